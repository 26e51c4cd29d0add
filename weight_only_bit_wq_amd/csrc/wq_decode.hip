// wq_decode.hip -- decode-path planning and dispatch over b (the kernels are
// instantiated one bit width per translation unit, wq_decode_b<b>.hip).
#include "wq_launch.h"

#include <algorithm>
#include <cstdlib>

namespace wq {

constexpr int kGroupSize = 128;

template <int B>
hipError_t decode_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                    bool tiled, const uint16_t *scales, uint16_t *Y, void *ws,
                    const DecodePlan &p, hipStream_t stream);
extern template hipError_t decode_b<2>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);
extern template hipError_t decode_b<3>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);
extern template hipError_t decode_b<4>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);
extern template hipError_t decode_b<5>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);
extern template hipError_t decode_b<6>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);
extern template hipError_t decode_b<7>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);
extern template hipError_t decode_b<8>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, uint16_t *, void *, const DecodePlan &, hipStream_t);

static int decode_mt(int64_t M) {
    if (M <= 1) return 1;
    if (M <= 2) return 2;
    if (M <= 4) return 4;
    if (M <= 8) return 8;
    return 16;
}

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int b) {
    (void)b;
    DecodePlan p{};
    const int G = (int)(K / kGroupSize);
    p.mt = decode_mt(M);
    p.rowblocks = (int)((N + 63) / 64);
    // Groups per split: a multiple of the 4 waves, two groups per wave by
    // default (enough workgroups to fill 256 CUs at the layer shapes used
    // here).  Row counts beyond the counter region run without splitting.
    int gps = 8;
    if (const char *e = std::getenv("WQ_DECODE_GPS")) gps = std::max(1, std::atoi(e));
    gps = std::min(gps, G);
    if (p.rowblocks > kWsMaxCounters) gps = G;
    p.gps = gps;
    p.splits = (G + gps - 1) / gps;
    if (p.splits > 1)
        p.ws_bytes = kWsScratchOffset + (int64_t)p.splits * p.mt * p.rowblocks * 64 * 4;
    else
        p.ws_bytes = 0;
    return p;
}

hipError_t launch_decode(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                         bool tiled, const uint16_t *scales, int b, uint16_t *Y, void *ws,
                         const DecodePlan &p, hipStream_t stream) {
    switch (b) {
        case 2: return decode_b<2>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 3: return decode_b<3>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 4: return decode_b<4>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 5: return decode_b<5>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 6: return decode_b<6>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 7: return decode_b<7>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 8: return decode_b<8>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
