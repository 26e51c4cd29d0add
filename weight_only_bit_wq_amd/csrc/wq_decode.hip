// wq_decode.hip -- decode-path planning and dispatch over b (the kernels are
// instantiated one bit width per translation unit, wq_decode_b<b>.hip).
#include "wq_launch.h"
#include "wq_device.h"

#include <algorithm>
#include <cstdlib>

namespace wq {

constexpr int kGroupSize = 128;
constexpr int kRowWaves = 4;  // waves per workgroup of the row kernel
constexpr int kRowsUpfrontGroups = 64;  // the row kernel's up-front form (kRowUpfrontMaxG)

template <int B, class GT>
hipError_t decode_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                    bool tiled, const uint16_t *scales, const uint8_t *zeros, uint16_t *Y,
                    void *ws, const DecodePlan &p, const GT &gt, hipStream_t stream);
extern template hipError_t decode_b<2, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<2, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);
extern template hipError_t decode_b<3, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<3, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);
extern template hipError_t decode_b<4, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<4, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);
extern template hipError_t decode_b<5, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<5, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);
extern template hipError_t decode_b<6, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<6, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);
extern template hipError_t decode_b<7, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<7, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);
extern template hipError_t decode_b<8, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const NoGroups &, hipStream_t);
extern template hipError_t decode_b<8, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t, const void *, bool, const uint16_t *, const uint8_t *, uint16_t *, void *, const DecodePlan &, const GroupTable &, hipStream_t);

static int decode_mt(int64_t M) {
    if (M <= 1) return 1;
    if (M <= 4) return 4;
    if (M <= 8) return 8;
    return 16;
}

// The one-row kernel's shape: rows per wave (8, or 4; 0 takes the split-K
// kernel) and the waves of a workgroup that share those rows' groups (1, 2
// or 4).  8 rows per wave, and the fewest sharing waves that give at least
// 3072 waves (three per SIMD: each wave then walks a few slots) and at most
// two slots per lane where 4 waves allow it (measured on MI355X at K 5120 ->
// N 17408: loading both slots at the start beat a slot-ahead ring by 2-5%);
// 4 rows per wave if 8 leave fewer than 8 groups per lane class; the
// split-K kernel for small layers with more than 64 groups (see below) and
// K beyond what the row kernel stages.  WQ_DECODE_ROWS (0, 4 or 8),
// WQ_DECODE_ROW_WAVES (1, 2, 4) and WQ_DECODE_ROW_TMAX (0, 2, 3: slots per
// lane loaded at the start) force a choice.
static void decode_rows_shape(int64_t M, int64_t N, int64_t K, int &rw, int &s) {
    rw = 0;
    s = 1;
    if (M != 1 || K > kRowKernelMaxK) return;
    const int G = (int)(K / kGroupSize);
    // The row kernel whenever it loads all of a lane's slots up front (at
    // most kRowsUpfrontGroups groups) or the layer has at least 1024 waves of
    // 4 rows; the split-K kernel keeps smaller layers with longer rows.
    // Measured at b = 6, alternating on one box: K 5120 -> N 256 / 1088 /
    // 2176 3.7 / 4.1 / 5.4 us against 6.2 / 7.1 / 7.3 (split-K), K 3840 ->
    // N 3200 4.5 against 8.2; with more groups the row kernel walks its
    // slots one ahead and was slower at K 10240 -> N 2560 (8.2 against 7.0)
    // and K 17408 -> N 1088 / 3200, faster only at K 17408 -> N 2176.
    rw = (G <= kRowsUpfrontGroups || (N + 3) / 4 >= 1024) ? (G >= 8 ? 8 : 4) : 0;
    if (const char *e = std::getenv("WQ_DECODE_ROWS")) {
        const int f = std::atoi(e);
        rw = f == 4 || f == 8 ? f : 0;
    }
    if (!rw) return;
    const int C = 64 / rw;
    const int64_t sets = (N + rw - 1) / rw;
    while (s < 4 && sets * s < 3072 && G >= C * s * 2) s *= 2;
    // More sharing waves while a lane would have over two slots: with at
    // most two, every slot is loaded at the start.
    while (s < 4 && G > 2 * C * s) s *= 2;
    if (const char *e = std::getenv("WQ_DECODE_ROW_WAVES")) {
        const int f = std::atoi(e);
        if (f == 1 || f == 2 || f == 4) s = f;
    }
}

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int b, bool rows_ok) {
    DecodePlan p{};
    const int G = (int)(K / kGroupSize);
    p.mt = decode_mt(M);
    p.rowblocks = (int)((N + 63) / 64);
    int rs = 1;
    if (rows_ok) decode_rows_shape(M, N, K, p.rw, rs);
    if (p.rw) {
        p.tmax = 3;
        if (const char *e = std::getenv("WQ_DECODE_ROW_TMAX")) p.tmax = std::atoi(e);
        p.splits = rs;  // waves of a workgroup sharing a row set's groups
        p.gps = G;
        p.waves = kRowWaves;
        p.tstride = 1;
        p.ws_bytes = 0;
        return p;
    }
    // Measured on MI355X (K 5120 -> N 17408 and K 17408 -> N 5120): with
    // many 64-row blocks, 8 waves per workgroup and one group per wave (K
    // split in chunks of 8 groups); with fewer than 192 row blocks, K split
    // so that ~240 workgroups are in flight, 16 waves for one row of A and 8
    // for the matrix-core row tiles (a sweep of 4/8/16 waves and 2..16 splits
    // at M = 4, 8, 16 found these plans best or within noise of it).
    int waves, splits;
    if (p.rowblocks >= 192) {
        // 16-row tiles up to b = 6: 4 waves of two groups each.  Measured
        // at K 5120 -> N 17408, M = 9, 12, 16, alternating on one box: b = 6
        // ~1.0 us faster, b = 5 0.1-0.3 us; b = 7 0.1-0.2 us slower.
        waves = (p.mt == 16 && b <= 6) ? 4 : 8;
        splits = (G + 7) / 8;
    } else {
        waves = p.mt == 1 ? 16 : 8;
        splits = std::max(1, std::min(G / waves, (240 + p.rowblocks - 1) / p.rowblocks));
    }
    if (const char *e = std::getenv("WQ_DECODE_WAVES")) waves = std::atoi(e);
    if (const char *e = std::getenv("WQ_DECODE_SPLITS")) splits = std::max(1, std::atoi(e));
    if (!(waves == 4 || waves == 8 || (waves == 16 && p.mt <= 4)))
        waves = 4;
    // One ticket per (row block, storing wave).
    if ((int64_t)p.rowblocks * std::min(waves, p.mt) > kWsMaxCounters) splits = 1;
    splits = std::min(std::min(splits, G), kDecodeMaxSplits);
    p.waves = waves;
    // Tickets 32 counters (one 128-byte line) apart where the counter region
    // allows: packed together, the tickets of neighbouring row blocks share a
    // line and their device-scope atomics queue behind each other.
    const int64_t tickets = (int64_t)p.rowblocks * std::min(waves, p.mt);
    p.tstride = 1;
    while (p.tstride < 32 && tickets * p.tstride * 2 <= kWsMaxCounters) p.tstride *= 2;
    p.gps = (G + splits - 1) / splits;
    p.splits = (G + p.gps - 1) / p.gps;
    // Row tiles of 8 and 16 with a K split store their partials and leave;
    // a second kernel adds them.  Measured on MI355X at K 5120 -> N 17408,
    // b = 5, 6, 7: 1.2-2.6 us faster per call at M = 16 than the in-kernel
    // hand-off (whose last workgroup per row block waits out a store, a
    // ticket and a load round trip), and up to 1.5 us slower at M = 4,
    // where the second launch costs more than the hand-off it saves.
    // Grouped launches (rows_ok false) keep the hand-off.  WQ_DECODE_REDUCE
    // (0 or 1) forces the choice for non-grouped launches.
    p.reduce = rows_ok && p.splits > 1 && p.mt >= 8;
    if (const char *e = std::getenv("WQ_DECODE_REDUCE"))
        p.reduce = rows_ok && p.splits > 1 && std::atoi(e) != 0;
    if (p.splits > 1)
        p.ws_bytes = kWsScratchOffset + (int64_t)p.splits * p.mt * p.rowblocks * 64 * 4;
    else
        p.ws_bytes = 0;
    return p;
}

hipError_t launch_decode(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                         bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                         uint16_t *Y, void *ws, const DecodePlan &p, hipStream_t stream) {
    switch (b) {
        case 2: return decode_b<2>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
        case 3: return decode_b<3>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
        case 4: return decode_b<4>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
        case 5: return decode_b<5>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
        case 6: return decode_b<6>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
        case 7: return decode_b<7>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
        case 8: return decode_b<8>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, NoGroups{}, stream);
    }
    return hipErrorInvalidValue;
}

// One thread per 4 consecutive columns of one row: the splits' float4s
// added in split order (the order and rounding of the in-kernel hand-off),
// rounded to bf16 once.  All loads go out before the first add (indices
// past the last split repeat it and are not added).  At M = 16 on the
// 5120 -> 17408 layer the kernel takes ~4 us (5.6 MB read by one workgroup
// per compute unit: about one launch and one memory round trip).
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float *__restrict__ part,
                                                            int splits, int mt, int M, int N,
                                                            int npad, uint16_t *__restrict__ Y) {
    const int64_t q = npad / 4;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int m = (int)(t / q);
    const int64_t n = (t - (int64_t)m * q) * 4;
    if (m >= M || n >= N) return;
    const float4 *p = reinterpret_cast<const float4 *>(part + (int64_t)m * npad + n);
    const int64_t step = (int64_t)mt * q;  // float4s from one split to the next
    float4 v[kDecodeMaxSplits];
#pragma unroll
    for (int s = 0; s < kDecodeMaxSplits; ++s) v[s] = p[min(s, splits - 1) * step];
    float4 acc = v[0];
#pragma unroll
    for (int s = 1; s < kDecodeMaxSplits; ++s) {
        if (s < splits) {
            acc.x += v[s].x;
            acc.y += v[s].y;
            acc.z += v[s].z;
            acc.w += v[s].w;
        }
    }
    uint16_t *y = Y + (int64_t)m * N + n;
    y[0] = f32_to_bf16_rne(acc.x);
    if (n + 1 < N) y[1] = f32_to_bf16_rne(acc.y);
    if (n + 2 < N) y[2] = f32_to_bf16_rne(acc.z);
    if (n + 3 < N) y[3] = f32_to_bf16_rne(acc.w);
}

hipError_t launch_decode_reduce(const float *part, int splits, int mt, int64_t M, int64_t N,
                                int rowblocks, uint16_t *Y, hipStream_t stream) {
    const int npad = rowblocks * 64;
    const int64_t threads = M * (npad / 4);
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, stream, part, splits, mt, (int)M, (int)N, npad, Y);
    return hipGetLastError();
}

hipError_t launch_decode_grouped(const uint16_t *A, int64_t N, int64_t K, const void *W,
                                 const uint8_t *zeros, int b, uint16_t *Y, void *ws,
                                 const DecodePlan &p, const GroupTable &gt, hipStream_t stream) {
    switch (b) {
        case 2: return decode_b<2>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
        case 3: return decode_b<3>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
        case 4: return decode_b<4>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
        case 5: return decode_b<5>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
        case 6: return decode_b<6>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
        case 7: return decode_b<7>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
        case 8: return decode_b<8>(A, 0, N, K, W, true, nullptr, zeros, Y, ws, p, gt, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
