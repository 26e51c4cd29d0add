// wq_launch.h -- host-side launchers of the libwq kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// ---- repack / unpack (wq_unpack.hip) ----
hipError_t launch_repack_tiled(const uint32_t *packed, const uint16_t *scales, int64_t N,
                               int64_t K, int b, bool per_channel, void *out, hipStream_t stream);
hipError_t launch_unpack(const void *W, bool tiled, const uint16_t *scales_unused, int64_t N,
                         int64_t K, int b, uint8_t *codes, hipStream_t stream);

// Every workspace starts with this many bytes of counters that must be zero
// before a call and are zero again after it (whatever the op or shape), so
// one workspace can serve any sequence of stream-ordered calls.  Scratch that
// need not start at zero follows at kWsScratchOffset.
constexpr int64_t kWsCounterBytes = 65536;
constexpr int kWsMaxCounters = (int)(kWsCounterBytes / 4);
constexpr int64_t kWsScratchOffset = kWsCounterBytes;

// ---- grouped (mixture-of-experts) launches ----
// One launch covers several experts: entry i is expert e[i] with rows
// [m0[i], m0[i] + me[i]) of A and Y.  Passed by value as a kernel argument
// (the host knows the offsets), so nothing is allocated or copied.  The
// decode kernel takes one entry per expert with rows; the prefill kernel
// one entry per 256-row tile.
constexpr int kMaxGroups = 240;
struct NoGroups {
    static constexpr bool kGrouped = false;
};
struct GroupTable {
    static constexpr bool kGrouped = true;
    int n;                 // entries
    int per;               // decode: 64-row blocks per expert (grid blocks per entry)
    int64_t expert_bytes;  // stride of the expert blobs
    int e[kMaxGroups];
    int m0[kMaxGroups];
    int me[kMaxGroups];
};

// ---- decode path, M <= kDecodeMaxM (wq_decode.hip) ----
constexpr int kDecodeMaxM = 16;
constexpr int kDecodeMaxSplits = 16;  // K splits of the vector-ALU decode kernel

struct DecodePlan {
    int mt;         // rows of A handled per kernel instance (template M tile)
    int splits;     // K splits across workgroups (row kernel: waves sharing a row set)
    int gps;        // groups per split
    int waves;      // waves per workgroup (4, 8 or 16; 16 only for mt <= 4)
    int rowblocks;  // ceil(N / 64)
    int tstride;    // counters from one split-K ticket to the next (spreads them over cache lines)
    int rw;         // one row of A without a K split: rows per wave of the row kernel (8 or 4); 0 = split-K kernel
    int tmax;       // row kernel: load every slot at the start when a lane has at most tmax (2 or 3; 0 never)
    int reduce;     // K split summed by a second kernel (no tickets): 1, or 0 for the in-kernel hand-off
    int64_t ws_bytes;
};
// The row kernel stages a row of A in LDS, 272 bytes per group of 128:
// K <= 24576 keeps that within 52 KB.
constexpr int64_t kRowKernelMaxK = 24576;
// rows_ok: the one-row kernel may be chosen (not for grouped launches).
DecodePlan decode_plan(int64_t M, int64_t N, int64_t K, int b, bool rows_ok = true);

hipError_t launch_decode(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                         bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                         uint16_t *Y, void *ws, const DecodePlan &plan, hipStream_t stream);
// Sum of the split-K partials that the decode kernel stored at `part`
// (split s, row m, column n at (s * mt + m) * 64 * rowblocks + n), in split
// order, written to Y [M, N] as bf16.
hipError_t launch_decode_reduce(const float *part, int splits, int mt, int64_t M, int64_t N,
                                int rowblocks, uint16_t *Y, hipStream_t stream);
// Grouped decode: every entry of gt has at most kDecodeMaxM rows; the plan
// is decode_plan(max rows, entries * N, K, b) with rowblocks = entries *
// ceil(N / 64).  Tiled layout.
hipError_t launch_decode_grouped(const uint16_t *A, int64_t N, int64_t K, const void *W,
                                 const uint8_t *zeros, int b, uint16_t *Y, void *ws,
                                 const DecodePlan &plan, const GroupTable &gt,
                                 hipStream_t stream);

// ---- prefill path, M > kDecodeMaxM (wq_prefill.hip) ----
int64_t prefill_ws_bytes(int64_t M, int64_t N, int64_t K, int b);
hipError_t launch_prefill(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                          uint16_t *Y, void *ws, hipStream_t stream);

// ---- quantized embedding gather (wq_embed.hip) ----
hipError_t launch_embed(const void *W, const uint16_t *scales, const uint8_t *zeros,
                        bool per_channel, int64_t V, int64_t K, int b, const int64_t *ids,
                        int64_t T, uint16_t *Y, hipStream_t stream);

// Grouped prefill: one entry of gt per m-tile of tile_m rows
// (kPrefillTileM or kPrefillSmallTileM, one size per launch); no K split,
// no workspace.
constexpr int kPrefillTileM = 256;
constexpr int kPrefillSmallTileM = 64;
hipError_t launch_prefill_grouped(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                                  const void *W, const uint8_t *zeros, int b, uint16_t *Y,
                                  const GroupTable &gt, int tile_m, hipStream_t stream);

// ---- W4A8 (wq_a8.hip) ----
hipError_t launch_quant_act(const uint16_t *A, int64_t M, int64_t K, int8_t *Aq, float *sa,
                            hipStream_t stream);
int64_t a8_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_a8(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                          void *Y, bool out_f32, void *ws, hipStream_t stream);

}  // namespace wq
