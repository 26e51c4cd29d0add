// wq_decode_mfma.hip -- WNA16 skinny GEMM on the matrix cores (2 <= M <= 16).
//
// Decode-shape batches are bound by the weight stream ("vLLM Quantization",
// Key points: decode waits on memory), but with several activation rows the
// per-row dot products outgrow the vector ALUs.  Here the product runs on
// v_mfma_f32_16x16x32_bf16 with the activations (M rows, zero-padded to 16)
// as the A operand and 16 weight rows as the B operand.
//
// Work split.  A workgroup owns 16 * RB weight rows and a range of groups;
// its KS waves take contiguous sub-ranges and are reduced through LDS at the
// end.  Per group a wave
//   1. copies its rows' slots (b 16-byte chunks per row) into a private LDS
//      buffer with coalesced 16-byte loads (prefetched one group ahead);
//   2. reads back, per lane, one quarter slot (32 codes = B dwords) of one
//      row: lane l takes row l % 16 of each 16-row block and quarter l / 16,
//      which is the B-operand layout (column n = l % 16, k-chunk l / 16);
//   3. unpacks the quarter to 16 bf16 pairs (128 + c, exact) and runs 4
//      MFMAs per 16-row block (k = 32 q + 8 s + t for step s, lane chunk q);
//      the activations use the same k order;
//   4. folds tot += s[n, g] * (P + Q) in fp32, where Q is the group's offset
//      term -(128 + 2^(b-1)) * sum_k a[m, k], made by 4 more MFMAs with a
//      constant B operand, so no code or scale is rounded.
// The RB + 1 accumulation chains of a group are interleaved so that no MFMA
// waits on the one before it.  K can also be split across workgroups; the
// last split of a row block adds the partials in split order.
#include <algorithm>
#include <cstdlib>

#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

// Bytes of dynamic LDS per wave: the staged slots of 16 * RB rows, or the
// wave's partial sums (RB blocks of 64 lanes x 4 floats) at the end.
constexpr int kMaxMfmaSplits = 16;

__host__ __device__ constexpr int mfma_wave_lds(int b, int rb) {
    return (rb * 16 * b * 16 > rb * 1024) ? rb * 16 * b * 16 : rb * 1024;
}

template <int B, class WL, int RB>
__global__ __launch_bounds__(256) void decode_mfma_kernel(const uint16_t *__restrict__ A, int M,
                                                          int N, int K, WL wl,
                                                          uint16_t *__restrict__ Y,
                                                          float *__restrict__ part,
                                                          unsigned *__restrict__ counters,
                                                          int splits) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    __shared__ unsigned ticket_sh;
    constexpr int kRows = 16 * RB;             // weight rows per workgroup
    constexpr int kChunks = kRows * B;         // 16-byte chunks per group
    constexpr int kLoads = (kChunks + 63) / 64;
    constexpr int kSlotDw = 4 * B;             // dwords per row slot

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = blockDim.x >> 6;
    const int G = K / kGroup;
    // Workgroup (row block R, K split sp); the splits of a row block are
    // adjacent in launch order.
    const int R = blockIdx.x / splits;
    const int sp = blockIdx.x - R * splits;
    const int64_t n0 = (int64_t)R * kRows;
    uint32_t *stage = reinterpret_cast<uint32_t *>(dyn_lds + w * mfma_wave_lds(B, RB));

    const int r = lane & 15;
    const int q = lane >> 4;

    // ---- 1. coalesced copy of the group's slots: chunk c of kChunks ----
    // Tiled: plane-major (c = plane * kRows + row), contiguous per plane.
    // Dense: row-major (c = row * B + plane), contiguous per row slot.
    int64_t goff[kLoads];  // byte offset of the chunk for group 0
    int soff[kLoads];      // its LDS dword offset (row-major slots)
    bool cok[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int c = lane + 64 * i;
        cok[i] = c < kChunks;
        const int cc = cok[i] ? c : 0;
        int row, plane;
        if constexpr (WL::kTiled) {
            row = cc % kRows;
            plane = cc / kRows;
        } else {
            row = cc / B;
            plane = cc % B;
        }
        const int64_t n = min(n0 + row, (int64_t)N - 1);
        goff[i] = (int64_t)(wl.slot0(n) - wl.slot0(0)) + plane * (WL::kTiled ? 1024 : 16);
        soff[i] = row * kSlotDw + 4 * plane;
    }
    const uint8_t *wbase = wl.slot0(0);
    const int64_t gstep = wl.slot_step();

    // Activations: lane row m = l % 16 (clamped), chunk q.
    const int m = min(r, M - 1);
    const uint16_t *arow = A + (int64_t)m * K + 32 * q;
    // Scales of this lane's rows.
    const uint8_t *sc0[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) sc0[t] = wl.scale0(min(n0 + 16 * t + r, (int64_t)N - 1));
    const int64_t sstep = wl.scale_step();

    // Everything a group needs is fetched one group ahead.
    u32x4 gbuf[kLoads], anext[4];
    uint16_t snext[RB];
    auto fetch = [&](int g) __attribute__((always_inline)) {
        const uint8_t *p = wbase + (int64_t)g * gstep;
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            gbuf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + goff[i]));
#pragma unroll
        for (int s = 0; s < 4; ++s)
            anext[s] = *reinterpret_cast<const u32x4 *>(arow + g * kGroup + 8 * s);
#pragma unroll
        for (int t = 0; t < RB; ++t)
            snext[t] = *reinterpret_cast<const uint16_t *>(sc0[t] + (int64_t)g * sstep);
    };

    const uint32_t mask = __builtin_amdgcn_readfirstlane(pair_mask<B < 8 ? B : 7>());
    const uint32_t magic = in_vgpr(kBf16Magic128x2);
    // -(128 + 2^(b-1)) (b = 8: -128) as a bf16 pair, exact.
    constexpr float kOff = (B == 8) ? 128.0f : (float)(128 + (1 << (B - 1)));
    const uint32_t negoff = (uint32_t)f32_to_bf16_rne(-kOff) * 0x00010001u;
    const bf16x8_t negoff8 = __builtin_bit_cast(bf16x8_t, u32x4{negoff, negoff, negoff, negoff});

    f32x4_t tot[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) tot[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Groups of this split, then of this wave.
    const int gs0 = (int)(((int64_t)G * sp) / splits);
    const int gs1 = (int)(((int64_t)G * (sp + 1)) / splits);
    const int g0 = gs0 + (int)(((int64_t)(gs1 - gs0) * w) / KS);
    const int g1 = gs0 + (int)(((int64_t)(gs1 - gs0) * (w + 1)) / KS);
    if (g0 < g1) fetch(g0);
    for (int g = g0; g < g1; ++g) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            if (cok[i]) *reinterpret_cast<u32x4 *>(stage + soff[i]) = gbuf[i];
        u32x4 areg[4];
        float sc[RB];
#pragma unroll
        for (int s = 0; s < 4; ++s) areg[s] = anext[s];
#pragma unroll
        for (int t = 0; t < RB; ++t) sc[t] = bf16_to_f32(snext[t]);
        if (g + 1 < g1) fetch(g + 1);
        // This lane's quarters, read back before any MFMA of the group is
        // issued.  (Issued after the dependent offset-term chain below, the
        // LDS returns could be allocated to that chain's accumulator
        // registers while it is still in flight; on the device that raced
        // and corrupted the codes.)
        uint32_t cw[RB][B];
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const uint32_t *src = stage + (16 * t + r) * kSlotDw + q * B;
#pragma unroll
            for (int e = 0; e < B; ++e) cw[t][e] = src[e];
        }
        __builtin_amdgcn_sched_barrier(0);
        // RB + 1 independent accumulation chains, interleaved (step s
        // outer): the blocks' codes, and the group's offset term (constant B
        // operand) shared by every block.  No MFMA depends on the one just
        // before it.
        uint32_t pr[RB][16];
#pragma unroll
        for (int t = 0; t < RB; ++t) QuarterPairs<B, 0>::run(cw[t], mask, magic, pr[t]);
        f32x4_t P[RB], Q = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < RB; ++t) P[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, areg[s]);
#pragma unroll
            for (int t = 0; t < RB; ++t)
                P[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a,
                    __builtin_bit_cast(bf16x8_t, u32x4{pr[t][4 * s], pr[t][4 * s + 1],
                                                       pr[t][4 * s + 2], pr[t][4 * s + 3]}),
                    P[t], 0, 0, 0);
            Q = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, negoff8, Q, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < RB; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[t][i] = fmaf(sc[t], P[t][i] + Q[i], tot[t][i]);
    }

    // ---- reduce the KS waves' partial sums through LDS ----
    __syncthreads();  // every wave is done with its staging buffer
    f32x4_t *red = reinterpret_cast<f32x4_t *>(dyn_lds + w * mfma_wave_lds(B, RB));
#pragma unroll
    for (int t = 0; t < RB; ++t) red[t * 64 + lane] = tot[t];
    __syncthreads();
    // D layout: lane l holds column n = l % 16, rows 4 (l / 16) + i.
    const int64_t Npad = (int64_t)(gridDim.x / splits) * kRows;
    for (int t = w; t < RB; t += KS) {
        f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int v = 0; v < KS; ++v)
            acc += reinterpret_cast<const f32x4_t *>(dyn_lds + v * mfma_wave_lds(B, RB))[t * 64 + lane];
        const int64_t n = n0 + 16 * t + r;
        if (splits == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mo = 4 * q + i;
                if (mo < M && n < N) Y[(int64_t)mo * N + n] = f32_to_bf16_rne(acc[i]);
            }
        } else {
            // Partials move through device-scope relaxed atomics (coherent
            // across the XCDs' L2s without an L2 write-back/invalidate).
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * q + i < M)
                    __hip_atomic_store(&part[((int64_t)sp * 16 + 4 * q + i) * Npad + n], acc[i],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (splits == 1) return;
    wait_vm_stores();
    __syncthreads();  // every wave's partial stores have completed
    if (threadIdx.x == 0)
        ticket_sh = __hip_atomic_fetch_add(&counters[R], 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket_sh != (unsigned)(splits - 1)) return;
    // Last split of the row block: add the partials in split order.  All of
    // an output's loads are issued before its adds (they are independent).
    for (int e = threadIdx.x; e < M * kRows; e += blockDim.x) {
        const int mo = e / kRows;
        const int64_t n = n0 + (e - mo * kRows);
        if (n >= N) continue;
        float v[kMaxMfmaSplits];
#pragma unroll
        for (int t = 0; t < kMaxMfmaSplits; ++t)
            v[t] = t < splits ? __hip_atomic_load(&part[((int64_t)t * 16 + mo) * Npad + n],
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : 0.0f;
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < kMaxMfmaSplits; ++t)
            if (t < splits) sum += v[t];
        Y[(int64_t)mo * N + n] = f32_to_bf16_rne(sum);
    }
    if (threadIdx.x == 0)  // leave the counter region zero
        __hip_atomic_store(&counters[R], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int B, int RB>
hipError_t launch_rb(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                     bool tiled, const uint16_t *scales, uint16_t *Y, void *ws,
                     const MfmaDecodePlan &p, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int64_t rowblocks = (N + 16 * RB - 1) / (16 * RB);
    const dim3 grid((unsigned)(rowblocks * p.splits));
    const dim3 block((unsigned)(64 * p.ks));
    const size_t lds = (size_t)p.ks * mfma_wave_lds(B, RB);
    float *part = nullptr;
    unsigned *counters = nullptr;
    if (p.splits > 1) {
        counters = static_cast<unsigned *>(ws);
        part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    }
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((decode_mfma_kernel<B, TiledW, RB>), grid, block, lds, stream, A,
                           (int)M, (int)N, (int)K, wl, Y, part, counters, p.splits);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((decode_mfma_kernel<B, DenseW, RB>), grid, block, lds, stream, A,
                           (int)M, (int)N, (int)K, wl, Y, part, counters, p.splits);
    }
    return hipGetLastError();
}

template <int B>
hipError_t launch_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W, bool tiled,
                    const uint16_t *scales, uint16_t *Y, void *ws, const MfmaDecodePlan &p,
                    hipStream_t stream) {
    switch (p.rb) {
        case 4: return launch_rb<B, 4>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 2: return launch_rb<B, 2>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        default: return launch_rb<B, 1>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
    }
}

}  // namespace

// 32-row blocks (RB = 2: 109-120 VGPRs, four waves per SIMD; RB = 4 needs
// 167-184, two per SIMD, and RB = 1 reloads the activations for every 16
// rows); K splits across workgroups only up to about 512 workgroups (the
// 5120 -> 17408 layer then runs unsplit, without a hand-off), with at least
// 4 groups each; 4 waves per workgroup with at least 2 groups each.
// Measured on the 5120 x 17408 and 17408 x 5120 layers (b = 6, M = 8 and
// 16) against RB = 1 and 4, 768 to 4096 workgroups and 1, 2 or 8 waves:
// 10-16% faster than 64-row blocks at 1024 workgroups of 2 waves.
// WQ_DMFMA_RB, WQ_DMFMA_TARGET_WGS and WQ_DMFMA_KS override the three
// choices.  Row blocks beyond the counter region fall back to one split.
MfmaDecodePlan decode_mfma_plan(int64_t, int64_t N, int64_t K, int) {
    MfmaDecodePlan p;
    static const int rb_env = [] {
        const char *e = std::getenv("WQ_DMFMA_RB");
        const int v = e ? std::atoi(e) : 2;
        return (v == 1 || v == 4) ? v : 2;
    }();
    p.rb = rb_env;
    const int64_t rowblocks = (N + 16 * p.rb - 1) / (16 * p.rb);
    const int G = (int)(K / kGroup);
    static const int target = [] {
        const char *e = std::getenv("WQ_DMFMA_TARGET_WGS");
        return e ? std::atoi(e) : 512;
    }();
    int64_t splits = (target + rowblocks - 1) / rowblocks;
    splits = std::min<int64_t>(splits, std::max(1, G / 4));
    splits = std::min<int64_t>(splits, kMaxMfmaSplits);
    if (rowblocks > kWsMaxCounters) splits = 1;
    p.splits = (int)std::max<int64_t>(1, splits);
    const int gps = (G + p.splits - 1) / p.splits;
    static const int ks_max = [] {
        const char *e = std::getenv("WQ_DMFMA_KS");
        return e ? std::atoi(e) : 4;
    }();
    p.ks = std::max(1, std::min(std::min(ks_max, 4), gps / 2));
    p.ws_bytes = kWsScratchOffset +
                 (p.splits > 1 ? (int64_t)p.splits * 16 * rowblocks * 16 * p.rb * 4 : 0);
    return p;
}

hipError_t launch_decode_mfma(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                              bool tiled, const uint16_t *scales, int b, uint16_t *Y, void *ws,
                              const MfmaDecodePlan &p, hipStream_t stream) {
    switch (b) {
        case 2: return launch_b<2>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 3: return launch_b<3>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 4: return launch_b<4>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 5: return launch_b<5>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 6: return launch_b<6>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 7: return launch_b<7>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
        case 8: return launch_b<8>(A, M, N, K, W, tiled, scales, Y, ws, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
