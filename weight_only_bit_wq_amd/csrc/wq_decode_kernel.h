// wq_decode_kernel.h -- WNA16 decode path (M <= 16): HBM-bound skinny GEMM.
//
// Small batches only read weights ("vLLM Quantization", Key points: at small
// batch decode waits on memory, so shrinking weights speeds it up).  The
// kernel is built so that the packed weights are read exactly once, with
// 128-bit loads, and everything else hides under that stream.
//
// Work decomposition
//   - A lane owns one output row n and, in turn, whole groups (row, g): the
//     b 16-byte chunks of a group (128 codes) are loaded into 4b VGPRs and
//     unpacked in registers.  In the tiled layout the 64 lanes of a wave read
//     one 1 KB plane per load instruction.
//   - All lanes of a wave work on the same group g.  With one row of A the
//     128 activations of that group are wave-uniform: they are read with
//     scalar loads and fed to v_dot2_f32_bf16 as its SGPR operand.  With 2..16
//     rows (padded to a row tile MT of 4, 8 or 16) the products run on the
//     matrix cores as 4x4x4 blocks that keep a lane on its row (see the
//     matrix-core group terms below).
//   - A workgroup (W waves) covers 64 rows and `gps` consecutive groups, the
//     waves interleaving groups; `splits` workgroups share one 64-row block.
//     Many small workgroups (rather than one per compute unit) let the
//     dispatcher balance the stream: a compute unit whose loads come back
//     early simply takes more workgroups.
//   - Split K hands off through the workspace: after the waves' sums meet in
//     LDS, only the waves that own output rows stay; each stores its fp32
//     partials and takes a ticket per (block, wave); the last of the splits
//     adds them in split order (deterministic), writes bf16 and resets the
//     ticket (in the workspace's counter region) to zero.  Row tiles of 8
//     and 16 (plan.reduce) only store their partials, and a second kernel
//     adds them in the same order: no ticket, and no workgroup waits out
//     the store, ticket and load round trips at the end.
//
// Arithmetic: the codes of a slot are turned into exact signed values
// q = c - 2^(b-1) (bf16 pairs, see wq_device.h: one XOR per word, a
// sign-extending extract and an int -> float conversion per code, one pack
// per pair), multiplied by the activations with fp32 accumulation
// (v_dot2_f32_bf16 at one row, 4x4x4 matrix-core blocks at 2..16 rows), and
// the group scale applied once per group in fp32:
//     acc += s[n,g] * sum_{k in g} a_k * q_k
// Every product is exact, so the rounding error is bounded by the sum of
// |a * w| of the row's own terms (a row of midpoint codes gives exactly 0).
// Zero points (b = 4 and 8 only) replace 2^(b-1) by z: q = c - z, exact too
// (|c - z| <= 255).
#pragma once

#include "wq_device.h"
#include "wq_launch.h"

namespace wq {


template <int N_>
struct UVec;
template <>
struct UVec<4> { typedef unsigned type __attribute__((ext_vector_type(4))); };
template <>
struct UVec<8> { typedef unsigned type __attribute__((ext_vector_type(8))); };
template <>
struct UVec<16> { typedef unsigned type __attribute__((ext_vector_type(16))); };

// Pairs P0 + I .. P0 + CP - 1 of the slot against the activation pairs in
// av (CP pairs of the one row come in with one wide scalar load).  Pair p
// of the slot is pair p % 16 of its 32-code quarter p / 16.
template <int B, int CP, int P0, int I, bool ZP, bool I8>
struct DotChunk {
    typedef typename UVec<CP>::type vec;
    __device__ __forceinline__ static void run(const uint32_t *w, const uint32_t *o,
                                               const vec &av, int z, float &d) {
        constexpr int P = P0 + I;
        d = dot2_bf16(av[I], slot_pair<B, P, ZP, I8>(w, o, z), d);
        DotChunk<B, CP, P0, I + 1, ZP, I8>::run(w, o, av, z, d);
    }
};
template <int B, int CP, int P0, bool ZP, bool I8>
struct DotChunk<B, CP, P0, CP, ZP, I8> {
    typedef typename UVec<CP>::type vec;
    __device__ __forceinline__ static void run(const uint32_t *, const uint32_t *, const vec &,
                                               int, float &) {}
};

// Everything a lane reads from memory for one (row, group) slot: its b
// chunks, its scale and (with zero points) its zero point.  A slot is
// loaded whole before the previous one is computed: the vector-memory
// counter retires in issue order, so a load issued after the next slot's
// prefetch would make the current slot wait for that prefetch.
template <int B, int MT>
struct SlotRegs {
    uint32_t w[4 * B];
    uint16_t s;
    uint32_t z;  // zero point (only with zero points)
};
template <int B, int MT, bool ZP, class WL>
__device__ __forceinline__ void load_slot_regs(const WL &wl, int64_t nr, int g,
                                               const uint8_t *zrow, SlotRegs<B, MT> &r) {
    load_slot<B>(wl.chunks(nr, g), wl.chunk_stride(), r.w);
    r.s = wl.scale(nr, g);
    if constexpr (ZP) r.z = zrow[g];
}

// One (row, group) slot of lane's row against group g of the one row of A:
//     x = sum_k a[k] q_k   (times 2^(8-b) for arranged runs, I8)
// (the caller applies the group scale).  `a` points at the group's first
// activation pair (read with scalar loads: wave-uniform).  The slot's
// words are prepared in place (prep_runs).
template <int B, bool ZP, bool I8>
__device__ __forceinline__ float group_terms(uint32_t *w, const uint32_t *a, int z) {
    uint32_t o[int8_words<B, ZP, I8>() ? 32 : 1];
    prep_runs<B, ZP, I8, 4>(w, o, z);
    // All 64 activation pairs of the group come in with four wide scalar
    // loads issued together.
    typedef typename UVec<16>::type vec16;
    vec16 av[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) av[c] = *reinterpret_cast<const vec16 *>(a + 16 * c);
    float d = 0.0f;
    DotChunk<B, 16, 0, 0, ZP, I8>::run(w, o, av[0], z, d);
    DotChunk<B, 16, 16, 0, ZP, I8>::run(w, o, av[1], z, d);
    DotChunk<B, 16, 32, 0, ZP, I8>::run(w, o, av[2], z, d);
    DotChunk<B, 16, 48, 0, ZP, I8>::run(w, o, av[3], z, d);
    return d;
}

// ---------------------------------------------------------------------------
// Matrix-core group terms, for row tiles MT = 4, 8, 16.
//
// v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products, one per
// block of 4 lanes: B column j of block i is lane 4i + j (4 consecutive k),
// and that lane receives the column's 4 outputs (one per A row).  With the
// broadcast control CBSZ = 4 all 16 blocks take their A operand (4 rows x 4
// k) from block ABID.  So lanes stay weight rows, exactly as in the
// vector-ALU form: a lane's unpacked code pairs 2j, 2j+1 are its B operand
// for k-step j (k = 4j .. 4j+3), and it gets its row's dot products with 4
// rows of A at once.  One 16-byte register per lane holds the activations of
// 4 rows for the whole group: lane 4i + r holds row r's k = 8i .. 8i+7, so
// k-step 2i + h is dwords 2h, 2h+1 of that register with ABID = i.  Rows of
// A come in sets of 4 (MT / 4 sets, one MFMA chain each).
// ---------------------------------------------------------------------------
typedef short bf16x4_bits __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <int B, int Q, int J, bool ZP, bool I8>
struct MfmaSteps {
    __device__ __forceinline__ static void run(const uint32_t *w, const uint32_t *o,
                                               const u32x4 *av, int z, f32x4_t *d) {
        // k-step J: codes 4J .. 4J+3, pairs 2J and 2J+1 of the slot (pair p
        // is pair p % 16 of quarter p / 16).
        constexpr int P0 = 2 * J, P1 = 2 * J + 1;
        u32x2_t wp;
        wp.x = slot_pair<B, P0, ZP, I8>(w, o, z);
        wp.y = slot_pair<B, P1, ZP, I8>(w, o, z);
        const bf16x4_bits bw = __builtin_bit_cast(bf16x4_bits, wp);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            u32x2_t a;
            a.x = av[q][2 * (J & 1)];
            a.y = av[q][2 * (J & 1) + 1];
            d[q] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4_bits, a), bw,
                                                          d[q], 4, J >> 1, 0);
        }
        MfmaSteps<B, Q, J + 1, ZP, I8>::run(w, o, av, z, d);
    }
};
template <int B, int Q, bool ZP, bool I8>
struct MfmaSteps<B, Q, 32, ZP, I8> {
    __device__ __forceinline__ static void run(const uint32_t *, const uint32_t *, const u32x4 *,
                                               int, f32x4_t *) {}
};

// Everything a lane reads for one (row, group) slot on the matrix-core form:
// its b chunks, its scale and its 16-byte activation register per set.
template <int B, int MT>
struct SlotRegsMf {
    uint32_t w[4 * B];
    u32x4 av[MT / 4];
    uint16_t s;
    uint32_t z;  // zero point (only with zero points)
};
template <int B, int MT, bool ZP, class WL>
__device__ __forceinline__ void load_slot_regs_mf(const WL &wl, int64_t nr, int g,
                                                  const uint32_t *A2, const int *arow_off,
                                                  int lane, const uint8_t *zrow,
                                                  SlotRegsMf<B, MT> &r) {
    load_slot<B>(wl.chunks(nr, g), wl.chunk_stride(), r.w);
    r.s = wl.scale(nr, g);
    if constexpr (ZP) r.z = zrow[g];
#pragma unroll
    for (int q = 0; q < MT / 4; ++q)
        r.av[q] = *reinterpret_cast<const u32x4 *>(A2 + (int64_t)g * 64 + arow_off[q]);
}

// x[m] = sum_k a[m,k] q_k for the lane's row and rows m = 0 .. MT-1 of A,
// as in group_terms; the caller applies the group scale.
template <int B, int MT, bool ZP, bool I8>
__device__ __forceinline__ void group_terms_mf(uint32_t *w, const u32x4 *av, int z, float *x) {
    constexpr int Q = MT / 4;
    uint32_t o[int8_words<B, ZP, I8>() ? 32 : 1];
    prep_runs<B, ZP, I8, 4>(w, o, z);
    f32x4_t d[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) d[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    MfmaSteps<B, Q, 0, ZP, I8>::run(w, o, av, z, d);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        x[4 * q + 0] = d[q][0];
        x[4 * q + 1] = d[q][1];
        x[4 * q + 2] = d[q][2];
        x[4 * q + 3] = d[q][3];
    }
}

// ---------------------------------------------------------------------------
// Row tile 16 on v_mfma_f32_16x16x32_bf16: a quarter of the matrix-core time
// of four 4x4x4 chains (measured: the 4x4x4 chains took ~3 us of a 24 us
// call at K 5120 -> N 17408).  The 16x16x32 block takes 16 weight rows,
// each spread over 4 lanes (k-quarters), while the loads leave every lane
// with its own row's whole slot; so each lane's exact code pairs move by 4x4
// transposes of the wave's 16-lane quarters (below).  For row block cb (rows
// 16 cb .. 16 cb + 15 of the wave's 64) and k-step t, lane (c, q) = (l % 16,
// l / 16) supplies pairs 16 t + 4 q .. + 3 (codes 32 t + 8 q .. + 7) of row
// 16 cb + c as its B operand, and the same 8 k of row c of A as its A
// operand, and receives rows 4 q .. 4 q + 3 of A against weight row
// 16 cb + c.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

// x_r <- quarter r of (x0, x1, x2, x3) taken across: afterwards quarter q of
// x_r holds what quarter r of x_q held (two v_permlane32_swap, then two
// v_permlane16_swap).
__device__ __forceinline__ void transpose_quarters(uint32_t &x0, uint32_t &x1, uint32_t &x2,
                                                   uint32_t &x3) {
    // Upper halves of x0, x1 <-> lower halves of x2, x3.
    const auto a = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
    // Odd quarters of the first <-> even quarters of the second.
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    x0 = c[0];
    x1 = c[1];
    x2 = d[0];
    x3 = d[1];
}

// x[4 cb + r] = sum_k a[4 q + r, k] q_k of weight row 16 cb + c (lane (c, q)),
// unscaled; av[t] holds the lane's 8 activations of k-step t.
template <int B, bool ZP, bool I8>
__device__ __forceinline__ void group_terms_mf16(uint32_t *w, const u32x4 *av, int z, float *x) {
    uint32_t o[int8_words<B, ZP, I8>() ? 32 : 1];
    prep_runs<B, ZP, I8, 4>(w, o, z);
    f32x4_t d[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) d[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    static_for<0, 4>([&](auto tc) __attribute__((always_inline)) {
        constexpr int T = decltype(tc)::value;
        uint32_t y[4][4];  // [pair i of the 8 codes][row block]
        static_for<0, 4>([&](auto ic) __attribute__((always_inline)) {
            constexpr int I = decltype(ic)::value;
            uint32_t x0 = slot_pair<B, 16 * T + 0 + I, ZP, I8>(w, o, z);
            uint32_t x1 = slot_pair<B, 16 * T + 4 + I, ZP, I8>(w, o, z);
            uint32_t x2 = slot_pair<B, 16 * T + 8 + I, ZP, I8>(w, o, z);
            uint32_t x3 = slot_pair<B, 16 * T + 12 + I, ZP, I8>(w, o, z);
            transpose_quarters(x0, x1, x2, x3);
            y[I][0] = x0;
            y[I][1] = x1;
            y[I][2] = x2;
            y[I][3] = x3;
        });
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            u32x4 bv;
            bv.x = y[0][cb];
            bv.y = y[1][cb];
            bv.z = y[2][cb];
            bv.w = y[3][cb];
            d[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, av[T]),
                                                            __builtin_bit_cast(bf16x8_v, bv),
                                                            d[cb], 0, 0, 0);
        }
    });
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[4 * cb + r] = d[cb][r];
}

// The lane's own row scale as seen by lane (c, q) for rows 16 cb + c.
__device__ __forceinline__ void row_block_scales(float sc, float *out) {
    uint32_t x0 = __float_as_uint(sc), x1 = x0, x2 = x0, x3 = x0;
    transpose_quarters(x0, x1, x2, x3);
    out[0] = __uint_as_float(x0);
    out[1] = __uint_as_float(x1);
    out[2] = __uint_as_float(x2);
    out[3] = __uint_as_float(x3);
}

// ONE: every wave has at most one group (gps <= W, the plan for large
// layers): no prefetch register set, so more waves fit per SIMD.  Used for
// the matrix-core row tiles; with one row of A the prefetching form measured
// 3.5% faster even then, so it keeps that one.
// GT: NoGroups, or a GroupTable (one entry per expert; the grid's 64-row
// blocks run entry by entry, and each workgroup rebases A, Y, the weights
// and the zero points to its expert).
template <int B, int MT, int W, class WL, bool ONE, bool ZP, class GT>
__global__ __launch_bounds__(64 * W) void decode_kernel(const uint16_t *__restrict__ A, int M,
                                                        int N, int K, WL wl,
                                                        const uint8_t *__restrict__ zeros,
                                                        uint16_t *__restrict__ Y,
                                                        float *__restrict__ part,
                                                        unsigned *__restrict__ counters,
                                                        int splits, int gps, int tstride,
                                                        const GT gt) {
    static_assert(W * MT <= 128, "LDS reduction table");
    static_assert(MT == 1 || MT % 4 == 0, "row tiles above 1 take the matrix-core form");
    constexpr bool MF = MT >= 4;
    constexpr bool MF16 = MT == 16;  // 16x16x32 blocks (4x4x4 below)
    constexpr bool I8 = WL::kTiled && int8_ready<B>() && !ZP;  // arranged runs
    constexpr float kSInv = operand_scale_inv<B, I8, ZP>();
    __shared__ float red[W][MT][64];

    const int G = K / kGroup;
    const int RB = blockIdx.x / splits;  // 64-row block of the grid (tickets, partials)
    const int s = blockIdx.x - RB * splits;
    int R = RB;  // 64-row block within the weights
    if constexpr (GT::kGrouped) {
        const int gi = RB / gt.per;
        R = RB - gi * gt.per;
        const int e = gt.e[gi];
        A += (int64_t)gt.m0[gi] * K;
        Y += (int64_t)gt.m0[gi] * N;
        M = gt.me[gi];
        wl.w += (int64_t)e * gt.expert_bytes;
        if constexpr (ZP) zeros += (int64_t)e * N * G;
    }
    const int g_begin = s * gps;
    const int g_end = min(G, g_begin + gps);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int Kp = K / 2;  // activation pairs per row
    const uint32_t *A2 = reinterpret_cast<const uint32_t *>(A);

    const int64_t n = (int64_t)R * 64 + lane;
    // Dense rows beyond N do not exist: read row N-1 and drop the result.
    // Tiled blobs hold zero-padded rows, so nothing to clamp there.
    const int64_t nr = (WL::kTiled || n < N) ? n : (int64_t)N - 1;
    // Zero points are [N, G] in either layout: padded tile rows read row N-1.
    const uint8_t *zrow = ZP ? zeros + (n < N ? n : (int64_t)N - 1) * G : nullptr;

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    // Matrix-core form, activation dwords of a group: 4x4x4, lane 4i + r
    // reads row 4q + r of set q, k = 8i .. 8i + 7; 16x16x32, lane (c, q)
    // reads row c, k = 32 t + 8 q .. + 7 for k-step t.  Rows past M repeat
    // row M-1; their outputs are dropped.
    int arow_off[MF ? MT / 4 : 1];
#pragma unroll
    for (int q = 0; q < (MF ? MT / 4 : 1); ++q)
        arow_off[q] = MF16 ? min(lane & 15, M - 1) * Kp + 16 * q + 4 * (lane >> 4)
                           : min(4 * q + (lane & 3), M - 1) * Kp + 4 * (lane >> 2);

    // Each wave walks groups g_begin + wave, + W, ...; the next group's chunks
    // are loaded before the current one is computed.
    if constexpr (MF && ONE) {
        const int g = g_begin + wave;
        if (g < g_end) {
            SlotRegsMf<B, MT> cur;
            load_slot_regs_mf<B, MT, ZP>(wl, nr, g, A2, arow_off, lane, zrow, cur);
            float x[MT];
            const float sc = bf16_to_f32(cur.s) * kSInv;
            if constexpr (MF16) {
                group_terms_mf16<B, ZP, I8>(cur.w, cur.av, (int)cur.z, x);
                float sb[4];
                row_block_scales(sc, sb);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = sb[m >> 2] * x[m];
            } else {
                group_terms_mf<B, MT, ZP, I8>(cur.w, cur.av, (int)cur.z, x);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = sc * x[m];
            }
        }
    } else if constexpr (MF) {
        SlotRegsMf<B, MT> cur, nxt;
        int g = g_begin + wave;
        if (g < g_end) load_slot_regs_mf<B, MT, ZP>(wl, nr, g, A2, arow_off, lane, zrow, cur);
        for (; g < g_end; g += W) {
            const int gn = g + W;
            if (gn < g_end)
                load_slot_regs_mf<B, MT, ZP>(wl, nr, gn, A2, arow_off, lane, zrow, nxt);
            float x[MT];
            const float sc = bf16_to_f32(cur.s) * kSInv;
            if constexpr (MF16) {
                group_terms_mf16<B, ZP, I8>(cur.w, cur.av, (int)cur.z, x);
                float sb[4];
                row_block_scales(sc, sb);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = fmaf(sb[m >> 2], x[m], acc[m]);
            } else {
                group_terms_mf<B, MT, ZP, I8>(cur.w, cur.av, (int)cur.z, x);
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] = fmaf(sc, x[m], acc[m]);
            }
            cur = nxt;
        }
    } else if constexpr (ONE) {
        const int g = g_begin + wave;
        if (g < g_end) {
            SlotRegs<B, MT> cur;
            load_slot_regs<B, MT, ZP>(wl, nr, g, zrow, cur);
            acc[0] = bf16_to_f32(cur.s) * kSInv *
                     group_terms<B, ZP, I8>(cur.w, A2 + (int64_t)g * 64, (int)cur.z);
        }
    } else {
        SlotRegs<B, MT> cur, nxt;
        int g = g_begin + wave;
        if (g < g_end) load_slot_regs<B, MT, ZP>(wl, nr, g, zrow, cur);
        for (; g < g_end; g += W) {
            const int gn = g + W;
            if (gn < g_end) load_slot_regs<B, MT, ZP>(wl, nr, gn, zrow, nxt);
            const float x = group_terms<B, ZP, I8>(cur.w, A2 + (int64_t)g * 64, (int)cur.z);
            acc[0] = fmaf(bf16_to_f32(cur.s) * kSInv, x, acc[0]);
            cur = nxt;
        }
    }

    // 16x16x32: acc[4 cb + r] is row 4 q + r of A against weight row 16 cb + c.
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if constexpr (MF16) red[wave][4 * (lane >> 4) + (m & 3)][16 * (m >> 2) + (lane & 15)] = acc[m];
        else red[wave][m][lane] = acc[m];
    }
    __syncthreads();

    // Rows m of A are summed over the waves by wave m % W; the other waves
    // are done and leave now, so that only the waves holding outputs stay
    // through the split-K hand-off (their compute unit can take new
    // workgroups meanwhile).
    const int storing = min(W, MT);
    if (wave >= storing) return;
    float v[(MT + W - 1) / W];
#pragma unroll
    for (int i = 0; i < (MT + W - 1) / W; ++i) {
        const int m = wave + i * W;
        v[i] = 0.0f;
        if (m < MT) {
            v[i] = red[0][m][lane];
#pragma unroll
            for (int w2 = 1; w2 < W; ++w2) v[i] += red[w2][m][lane];
        }
    }
    if (splits == 1) {
#pragma unroll
        for (int i = 0; i < (MT + W - 1) / W; ++i) {
            const int m = wave + i * W;
            if (m < MT && m < M && n < N) Y[(int64_t)m * N + n] = f32_to_bf16_rne(v[i]);
        }
        return;
    }

    const int Npad = (int)(gridDim.x / splits) * 64;
    const int64_t np = (int64_t)RB * 64 + lane;  // partial-sum column
    // No counters: a second kernel adds the partials (stream order makes
    // these stores visible to it).
    if (counters == nullptr) {
#pragma unroll
        for (int i = 0; i < (MT + W - 1) / W; ++i) {
            const int m = wave + i * W;
            if (m < MT) part[((int64_t)s * MT + m) * Npad + np] = v[i];
        }
        return;
    }

    // Cross-workgroup reduction, per storing wave (rows m = wave + i W of
    // this 64-row block).  Shared data moves through device-scope relaxed
    // atomics (coherent across the XCDs' L2s without the L2
    // write-back/invalidate an agent-scope fence costs): the partials are
    // atomic stores, the wave waits for their completion before its ticket
    // RMW, and the last of the `splits` waves with this (block, wave) reads
    // them back with atomic loads, adds them in split order (deterministic)
    // and resets the ticket.
    unsigned *ticket = counters + ((int64_t)RB * storing + wave) * tstride;
#pragma unroll
    for (int i = 0; i < (MT + W - 1) / W; ++i) {
        const int m = wave + i * W;
        if (m < MT)
            __hip_atomic_store(&part[((int64_t)s * MT + m) * Npad + np], v[i], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vm_stores();
    unsigned tk = 0;
    if (lane == 0) tk = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(tk) != (unsigned)(splits - 1)) return;
    // The partial loads below follow the ticket (a compiler barrier: the
    // hardware has already returned the ticket, whose value chose this path).
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // All of an output's partial loads are issued before its adds, without
    // branches (indices past the last split repeat it and are not added): one
    // at a time, or behind a branch the compiler waits on, they would put
    // extra round trips on the kernel's tail.
#pragma unroll
    for (int i = 0; i < (MT + W - 1) / W; ++i) {
        const int m = wave + i * W;
        if (m >= MT) continue;
        float p[kDecodeMaxSplits];
#pragma unroll
        for (int t = 0; t < kDecodeMaxSplits; ++t)
            p[t] = __hip_atomic_load(&part[((int64_t)min(t, splits - 1) * MT + m) * Npad + np],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float sum = p[0];
#pragma unroll
        for (int t = 1; t < kDecodeMaxSplits; ++t)
            if (t < splits) sum += p[t];
        if (m < M && n < N) Y[(int64_t)m * N + n] = f32_to_bf16_rne(sum);
    }
    if (lane == 0)  // leave the counter region zero
        __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// One-row decode without a cross-workgroup K split (the row kernel).
//
// A wave owns RW rows of the weights (8, or 4) and a share of K: lane l
// works on row l % RW, and on groups g = j + C (S t + s), t = 0, 1, ...,
// with C = 64 / RW lane classes, j = l / RW and s the wave's share
// among the S waves of its workgroup that hold the same rows.  Each lane
// loads whole slots (b 16-byte chunks; in the tiled layout the RW rows of
// one class are 16 * RW consecutive bytes of a plane, whole cache lines),
// turns the codes into exact bf16 pairs and multiplies them with the
// group's activations on the matrix cores (4x4x4 blocks, see RowChunks;
// the vector ALU only converts), which the workgroup stages once in LDS
// (groups 272 bytes apart, so 16 consecutive groups start on distinct
// 16-byte bank groups and the C classes' reads do not conflict).  The group
// scale is applied once per group in fp32.  The C partial sums of a row are
// added with DPP and the S waves' sums in LDS, in a fixed order, and one
// lane writes the bf16 output: no cross-workgroup hand-off and no
// workspace.  A wave's time is about one memory round trip per slot it
// waits on, so lanes with few slots (two, or three up to b = 6) load them
// all at the start and the whole layer is requested at once; otherwise the
// next slot is in flight while one is computed.
// ---------------------------------------------------------------------------
constexpr int kRowActStride = 272;  // LDS bytes per group of staged activations
constexpr int kRowWaves = 4;        // waves per workgroup
constexpr int kRowActRegs = 16;     // activation dwords a lane stages up front
constexpr int kRowUpfrontMaxG = kRowWaves * kRowActRegs;  // groups the up-front form takes

// Sum of v over the C lanes of a row (lanes r, r + RW, r + 2 RW, ...;
// RW = 8 or 4); every such lane receives it.  Fixed order: deterministic.
template <int RW>
__device__ __forceinline__ float class_sum(float v) {
    if constexpr (RW == 4) v = dpp_add<0x124, 0xF>(v);  // row_ror:4
    v = dpp_add<0x128, 0xF>(v);                         // row_ror:8
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                      false, false);
    v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                      false, false);
    return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// Activation chunk I of the group (8 k, staged in LDS at ab) against codes
// 8I .. 8I+7 of the slot: two k-steps of v_mfma_f32_4x4x4_16b_bf16, one per
// accumulator chain.  The 4 lanes of an MFMA block are 4 rows of one lane
// class, so they hold the same activations: block i's A operand has that
// chunk's 4 k in all four of its rows, its B column j is lane 4i + j's 4
// exact codes, and every row of its output column j is the lane's dot
// product.  Chunk I+1 is read ahead; the fence keeps the compiler from
// hoisting every read and conversion of the slot.
template <int B, bool ZP, bool I8, int I>
struct RowChunks {
    // One k-step: pairs Q, Q+1 of the slot against activation dwords E, E+1.
    template <int Q, int E>
    __device__ __forceinline__ static void step(const uint32_t *w, const uint32_t *o, u32x4 av,
                                                int z, f32x4_t &d) {
        u32x2_t wp, a;
        wp.x = slot_pair<B, Q, ZP, I8>(w, o, z);
        wp.y = slot_pair<B, Q + 1, ZP, I8>(w, o, z);
        a.x = av[E];
        a.y = av[E + 1];
        d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(bf16x4_bits, a),
                                                   __builtin_bit_cast(bf16x4_bits, wp), d, 0, 0,
                                                   0);
    }
    __device__ __forceinline__ static void run(const uint32_t *w, const uint32_t *o,
                                               const uint8_t *ab, int z, u32x4 av, f32x4_t *d) {
        u32x4 nx = av;
        if constexpr (I + 1 < 16) nx = *reinterpret_cast<const u32x4 *>(ab + 16 * (I + 1));
        constexpr int P = 4 * I;
        step<P, 0>(w, o, av, z, d[0]);
        step<P + 2, 2>(w, o, av, z, d[1]);
        __builtin_amdgcn_sched_barrier(0);
        RowChunks<B, ZP, I8, I + 1>::run(w, o, ab, z, nx, d);
    }
};
template <int B, bool ZP, bool I8>
struct RowChunks<B, ZP, I8, 16> {
    __device__ __forceinline__ static void run(const uint32_t *, const uint32_t *,
                                               const uint8_t *, int, u32x4, f32x4_t *) {}
};

// TMAX > 0: every lane has at most TMAX slots, all loaded at the start (the
// whole layer is requested at once and each slot is computed as it lands);
// 0: any number of slots, the next one loaded while one is computed.
template <int B, int RW, int S, class WL, bool ZP, int TMAX>
__global__ __launch_bounds__(64 * kRowWaves, (TMAX > 0 || (B == 7 && !WL::kTiled) || (B == 8 && ZP)) ? 4 : 5) void decode_rows_kernel(
        const uint16_t *__restrict__ A, int N, int K, WL wl, const uint8_t *__restrict__ zeros,
        uint16_t *__restrict__ Y) {
    constexpr int C = 64 / RW;
    constexpr int RO = kRowWaves / S;  // row sets per workgroup
    constexpr bool I8 = WL::kTiled && int8_ready<B>() && !ZP;  // arranged runs
    constexpr float kSInv = operand_scale_inv<B, I8, ZP>();
    extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];
    __shared__ float red[S > 1 ? RO : 1][S][RW];
    const int G = K / kGroup;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ro = wave / S, sw = wave % S;
    // Lane l: row l % RW of the wave's row set, class j = l / RW (so each
    // 4-lane MFMA block is 4 rows of one class).
    const int j = lane / RW;
    const int rr = lane % RW;
    // Workgroup b runs on XCD b % 8; the row sets of one 64-row block share
    // its tiles' scale lines, so consecutive row sets go to one XCD (one L2
    // fetch per line): XCD x takes a contiguous run of the grid.
    int blk = blockIdx.x;
    if ((gridDim.x & 7) == 0) blk = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int64_t n = ((int64_t)blk * RO + ro) * RW + rr;
    // Dense rows beyond N do not exist: read row N-1 and drop the result.
    // Tiled blobs hold zero-padded rows (RW divides 64), so nothing to clamp.
    const int64_t nr = (WL::kTiled || n < N) ? n : (int64_t)N - 1;
    const uint8_t *zrow = ZP ? zeros + (n < N ? n : (int64_t)N - 1) * G : nullptr;
    // Slots of this wave's lanes: groups j + C (S t + sw) below G.
    const int T = (G - C * sw + C * S - 1) / (C * S);

    // Activations into LDS, one group (256 bytes) per wave-wide step, each
    // lane 4 bytes at the group's padded place.  The rolled form loads
    // them straight into LDS (no registers held); the all-slots-up-front
    // form (launched for at most kRowUpfrontMaxG groups, so at most
    // kRowActRegs per wave) goes through registers, so that the compiler's
    // waits see which loads the LDS writes depend on and the slot loads
    // stay in flight past them.
    constexpr int kActRegs = kRowActRegs;
    uint32_t areg[TMAX > 0 ? kActRegs : 1];
    if constexpr (TMAX > 0) {
        const uint32_t *A32 = reinterpret_cast<const uint32_t *>(A);
#pragma unroll
        for (int i = 0; i < kActRegs; ++i)
            areg[i] = A32[(int64_t)min(wave + kRowWaves * i, G - 1) * (kGroup / 2) + lane];
    } else {
        for (int g = wave; g < G; g += kRowWaves)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(A + (int64_t)g * kGroup + 2 * lane),
                (__attribute__((address_space(3))) void *)(act_lds + g * kRowActStride), 4, 0, 0);
    }

    auto load = [&](int t, SlotRegs<B, 1> &r) __attribute__((always_inline)) {
        const int g = min(j + C * (S * t + sw), G - 1);
        load_slot<B>(wl.chunks(nr, g), wl.chunk_stride(), r.w);
        r.s = wl.scale(nr, g);
        if constexpr (ZP) r.z = zrow[g];
    };
    float acc = 0.0f;
    auto compute = [&](int t, SlotRegs<B, 1> &r) __attribute__((always_inline)) {
        const int g = j + C * (S * t + sw);
        const int gc = min(g, G - 1);
        uint32_t o[int8_words<B, ZP, I8>() ? 32 : 1];
        prep_runs<B, ZP, I8, 4>(r.w, o, (int)r.z);
        f32x4_t d[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
        const uint8_t *ab = act_lds + gc * kRowActStride;
        RowChunks<B, ZP, I8, 0>::run(r.w, o, ab, (int)r.z, *reinterpret_cast<const u32x4 *>(ab),
                                     d);
        const float v = fmaf(bf16_to_f32(r.s) * kSInv, d[0][0] + d[1][0], acc);
        acc = g < G ? v : acc;
    };

    if constexpr (TMAX > 0) {
        // All slots at once, after the activations' loads: each slot is B
        // chunk loads, the scale and the zero point, TMAX slots for every
        // wave.  A slot past the lane's last group (the wave has fewer than
        // TMAX, or G is not a multiple of the C classes) reads row 0's first
        // slot instead: one line that all such loads share, so no slot is
        // fetched twice.
        SlotRegs<B, 1> r[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            const int g = j + C * (S * t + sw);
            const bool real = g < G;
            load_slot<B>(real ? wl.chunks(nr, g) : wl.chunks(0, 0), wl.chunk_stride(), r[t].w);
            r[t].s = real ? wl.scale(nr, g) : wl.scale(0, 0);
            if constexpr (ZP) r[t].z = real ? zrow[g] : zeros[0];
        }
        // The activations' LDS writes wait for their own loads only; the
        // barrier then orders LDS (the slot loads stay in flight).
#pragma unroll
        for (int i = 0; i < kActRegs; ++i) {
            const int g = wave + kRowWaves * i;
            if (g < G) *reinterpret_cast<uint32_t *>(act_lds + g * kRowActStride + 4 * lane) = areg[i];
        }
        lds_barrier();
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if (t < T) compute(t, r[t]);
    } else if constexpr (I8) {
        // One slot buffer: slot t is decoded to its int8 words first, which
        // frees the buffer for slot t + 1's loads before slot t's products.
        SlotRegs<B, 1> r;
        if (T > 0) load(0, r);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): activations and first slot
        __syncthreads();
        for (int t = 0; t < T; ++t) {
            const int g = j + C * (S * t + sw);
            const int gc = min(g, G - 1);
            uint32_t o[32];
            prep_runs<B, ZP, true, 4>(r.w, o, 0);
            const float sc = bf16_to_f32(r.s) * kSInv;
            if (t + 1 < T) load(t + 1, r);
            f32x4_t d[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
            const uint8_t *ab = act_lds + gc * kRowActStride;
            RowChunks<B, ZP, true, 0>::run(nullptr, o, ab, 0, *reinterpret_cast<const u32x4 *>(ab),
                                           d);
            const float v = fmaf(sc, d[0][0] + d[1][0], acc);
            acc = g < G ? v : acc;
        }
    } else {
        SlotRegs<B, 1> cur, nxt;
        if (T > 0) load(0, cur);
        // The activations (and the first slot, issued with them) have landed
        // for this wave; after the barrier, for every wave.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        // Slot t + 1 is loaded before slot t is computed (loads retire in
        // issue order, so slot t's wait leaves t + 1 in flight).
        for (int t = 0; t < T; ++t) {
            if (t + 1 < T) load(t + 1, nxt);
            compute(t, cur);
            cur = nxt;
        }
    }
    const float y = class_sum<RW>(acc);
    if constexpr (S == 1) {
        if (j == 0 && n < N) Y[n] = f32_to_bf16_rne(y);
    } else {
        if (j == 0) red[ro][sw][rr] = y;
        __syncthreads();
        if (sw == 0 && j == 0 && n < N) {
            float v = red[ro][0][rr];
#pragma unroll
            for (int i = 1; i < S; ++i) v += red[ro][i][rr];
            Y[n] = f32_to_bf16_rne(v);
        }
    }
}

template <int B, int RW, int S, class WL, bool ZP>
static void launch_rows_kernel(const uint16_t *A, int64_t N, int64_t K, const WL &wl,
                               const uint8_t *zeros, uint16_t *Y, int tmax, hipStream_t stream) {
    constexpr int RO = kRowWaves / S;
    constexpr int C = 64 / RW;
    const int64_t sets = (N + RW - 1) / RW;
    const dim3 grid((unsigned)((sets + RO - 1) / RO));
    const int G = (int)(K / kGroup);
    const size_t lds = (size_t)G * kRowActStride;
    const int T = (G + C * S - 1) / (C * S);  // most slots of any lane
    // Three slots in registers fit up to b = 6 (b = 7, 8 would spill); the
    // up-front form stages at most kRowUpfrontMaxG groups of activations.
    if (G > kRowUpfrontMaxG) tmax = 0;
    if (tmax >= 2 && T <= 2) {
        hipLaunchKernelGGL((decode_rows_kernel<B, RW, S, WL, ZP, 2>), grid, dim3(64 * kRowWaves),
                           lds, stream, A, (int)N, (int)K, wl, zeros, Y);
        return;
    }
    if constexpr (B <= 6) {
        if (tmax >= 3 && T <= 3) {
            hipLaunchKernelGGL((decode_rows_kernel<B, RW, S, WL, ZP, 3>), grid,
                               dim3(64 * kRowWaves), lds, stream, A, (int)N, (int)K, wl, zeros,
                               Y);
            return;
        }
    }
    hipLaunchKernelGGL((decode_rows_kernel<B, RW, S, WL, ZP, 0>), grid, dim3(64 * kRowWaves), lds,
                       stream, A, (int)N, (int)K, wl, zeros, Y);
}

template <int B, int RW, class WL, bool ZP>
static void launch_rows_s(const uint16_t *A, int64_t N, int64_t K, const WL &wl,
                          const uint8_t *zeros, uint16_t *Y, int s, int tmax,
                          hipStream_t stream) {
    if (s == 4) launch_rows_kernel<B, RW, 4, WL, ZP>(A, N, K, wl, zeros, Y, tmax, stream);
    else if (s == 2) launch_rows_kernel<B, RW, 2, WL, ZP>(A, N, K, wl, zeros, Y, tmax, stream);
    else launch_rows_kernel<B, RW, 1, WL, ZP>(A, N, K, wl, zeros, Y, tmax, stream);
}

template <int B, class WL>
static hipError_t launch_rows(const uint16_t *A, int64_t N, int64_t K, const WL &wl,
                              const uint8_t *zeros, uint16_t *Y, int rw, int s, int tmax,
                              hipStream_t stream) {
    if (zeros) {
        if constexpr (B == 4 || B == 8) {
            if (rw == 8) launch_rows_s<B, 8, WL, true>(A, N, K, wl, zeros, Y, s, tmax, stream);
            else launch_rows_s<B, 4, WL, true>(A, N, K, wl, zeros, Y, s, tmax, stream);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        if (rw == 8) launch_rows_s<B, 8, WL, false>(A, N, K, wl, nullptr, Y, s, tmax, stream);
        else launch_rows_s<B, 4, WL, false>(A, N, K, wl, nullptr, Y, s, tmax, stream);
    }
    return hipGetLastError();
}

template <int B, int MT, int W, class WL, bool ZP, class GT>
static void launch_decode_kernel(bool one, const uint16_t *A, int64_t M, int64_t N, int64_t K,
                                 const WL &wl, const uint8_t *zeros, uint16_t *Y, float *part,
                                 unsigned *counters, const DecodePlan &p, const GT &gt,
                                 hipStream_t stream) {
    const dim3 grid((unsigned)(p.rowblocks * p.splits));
    if (one)
        hipLaunchKernelGGL((decode_kernel<B, MT, W, WL, true, ZP, GT>), grid, dim3(64 * W), 0,
                           stream, A, (int)M, (int)N, (int)K, wl, zeros, Y, part, counters,
                           p.splits, p.gps, p.tstride, gt);
    else
        hipLaunchKernelGGL((decode_kernel<B, MT, W, WL, false, ZP, GT>), grid, dim3(64 * W), 0,
                           stream, A, (int)M, (int)N, (int)K, wl, zeros, Y, part, counters,
                           p.splits, p.gps, p.tstride, gt);
}

template <int B, int MT, int W, class WL, class GT>
static hipError_t launch_decode_zp(bool one, const uint16_t *A, int64_t M, int64_t N, int64_t K,
                                   const WL &wl, const uint8_t *zeros, uint16_t *Y, float *part,
                                   unsigned *counters, const DecodePlan &p, const GT &gt,
                                   hipStream_t stream) {
    if (!zeros) {
        launch_decode_kernel<B, MT, W, WL, false>(one, A, M, N, K, wl, nullptr, Y, part,
                                                  counters, p, gt, stream);
    } else if constexpr (B == 4 || B == 8) {  // the widths with an asymmetric form
        launch_decode_kernel<B, MT, W, WL, true>(one, A, M, N, K, wl, zeros, Y, part, counters,
                                                 p, gt, stream);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int B, int MT, int W, class GT>
hipError_t decode_bmw(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W_,
                      bool tiled, const uint16_t *scales, const uint8_t *zeros, uint16_t *Y,
                      void *ws, const DecodePlan &p, const GT &gt, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    float *part = nullptr;
    unsigned *counters = nullptr;
    if (p.splits > 1) {
        if (!p.reduce) counters = static_cast<unsigned *>(ws);
        part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    }
    const bool one = MT > 1 && p.gps <= W;
    hipError_t e;
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W_), G, B};
        e = launch_decode_zp<B, MT, W>(one, A, M, N, K, wl, zeros, Y, part, counters, p, gt,
                                       stream);
    } else if constexpr (GT::kGrouped) {
        return hipErrorInvalidValue;  // grouped launches take the tiled layout
    } else {
        DenseW wl{static_cast<const uint8_t *>(W_), scales, (int64_t)16 * B * G, G, B};
        e = launch_decode_zp<B, MT, W>(one, A, M, N, K, wl, zeros, Y, part, counters, p, gt,
                                       stream);
    }
    if (e != hipSuccess || p.splits == 1 || !p.reduce) return e;
    if constexpr (GT::kGrouped) return hipErrorInvalidValue;  // grouped plans keep the hand-off
    return launch_decode_reduce(part, p.splits, MT, M, N, p.rowblocks, Y, stream);
}

template <int B, int MT, class GT>
hipError_t decode_bm(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W_,
                     bool tiled, const uint16_t *scales, const uint8_t *zeros, uint16_t *Y,
                     void *ws, const DecodePlan &p, const GT &gt, hipStream_t stream) {
    if constexpr (MT <= 4) {
        if (p.waves == 16)
            return decode_bmw<B, MT, 16>(A, M, N, K, W_, tiled, scales, zeros, Y, ws, p, gt,
                                         stream);
    }
    if (p.waves == 8)
        return decode_bmw<B, MT, 8>(A, M, N, K, W_, tiled, scales, zeros, Y, ws, p, gt, stream);
    if (p.waves == 4)
        return decode_bmw<B, MT, 4>(A, M, N, K, W_, tiled, scales, zeros, Y, ws, p, gt, stream);
    return hipErrorInvalidValue;
}

template <int B, class GT>
hipError_t decode_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                    bool tiled, const uint16_t *scales, const uint8_t *zeros, uint16_t *Y,
                    void *ws, const DecodePlan &p, const GT &gt, hipStream_t stream) {
    if constexpr (!GT::kGrouped) {
        if (p.rw) {
            const int G = (int)(K / kGroup);
            if (tiled)
                return launch_rows<B>(A, N, K, TiledW{static_cast<const uint8_t *>(W), G, B},
                                      zeros, Y, p.rw, p.splits, p.tmax, stream);
            return launch_rows<B>(A, N, K,
                                  DenseW{static_cast<const uint8_t *>(W), scales,
                                         (int64_t)16 * B * G, G, B},
                                  zeros, Y, p.rw, p.splits, p.tmax, stream);
        }
    }
    switch (p.mt) {
        case 1: return decode_bm<B, 1>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, gt, stream);
        case 4: return decode_bm<B, 4>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, gt, stream);
        case 8: return decode_bm<B, 8>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, gt, stream);
        case 16:
            return decode_bm<B, 16>(A, M, N, K, W, tiled, scales, zeros, Y, ws, p, gt, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
