// wq_prefill.hip -- WNA16 prefill path (M > 16): LDS-tiled bf16 MFMA GEMM.
//
// At large batch the layer is compute-bound ("vLLM Quantization", Key points
// and Pitfalls: weight-only gains fade as batch grows), so codes are
// dequantized once per workgroup tile into LDS and the product runs on the
// matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// Exactness.  The B operand holds 128 + c as bf16 (exact for c < 128; b = 8
// uses byte conversion, offset 128), so the integer codes are never rounded.
// Each group of 128 k is accumulated into its own fp32 block P_g and folded
// as  total += s[n,g] * P_g  in fp32.  The constant part
//     -(128 + 2^(b-1)) * sum_g s[n,g] * sum_{k in g} a[m,k]
// is a small product over groups: a pre-pass writes, per (row m, group g),
// v = -(128 + 2^(b-1)) * sum_{k in g} a[m,k] split exactly into three bf16
// terms (hi + mid + lo, error ~2^-24 |v|) at k' = 3g + t, and the main loop
// multiplies that against s[n, k'/3] as extra "pseudo-groups" with scale 1.
// No scale or code is ever rounded to bf16.
//
// Tiling.  Workgroup 256 (m) x 128 (n), 8 waves of 64 x 64 (two per SIMD),
// each as 2 x 2 MFMA blocks of 32 x 32 run in two staggered halves.  K runs
// in whole groups of 128 through LDS (A in two phase-shifted halves, B
// unpacked to bf16 once per workgroup, double-buffered), register-staged.
// Workgroups an XCD runs together share an A row block.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPM = 256;          // workgroup rows (m)
constexpr int kPN = 128;          // workgroup cols (n)
constexpr int kPseudoK = 128;     // k' per pseudo-group

// Pre-pass: per (row m, group g) v = -off * sum_{k in g} a[m,k], written as
// three bf16 terms at k' = 3g + {0,1,2} of a [M, Kp] bf16 matrix (zero beyond
// 3G).  One workgroup of 256 threads per row; 16 threads per group, fixed
// reduction order.
__global__ __launch_bounds__(256) void group_sum_split_kernel(const uint16_t *__restrict__ A,
                                                              int K, int Kp, float off,
                                                              uint16_t *__restrict__ Ap) {
    const int64_t m = blockIdx.x;
    const int G = K / kGroup;
    const int t = threadIdx.x;
    uint16_t *out = Ap + m * Kp;
    for (int k = 3 * G + t; k < Kp; k += 256) out[k] = 0;
    for (int base = 0; base < K; base += 256 * 8) {
        const int k0 = base + 8 * t;
        float s = 0.0f;
        if (k0 < K) {
            const uint4 v = *reinterpret_cast<const uint4 *>(A + m * K + k0);
            s = dot2_bf16(v.x, 0x3F803F80u, s);
            s = dot2_bf16(v.y, 0x3F803F80u, s);
            s = dot2_bf16(v.z, 0x3F803F80u, s);
            s = dot2_bf16(v.w, 0x3F803F80u, s);
        }
        // 16 consecutive threads hold one group (16 x 8 = 128 k).
        s += __shfl_xor(s, 1, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 8, 16);
        if ((t & 15) == 0 && k0 < K) {
            const int g = k0 / kGroup;
            const float v = -off * s;
            const uint16_t hi = f32_to_bf16_rne(v);
            const float r1 = v - bf16_to_f32(hi);
            const uint16_t mid = f32_to_bf16_rne(r1);
            const float r2 = r1 - bf16_to_f32(mid);
            out[3 * g + 0] = hi;
            out[3 * g + 1] = mid;
            out[3 * g + 2] = f32_to_bf16_rne(r2);
        }
    }
}

// LDS tiles are rows of 16-byte chunks (8 bf16 of k), 16 chunks (one group
// of 128 k, 256 bytes) per row; chunk c of row r sits at r*16 + (c ^ (r &
// 15)).  LDS serves a 128-bit read 16 lanes at a time over 64 banks, and
// the 16 consecutive rows such a lane group reads (one chunk each) land on
// 16 distinct 16-byte bank groups; the loaders' row-wise writes (16 chunks
// of one row per 16 lanes) are conflict free too, with no padding.
__device__ __forceinline__ int swz16(int row, int chunk) {
    return row * 16 + (chunk ^ (row & 15));
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Workgroup: 512 threads = 8 waves (two per SIMD) over a 256 (m) x 128 (n)
// output tile; wave (wm, wn) owns rows 64 wm .. +64 and columns 64 wn .. +64
// as 2 x 2 blocks (i, j) of 32 x 32 (v_mfma_f32_32x32x16_bf16: lane l holds
// A row l%32 and B column l%32 at k-chunk l/32; result element r of lane l
// is row 8(r/4) + 4(l/32) + r%4, column l%32).  Per block two fp32 sets live
// in VGPRs: P (the current group) and tot (the folded sum).
//
// Staggered halves.  Folding a group (tot += s * P, one FMA per output
// element) must read P after the group's last MFMA on it has completed and
// before the next group's first MFMA overwrites it.  So each group runs in
// two phases of 16 MFMA slots: phase 0 runs the 8 k-steps of blocks (0, *),
// phase 1 those of blocks (1, *) (two accumulation chains each, alternating
// j).  Phase 0 folds the (1, *) blocks of the previous group and phase 1 the
// (0, *) blocks of this one, whose MFMAs finished a phase earlier: two FMAs
// per slot, no wait on the matrix pipe.  The 32 x 32 x 16 MFMA holds the
// matrix pipe about four times as long as the issue port, so the fold and
// the code unpack (about 1.5 VALU per slot) issue beside it.
//
// LDS.  A is held one group at a time as two halves: half h has, for every
// wave, its 32 rows of block row h (128 rows x 128 k, 32 KB); half 0 is read
// in phase 0 and refilled with the next group during phase 1, half 1 the
// other way round.  B (128 rows x 128 k, 32 KB) is double-buffered by group
// and the group's scales sit beside it.  The NP pseudo-groups run first,
// unpipelined (A from the pre-pass matrix, B = scales, scale 1); the G real
// groups are software-pipelined:
//   group g, phase 0: fold (1, *) of g-1; unpack codes of g+1 into the other
//     B buffer (one pair every other slot, both phases); fetch the codes of
//     g+2 (a second register set) at slot 1; write A half 1 of g (fetched in
//     phase 1 of g-1) at slots 4-7, a 16-byte piece each; fetch A half 0 of
//     g+1 at slot 8; barrier after slot 13, then read phase 1's first k-step;
//   group g, phase 1: fold (0, *) of g; finish the unpack by slot 11 (with
//     the scales of g+1); write A half 0 of g+1 at slots 4-7, fetch A half 1
//     of g+1 at slot 8; barrier after slot 13, then read the first k-step of
//     group g+1's phase 0; the codes of g+2 move to the first set.
// Operands run one k-step ahead; the next phase's first k-step is read
// right after the barrier, under the phase's last four MFMAs.
template <int B, class WL>
__global__ __launch_bounds__(512) void prefill_kernel(const uint16_t *__restrict__ A,
                                                      const uint16_t *__restrict__ Ap, int M,
                                                      int N, int K, int Kp, WL wl,
                                                      uint16_t *__restrict__ Y, int mtiles,
                                                      int ntiles, int splits,
                                                      float *__restrict__ part, int64_t mnp) {
    __shared__ u32x4 Ah[2][kPN * 16];   // [half][128 rows x 16 chunks]
    __shared__ u32x4 Bsm[2][kPN * 16];  // [group buffer][128 rows x 16 chunks]
    __shared__ float Ss[2][kPN];

    const int G = K / kGroup;
    const int NP = Kp / kPseudoK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Block b runs on XCD b % 8: give each XCD a contiguous run of logical
    // tiles, n fastest, so the tiles an XCD runs together share A rows.
    // With K split `splits` ways, logical = split * tiles + tile.
    const int tiles = mtiles * ntiles;
    const int total = tiles * splits;
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int sp = logical / tiles;
    const int tile = logical - sp * tiles;
    const int bm = tile / ntiles;
    const int bn = tile - bm * ntiles;
    // This workgroup's groups; the pseudo-groups go with split 0.
    const int g_lo = (int)(((int64_t)G * sp) / splits);
    const int g_hi = (int)(((int64_t)G * (sp + 1)) / splits);
    const int64_t m0 = (int64_t)bm * kPM;
    const int64_t n0 = (int64_t)bn * kPN;

    const uint32_t mask = __builtin_amdgcn_readfirstlane(pair_mask<B < 8 ? B : 7>());
    const uint32_t magic = in_vgpr(kBf16Magic128x2);

    // A loader: chunk ac of half rows hr = ar + 32 u (u < 4), which are tile
    // rows 64 u + 32 h + ar.  Rows beyond M read row M-1 (results dropped).
    const int ac = tid & 15;
    const int ar = tid >> 4;
    const int mlim = (int)min((int64_t)M - 1 - m0, (int64_t)kPM - 1);
    int arow_g[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 4; ++u) arow_g[h][u] = min(64 * u + 32 * h + ar, mlim);
    const uint16_t *A_blk = A + m0 * K;
    const uint16_t *Ap_blk = Ap + m0 * Kp;
    int a_lds[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a_lds[u] = swz16(ar + 32 * u, ac);

    // B loader: row brow, quarter bq (wave-uniform) of each group.
    const int brow = tid & (kPN - 1);
    const int bq = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int64_t bn_read = min(n0 + brow, (int64_t)N - 1);
    const uint8_t *bslot0 = wl.slot0(bn_read);
    const uint8_t *bscale0 = wl.scale0(bn_read);
    const int bstep = (int)wl.slot_step();
    const int sstep = (int)wl.scale_step();

    // MFMA operand rows (in an A half and in B) and k-chunk half of this lane.
    const int arow = wm * 32 + (lane & 31);
    const int bmrow = wn * 64 + (lane & 31);
    const int khalf = lane >> 5;

    u32x4 areg[4];
    uint32_t creg[B], cnext[B];
    f32x16_t tot[2][2], P[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                tot[i][j][r] = 0.0f;
                P[i][j][r] = 0.0f;
            }
        }

    // A half h of real group g (clamped to this split's last one) into areg
    // / from areg into LDS.
    auto load_a = [&](int g, int h) __attribute__((always_inline)) {
        const uint16_t *src = A_blk + min(g, g_hi - 1) * kGroup + 8 * ac;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            areg[u] = *reinterpret_cast<const u32x4 *>(src + __mul24(arow_g[h][u], K));
    };
    // One of the four 16-byte pieces (spread over four slots, so the LDS
    // write queue never takes a whole phase's worth at once).
    auto store_a = [&](int h, int u) __attribute__((always_inline)) {
        Ah[h][a_lds[u]] = areg[u];
    };
    // Quarter bq of real group g's codes (clamped to the last group): B
    // dwords at per-wave offsets held in scalar registers.
    int qoff[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
        const int d = bq * B + e;
        qoff[e] = __builtin_amdgcn_readfirstlane((d >> 2) * (WL::kTiled ? 1024 : 16) + (d & 3) * 4);
    }
    auto load_codes = [&](int g, uint32_t(&dst)[B]) __attribute__((always_inline)) {
        const uint8_t *slot = bslot0 + (int64_t)min(g, g_hi - 1) * bstep;
#pragma unroll
        for (int e = 0; e < B; ++e) dst[e] = *reinterpret_cast<const uint32_t *>(slot + qoff[e]);
    };
    // Chunk C (pairs 4C .. 4C+3, 8 codes) of the B operand (128 + c as bf16)
    // from creg into B buffer buf.
    auto fill_chunk = [&](int buf, auto cconst) __attribute__((always_inline)) {
        constexpr int C = decltype(cconst)::value;
        const u32x4 v{quarter_pair<B, 4 * C>(creg, mask, magic),
                      quarter_pair<B, 4 * C + 1>(creg, mask, magic),
                      quarter_pair<B, 4 * C + 2>(creg, mask, magic),
                      quarter_pair<B, 4 * C + 3>(creg, mask, magic)};
        Bsm[buf][swz16(brow, 4 * bq + C)] = v;
    };
    // Group g's scales into Ss[buf] (the four quarter waves of a row store
    // the same value: no branch).
    auto store_scale = [&](int g, int buf) __attribute__((always_inline)) {
        Ss[buf][brow] =
            bf16_to_f32(*reinterpret_cast<const uint16_t *>(bscale0 + min(g, g_hi - 1) * sstep));
    };
    // Slice q (of 16) of folding block row i with column scales sq: the
    // slot's two FMAs.
    auto fold_slice = [&](int i, int q, const float(&sq)[2]) __attribute__((always_inline)) {
        const int j = q >> 3, r = 2 * (q & 7);
        tot[i][j][r] = fmaf(sq[j], P[i][j][r], tot[i][j][r]);
        tot[i][j][r + 1] = fmaf(sq[j], P[i][j][r + 1], tot[i][j][r + 1]);
    };

    // Operands of one k-step (A half ah, B buffer gb): sets 0 and 1 hold
    // k-steps of the running phase in turn, set 2 the next phase's k-step 0.
    bf16x8_t af[3], bfr[3][2];
    auto read_ops = [&](int ah, int gbuf, int kk, int e) __attribute__((always_inline)) {
        af[e] = __builtin_bit_cast(bf16x8_t, Ah[ah][swz16(arow, 2 * kk + khalf)]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bfr[e][j] = __builtin_bit_cast(bf16x8_t, Bsm[gbuf][swz16(bmrow + 32 * j, 2 * kk + khalf)]);
    };

    // One phase: the 8 k-steps of blocks (I, 0), (I, 1) from A half I and B
    // buffer gbuf, starting from k-step 0's operands in set 2; k-step kk+1 is
    // read into set (kk+1) & 1 at the start of k-step kk.  After each MFMA,
    // hook(slot) issues a slice of the other work and the pair is fenced, so
    // the order written here is the issue order.  With NEXT, the workgroup
    // barrier follows slot 13: by then every operand read of this phase has
    // been issued (the last one, k-step 7's, at the start of k-step 6), so
    // no wave past the barrier can overwrite a buffer another wave still
    // has to read; and every LDS write the next phase needs is issued in the
    // hooks before it.  Then the next phase's k-step 0 (A half na, B buffer
    // ngb) is read into set 2, under the phase's last two MFMAs.
    auto phase = [&](auto iconst, int gbuf, auto nconst, int na, int ngb, auto &&hook)
        __attribute__((always_inline)) {
        constexpr int I = decltype(iconst)::value;
        constexpr bool NEXT = decltype(nconst)::value;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (kk + 1 < 8) read_ops(I, gbuf, kk + 1, (kk + 1) & 1);
            const int e = kk == 0 ? 2 : (kk & 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x16_t c = P[I][j];
                if (kk == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) c[r] = 0.0f;
                }
                P[I][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[e], bfr[e][j], c, 0, 0, 0);
                const int slot = 2 * kk + j;
                hook(slot);
                if (NEXT && slot == 13) {
                    lds_barrier();
                    read_ops(na, ngb, 0, 2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    float sq_prev[2] = {0.0f, 0.0f};

    // ---- pseudo-groups (scale 1), not pipelined: A' from the pre-pass
    // matrix, B' = s[n, k'/3] (zero beyond 3G) ----
    {
        const float one[2] = {1.0f, 1.0f};
        for (int ps = 0; ps < (sp == 0 ? NP : 0); ++ps) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint16_t *src = Ap_blk + ps * kPseudoK + 8 * ac;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    areg[u] = *reinterpret_cast<const u32x4 *>(src + __mul24(arow_g[h][u], Kp));
#pragma unroll
                for (int u = 0; u < 4; ++u) store_a(h, u);
            }
            const int k0 = ps * kPseudoK + 32 * bq;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                uint32_t pr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int ka = k0 + 8 * u + 2 * e, kb = ka + 1;
                    const uint32_t sa = *reinterpret_cast<const uint16_t *>(
                        bscale0 + min(ka / 3, G - 1) * sstep);
                    const uint32_t sb = *reinterpret_cast<const uint16_t *>(
                        bscale0 + min(kb / 3, G - 1) * sstep);
                    pr[e] = (ka < 3 * G ? sa : 0u) | ((kb < 3 * G ? sb : 0u) << 16);
                }
                Bsm[0][swz16(brow, 4 * bq + u)] = u32x4{pr[0], pr[1], pr[2], pr[3]};
            }
            lds_barrier();
            read_ops(0, 0, 0, 2);
            phase(std::integral_constant<int, 0>{}, 0, std::integral_constant<bool, false>{}, 0,
                  0, [&](int slot) { fold_slice(1, slot, sq_prev); });
            sq_prev[0] = one[0];
            sq_prev[1] = one[1];
            read_ops(1, 0, 0, 2);
            phase(std::integral_constant<int, 1>{}, 0, std::integral_constant<bool, false>{}, 0,
                  0, [&](int slot) { fold_slice(0, slot, one); });
            lds_barrier();
        }
    }

    // ---- real groups, software-pipelined ----
    {
        // Prologue: group g_lo's B, scales and both A halves in LDS; the
        // codes of g_lo + 1 in registers.
        load_codes(g_lo, creg);
        fill_chunk(0, std::integral_constant<int, 0>{});
        fill_chunk(0, std::integral_constant<int, 1>{});
        fill_chunk(0, std::integral_constant<int, 2>{});
        fill_chunk(0, std::integral_constant<int, 3>{});
        store_scale(g_lo, 0);
        load_a(g_lo, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) store_a(0, u);
        load_a(g_lo, 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) store_a(1, u);
        load_codes(g_lo + 1, creg);
        lds_barrier();
        read_ops(0, 0, 0, 2);

        for (int g = g_lo; g < g_hi; ++g) {
            const int gb = (g - g_lo) & 1, nb = gb ^ 1;
            const bool first = g == g_lo;
            uint32_t pairs[16];
            // Unpack pair p of group g+1 at global slot 2p (p < 14), pairs
            // 14 and 15 at slot 27; a 16-byte chunk goes to LDS every four.
            auto unpack = [&](int sigma) __attribute__((always_inline)) {
                int p0 = -1, p1 = -1;
                if (sigma < 28 && (sigma & 1) == 0) p0 = sigma >> 1;
                if (sigma == 27) { p0 = 14; p1 = 15; }
                if (p0 >= 0) pairs[p0] = quarter_pair_dyn<B>(p0, creg, mask, magic);
                if (p1 >= 0) pairs[p1] = quarter_pair_dyn<B>(p1, creg, mask, magic);
                const int last = p1 >= 0 ? p1 : p0;
                if (last >= 0 && (last & 3) == 3)
                    Bsm[nb][swz16(brow, 4 * bq + (last >> 2))] =
                        u32x4{pairs[last - 3], pairs[last - 2], pairs[last - 1], pairs[last]};
            };
            // Phase 0: blocks (0, *) of g; fold (1, *) of g-1.
            phase(std::integral_constant<int, 0>{}, gb, std::integral_constant<bool, true>{}, 1,
                  gb, [&](int slot) {
                      fold_slice(1, slot, sq_prev);
                      unpack(slot);
                      if (slot == 1) load_codes(g + 2, cnext);
                      if (slot >= 4 && slot <= 7 && !first) store_a(1, slot - 4);
                      if (slot == 8) load_a(g + 1, 0);
                  });
            // Phase 1: blocks (1, *) of g; fold (0, *) of g.
            float sq[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) sq[j] = Ss[gb][wn * 64 + 32 * j + (lane & 31)];
            phase(std::integral_constant<int, 1>{}, gb, std::integral_constant<bool, true>{}, 0,
                  nb, [&](int slot) {
                      fold_slice(0, slot, sq);
                      unpack(16 + slot);
                      if (slot == 11) store_scale(g + 1, nb);
                      if (slot == 15) {
#pragma unroll
                          for (int e = 0; e < B; ++e) creg[e] = cnext[e];
                      }
                      if (slot >= 4 && slot <= 7) store_a(0, slot - 4);
                      if (slot == 8) load_a(g + 1, 1);
                  });
            sq_prev[0] = sq[0];
            sq_prev[1] = sq[1];
        }
        // The last group's (1, *) blocks.
#pragma unroll
        for (int q = 0; q < 16; ++q) fold_slice(1, q, sq_prev);
    }

    // Output element r of block (i, j): row 8(r/4) + 4(lane/32) + r%4,
    // column lane%32.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (m < M && n < N) {
                    if (splits == 1)
                        Y[m * N + n] = f32_to_bf16_rne(tot[i][j][r]);
                    else
                        part[(int64_t)sp * mnp + m * N + n] = tot[i][j][r];
                }
            }
        }
}

// Y = bf16(sum over splits of part[s]) in split order (deterministic); four
// consecutive outputs per thread.  Split s's partials start at s * mnp
// (M * N rounded up to 64 floats, so the vector loads stay aligned).
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float *__restrict__ part,
                                                             int splits, int64_t MN, int64_t mnp,
                                                             uint16_t *__restrict__ Y) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= MN) return;
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(part + e);
    for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const f32x4_t *>(part + s * mnp + e);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (e + i < MN) Y[e + i] = f32_to_bf16_rne(acc[i]);
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

static int pseudo_kp(int64_t K) {
    const int G = (int)(K / kGroup);
    return (3 * G + kPseudoK - 1) / kPseudoK * kPseudoK;
}

// K splits: when the tiles alone leave compute units idle, split K so that
// tiles x splits is just under 256 (one workgroup per compute unit), at
// least 8 groups per split; between 192 and 383 tiles, 2 splits (the second
// round of workgroups would otherwise run nearly empty).  Measured at M =
// 512: 17408 -> 5120 (80 tiles) best at 3 splits, 174 vs 365 us unsplit;
// 5120 -> 17408 (272 tiles) 219 us at 2 splits vs 240 us.
// WQ_PREFILL_SPLITS forces a split count.
static int prefill_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + kPM - 1) / kPM) * ((N + kPN - 1) / kPN);
    const int G = (int)(K / kGroup);
    static const int forced = [] {
        const char *e = std::getenv("WQ_PREFILL_SPLITS");
        return e ? std::atoi(e) : 0;
    }();
    if (forced > 0) return std::max(1, std::min(forced, G));
    if (tiles >= 384) return 1;
    if (tiles >= 192) return G >= 16 ? 2 : 1;
    int s = (int)std::max<int64_t>(1, 256 / tiles);
    return std::max(1, std::min(s, G / 8));
}

static int64_t prefill_mnp(int64_t M, int64_t N) { return (M * N + 63) / 64 * 64; }

// Workspace: the shared counter region (unused here), then the pre-pass
// matrix [M, Kp] bf16, then (K split) the fp32 partial outputs, split s at
// s * mnp floats.
int64_t prefill_ws_bytes(int64_t M, int64_t N, int64_t K, int) {
    const int s = prefill_splits(M, N, K);
    return kWsScratchOffset + align256(M * pseudo_kp(K) * 2) +
           (s > 1 ? s * prefill_mnp(M, N) * 4 : 0);
}

template <int B>
static hipError_t prefill_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                            bool tiled, const uint16_t *scales, uint16_t *Y, void *ws,
                            hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int Kp = pseudo_kp(K);
    uint16_t *Ap = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    const int splits = prefill_splits(M, N, K);
    float *part = splits > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                         kWsScratchOffset + align256(M * Kp * 2))
                             : nullptr;
    const float off = (B == 8) ? 128.0f : (float)(128 + (1 << (B - 1)));
    hipLaunchKernelGGL(group_sum_split_kernel, dim3((unsigned)M), dim3(256), 0, stream, A, (int)K,
                       Kp, off, Ap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int mtiles = (int)((M + kPM - 1) / kPM);
    const int ntiles = (int)((N + kPN - 1) / kPN);
    const dim3 grid((unsigned)(mtiles * ntiles * splits));
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((prefill_kernel<B, TiledW>), grid, dim3(512), 0, stream, A, Ap,
                           (int)M, (int)N, (int)K, Kp, wl, Y, mtiles, ntiles, splits, part,
                           prefill_mnp(M, N));
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((prefill_kernel<B, DenseW>), grid, dim3(512), 0, stream, A, Ap,
                           (int)M, (int)N, (int)K, Kp, wl, Y, mtiles, ntiles, splits, part,
                           prefill_mnp(M, N));
    }
    e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t MN = M * N;
    const int64_t threads = (MN + 3) / 4;
    hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, part, splits, MN, prefill_mnp(M, N), Y);
    return hipGetLastError();
}

hipError_t launch_prefill(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, int b, uint16_t *Y, void *ws,
                          hipStream_t stream) {
    switch (b) {
        case 2: return prefill_b<2>(A, M, N, K, W, tiled, scales, Y, ws, stream);
        case 3: return prefill_b<3>(A, M, N, K, W, tiled, scales, Y, ws, stream);
        case 4: return prefill_b<4>(A, M, N, K, W, tiled, scales, Y, ws, stream);
        case 5: return prefill_b<5>(A, M, N, K, W, tiled, scales, Y, ws, stream);
        case 6: return prefill_b<6>(A, M, N, K, W, tiled, scales, Y, ws, stream);
        case 7: return prefill_b<7>(A, M, N, K, W, tiled, scales, Y, ws, stream);
        case 8: return prefill_b<8>(A, M, N, K, W, tiled, scales, Y, ws, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
