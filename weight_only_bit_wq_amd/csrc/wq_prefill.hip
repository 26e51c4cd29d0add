// wq_prefill.hip -- WNA16 prefill path (M > 16): LDS-tiled bf16 MFMA GEMM.
//
// At large batch the layer is compute-bound ("vLLM Quantization", Key points
// and Pitfalls: weight-only gains fade as batch grows), so codes are
// dequantized once per workgroup tile into LDS and the product runs on the
// matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.
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
// Tiling.  Workgroup 256 (m) x 128 (n), 8 waves of 64 x 64 (two per SIMD).
// K runs in LDS stages of 64 for A and whole groups of 128 for B (unpacked
// to bf16 in LDS once per workgroup), double-buffered, register-staged.
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
constexpr int kPK = 64;           // k per LDS stage
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

// LDS tiles are rows of 16-byte chunks (8 bf16 of k).  Chunk c of row r is
// stored at position c ^ (r mod 8) (A: 8 chunks per row) or c ^ (r mod 16)
// (B: 16 chunks per row), so the 16 rows one MFMA operand read touches sit on
// 16 distinct bank groups and the loaders' row-major writes stay conflict
// free (no padding).
__device__ __forceinline__ int swz8(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }
__device__ __forceinline__ int swz16(int row, int chunk) {
    return row * 16 + (chunk ^ (row & 15));
}

// Workgroup: 512 threads = 8 waves (two per SIMD) over a 256 (m) x 128 (n)
// output tile; wave (wm, wn) owns rows 64 wm .. +64 and columns 64 wn .. +64
// as 4 x 4 MFMA blocks of 16 x 16.  Per block two fp32 sets live in VGPRs:
// P (the current group) and tot (the folded sum).
//
// The NP pseudo-groups run first, unpipelined (A from the pre-pass matrix,
// B = scales, scale 1).  The G real groups are software-pipelined.  LDS: A
// per 64-k stage (two buffers, 32 KB each), B per 128-k group (two buffers,
// 32 KB each), the group scales per group (two buffers).  Group g (stages
// 2g, 2g+1):
//   stage 2g:   MFMA (A buf 0, B buf g&1, k 0..63); fold row block 3 of
//               group g-1; write A stage 2g+1 to A buf 1; fetch A stage
//               2g+2; unpack group g+1 into B buf (g+1)&1 and its scales
//               into Ss; fetch the codes of group g+2;            barrier
//   stage 2g+1: MFMA (A buf 1, B buf g&1, k 64..127); fold row blocks 0..2
//               of group g; write A stage 2g+2 to A buf 0; fetch A stage
//               2g+3;                                              barrier
// Each MFMA is followed by a small slice of the other work, in a fixed
// order: an MFMA occupies the SIMD's issue port for about two VALU slots
// and the matrix pipe for four, so about two VALU operations per MFMA issue
// for free.
template <int B, class WL>
__global__ __launch_bounds__(512) void prefill_kernel(const uint16_t *__restrict__ A,
                                                      const uint16_t *__restrict__ Ap, int M,
                                                      int N, int K, int Kp, WL wl,
                                                      uint16_t *__restrict__ Y, int mtiles,
                                                      int ntiles, int splits,
                                                      float *__restrict__ part, int64_t mnp) {
    __shared__ u32x4 Asm[2][kPM * 8];   // [stage buffer][256 rows x 8 chunks]
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

    // A loader: rows ar + 64 i (i < 4), chunk ac.  Rows beyond M read row
    // M-1 (their results are dropped).
    const int ac = tid & 7;
    const int ar = tid >> 3;
    const int mlim = (int)min((int64_t)M - 1 - m0, (int64_t)kPM - 1);
    int arows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arows[i] = min(ar + 64 * i, mlim);
    const uint16_t *A_blk = A + m0 * K;
    const uint16_t *Ap_blk = Ap + m0 * Kp;
    const int a_lds = swz8(ar, ac);  // + 512 i

    // B loader: row brow, quarter bq (wave-uniform) of each group.
    const int brow = tid & (kPN - 1);
    const int bq = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int64_t bn_read = min(n0 + brow, (int64_t)N - 1);
    const uint8_t *bslot0 = wl.slot0(bn_read);
    const uint8_t *bscale0 = wl.scale0(bn_read);
    const int bstep = (int)wl.slot_step();
    const int sstep = (int)wl.scale_step();

    // MFMA operand rows and k-chunk of this lane.
    const int arow = wm * 64 + (lane & 15);
    const int bmrow = wn * 64 + (lane & 15);
    const int q = lane >> 4;

    u32x4 areg[4];
    uint32_t creg[B];
    f32x4_t tot[4][4], P[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Real stage s (64 k of group s/2), clamped to this split's last one.
    auto load_a = [&](int s) __attribute__((always_inline)) {
        s = min(s, 2 * g_hi - 1);
        const uint16_t *src = A_blk + (s >> 1) * kGroup + (s & 1) * kPK;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            areg[i] = *reinterpret_cast<const u32x4 *>(src + __mul24(arows[i], K) + 8 * ac);
    };
    auto store_a = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Asm[buf][a_lds + 512 * i] = areg[i];
    };
    // Quarter bq of real group g's codes (clamped to the last group): B
    // dwords at per-wave offsets held in scalar registers.
    int qoff[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
        const int d = bq * B + e;
        qoff[e] = __builtin_amdgcn_readfirstlane((d >> 2) * (WL::kTiled ? 1024 : 16) + (d & 3) * 4);
    }
    auto load_codes = [&](int g) __attribute__((always_inline)) {
        const uint8_t *slot = bslot0 + (int64_t)min(g, g_hi - 1) * bstep;
#pragma unroll
        for (int e = 0; e < B; ++e) creg[e] = *reinterpret_cast<const uint32_t *>(slot + qoff[e]);
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
    auto fold_block = [&](int i, int j, const float(&sq)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[i][j][r] = fmaf(sq[j], P[i][j][r], tot[i][j][r]);
    };

    // One 64-k stage of the wave's 4 x 4 blocks: 8 steps (k-step kk, row
    // block i) of 4 MFMAs.  After each MFMA, hook(step, j) issues a slice of
    // the stage's other work (about one MFMA's worth of VALU), and the pair
    // is fenced, so the order written here is the issue order: the matrix
    // core always has queued work while the VALU slices issue.  Operands of
    // step s+1 are read from LDS at the start of step s.  H = 0 opens a
    // group: k-step 0 starts each block from zero.
    auto mfma_stage = [&](int abuf, int gbuf, auto hconst, auto &&hook)
        __attribute__((always_inline)) {
        constexpr int H = decltype(hconst)::value;
        const u32x4 *as = Asm[abuf];
        const u32x4 *bs = Bsm[gbuf];
        bf16x8_t bfr[2][4], af[2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bfr[0][j] = __builtin_bit_cast(bf16x8_t, bs[swz16(bmrow + 16 * j, 8 * H + q)]);
        af[0] = __builtin_bit_cast(bf16x8_t, as[swz8(arow, q)]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int step = 0; step < 8; ++step) {
            const int kk = step >> 2, i = step & 3;
            if (i < 3) {
                af[(step + 1) & 1] =
                    __builtin_bit_cast(bf16x8_t, as[swz8(arow + 16 * (i + 1), 4 * kk + q)]);
            } else if (kk == 0) {
                af[(step + 1) & 1] = __builtin_bit_cast(bf16x8_t, as[swz8(arow, 4 + q)]);
            }
            if (step == 2) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bfr[1][j] = __builtin_bit_cast(bf16x8_t,
                                                   bs[swz16(bmrow + 16 * j, 8 * H + 4 + q)]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    af[step & 1], bfr[kk][j],
                    (H == 0 && kk == 0) ? f32x4_t{0.0f, 0.0f, 0.0f, 0.0f} : P[i][j], 0, 0, 0);
                hook(step, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Folding group t (scales sq) runs one row block behind its last
    // k-step: rows 0..2 during steps 5..7 of its closing stage, row 3
    // during step 0 of the next group's opening stage (before step 3
    // restarts P[3]).  P starts at zero, so the first such row-3 fold adds
    // nothing.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) P[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float sq_prev[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // ---- pseudo-groups (scale 1), not pipelined: A' from the pre-pass
    // matrix, B' = s[n, k'/3] (zero beyond 3G) ----
    {
        const float one[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        for (int ps = 0; ps < (sp == 0 ? NP : 0); ++ps) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint16_t *src = Ap_blk + ps * kPseudoK + h * kPK;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    areg[i] = *reinterpret_cast<const u32x4 *>(src + __mul24(arows[i], Kp) + 8 * ac);
                store_a(h);
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
            mfma_stage(0, 0, std::integral_constant<int, 0>{}, [&](int step, int j) {
                if (step == 0) fold_block(3, j, sq_prev);
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) sq_prev[j] = one[j];
            mfma_stage(1, 0, std::integral_constant<int, 1>{}, [&](int step, int j) {
                if (step >= 5) fold_block(step - 5, j, one);
            });
            lds_barrier();
        }
    }

    // ---- real groups, software-pipelined ----
    {
        // Prologue: group 0's B and scales, A stage 0 in LDS, A stage 1 and
        // the codes of group 1 in registers.
        load_codes(g_lo);
        fill_chunk(0, std::integral_constant<int, 0>{});
        fill_chunk(0, std::integral_constant<int, 1>{});
        fill_chunk(0, std::integral_constant<int, 2>{});
        fill_chunk(0, std::integral_constant<int, 3>{});
        store_scale(g_lo, 0);
        load_a(2 * g_lo);
        store_a(0);
        load_a(2 * g_lo + 1);
        load_codes(g_lo + 1);
        lds_barrier();

        for (int g = g_lo; g < g_hi; ++g) {
            const int gb = (g - g_lo) & 1, nb = gb ^ 1;
            float sq[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sq[j] = Ss[gb][wn * 64 + 16 * j + (lane & 15)];
            // stage 2g (A buffer 0): finish folding the previous group; write
            // A stage 2g+1, fetch A stage 2g+2; unpack group g+1 into the
            // other B buffer (past the end: a harmless rewrite of a buffer
            // nobody reads), one code pair per MFMA; fetch the codes of group
            // g+2.
            uint32_t pairs[16];
            mfma_stage(0, gb, std::integral_constant<int, 0>{}, [&](int step, int j) {
                if (step == 0) fold_block(3, j, sq_prev);
                if (step == 1 && j == 0) store_a(1);
                if (step == 2 && j == 0) load_a(2 * g + 2);
                if (step >= 4) {
                    const int pr = 4 * (step - 4) + j;
                    pairs[pr] = quarter_pair_dyn<B>(pr, creg, mask, magic);
                    if (j == 3)
                        Bsm[nb][swz16(brow, 4 * bq + (step - 4))] =
                            u32x4{pairs[pr - 3], pairs[pr - 2], pairs[pr - 1], pairs[pr]};
                    if (step == 7 && j == 3) {
                        store_scale(g + 1, nb);
                        load_codes(g + 2);
                    }
                }
            });
            lds_barrier();
            // stage 2g+1 (A buffer 1): write A stage 2g+2, fetch A stage
            // 2g+3; fold rows 0..2 of group g.
            mfma_stage(1, gb, std::integral_constant<int, 1>{}, [&](int step, int j) {
                if (step == 1 && j == 0) store_a(0);
                if (step == 2 && j == 0) load_a(2 * g + 3);
                if (step >= 5) fold_block(step - 5, j, sq);
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) sq_prev[j] = sq[j];
            lds_barrier();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) fold_block(3, j, sq_prev);
    }

    // Output element r of block (i, j): row 4*(lane/16) + r, column lane%16.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
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
