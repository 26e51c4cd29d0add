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
// Tiling.  Workgroup 256 (m) x 128 (n), 4 waves as 2 x 2, each wave 128 x 64
// = 8 x 4 MFMA blocks of 16 x 16.  K runs in stages of 64 (half a group),
// double-buffered in LDS; the next stage is fetched into registers while the
// current one is multiplied, then written (A) or unpacked (B) into the other
// buffer.  Workgroups an XCD runs together share an A row block.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPM = 256;          // workgroup rows (m)
constexpr int kPN = 128;          // workgroup cols (n)
constexpr int kPK = 64;           // k per LDS stage
constexpr int kPRow = kPK + 8;    // bf16 per LDS row (16-byte pad)
constexpr int kPseudoK = 128;     // k' per pseudo-group

// Codes 2P, 2P+1 of a 32-code quarter slot held in B words.
template <int B, int P>
struct QSel {
    static constexpr int o0 = 2 * P * B;
    static constexpr int o1 = o0 + B;
    static constexpr int byte0 = o0 >> 3;
    static constexpr int byte1 = o1 >> 3;
    static constexpr int word = byte0 >> 2;
    static constexpr int base = 4 * word;
    static constexpr uint32_t sel = (uint32_t)(byte0 - base) |
                                    ((uint32_t)(byte0 + 1 - base) << 8) |
                                    ((uint32_t)(byte1 - base) << 16) |
                                    ((uint32_t)(byte1 + 1 - base) << 24);
    static constexpr int sh0 = o0 & 7;
    static constexpr int sh1 = o1 & 7;
    static constexpr bool has_hi = word + 1 < B;
};

template <int B, int P>
__device__ __forceinline__ uint32_t quarter_pair(const uint32_t *w, uint32_t mask,
                                                 uint32_t magic) {
    if constexpr (B == 8) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const uint32_t x = w[P >> 1];
        f32x2 f;
        f.x = (float)((x >> (16 * (P & 1))) & 0xFFu);
        f.y = (float)((x >> (16 * (P & 1) + 8)) & 0xFFu);
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    } else {
        using S = QSel<B, P>;
        const uint32_t lo = w[S::word];
        const uint32_t hi = S::has_hi ? w[S::word + 1] : 0u;
        uint32_t x = __builtin_amdgcn_perm(hi, lo, S::sel);
        if constexpr (S::sh0 != 0 || S::sh1 != 0) x = pk_shr16(x, S::sh0, S::sh1);
        return and_or(x, mask, magic);
    }
}

template <int B, int P>
struct QuarterPairs {
    __device__ __forceinline__ static void run(const uint32_t *w, uint32_t mask, uint32_t magic,
                                               uint32_t *out) {
        out[P] = quarter_pair<B, P>(w, mask, magic);
        QuarterPairs<B, P + 1>::run(w, mask, magic, out);
    }
};
template <int B>
struct QuarterPairs<B, 16> {
    __device__ __forceinline__ static void run(const uint32_t *, uint32_t, uint32_t,
                                               uint32_t *) {}
};

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

// One LDS stage (64 k = two 16x16x32 k-steps) of a wave's 8 x 4 blocks.
// FIRST: the stage opens a group, so the first k-step starts from zero.
template <bool FIRST>
__device__ __forceinline__ void compute_stage(const uint16_t *as, const uint16_t *bs, int arow,
                                              int brow_w, int kq, f32x4_t (&P)[8][4]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t bfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8_t *>(
                &bs[(brow_w + 16 * j) * kPRow + 32 * kk + kq]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t *>(
                &as[(arow + 16 * i) * kPRow + 32 * kk + kq]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (FIRST && kk == 0)
                    P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af, bfr[j], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                else
                    P[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], P[i][j], 0, 0, 0);
            }
        }
    }
}

template <int B, class WL>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ Ap, int M,
                                                         int N, int K, int Kp, WL wl,
                                                         uint16_t *__restrict__ Y, int mtiles,
                                                         int ntiles) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kPM * kPRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kPN * kPRow];
    __shared__ float Ss[2][kPN];

    const int G = K / kGroup;
    const int nreal = 2 * G;                      // stages of real groups
    const int nstages = nreal + 2 * (Kp / kPseudoK);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Block b runs on XCD b % 8: give each XCD a contiguous run of logical
    // tiles, n fastest, so the tiles an XCD runs together share A rows.
    const int total = mtiles * ntiles;
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bm = logical / ntiles;
    const int bn = logical - bm * ntiles;
    const int64_t m0 = (int64_t)bm * kPM;
    const int64_t n0 = (int64_t)bn * kPN;

    const uint32_t mask = __builtin_amdgcn_readfirstlane(pair_mask<B < 8 ? B : 7>());
    const uint32_t magic = in_vgpr(kBf16Magic128x2);

    // Loader roles.  A: 256 rows x 64 k = 2048 uint4, 8 per thread: rows
    // arow0 + 32 i, 16-byte column ac.  Rows beyond M read row M-1 (results
    // dropped).  B: row brow of the tile, half bpart of the stage's 64 codes
    // (a quarter slot of 32 codes = B dwords).
    const int arow0 = tid >> 3, ac = tid & 7;
    int aoff[8], apoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t m = min(m0 + arow0 + 32 * i, (int64_t)M - 1);
        aoff[i] = (int)((m - m0) * K) + 8 * ac;
        apoff[i] = (int)((m - m0) * Kp) + 8 * ac;
    }
    const uint16_t *A_blk = A + m0 * K;
    const uint16_t *Ap_blk = Ap + m0 * Kp;
    const int brow = tid & 127;
    const int bpart = tid >> 7;
    const int64_t bn_row = n0 + brow;
    const int64_t bn_read = bn_row < N ? bn_row : (int64_t)N - 1;
    const uint8_t *bslot0 = wl.slot0(bn_read);
    const uint8_t *bscale0 = wl.scale0(bn_read);
    const int64_t bstep = wl.slot_step();
    const int64_t sstep = wl.scale_step();

    uint4 areg[8];
    uint32_t breg[16];
    float sreg = 1.0f;

    auto fetch = [&](int s) {
        const int grp = s >> 1, h = s & 1;
        if (s < nreal) {
            const uint16_t *src = A_blk + grp * kGroup + h * kPK;
#pragma unroll
            for (int i = 0; i < 8; ++i) areg[i] = *reinterpret_cast<const uint4 *>(src + aoff[i]);
            const uint8_t *slot = bslot0 + grp * bstep;
            const int qi = 2 * h + bpart;  // quarter of the slot
            if (qi == 0) {
#pragma unroll
                for (int e = 0; e < B; ++e)
                    breg[e] = *reinterpret_cast<const uint32_t *>(slot + WL::dword_off(e));
            } else if (qi == 1) {
#pragma unroll
                for (int e = 0; e < B; ++e)
                    breg[e] = *reinterpret_cast<const uint32_t *>(slot + WL::dword_off(B + e));
            } else if (qi == 2) {
#pragma unroll
                for (int e = 0; e < B; ++e)
                    breg[e] = *reinterpret_cast<const uint32_t *>(slot + WL::dword_off(2 * B + e));
            } else {
#pragma unroll
                for (int e = 0; e < B; ++e)
                    breg[e] = *reinterpret_cast<const uint32_t *>(slot + WL::dword_off(3 * B + e));
            }
            sreg = bf16_to_f32(*reinterpret_cast<const uint16_t *>(bscale0 + grp * sstep));
        } else {
            const int kbase = (s - nreal) * kPK;
            const uint16_t *src = Ap_blk + kbase;
#pragma unroll
            for (int i = 0; i < 8; ++i) areg[i] = *reinterpret_cast<const uint4 *>(src + apoff[i]);
            // S'[n][k'] = s[n][k'/3] for k' < 3G, else 0: 32 values, 16 pairs.
            const int k0 = kbase + 32 * bpart;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ka = k0 + 2 * e, kb = ka + 1;
                const uint32_t sa =
                    ka < 3 * G ? *reinterpret_cast<const uint16_t *>(bscale0 + (ka / 3) * sstep) : 0u;
                const uint32_t sb =
                    kb < 3 * G ? *reinterpret_cast<const uint16_t *>(bscale0 + (kb / 3) * sstep) : 0u;
                breg[e] = sa | (sb << 16);
            }
            sreg = 1.0f;
        }
    };

    auto store = [&](int s, int buf) {
        uint16_t *as = As[buf];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = tid + 256 * i;
            const int row = idx >> 3, c = idx & 7;
            *reinterpret_cast<uint4 *>(&as[row * kPRow + 8 * c]) = areg[i];
        }
        uint32_t pairs[16];
        if (s < nreal) {
            QuarterPairs<B, 0>::run(breg, mask, magic, pairs);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) pairs[e] = breg[e];
        }
        uint4 *bs = reinterpret_cast<uint4 *>(&Bs[buf][brow * kPRow + 32 * bpart]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bs[i] = make_uint4(pairs[4 * i], pairs[4 * i + 1], pairs[4 * i + 2], pairs[4 * i + 3]);
        if (bpart == 0) Ss[buf][brow] = sreg;
    };

    f32x4_t tot[8][4], P[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[i][j][r] = 0.0f;

    fetch(0);
    store(0, 0);
    __syncthreads();

    const int arow = wm * 128 + (lane & 15);
    const int brow_w = wn * 64 + (lane & 15);
    const int kq = 8 * (lane >> 4);

    for (int s = 0; s < nstages; ++s) {
        const int buf = s & 1;
        if (s + 1 < nstages) fetch(s + 1);

        const uint16_t *as = As[buf];
        const uint16_t *bs = Bs[buf];
        if ((s & 1) == 0)
            compute_stage<true>(as, bs, arow, brow_w, kq, P);
        else
            compute_stage<false>(as, bs, arow, brow_w, kq, P);
        if (s & 1) {  // group complete: total += s[n, g] * P
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sc = Ss[buf][wn * 64 + 16 * j + (lane & 15)];
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tot[i][j][r] = fmaf(sc, P[i][j][r], tot[i][j][r]);
            }
        }
        if (s + 1 < nstages) store(s + 1, buf ^ 1);
        __syncthreads();
    }

    // Output element r of block (i, j): row 4*(lane/16) + r, column lane%16.
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + wn * 64 + 16 * j + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 128 + 16 * i + 4 * (lane >> 4) + r;
                if (m < M && n < N) Y[m * N + n] = f32_to_bf16_rne(tot[i][j][r]);
            }
        }
}

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

static int pseudo_kp(int64_t K) {
    const int G = (int)(K / kGroup);
    return (3 * G + kPseudoK - 1) / kPseudoK * kPseudoK;
}

// Workspace: the shared counter region (unused here), then the pre-pass
// matrix [M, Kp] bf16.
int64_t prefill_ws_bytes(int64_t M, int64_t, int64_t K, int) {
    return kWsScratchOffset + align256(M * pseudo_kp(K) * 2);
}

template <int B>
static hipError_t prefill_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                            bool tiled, const uint16_t *scales, uint16_t *Y, void *ws,
                            hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int Kp = pseudo_kp(K);
    uint16_t *Ap = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    const float off = (B == 8) ? 128.0f : (float)(128 + (1 << (B - 1)));
    hipLaunchKernelGGL(group_sum_split_kernel, dim3((unsigned)M), dim3(256), 0, stream, A, (int)K,
                       Kp, off, Ap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int mtiles = (int)((M + kPM - 1) / kPM);
    const int ntiles = (int)((N + kPN - 1) / kPN);
    const dim3 grid((unsigned)(mtiles * ntiles));
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((prefill_kernel<B, TiledW>), grid, dim3(256), 0, stream, A, Ap,
                           (int)M, (int)N, (int)K, Kp, wl, Y, mtiles, ntiles);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((prefill_kernel<B, DenseW>), grid, dim3(256), 0, stream, A, Ap,
                           (int)M, (int)N, (int)K, Kp, wl, Y, mtiles, ntiles);
    }
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
