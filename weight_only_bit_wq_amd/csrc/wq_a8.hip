// wq_a8.hip -- int8 activations on b-bit weights (b = 4: W4A8).
//
// club-3090 discussion #733, "Under the hood": activations are quantized per
// token to int8 at run time, the int4 weights widen to int8 without loss and
// the product runs on int8 matrix units; the same int4 checkpoint and group
// scales as the weight-only path are used.  ("Which slugs": the widening has
// to be lossless, which is why a float format is refused there; integer
// codes of any b <= 8 widen losslessly, so every b runs here, b = 8 being
// W8A8.)  Here:
//   1. quant_act_kernel: s_a[m] = max|a| / 127 (fp32, IEEE division),
//      Aq = clamp(rint(a / s_a), -127, 127), zero row -> 0.
//   2. gemm_a8_kernel: int8 MFMA (v_mfma_i32_16x16x64_i8) with exact int32
//      sums per group of 128, folded in fp32 with the group scale, times s_a.
//
// Lossless widening with one AND per four codes: XOR-ing a nibble c with 8
// gives the 4-bit two's-complement encoding of c - 8; placed in the high
// nibble of a byte it reads as the int8 value 16 * (c - 8).  The factor 16 is
// removed exactly by using s/16 as the group scale.  A 32-bit word of eight
// codes yields two int8x4 registers: even codes ((x << 4) & 0xF0F0F0F0) and
// odd codes (x & 0xF0F0F0F0), so within every 8 consecutive k the B operand
// is ordered (0,2,4,6,1,3,5,7); the activation bytes are written in the same
// order, which leaves the contraction unchanged.
//
// Other widths, same idea: the b-bit field c ^ 2^(b-1) is the b-bit two's
// complement of c - 2^(b-1); shifted to the top of its byte it reads as the
// int8 value (c - 2^(b-1)) * 2^(8-b), and the group scale becomes
// s / 2^(8-b) (exact).  Codes are pulled out in pairs with the unpacker's
// byte-window selectors, four fields packed into a dword with one v_perm_b32,
// then shifted and XOR-ed (b = 8: the code bytes XOR 0x80); in the tiled
// layout the runs of b = 5, 6, 7 are stored arranged (wq_device.h) and
// decode to those int8 values with a few masks and bit-field inserts.  The
// k order is the natural one for b != 4, and the activations are written in
// it.
// Group sums stay exact: |Aq| <= 127, |w * 2^(8-b)| <= 128, 128 terms.
//
// Zero points (b = 4 only: at b = 8, c - z can leave the int8 range): the
// nibbles go to the low half of their bytes (even and odd codes apart, the
// same k order), and ((c | 0x80) - z) ^ 0x80 per byte is the int8 c - z
// (128 + c - z lies in 113..143, so no byte borrows from its neighbour); the
// group scale is s itself.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 activations (one uint4 of bf16) -> 8 int8 codes, as two dwords.
// PERM: order (0,2,4,6 | 1,3,5,7) for the GEMM; else natural order.
template <bool PERM>
__device__ __forceinline__ uint2 quant8(uint4 v, float s, bool zero) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float a = __uint_as_float(h ? (in[i] & 0xFFFF0000u) : (in[i] << 16));
            float r = zero ? 0.0f : rintf(a / s);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            q[2 * i + h] = (uint32_t)(int)r & 0xFFu;
        }
    }
    uint2 out;
    if (PERM) {
        out.x = q[0] | (q[2] << 8) | (q[4] << 16) | (q[6] << 24);
        out.y = q[1] | (q[3] << 8) | (q[5] << 16) | (q[7] << 24);
    } else {
        out.x = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        out.y = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
    }
    return out;
}

// Codes 2P, 2P+1 of a 32-code quarter slot held in B words, as the low bits
// of the two 16-bit halves (masked).
template <int B, int P>
__device__ __forceinline__ uint32_t quarter_fields(const uint32_t *w) {
    using S = QSel<B, P>;
    const uint32_t lo = w[S::word];
    const uint32_t hi = S::has_hi ? w[S::word + 1] : 0u;
    uint32_t x = __builtin_amdgcn_perm(hi, lo, S::sel);
    if constexpr (S::sh0 != 0 || S::sh1 != 0) x = pk_shr16(x, S::sh0, S::sh1);
    return x & pair_mask<B>();
}

// Codes 4I .. 4I+3 of a quarter as four int8 (c - 2^(b-1)) * 2^(8-b), in order.
template <int B, int I>
__device__ __forceinline__ uint32_t widen4(const uint32_t *w) {
    if constexpr (B == 8) {
        return w[I] ^ 0x80808080u;
    } else {
        const uint32_t x = __builtin_amdgcn_perm(quarter_fields<B, 2 * I + 1>(w),
                                                 quarter_fields<B, 2 * I>(w), 0x06040200u);
        return (x << (8 - B)) ^ 0x80808080u;
    }
}

// Quarter q (dwords [B q, B q + B)) of the slot starting at `slot`, with q
// wave-uniform: 16-byte loads when B % 4 == 0, 8-byte when B is even (a pair
// never crosses a 16-byte chunk), else dwords.
template <class WL, int B>
__device__ __forceinline__ void load_quarter(const uint8_t *slot, int q, uint32_t *w) {
    const int d0 = B * q;
    if constexpr (B % 4 == 0) {
#pragma unroll
        for (int i = 0; i < B / 4; ++i) {
            const u32x4 v = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(slot + WL::dword_off(d0 + 4 * i)));
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else if constexpr (B % 2 == 0) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < B / 2; ++i) {
            const u32x2 v = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2 *>(slot + WL::dword_off(d0 + 2 * i)));
            w[2 * i] = v.x; w[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int e = 0; e < B; ++e)
            w[e] = __builtin_nontemporal_load(
                reinterpret_cast<const uint32_t *>(slot + WL::dword_off(d0 + e)));
    }
}

// One workgroup (256 threads) per activation row.
template <bool PERM>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t *__restrict__ A, int K,
                                                        int8_t *__restrict__ Aq,
                                                        float *__restrict__ sa) {
    __shared__ float wmax[4];
    const int64_t m = blockIdx.x;
    const uint4 *row = reinterpret_cast<const uint4 *>(A + m * K);
    const int nv = K / 8;
    float amax = 0.0f;
    for (int i = threadIdx.x; i < nv; i += 256) {
        const uint4 v = row[i];
        const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = fmaxf(amax, fabsf(__uint_as_float(in[j] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(in[j] & 0xFFFF0000u)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax / 127.0f;
    const bool zero = !(amax > 0.0f);
    if (threadIdx.x == 0) sa[m] = s;
    uint2 *out = reinterpret_cast<uint2 *>(Aq + m * K);
    for (int i = threadIdx.x; i < nv; i += 256) out[i] = quant8<PERM>(row[i], s, zero);
}

hipError_t launch_quant_act(const uint16_t *A, int64_t M, int64_t K, int8_t *Aq, float *sa,
                            hipStream_t stream) {
    hipLaunchKernelGGL((quant_act_kernel<false>), dim3((unsigned)M), dim3(256), 0, stream, A,
                       (int)K, Aq, sa);
    return hipGetLastError();
}

constexpr int kABM = 256, kABN = 128;

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace: the shared counter region (unused here, left zero), then Aq
// (GEMM k-order) and s_a.
int64_t a8_ws_bytes(int64_t M, int64_t, int64_t K) {
    return kWsScratchOffset + align256(M * K) + align256(M * 4);
}

// LDS rows of 128 bytes (8 chunks of 16 int8 = 16 k); chunk c of row r sits
// at c ^ (r mod 8), so an operand read (16 rows, one chunk) and the loaders'
// row-major writes are conflict free.
__device__ __forceinline__ int a8_swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// Workgroup: 512 threads = 8 waves (two per SIMD) over a 256 (m) x 128 (n)
// tile; wave (wm, wn) owns 64 x 64 = 4 x 4 blocks of v_mfma_i32_16x16x64_i8.
// Per group of 128 k: 2 k-steps x 16 MFMAs into exact int32 sums P, then
// tot += (s/16) * float(P) (fp32).  A (int8, GEMM k-order) and the widened
// B of a group sit in LDS (double-buffered, 32 + 16 KB per buffer); the next
// group's A and codes are fetched into registers during the current one.
// The fold runs one row block behind the group's last MFMAs (row 3 during
// the next group's first k-step), one block per MFMA, so it issues in the
// matrix core's shadow.
template <class WL, int B, bool ZP>
__global__ __launch_bounds__(512) void gemm_a8_kernel(const int8_t *__restrict__ Aq,
                                                      const float *__restrict__ sa, int M, int N,
                                                      int K, WL wl,
                                                      const uint8_t *__restrict__ zeros,
                                                      void *__restrict__ Y,
                                                      bool out_f32, int mtiles, int ntiles) {
    __shared__ u32x4 Asm[2][kABM * 8];  // 2 x 32 KB
    __shared__ u32x4 Bsm[2][kABN * 8];  // 2 x 16 KB
    __shared__ float Ss[2][kABN];

    const int G = K / kGroup;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Block b runs on XCD b % 8: each XCD takes a contiguous run of logical
    // tiles, n fastest, so the tiles it runs together share A rows.
    const int total = mtiles * ntiles;
    int logical = blockIdx.x;
    if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bm = logical / ntiles;
    const int bn = logical - bm * ntiles;
    const int64_t m0 = (int64_t)bm * kABM;
    const int64_t n0 = (int64_t)bn * kABN;

    // A loader: rows ar + 64 i (i < 4), chunk ac; rows beyond M read row M-1.
    const int ac = tid & 7;
    const int ar = tid >> 3;
    const int mlim = (int)min((int64_t)M - 1 - m0, (int64_t)kABM - 1);
    int arows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arows[i] = min(ar + 64 * i, mlim);
    const int8_t *A_blk = Aq + m0 * K;
    const int a_lds = a8_swz(ar, ac);  // + 512 i

    // B loader: row brow, quarter bj (wave-uniform) = codes 32 bj .. +32 of
    // the group (b = 4: 16-byte chunk bj); widened to int8 it fills LDS
    // chunks 2 bj and 2 bj + 1.
    const int brow = tid & (kABN - 1);
    const int bj = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int64_t bn_read = min(n0 + brow, (int64_t)N - 1);
    const uint8_t *bslot0 = wl.slot0(bn_read);
    const uint8_t *bscale0 = wl.scale0(bn_read);
    const int bstep = (int)wl.slot_step();
    const int sstep = (int)wl.scale_step();
    const uint8_t *zrow = ZP ? zeros + bn_read * G : nullptr;  // zero points [N, G]

    // MFMA operand rows and k-chunk of this lane.
    const int arow = wm * 64 + (lane & 15);
    const int bmrow = wn * 64 + (lane & 15);
    const int q = lane >> 4;

    u32x4 areg[4];
    uint32_t breg[B];
    uint16_t sreg;
    uint32_t zreg = 0;
    i32x4_t P[4][4];
    f32x4_t tot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tot[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            P[i][j] = i32x4_t{0, 0, 0, 0};
        }

    auto fetch = [&](int g) __attribute__((always_inline)) {  // clamped to the last group
        g = min(g, G - 1);
        const int8_t *src = A_blk + (int64_t)g * kGroup + 16 * ac;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            areg[i] = *reinterpret_cast<const u32x4 *>(src + (int64_t)arows[i] * K);
        load_quarter<WL, B>(bslot0 + (int64_t)g * bstep, bj, breg);
        sreg = *reinterpret_cast<const uint16_t *>(bscale0 + (int64_t)g * sstep);
        if constexpr (ZP) zreg = zrow[g];
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Asm[buf][a_lds + 512 * i] = areg[i];
        if constexpr (ZP) {  // b = 4: int8 c - z, codes ordered as below
            const u32x4 x = u32x4{breg[0], breg[1], breg[2], breg[3]};
            const uint32_t zb = zreg * 0x01010101u;
            auto lo = [&](uint32_t v) {
                return (((v & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
            };
            auto hi = [&](uint32_t v) {
                return ((((v >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
            };
            Bsm[buf][a8_swz(brow, 2 * bj)] = u32x4{lo(x.x), hi(x.x), lo(x.y), hi(x.y)};
            Bsm[buf][a8_swz(brow, 2 * bj + 1)] = u32x4{lo(x.z), hi(x.z), lo(x.w), hi(x.w)};
        } else if constexpr (B == 4) {
            const u32x4 x = u32x4{breg[0], breg[1], breg[2], breg[3]} ^ 0x88888888u;
            Bsm[buf][a8_swz(brow, 2 * bj)] =
                u32x4{(x.x << 4) & 0xF0F0F0F0u, x.x & 0xF0F0F0F0u, (x.y << 4) & 0xF0F0F0F0u,
                      x.y & 0xF0F0F0F0u};
            Bsm[buf][a8_swz(brow, 2 * bj + 1)] =
                u32x4{(x.z << 4) & 0xF0F0F0F0u, x.z & 0xF0F0F0F0u, (x.w << 4) & 0xF0F0F0F0u,
                      x.w & 0xF0F0F0F0u};
        } else if constexpr (WL::kTiled && int8_ready<B>()) {
            // The tiled layout's arranged run decodes straight to the int8
            // values q * 2^(8-b), natural order.
            uint32_t o[8];
            run_int8<B>(breg, o);
            Bsm[buf][a8_swz(brow, 2 * bj)] = u32x4{o[0], o[1], o[2], o[3]};
            Bsm[buf][a8_swz(brow, 2 * bj + 1)] = u32x4{o[4], o[5], o[6], o[7]};
        } else {
            Bsm[buf][a8_swz(brow, 2 * bj)] = u32x4{widen4<B, 0>(breg), widen4<B, 1>(breg),
                                                   widen4<B, 2>(breg), widen4<B, 3>(breg)};
            Bsm[buf][a8_swz(brow, 2 * bj + 1)] = u32x4{widen4<B, 4>(breg), widen4<B, 5>(breg),
                                                       widen4<B, 6>(breg), widen4<B, 7>(breg)};
        }
        // The four chunk waves of a row store the same value: no branch.
        Ss[buf][brow] = bf16_to_f32(sreg) * (ZP ? 1.0f : 1.0f / (float)(1 << (8 - B)));
    };
    auto fold_block = [&](int i, int j, const float(&sq)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[i][j][r] = fmaf(sq[j], (float)P[i][j][r], tot[i][j][r]);
    };

    float sq_prev[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    fetch(0);
    store(0);
    fetch(1);
    lds_barrier();

    for (int g = 0; g < G; ++g) {
        const int gb = g & 1;
        float sq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sq[j] = Ss[gb][wn * 64 + 16 * j + (lane & 15)];
        const u32x4 *as = Asm[gb];
        const u32x4 *bs = Bsm[gb];
        i32x4_t bfr[2][4], af[2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bfr[0][j] = __builtin_bit_cast(i32x4_t, bs[a8_swz(bmrow + 16 * j, q)]);
        af[0] = __builtin_bit_cast(i32x4_t, as[a8_swz(arow, q)]);
        __builtin_amdgcn_sched_barrier(0);
        // 8 steps (k-step kk, row block i) of 4 MFMAs; each MFMA is followed
        // by its slice of the other work, fenced so this is the issue order.
#pragma unroll
        for (int step = 0; step < 8; ++step) {
            const int kk = step >> 2, i = step & 3;
            if (i < 3)
                af[(step + 1) & 1] =
                    __builtin_bit_cast(i32x4_t, as[a8_swz(arow + 16 * (i + 1), 4 * kk + q)]);
            else if (kk == 0)
                af[(step + 1) & 1] = __builtin_bit_cast(i32x4_t, as[a8_swz(arow, 4 + q)]);
            if (step == 2) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bfr[1][j] = __builtin_bit_cast(i32x4_t, bs[a8_swz(bmrow + 16 * j, 4 + q)]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                P[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    af[step & 1], bfr[kk][j], kk == 0 ? i32x4_t{0, 0, 0, 0} : P[i][j], 0, 0, 0);
                if (step == 0) fold_block(3, j, sq_prev);  // previous group's row 3
                if (step >= 5) fold_block(step - 5, j, sq);
                if (step == 3 && j == 0) store(gb ^ 1);    // group g+1 into the other buffer
                if (step == 4 && j == 0) fetch(g + 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sq_prev[j] = sq[j];
        lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) fold_block(3, j, sq_prev);

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
                    const float y = sa[m] * tot[i][j][r];
                    if (out_f32)
                        static_cast<float *>(Y)[m * N + n] = y;
                    else
                        static_cast<uint16_t *>(Y)[m * N + n] = f32_to_bf16_rne(y);
                }
            }
        }
}

template <int B, bool ZP>
static hipError_t launch_gemm_a8_b(const int8_t *Aq, const float *sa, int64_t M, int64_t N,
                                   int64_t K, const void *W, bool tiled, const uint16_t *scales,
                                   const uint8_t *zeros, void *Y, bool out_f32,
                                   hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int mtiles = (int)((M + kABM - 1) / kABM);
    const int ntiles = (int)((N + kABN - 1) / kABN);
    const dim3 grid((unsigned)(mtiles * ntiles));
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((gemm_a8_kernel<TiledW, B, ZP>), grid, dim3(512), 0, stream, Aq, sa,
                           (int)M, (int)N, (int)K, wl, zeros, Y, out_f32, mtiles, ntiles);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((gemm_a8_kernel<DenseW, B, ZP>), grid, dim3(512), 0, stream, Aq, sa,
                           (int)M, (int)N, (int)K, wl, zeros, Y, out_f32, mtiles, ntiles);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_a8(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                          void *Y, bool out_f32, void *ws, hipStream_t stream) {
    int8_t *Aq = reinterpret_cast<int8_t *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    float *sa = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kWsScratchOffset +
                                          align256(M * K));
    // b = 4 takes the (0,2,4,6,1,3,5,7) k order of its widening; others the natural one.
    if (b == 4)
        hipLaunchKernelGGL((quant_act_kernel<true>), dim3((unsigned)M), dim3(256), 0, stream, A,
                           (int)K, Aq, sa);
    else
        hipLaunchKernelGGL((quant_act_kernel<false>), dim3((unsigned)M), dim3(256), 0, stream, A,
                           (int)K, Aq, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (zeros) {  // b = 4 only (checked at the boundary)
        if (b != 4) return hipErrorInvalidValue;
        return launch_gemm_a8_b<4, true>(Aq, sa, M, N, K, W, tiled, scales, zeros, Y, out_f32,
                                         stream);
    }
    switch (b) {
        case 2:
            return launch_gemm_a8_b<2, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
        case 3:
            return launch_gemm_a8_b<3, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
        case 4:
            return launch_gemm_a8_b<4, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
        case 5:
            return launch_gemm_a8_b<5, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
        case 6:
            return launch_gemm_a8_b<6, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
        case 7:
            return launch_gemm_a8_b<7, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
        case 8:
            return launch_gemm_a8_b<8, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
