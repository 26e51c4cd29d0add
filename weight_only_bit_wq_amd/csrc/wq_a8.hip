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
//   2. gemm_a8_kernel: int8 MFMA (v_mfma_i32_32x32x32_i8) with exact int32
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
#include <type_traits>

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
// never crosses a 16-byte chunk), else dwords.  Ordinary (temporal) loads:
// every M-tile of the layer reads the same codes again.
template <class WL, int B>
__device__ __forceinline__ void load_quarter(const uint8_t *slot, int q, uint32_t *w) {
    const int d0 = B * q;
    if constexpr (B % 4 == 0) {
#pragma unroll
        for (int i = 0; i < B / 4; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(slot + WL::dword_off(d0 + 4 * i));
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else if constexpr (B % 2 == 0) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < B / 2; ++i) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(slot + WL::dword_off(d0 + 2 * i));
            w[2 * i] = v.x; w[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int e = 0; e < B; ++e)
            w[e] = *reinterpret_cast<const uint32_t *>(slot + WL::dword_off(d0 + e));
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

constexpr int kABM = 256, kABN = 128;  // workgroup tile (m x n)
constexpr int kAW = kABM / 32;          // waves: (kABM / 64) x 2 of 64 x 64
constexpr int kAQ = 4 * kABN / (64 * kAW);  // 32-code quarters each thread stages per group

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Tail balance.  One workgroup per compute unit (the tile's LDS buffers
// take 97 KB) and 256 compute units, so the tiles run in rounds of 256.
// When the last round would be at most half full (M = 2048 at N = 17408:
// 1088 tiles, 4 rounds and 64 tiles), its tiles are split along K into up
// to 4 parts (at least 4 groups each), which fill the last round with
// shorter workgroups; they store fp32 partials and a second kernel adds
// them in split order.  (Measured on MI355X at K 5120 -> N 17408: M = 2048
// took 98% of the time of M = 2304, 12.5% more work.)  The split tiles are
// the last in logical order and run last.
constexpr int kA8Slots = 256;
struct A8Plan {
    int tiles;   // all tiles
    int full;    // tiles run whole (the first `full` in logical order)
    int splits;  // K parts of each remaining tile (1: none)
};
static A8Plan a8_plan(int64_t M, int64_t N, int64_t K) {
    A8Plan p;
    p.tiles = (int)(((M + kABM - 1) / kABM) * ((N + kABN - 1) / kABN));
    p.full = p.tiles;
    p.splits = 1;
    const int G = (int)(K / kGroup);
    const int r = p.tiles % kA8Slots;
    if (p.tiles >= kA8Slots && r > 0 && 2 * r <= kA8Slots) {
        const int s = std::min(std::min(kA8Slots / r, 4), G / 4);
        if (s >= 2) {
            p.full = p.tiles - r;
            p.splits = s;
        }
    }
    return p;
}
static int64_t a8_part_bytes(const A8Plan &p) {
    return (int64_t)(p.tiles - p.full) * p.splits * kABM * kABN * 4;
}

// Workspace: the shared counter region (unused here, left zero), then Aq
// (GEMM k-order), s_a and the tail tiles' partials.
int64_t a8_ws_bytes(int64_t M, int64_t N, int64_t K) {
    return kWsScratchOffset + align256(M * K) + align256(M * 4) +
           align256(a8_part_bytes(a8_plan(M, N, K)));
}

// LDS rows of 128 bytes (8 chunks of 16 int8 = 16 k); chunk c of row r sits
// at c ^ ((r / 2) mod 8): the 16 consecutive rows of one chunk that an
// operand read or a code store touches land in 16 distinct 16-byte bank
// groups (row parity picks the half of the 256 bytes, r / 2 the slot).
__device__ __forceinline__ int a8_swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Workgroup: 512 threads = 8 waves (two per SIMD) over a 256 (m) x 128 (n)
// tile; wave (wm, wn) owns 64 x 64 = 2 x 2 blocks of v_mfma_i32_32x32x32_i8
// (lane l: row / column l % 32 of a block's operands, k-half l / 32 of the
// k-step; result column l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4 in
// register r).  Per group of 128 k: 4 k-steps x 4 MFMAs into exact int32
// sums P, then tot += (s/16) * float(P) (fp32): 64 conversions and FMAs per
// lane, as much vector-ALU time as the MFMAs take on the matrix cores.  The
// fold is spread evenly over the MFMA slots: each group runs block row 0,
// then block row 1, each over the four k-steps, and every MFMA slot folds 4
// sums of the block row the matrix core is not writing (see group below).
// Data: A (int8, GEMM k-order) goes global -> LDS by direct loads, the codes
// through registers (widened to int8 on their way into LDS), both double-
// buffered in separate LDS objects (so the compiler sees that the reads of
// one buffer do not wait for loads into the other).  At the start of group
// g a wave stores group g + 1's widened codes (fetched during g - 1), then
// issues group g + 2's code fetch and group g + 1's A loads.
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <class WL, int B, bool ZP>
__global__ __launch_bounds__(64 * kAW) void gemm_a8_kernel(const int8_t *__restrict__ Aq,
                                                      const float *__restrict__ sa, int M, int N,
                                                      int K, WL wl,
                                                      const uint8_t *__restrict__ zeros,
                                                      void *__restrict__ Y,
                                                      bool out_f32, int mtiles, int ntiles,
                                                      int nfull, int tsplits,
                                                      float *__restrict__ part) {
    __shared__ u32x4 As0[kABM * 8];  // 128 bytes per row: 32 KB each
    __shared__ u32x4 As1[kABM * 8];
    __shared__ u32x4 Bs0[kABN * 8];  // 16 KB each
    __shared__ u32x4 Bs1[kABN * 8];
    __shared__ float Ss[2][kABN];

    const int G = K / kGroup;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Block b < nfull runs whole tile b, remapped: block b runs on XCD
    // b % 8, and each XCD takes a contiguous run of logical tiles, n fastest,
    // so the tiles it runs together share A rows.  Blocks past nfull run
    // part sp of the K split of tile nfull + (b - nfull) / tsplits.
    const int b = blockIdx.x;
    int logical = b, sp = 0, g_lo = 0, g_hi = G;
    if (b < nfull) {
        if ((nfull & 7) == 0) logical = (b & 7) * (nfull >> 3) + (b >> 3);
    } else {
        const int j = b - nfull;
        logical = nfull + j / tsplits;
        sp = j - (j / tsplits) * tsplits;
        g_lo = (int)((int64_t)G * sp / tsplits);
        g_hi = (int)((int64_t)G * (sp + 1) / tsplits);
    }
    const int bm = logical / ntiles;
    const int bn = logical - bm * ntiles;
    const int64_t m0 = (int64_t)bm * kABM;
    const int64_t n0 = (int64_t)bn * kABN;

    // A direct loads: instruction u of wave w fills LDS slots 64 (w + W u)
    // .. +63 (W waves), rows 8 (w + W u) .. +7; lane l writes slot l of them:
    // row 8 (w + W u) + l / 8, physical chunk l % 8, which holds logical
    // chunk (l % 8) ^ ((row / 2) % 8) (a8_swz).  Rows beyond M read row M-1.
    constexpr int AU = kABM / (8 * kAW);  // direct loads per wave per group
    const int mlim = (int)min((int64_t)M - 1 - m0, (int64_t)kABM - 1);
    const int8_t *A_blk = Aq + m0 * K;
    uint32_t aoff[AU];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
        const int row = 8 * (wave + kAW * u) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        aoff[u] = (uint32_t)(min(row, mlim) * K + 16 * chunk);
    }
    auto dma_a = [&](int g, u32x4 *dst) __attribute__((always_inline)) {
        g = min(g, g_hi - 1);
        const int8_t *src = A_blk + (int64_t)g * kGroup;
#pragma unroll
        for (int u = 0; u < AU; ++u)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(src + aoff[u]),
                (__attribute__((address_space(3))) void *)&dst[64 * (wave + kAW * u)], 16, 0, 0);
    };

    // B loader: row brow, quarters bj + (64 kAW / kABN) i (i < kAQ, wave-
    // uniform) = codes 32 q .. +32 of the group (b = 4: 16-byte chunk q);
    // widened to int8 quarter q fills LDS chunks 2 q and 2 q + 1.
    const int brow = tid & (kABN - 1);
    const int bj = __builtin_amdgcn_readfirstlane(tid >> 7);
    constexpr int kQStep = 64 * kAW / kABN;
    const int64_t bn_read = min(n0 + brow, (int64_t)N - 1);
    const uint8_t *bslot0 = wl.slot0(bn_read);
    const uint8_t *bscale0 = wl.scale0(bn_read);
    const int bstep = (int)wl.slot_step();
    const int sstep = (int)wl.scale_step();
    const uint8_t *zrow = ZP ? zeros + bn_read * G : nullptr;  // zero points [N, G]

    // MFMA operand rows and k-half of this lane.
    const int r32 = lane & 31, hh = lane >> 5;
    const int arow = wm * 64 + r32;
    const int bmrow = wn * 64 + r32;

    uint32_t breg[kAQ][B];
    uint16_t sreg;
    uint32_t zreg = 0;
    i32x16_t P[2][2];  // [block row][block column]
    f32x16_t tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                tot[i][j][r] = 0.0f;
                P[i][j][r] = 0;
            }

    auto fetch_b = [&](int g) __attribute__((always_inline)) {  // clamped to the last group
        g = min(g, g_hi - 1);
#pragma unroll
        for (int i = 0; i < kAQ; ++i)
            load_quarter<WL, B>(bslot0 + (int64_t)g * bstep, bj + kQStep * i, breg[i]);
        sreg = *reinterpret_cast<const uint16_t *>(bscale0 + (int64_t)g * sstep);
        if constexpr (ZP) zreg = zrow[g];
    };
    auto store_b = [&](u32x4 *Bsm, float *Sr) __attribute__((always_inline)) {
#pragma unroll
      for (int qi = 0; qi < kAQ; ++qi) {
        const int bq = bj + kQStep * qi;
        const uint32_t *breg_q = breg[qi];
        if constexpr (ZP) {  // b = 4: int8 c - z, codes ordered as below
            const u32x4 x = u32x4{breg_q[0], breg_q[1], breg_q[2], breg_q[3]};
            const uint32_t zb = zreg * 0x01010101u;
            auto lo = [&](uint32_t v) {
                return (((v & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
            };
            auto hi = [&](uint32_t v) {
                return ((((v >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
            };
            Bsm[a8_swz(brow, 2 * bq)] = u32x4{lo(x.x), hi(x.x), lo(x.y), hi(x.y)};
            Bsm[a8_swz(brow, 2 * bq + 1)] = u32x4{lo(x.z), hi(x.z), lo(x.w), hi(x.w)};
        } else if constexpr (B == 4) {
            const u32x4 x = u32x4{breg_q[0], breg_q[1], breg_q[2], breg_q[3]} ^ 0x88888888u;
            Bsm[a8_swz(brow, 2 * bq)] =
                u32x4{(x.x << 4) & 0xF0F0F0F0u, x.x & 0xF0F0F0F0u, (x.y << 4) & 0xF0F0F0F0u,
                      x.y & 0xF0F0F0F0u};
            Bsm[a8_swz(brow, 2 * bq + 1)] =
                u32x4{(x.z << 4) & 0xF0F0F0F0u, x.z & 0xF0F0F0F0u, (x.w << 4) & 0xF0F0F0F0u,
                      x.w & 0xF0F0F0F0u};
        } else if constexpr (WL::kTiled && int8_ready<B>()) {
            // The tiled layout's arranged run decodes straight to the int8
            // values q * 2^(8-b), natural order.
            uint32_t o[8];
            run_int8<B>(breg_q, o);
            Bsm[a8_swz(brow, 2 * bq)] = u32x4{o[0], o[1], o[2], o[3]};
            Bsm[a8_swz(brow, 2 * bq + 1)] = u32x4{o[4], o[5], o[6], o[7]};
        } else {
            Bsm[a8_swz(brow, 2 * bq)] = u32x4{widen4<B, 0>(breg_q), widen4<B, 1>(breg_q),
                                              widen4<B, 2>(breg_q), widen4<B, 3>(breg_q)};
            Bsm[a8_swz(brow, 2 * bq + 1)] = u32x4{widen4<B, 4>(breg_q), widen4<B, 5>(breg_q),
                                                  widen4<B, 6>(breg_q), widen4<B, 7>(breg_q)};
        }
      }
        // The waves holding a row's quarters store the same value: no branch.
        Sr[brow] = bf16_to_f32(sreg) * (ZP ? 1.0f : 1.0f / (float)(1 << (8 - B)));
    };
    // tot += s * P for elements 4 q .. 4 q + 3 of block (i, j): four
    // conversions and four FMAs, pinned in their MFMA slot by an empty asm.
    auto fold4 = [&](int i, int j, int q, float sc) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
            float t = fmaf(sc, (float)P[i][j][r], tot[i][j][r]);
            asm volatile("" : "+v"(t));
            tot[i][j][r] = t;
        }
    };

    // Prologue: group g_lo's A and codes in buffer 0, group g_lo + 1's codes
    // in registers.
    dma_a(g_lo, As0);
    fetch_b(g_lo);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    store_b(Bs0, Ss[0]);
    fetch_b(g_lo + 1);

    // Each group runs in two phases of 8 MFMA slots: phase 0 runs block row
    // 0 (blocks (0, 0), (0, 1)) over the group's four k-steps and folds
    // block row 1 of the previous group; phase 1 runs block row 1 and folds
    // block row 0 of this group (block (0, 0) from phase 1's first slot, two
    // MFMAs after its last one; block (0, 1) from its fifth).  Every MFMA
    // slot carries the same fold work (4 conversions, 4 FMAs) in both waves
    // of a SIMD, so neither runs a long stretch of vector-ALU work with the
    // matrix core idle.  The B operands of the group's four k-steps are read
    // during phase 0 and kept for phase 1; the A operand one k-step ahead.
    float sq_prev[2] = {0.0f, 0.0f};
    auto group = [&](int g, auto bufc) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bufc)::value;
        const u32x4 *as = BUF ? As1 : As0;
        const u32x4 *bs = BUF ? Bs1 : Bs0;
        // Group g's A (loaded during g - 1) and codes (stored at the start
        // of g - 1) are in buffer BUF for every wave, and every wave is done
        // with the other buffer.  Fenced: the scheduler would otherwise move
        // the previous group's MFMAs and folds past this wait, which then
        // stalls on loads issued just before.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        store_b(BUF ? Bs0 : Bs1, Ss[BUF ^ 1]);  // group g + 1's codes
        fetch_b(g + 2);
        dma_a(g + 1, BUF ? As0 : As1);
        __builtin_amdgcn_sched_barrier(0);  // the loads go out now
        float sq[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) sq[j] = Ss[BUF][wn * 64 + 32 * j + r32];
        i32x4_t bf[4][2], af[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf[0][j] = __builtin_bit_cast(i32x4_t, bs[a8_swz(bmrow + 32 * j, hh)]);
        af[0] = __builtin_bit_cast(i32x4_t, as[a8_swz(arow, hh)]);
        static_for<0, 16>([&](auto sc) __attribute__((always_inline)) {
            constexpr int S = decltype(sc)::value;
            constexpr int PH = S >> 3, kk = (S & 7) >> 1, j = S & 1;
            if constexpr (j == 0) {
                if constexpr (kk + 1 < 4) {
                    af[(kk + 1) & 1] = __builtin_bit_cast(
                        i32x4_t, as[a8_swz(arow + 32 * PH, 2 * (kk + 1) + hh)]);
                    if constexpr (PH == 0) {
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj)
                            bf[kk + 1][jj] = __builtin_bit_cast(
                                i32x4_t, bs[a8_swz(bmrow + 32 * jj, 2 * (kk + 1) + hh)]);
                    }
                } else if constexpr (PH == 0) {
                    af[0] = __builtin_bit_cast(i32x4_t, as[a8_swz(arow + 32, hh)]);
                }
            }
            const i32x16_t zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            P[PH][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kk & 1], bf[kk][j],
                                                            kk == 0 ? zero : P[PH][j], 0, 0, 0);
            if constexpr (PH == 0) fold4(1, S >> 2, S & 3, sq_prev[S >> 2]);
            else fold4(0, (S - 8) >> 2, S & 3, sq[(S - 8) >> 2]);
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < 2; ++j) sq_prev[j] = sq[j];
    };
    int g = g_lo;
    for (; g + 1 < g_hi; g += 2) {
        group(g, std::integral_constant<int, 0>{});
        group(g + 1, std::integral_constant<int, 1>{});
    }
    if (g < g_hi) group(g, std::integral_constant<int, 0>{});
    // The last group's block row 1.
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) fold4(1, j, q, sq_prev[j]);
    // Drain the (clamped, unused) loads issued for the groups after the last:
    // no direct load may still be writing LDS when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Output register r of block (i, j): row 8 (r / 4) + 4 (lane / 32) + r % 4,
    // column lane % 32.  A part of a split tile stores its fp32 sums (before
    // the s_a factor) at [part][split tile][row of the tile][column].
    const int64_t mw = m0 + wm * 64 + 4 * hh;  // row of register 0, block row 0
    if (b >= nfull) {
        float *pt = part + ((int64_t)sp * (mtiles * ntiles - nfull) + (logical - nfull)) *
                                   (kABM * kABN);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t n = n0 + wn * 64 + 32 * j + r32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = mw + 32 * i + 8 * (r >> 2) + (r & 3);
                    if (m < M && n < N) pt[(m - m0) * kABN + (n - n0)] = tot[i][j][r];
                }
            }
        return;
    }
    // The s_a factors of the lane's 32 rows, all loaded before the first is
    // used (rows 4 q .. 4 q + 3 of a block row are consecutive: one 16-byte
    // load; past row M - 1 the loads read row M - 1).
    float sv[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t m = mw + 32 * i + 8 * q;
            if (m + 3 < M) {
                const f32x4_t v = *reinterpret_cast<const f32x4_t *>(sa + m);
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[i][4 * q + e] = v[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[i][4 * q + e] = sa[min(m + e, (int64_t)M - 1)];
            }
        }
    if (!out_f32 && m0 + kABM <= M && n0 + kABN <= N) {
        // A whole tile in bf16: each register's 64 values go to two 64-byte
        // row runs; the row offset is wave-uniform, the lane's offset fixed.
        uint16_t *Yw = static_cast<uint16_t *>(Y) + (m0 + wm * 64) * N + n0 + wn * 64;
        const uint32_t lo = (uint32_t)(4 * hh) * (uint32_t)N + (uint32_t)r32;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    (Yw + (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * N + 32 * j)[lo] =
                            f32_to_bf16_rne(sv[i][r] * tot[i][j][r]);
        return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = mw + 32 * i + 8 * (r >> 2) + (r & 3);
                if (m < M && n < N) {
                    const float y = sv[i][r] * tot[i][j][r];
                    if (out_f32)
                        static_cast<float *>(Y)[m * N + n] = y;
                    else
                        static_cast<uint16_t *>(Y)[m * N + n] = f32_to_bf16_rne(y);
                }
            }
        }
}

// The split tiles' outputs: thread t takes 4 consecutive columns of one row
// of split tile t / (kABM kABN / 4), adds the parts' sums in part order and
// applies s_a, as the whole-tile epilogue does.
__global__ __launch_bounds__(256) void a8_tail_reduce_kernel(const float *__restrict__ part,
                                                             const float *__restrict__ sa,
                                                             int splits, int nfull, int nsplit,
                                                             int ntiles, int M, int N,
                                                             void *__restrict__ Y, bool out_f32) {
    constexpr int kQuads = kABM * kABN / 4;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int ts = (int)(t / kQuads);
    if (ts >= nsplit) return;
    const int e = (int)(t - (int64_t)ts * kQuads) * 4;
    const int tile = nfull + ts;
    const int bm = tile / ntiles, bn = tile - (tile / ntiles) * ntiles;
    const int64_t m = (int64_t)bm * kABM + e / kABN;
    const int64_t n = (int64_t)bn * kABN + e % kABN;
    if (m >= M || n >= N) return;
    const int64_t stride = (int64_t)nsplit * (kABM * kABN);  // floats from one part to the next
    const float *p = part + (int64_t)ts * (kABM * kABN) + e;
    // All (at most 4) loads before the first add; indices past the last part
    // repeat it and are not added.
    float4 v[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = *reinterpret_cast<const float4 *>(p + min(s, splits - 1) * stride);
    float acc[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
    for (int s = 1; s < 4; ++s) {
        if (s < splits) {
            acc[0] += v[s].x;
            acc[1] += v[s].y;
            acc[2] += v[s].z;
            acc[3] += v[s].w;
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (n + c >= N) break;
        const float y = sa[m] * acc[c];
        if (out_f32)
            static_cast<float *>(Y)[m * N + n + c] = y;
        else
            static_cast<uint16_t *>(Y)[m * N + n + c] = f32_to_bf16_rne(y);
    }
}

template <int B, bool ZP>
static hipError_t launch_gemm_a8_b(const int8_t *Aq, const float *sa, int64_t M, int64_t N,
                                   int64_t K, const void *W, bool tiled, const uint16_t *scales,
                                   const uint8_t *zeros, void *Y, bool out_f32, float *part,
                                   hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int mtiles = (int)((M + kABM - 1) / kABM);
    const int ntiles = (int)((N + kABN - 1) / kABN);
    const A8Plan p = a8_plan(M, N, K);
    const int nsplit = p.tiles - p.full;
    const dim3 grid((unsigned)(p.full + nsplit * p.splits));
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((gemm_a8_kernel<TiledW, B, ZP>), grid, dim3(64 * kAW), 0, stream, Aq, sa,
                           (int)M, (int)N, (int)K, wl, zeros, Y, out_f32, mtiles, ntiles,
                           p.full, p.splits, part);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((gemm_a8_kernel<DenseW, B, ZP>), grid, dim3(64 * kAW), 0, stream, Aq, sa,
                           (int)M, (int)N, (int)K, wl, zeros, Y, out_f32, mtiles, ntiles,
                           p.full, p.splits, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit == 0) return e;
    const int64_t threads = (int64_t)nsplit * (kABM * kABN / 4);
    hipLaunchKernelGGL(a8_tail_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, stream, part, sa, p.splits, p.full, nsplit, ntiles, (int)M, (int)N, Y,
                       out_f32);
    return hipGetLastError();
}

hipError_t launch_gemm_a8(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                          void *Y, bool out_f32, void *ws, hipStream_t stream) {
    int8_t *Aq = reinterpret_cast<int8_t *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    float *sa = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kWsScratchOffset +
                                          align256(M * K));
    float *part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kWsScratchOffset +
                                            align256(M * K) + align256(M * 4));
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
                                         part, stream);
    }
    switch (b) {
        case 2:
            return launch_gemm_a8_b<2, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
        case 3:
            return launch_gemm_a8_b<3, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
        case 4:
            return launch_gemm_a8_b<4, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
        case 5:
            return launch_gemm_a8_b<5, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
        case 6:
            return launch_gemm_a8_b<6, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
        case 7:
            return launch_gemm_a8_b<7, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
        case 8:
            return launch_gemm_a8_b<8, false>(Aq, sa, M, N, K, W, tiled, scales, nullptr, Y,
                                              out_f32, part, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
