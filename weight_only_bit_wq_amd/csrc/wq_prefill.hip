// wq_prefill.hip -- WNA16 prefill path (M > 16): LDS-tiled bf16 MFMA GEMM.
//
// At large batch the layer is compute-bound ("vLLM Quantization", Key points
// and Pitfalls: weight-only gains fade as batch grows), so the codes are
// dequantized once per workgroup tile into LDS and the product runs on the
// matrix cores (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// Exactness: the B operand holds 128 + c as bf16 (exact for c < 128, built
// with the same perm/shift/and_or unpacker as the decode path; b = 8 uses
// byte conversion).  Each group of 128 k is accumulated into its own fp32
// block, then folded into the running total in fp32 as
//     total += s[n,g] * (P_g - (128 + 2^(b-1)) * sum_{k in g} a[m,k])
// so neither the codes nor the scale are ever rounded to bf16.
//
// Tiles: workgroup 128 (m) x 128 (n), 4 waves as 2 x 2, each wave 64 x 64
// = 2 x 2 MFMA blocks of 32 x 32.  One group (128 k) per LDS stage.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPBM = 128;          // workgroup rows (m)
constexpr int kPBN = 128;          // workgroup cols (n)
constexpr int kLdsRow = 128 + 8;   // bf16 per LDS row (16-byte pad against bank conflicts)

template <int B, int P>
struct DequantPairs {
    __device__ __forceinline__ static void run(const uint32_t *w, uint32_t mask, uint32_t magic,
                                               uint32_t *dst) {
        if constexpr (B == 8) {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            const uint32_t x = w[P >> 1];
            f32x2 f;
            f.x = (float)((x >> (16 * (P & 1))) & 0xFFu);
            f.y = (float)((x >> (16 * (P & 1) + 8)) & 0xFFu);
            dst[P] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
        } else {
            dst[P] = code_pair_bf16_plus128<B, P>(w, mask, magic);
        }
        DequantPairs<B, P + 1>::run(w, mask, magic, dst);
    }
};
template <int B>
struct DequantPairs<B, 64> {
    __device__ __forceinline__ static void run(const uint32_t *, uint32_t, uint32_t, uint32_t *) {}
};

template <int B, class WL>
__global__ __launch_bounds__(256) void prefill_kernel(const uint16_t *__restrict__ A, int M,
                                                      int N, int K, WL wl,
                                                      uint16_t *__restrict__ Y, int mtiles) {
    __shared__ __attribute__((aligned(16))) uint16_t As[kPBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kPBN * kLdsRow];
    __shared__ float asum_s[kPBM];
    __shared__ float scale_s[kPBN];

    const int G = K / kGroup;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int bm = blockIdx.x % mtiles;
    const int bn = blockIdx.x / mtiles;
    const int64_t m0 = (int64_t)bm * kPBM;
    const int64_t n0 = (int64_t)bn * kPBN;
    constexpr float kOff = (B == 8) ? 128.0f : (float)(128 + (1 << (B - 1)));

    const uint32_t mask = __builtin_amdgcn_readfirstlane(pair_mask<B < 8 ? B : 7>());
    const uint32_t magic = in_vgpr(kBf16Magic128x2);

    f32x16_t tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.0f;

    for (int g = 0; g < G; ++g) {
        // A tile: 128 rows x 128 k bf16 = 2048 uint4, 8 per thread.
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = tid + 256 * it;
            const int row = idx >> 4, c16 = idx & 15;
            const int64_t m = m0 + row;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < M)
                v = *reinterpret_cast<const uint4 *>(A + m * K + (int64_t)g * kGroup + c16 * 8);
            *reinterpret_cast<uint4 *>(&As[row * kLdsRow + c16 * 8]) = v;
        }
        // B tile: threads 0..127 unpack one slot (row n0 + t, group g) each.
        if (tid < kPBN) {
            const int64_t n = n0 + tid;
            const int64_t nr = n < N ? n : (int64_t)N - 1;
            uint32_t w[4 * B];
            load_slot<B>(wl.chunks(nr, g), wl.chunk_stride(), w);
            uint32_t pairs[64];
            DequantPairs<B, 0>::run(w, mask, magic, pairs);
            uint4 *dst = reinterpret_cast<uint4 *>(&Bs[tid * kLdsRow]);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                dst[i] = make_uint4(pairs[4 * i], pairs[4 * i + 1], pairs[4 * i + 2], pairs[4 * i + 3]);
            scale_s[tid] = bf16_to_f32(wl.scale(nr, g));
        }
        __syncthreads();
        // Activation sums of this group: thread pair (2r, 2r+1) sums row r.
        {
            const int row = tid >> 1, half = tid & 1;
            const uint32_t *ap = reinterpret_cast<const uint32_t *>(&As[row * kLdsRow + half * 64]);
            float sacc = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) sacc = dot2_bf16(ap[i], 0x3F803F80u, sacc);
            sacc += __shfl_xor(sacc, 1, 64);
            if (half == 0) asum_s[row] = sacc;
        }
        __syncthreads();

        f32x16_t P[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) P[i][j][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            bf16x8_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t *>(
                    &As[(wm * 64 + i * 32 + (lane & 31)) * kLdsRow + ks * 16 + (lane >> 5) * 8]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t *>(
                    &Bs[(wn * 64 + j * 32 + (lane & 31)) * kLdsRow + ks * 16 + (lane >> 5) * 8]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    P[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], P[i][j], 0, 0, 0);
        }
        // Fold the group: output element r of block (i, j) in this lane is
        // row 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of the block.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float s = scale_s[wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ml = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    tot[i][j][r] = fmaf(s, fmaf(-kOff, asum_s[ml], P[i][j][r]), tot[i][j][r]);
                }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) Y[m * N + n] = f32_to_bf16_rne(tot[i][j][r]);
            }
        }
}

int64_t prefill_ws_bytes(int64_t, int64_t, int64_t, int) { return 0; }

template <int B>
static hipError_t prefill_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                            bool tiled, const uint16_t *scales, uint16_t *Y, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int mtiles = (int)((M + kPBM - 1) / kPBM);
    const int ntiles = (int)((N + kPBN - 1) / kPBN);
    const dim3 grid((unsigned)(mtiles * ntiles));
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((prefill_kernel<B, TiledW>), grid, dim3(256), 0, stream, A, (int)M,
                           (int)N, (int)K, wl, Y, mtiles);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((prefill_kernel<B, DenseW>), grid, dim3(256), 0, stream, A, (int)M,
                           (int)N, (int)K, wl, Y, mtiles);
    }
    return hipGetLastError();
}

hipError_t launch_prefill(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, int b, uint16_t *Y, void *,
                          hipStream_t stream) {
    switch (b) {
        case 2: return prefill_b<2>(A, M, N, K, W, tiled, scales, Y, stream);
        case 3: return prefill_b<3>(A, M, N, K, W, tiled, scales, Y, stream);
        case 4: return prefill_b<4>(A, M, N, K, W, tiled, scales, Y, stream);
        case 5: return prefill_b<5>(A, M, N, K, W, tiled, scales, Y, stream);
        case 6: return prefill_b<6>(A, M, N, K, W, tiled, scales, Y, stream);
        case 7: return prefill_b<7>(A, M, N, K, W, tiled, scales, Y, stream);
        case 8: return prefill_b<8>(A, M, N, K, W, tiled, scales, Y, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
