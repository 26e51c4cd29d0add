// wq_a8.hip -- W4A8: per-token int8 activations on int4 weights.
//
// club-3090 discussion #733, "Under the hood": activations are quantized per
// token to int8 at run time, the int4 weights widen to int8 without loss and
// the product runs on int8 matrix units; the same int4 checkpoint and group
// scales as the weight-only path are used.  Here:
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
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

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

constexpr int kABM = 128, kABN = 128;
constexpr int kA8Row = 128 + 16;  // bytes per LDS row (pad)

static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace: the shared counter region (unused here, left zero), then Aq
// (GEMM k-order) and s_a.
int64_t a8_ws_bytes(int64_t M, int64_t, int64_t K) {
    return kWsScratchOffset + align256(M * K) + align256(M * 4);
}

template <class WL>
__global__ __launch_bounds__(256) void gemm_a8_kernel(const int8_t *__restrict__ Aq,
                                                      const float *__restrict__ sa, int M, int N,
                                                      int K, WL wl, void *__restrict__ Y,
                                                      bool out_f32, int mtiles) {
    __shared__ __attribute__((aligned(16))) uint8_t As[kABM * kA8Row];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[kABN * kA8Row];
    __shared__ float scale_s[kABN];

    const int G = K / kGroup;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int bm = blockIdx.x % mtiles;
    const int bn = blockIdx.x / mtiles;
    const int64_t m0 = (int64_t)bm * kABM;
    const int64_t n0 = (int64_t)bn * kABN;

    float tot[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.0f;

    for (int g = 0; g < G; ++g) {
        // A tile: 128 rows x 128 int8 (already in GEMM k-order), 4 uint4 per thread.
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + 256 * it;
            const int row = idx >> 3, c16 = idx & 7;
            const int64_t m = m0 + row;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < M)
                v = *reinterpret_cast<const uint4 *>(Aq + m * K + (int64_t)g * kGroup + c16 * 16);
            *reinterpret_cast<uint4 *>(&As[row * kA8Row + c16 * 16]) = v;
        }
        if (tid < kABN) {
            const int64_t n = n0 + tid;
            const int64_t nr = n < N ? n : (int64_t)N - 1;
            uint32_t w[16];
            load_slot<4>(wl.chunks(nr, g), wl.chunk_stride(), w);
            uint4 *dst = reinterpret_cast<uint4 *>(&Bs[tid * kA8Row]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t x0 = w[2 * i] ^ 0x88888888u, x1 = w[2 * i + 1] ^ 0x88888888u;
                dst[i] = make_uint4((x0 << 4) & 0xF0F0F0F0u, x0 & 0xF0F0F0F0u,
                                    (x1 << 4) & 0xF0F0F0F0u, x1 & 0xF0F0F0F0u);
            }
            scale_s[tid] = bf16_to_f32(wl.scale(nr, g)) * 0.0625f;
        }
        __syncthreads();

        i32x16_t P[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) P[i][j][r] = 0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            i32x4_t af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const i32x4_t *>(
                    &As[(wm * 64 + i * 32 + (lane & 31)) * kA8Row + ks * 32 + (lane >> 5) * 16]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const i32x4_t *>(
                    &Bs[(wn * 64 + j * 32 + (lane & 31)) * kA8Row + ks * 32 + (lane >> 5) * 16]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    P[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bfr[j], P[i][j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float s16 = scale_s[wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    tot[i][j][r] = fmaf(s16, (float)P[i][j][r], tot[i][j][r]);
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

hipError_t launch_gemm_a8(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, void *Y, bool out_f32, void *ws,
                          hipStream_t stream) {
    int8_t *Aq = reinterpret_cast<int8_t *>(static_cast<uint8_t *>(ws) + kWsScratchOffset);
    float *sa = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kWsScratchOffset +
                                          align256(M * K));
    hipLaunchKernelGGL((quant_act_kernel<true>), dim3((unsigned)M), dim3(256), 0, stream, A,
                       (int)K, Aq, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = (int)(K / kGroup);
    const int mtiles = (int)((M + kABM - 1) / kABM);
    const int ntiles = (int)((N + kABN - 1) / kABN);
    const dim3 grid((unsigned)(mtiles * ntiles));
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, 4};
        hipLaunchKernelGGL((gemm_a8_kernel<TiledW>), grid, dim3(256), 0, stream, Aq, sa, (int)M,
                           (int)N, (int)K, wl, Y, out_f32, mtiles);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), scales, (int64_t)16 * 4 * G, G, 4};
        hipLaunchKernelGGL((gemm_a8_kernel<DenseW>), grid, dim3(256), 0, stream, Aq, sa, (int)M,
                           (int)N, (int)K, wl, Y, out_f32, mtiles);
    }
    return hipGetLastError();
}

}  // namespace wq
