// ceilings.hip -- practical ceilings of MI355X for the two regimes of the
// quantized linear layer ("vLLM Quantization", Qwen3-8B demo: small batches
// wait on memory, big batches on compute).  Measurement kernels only: the
// benchmark times them next to the library's kernels so that each kernel can
// be placed against what the chip delivers, not only against its data sheet.
// Nothing here is part of libwq's hot path.
//
//   wqc_stream_read   a plain 128-bit streaming read: each workgroup reads
//                     one contiguous stretch of a buffer with 16-byte
//                     non-temporal loads, U loads in flight per lane, and
//                     folds the words into one value per thread (written to
//                     a sink so the loads are not removed).
//   wqc_mfma_loop     back-to-back MFMAs (bf16 32x32x16 / 16x16x32, int8
//                     16x16x64 / 32x32x32) on register operands into
//                     independent accumulators.
//   wqc_mfma_fold     the same MFMAs (bf16 32x32x16 or int8 32x32x32) with
//                     NV vector-ALU operations issued after each one: the
//                     per-group fold of the GEMM kernels (tot += s * P, one
//                     FMA per element for fp32 sums, an int -> float
//                     conversion and an FMA for int32 sums), which shares the
//                     issue port with the MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4v __attribute__((ext_vector_type(4)));

// Workgroup w reads bytes [w * chunk, min((w + 1) * chunk, bytes)) of buf;
// chunk16 (in 16-byte units) is rounded up by the host to a multiple of 256 U.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ buf,
                                                          int64_t n16, int64_t chunk16,
                                                          unsigned *__restrict__ sink) {
    const int64_t begin = (int64_t)blockIdx.x * chunk16;
    const int64_t end = begin + chunk16 < n16 ? begin + chunk16 : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = begin + threadIdx.x; i < end; i += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = i + 256 * u;
            v[u] = k < end ? __builtin_nontemporal_load(buf + k) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// C independent accumulators per wave; OP selects the instruction:
// 0 v_mfma_f32_32x32x16_bf16, 1 v_mfma_f32_16x16x32_bf16,
// 2 v_mfma_i32_16x16x64_i8, 3 v_mfma_i32_32x32x32_i8.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
template <int OP, int C>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
    i32x4v ai, bi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((lane + i) & 7);
        b[i] = (__bf16)(float)((lane * 3 + i) & 7);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ai[i] = (lane * 0x01030507) ^ (i * 0x11111111);
        bi[i] = (lane * 0x07050301) ^ (i * 0x01010101);
    }
    float s = 0.0f;
    if constexpr (OP == 0) {
        f32x16_t c[C];
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < C; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += c[j][r];
    } else if constexpr (OP == 1) {
        f32x4_t c[C];
#pragma unroll
        for (int j = 0; j < C; ++j) c[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < C; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    } else if constexpr (OP == 2) {
        i32x4_t c[C];
#pragma unroll
        for (int j = 0; j < C; ++j) c[j] = i32x4_t{0, 0, 0, 0};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < C; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, bi, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C; ++j) s += (float)(c[j][0] + c[j][1] + c[j][2] + c[j][3]);
    } else {
        i32x16_t c[C];
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[j][r] = 0;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < C; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, bi, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += (float)c[j][r];
    }
    sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// Two accumulator chains per wave; after each MFMA, NV vector-ALU ops fold
// 16 values of a finished block into fp32 totals.  OP 0: fp32 block of
// v_mfma_f32_32x32x16_bf16, one FMA per value; OP 1: int32 block of
// v_mfma_i32_32x32x32_i8, a conversion and an FMA per value (NV / 2
// values).  The folded values pass through an empty asm each time so the
// compiler can neither hoist nor drop the work.
template <int OP, int NV>
__global__ __launch_bounds__(256) void mfma_fold_kernel(int iters, float scale,
                                                        float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
    i32x4v ai, bi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((lane + i) & 7);
        b[i] = (__bf16)(float)((lane * 3 + i) & 7);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ai[i] = (lane * 0x01030507) ^ (i * 0x11111111);
        bi[i] = (lane * 0x07050301) ^ (i * 0x01010101);
    }
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = (float)r;
    float s = 0.0f;
    auto fold = [&](auto &q, int base) __attribute__((always_inline)) {
        if constexpr (OP == 0) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float x = q[(base + v) & 15];
                asm volatile("" : "+v"(x));
                t[(base + v) & 15] = fmaf(scale, x, t[(base + v) & 15]);
            }
        } else {
#pragma unroll
            for (int v = 0; v < NV / 2; ++v) {
                int x = q[(base + v) & 15];
                asm volatile("" : "+v"(x));
                t[(base + v) & 15] = fmaf(scale, (float)x, t[(base + v) & 15]);
            }
        }
    };
    if constexpr (OP == 0) {
        f32x16_t c0, c1, q;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            c0[r] = c1[r] = 0.0f;
            q[r] = (float)(lane * r);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
                fold(q, 2 * j * NV);
                __builtin_amdgcn_sched_barrier(0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
                fold(q, (2 * j + 1) * NV);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c0[r] + c1[r];
    } else {
        i32x16_t c0, c1, q;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            c0[r] = c1[r] = 0;
            q[r] = lane * r;
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, bi, c0, 0, 0, 0);
                fold(q, j * NV);
                __builtin_amdgcn_sched_barrier(0);
                c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ai, bi, c1, 0, 0, 0);
                fold(q, j * NV + 8);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s += (float)(c0[r] + c1[r]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s += t[r];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
}

template <int OP>
static void launch_fold(int nv, int wgs, int iters, float *sink, hipStream_t s) {
    switch (nv) {
        case 0: hipLaunchKernelGGL((mfma_fold_kernel<OP, 0>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
        case 2: hipLaunchKernelGGL((mfma_fold_kernel<OP, 2>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
        case 4: hipLaunchKernelGGL((mfma_fold_kernel<OP, 4>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
        case 6: hipLaunchKernelGGL((mfma_fold_kernel<OP, 6>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
        case 8: hipLaunchKernelGGL((mfma_fold_kernel<OP, 8>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
        case 10: hipLaunchKernelGGL((mfma_fold_kernel<OP, 10>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
        default: hipLaunchKernelGGL((mfma_fold_kernel<OP, 12>), dim3(wgs), dim3(256), 0, s, iters, 0.5f, sink); break;
    }
}

template <int OP>
static void launch_loop(int chains, int wgs, int iters, float *sink, hipStream_t s) {
    if (chains == 2)
        hipLaunchKernelGGL((mfma_loop_kernel<OP, 2>), dim3(wgs), dim3(256), 0, s, iters, sink);
    else if (chains == 8)
        hipLaunchKernelGGL((mfma_loop_kernel<OP, 8>), dim3(wgs), dim3(256), 0, s, iters, sink);
    else
        hipLaunchKernelGGL((mfma_loop_kernel<OP, 4>), dim3(wgs), dim3(256), 0, s, iters, sink);
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) at buf_d in `wgs` workgroups
// of 256 threads, U = unroll in {1, 2, 4, 8} loads in flight per lane.
// sink_d: wgs * 256 unsigned.  Returns a hipError_t value.
int wqc_stream_read(const void *buf_d, int64_t bytes, int wgs, int unroll, unsigned *sink_d,
                    void *stream) {
    if (!buf_d || !sink_d || bytes <= 0 || bytes % 16 || wgs <= 0) return (int)hipErrorInvalidValue;
    const int64_t n16 = bytes / 16;
    const int64_t per = 256 * (int64_t)unroll;
    int64_t chunk16 = (n16 + wgs - 1) / wgs;
    chunk16 = (chunk16 + per - 1) / per * per;
    hipStream_t s = (hipStream_t)stream;
    const u32x4 *b = static_cast<const u32x4 *>(buf_d);
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(wgs), dim3(256), 0, s, b, n16, chunk16, sink_d); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(wgs), dim3(256), 0, s, b, n16, chunk16, sink_d); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(wgs), dim3(256), 0, s, b, n16, chunk16, sink_d); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(wgs), dim3(256), 0, s, b, n16, chunk16, sink_d); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

// `wgs` workgroups of 4 waves, each wave `iters` x `chains` (2, 4 or 8)
// back-to-back MFMAs of instruction `op` (0: v_mfma_f32_32x32x16_bf16,
// 1: v_mfma_f32_16x16x32_bf16, 2: v_mfma_i32_16x16x64_i8,
// 3: v_mfma_i32_32x32x32_i8) into independent accumulators.  Work per
// call: wgs * 4 * iters * chains * (2 m n k) of that instruction.
// sink_d: wgs * 256 floats.  Returns a hipError_t value.
int wqc_mfma_loop(int op, int chains, int wgs, int iters, float *sink_d, void *stream) {
    if (!sink_d || wgs <= 0 || iters <= 0 || op < 0 || op > 3) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    switch (op) {
        case 0: launch_loop<0>(chains, wgs, iters, sink_d, s); break;
        case 1: launch_loop<1>(chains, wgs, iters, sink_d, s); break;
        case 2: launch_loop<2>(chains, wgs, iters, sink_d, s); break;
        default: launch_loop<3>(chains, wgs, iters, sink_d, s); break;
    }
    return (int)hipGetLastError();
}

// `wgs` workgroups of 4 waves, each wave `iters` x 16 MFMAs of instruction
// `op` (0: v_mfma_f32_32x32x16_bf16, 1: v_mfma_i32_32x32x32_i8) in two
// chains, with `nv` (0, 2, .., 12) vector-ALU fold operations after each.
// Work per call: wgs * 4 * iters * 16 * (2 m n k).  sink_d: wgs * 256
// floats.  Returns a hipError_t value.
int wqc_mfma_fold(int op, int nv, int wgs, int iters, float *sink_d, void *stream) {
    if (!sink_d || wgs <= 0 || iters <= 0 || op < 0 || op > 1 || nv < 0 || nv > 12 || nv % 2)
        return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    if (op == 0) launch_fold<0>(nv, wgs, iters, sink_d, s);
    else launch_fold<1>(nv, wgs, iters, sink_d, s);
    return (int)hipGetLastError();
}

}  // extern "C"
