// wq_unpack.hip -- the offline repack into the tiled layout, and the device
// unpacker export (codes out of either layout, through the same in-register
// unpacker the GEMMs use).
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

// One thread per (64-row block R, group g, row r in block): copies the b
// 16-byte chunks of that slot into plane j of the tile (lanes = rows, so each
// plane store is 1 KB contiguous per wave) and the scale after the planes.
// For b = 5, 6, 7 each 32-code run of the slot is first rewritten in the
// int8-ready arrangement (signed values, see wq_device.h); other widths keep
// the dense stream's bits.  Rows >= N are written as zero words and zero
// scales.  Scales are read at n * sG + g * sg: (G, 1) for group scales,
// (1, 0) for one scale per row (per-channel), which every group of the row
// then carries.
template <int B>
__global__ __launch_bounds__(256) void repack_tiled_kernel(const uint32_t *__restrict__ packed,
                                                          const uint16_t *__restrict__ scales,
                                                          int64_t N, int G, int sG, int sg,
                                                          int rowblocks,
                                                          uint8_t *__restrict__ out) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t slots = (int64_t)rowblocks * G * 64;
    if (tid >= slots) return;
    const int r = (int)(tid & 63);
    const int64_t tile_idx = tid >> 6;  // = R * G + g
    const int g = (int)(tile_idx % G);
    const int64_t R = tile_idx / G;
    const int64_t n = R * 64 + r;
    uint8_t *tile = out + tile_idx * (int64_t)tile_bytes(B);
    uint4 *dst = reinterpret_cast<uint4 *>(tile) + r;
    if (n < N) {
        const uint4 *src = reinterpret_cast<const uint4 *>(
            reinterpret_cast<const uint8_t *>(packed) + n * (int64_t)(16 * B * G) +
            (int64_t)g * 16 * B);
        if constexpr (int8_ready<B>()) {
            uint32_t w[4 * B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const uint4 c = src[j];
                w[4 * j] = c.x; w[4 * j + 1] = c.y; w[4 * j + 2] = c.z; w[4 * j + 3] = c.w;
            }
            constexpr uint32_t mask = (1u << B) - 1u;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t v[32], d[B];
#pragma unroll
                for (int k = 0; k < 32; ++k) {
                    const int o = k * B, i = o >> 5, sh = o & 31;
                    const uint64_t win = (uint64_t)w[q * B + i] |
                                         ((i + 1 < B) ? (uint64_t)w[q * B + i + 1] << 32 : 0ull);
                    v[k] = ((uint32_t)(win >> sh) & mask) ^ (1u << (B - 1));
                }
                arrange_run<B>(v, d);
#pragma unroll
                for (int i = 0; i < B; ++i) w[q * B + i] = d[i];
            }
#pragma unroll
            for (int j = 0; j < B; ++j)
                dst[j * 64] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < B; ++j) dst[j * 64] = src[j];
        }
        reinterpret_cast<uint16_t *>(tile + tile_code_bytes(B))[r] = scales[n * sG + g * sg];
    } else {
        const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < B; ++j) dst[j * 64] = z;
        reinterpret_cast<uint16_t *>(tile + tile_code_bytes(B))[r] = 0;
    }
}

// Four codes (pairs a = codes 0,1 and b = codes 2,3 as 16-bit halves) -> 4 bytes.
__device__ __forceinline__ uint32_t pairs_to_bytes(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x06040200u);
}

template <int B, int P>
struct UnpackStep {
    __device__ __forceinline__ static void run(const uint32_t *w, uint32_t *out) {
        out[P / 2] = pairs_to_bytes(code_pair<B, P>(w), code_pair<B, P + 1>(w));
        UnpackStep<B, P + 2>::run(w, out);
    }
};
template <int B>
struct UnpackStep<B, 64> {
    __device__ __forceinline__ static void run(const uint32_t *, uint32_t *) {}
};

// One thread per slot (row n, group g); writes 128 code bytes.
template <int B, class WL>
__global__ __launch_bounds__(256) void unpack_kernel(WL wl, int64_t N, int G, bool tiled,
                                                    uint8_t *__restrict__ codes) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t n;
    int g;
    if (tiled) {  // lanes = rows of one tile: coalesced plane loads
        const int64_t tile_idx = tid >> 6;
        g = (int)(tile_idx % G);
        n = (tile_idx / G) * 64 + (tid & 63);
    } else {      // lanes = consecutive groups of one row: contiguous loads
        n = tid / G;
        g = (int)(tid % G);
    }
    if (n >= N) return;
    uint32_t w[4 * B];
    load_slot<B>(wl.chunks(n, g), wl.chunk_stride(), w);
    uint32_t out[32];
    if constexpr (int8_ready<B>()) {
        if (tiled) {
            // Arranged runs: int8 q * 2^(8-b) per byte -> c = q + 2^(b-1).
            uint32_t o[32];
#pragma unroll
            for (int q = 0; q < 4; ++q) run_int8<B>(w + q * B, o + q * 8);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                uint32_t x = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int qv = (int)(int8_t)(uint8_t)(o[i] >> (8 * e)) >> (8 - B);
                    x |= (uint32_t)(qv + (1 << (B - 1))) << (8 * e);
                }
                out[i] = x;
            }
        } else {
            UnpackStep<B, 0>::run(w, out);
        }
    } else {
        UnpackStep<B, 0>::run(w, out);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes + n * (int64_t)G * kGroup + (int64_t)g * kGroup);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

template <int B>
static hipError_t repack_b(const uint32_t *packed, const uint16_t *scales, int64_t N, int G,
                           bool per_channel, void *out, hipStream_t stream) {
    const int rowblocks = (int)((N + 63) / 64);
    const int64_t slots = (int64_t)rowblocks * G * 64;
    const int64_t blocks = (slots + 255) / 256;
    hipLaunchKernelGGL(repack_tiled_kernel<B>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       packed, scales, N, G, per_channel ? 1 : G, per_channel ? 0 : 1, rowblocks,
                       static_cast<uint8_t *>(out));
    return hipGetLastError();
}

hipError_t launch_repack_tiled(const uint32_t *packed, const uint16_t *scales, int64_t N,
                               int64_t K, int b, bool per_channel, void *out, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    switch (b) {
        case 2: return repack_b<2>(packed, scales, N, G, per_channel, out, stream);
        case 3: return repack_b<3>(packed, scales, N, G, per_channel, out, stream);
        case 4: return repack_b<4>(packed, scales, N, G, per_channel, out, stream);
        case 5: return repack_b<5>(packed, scales, N, G, per_channel, out, stream);
        case 6: return repack_b<6>(packed, scales, N, G, per_channel, out, stream);
        case 7: return repack_b<7>(packed, scales, N, G, per_channel, out, stream);
        case 8: return repack_b<8>(packed, scales, N, G, per_channel, out, stream);
    }
    return hipErrorInvalidValue;
}

template <int B>
static hipError_t unpack_b(const void *W, bool tiled, int64_t N, int G, uint8_t *codes,
                           hipStream_t stream) {
    const int64_t rows = tiled ? (N + 63) / 64 * 64 : N;
    const int64_t threads = rows * G;
    const int64_t blocks = (threads + 255) / 256;
    if (tiled) {
        TiledW wl{static_cast<const uint8_t *>(W), G, B};
        hipLaunchKernelGGL((unpack_kernel<B, TiledW>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, wl, N, G, true, codes);
    } else {
        DenseW wl{static_cast<const uint8_t *>(W), nullptr, (int64_t)16 * B * G, G, B};
        hipLaunchKernelGGL((unpack_kernel<B, DenseW>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, wl, N, G, false, codes);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const void *W, bool tiled, const uint16_t *, int64_t N, int64_t K,
                         int b, uint8_t *codes, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    switch (b) {
        case 2: return unpack_b<2>(W, tiled, N, G, codes, stream);
        case 3: return unpack_b<3>(W, tiled, N, G, codes, stream);
        case 4: return unpack_b<4>(W, tiled, N, G, codes, stream);
        case 5: return unpack_b<5>(W, tiled, N, G, codes, stream);
        case 6: return unpack_b<6>(W, tiled, N, G, codes, stream);
        case 7: return unpack_b<7>(W, tiled, N, G, codes, stream);
        case 8: return unpack_b<8>(W, tiled, N, G, codes, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
