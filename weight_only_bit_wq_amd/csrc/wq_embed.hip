// wq_embed.hip -- quantized embedding gather on the dense (checkpoint) layout.
//
// The vocabulary layers are large: 248,320 x 5,120 in bf16 is 2.37 GiB per
// layer, and int8 with group scales is the recommended trade ("vLLM Can Run
// INT5-7", section 3).  The model card "Qwen3.8-27B-INT6-Mixed-AutoRound"
// (Findings) explains why a 5/6/7-bit embed_tokens cannot load: the existing
// gather indexes codes as if 32 // b of them fit in each word, which does not
// match the dense ceil(K * b / 32)-word rows once codes straddle words.  This
// gather reads exactly that dense layout, for every b in 2..8.
//
// One thread per (token t, chunk j of 8 codes), blocks of 128 chunks of one
// token.  Eight b-bit codes are
// exactly b bytes, so chunk j of a dense row starts at byte b*j: lanes of a
// wave read consecutive b-byte pieces (one contiguous 64*b-byte range per
// load) and write consecutive 16-byte pieces of Y (one contiguous 1 KB range
// per store).  A lane loads the dwords that hold its b bytes (two, three for
// b = 7 at some offsets; addresses clamped to the row so none leaves it),
// shifts them by 8 * (b*j mod 4) bits so code i sits at bit b*i of a 64-bit
// window, extracts the 8 codes at those compile-time offsets and writes
//     Y[t, 8j + i] = bf16_rne(s[id, j/16] * (c_i - z[id, j/16]))      (id = ids[t])
// with z = 2^(b-1) for symmetric groups (the zero points exist for b = 4 and
// 8; a per-channel scale is s[id] for every group).  c - z is formed exactly
// in fp32 and then multiplied by the scale (a product, so a zero code under
// a negative scale gives -0 as the exact product does); the product has at
// most 16 significant bits, so it is exact in fp32 and the one rounding is
// the bf16 conversion.  Ids outside [0, V)
// give rows of zeros: the rows of a vocabulary shard that belong to other
// shards.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

typedef float f32x2_e __attribute__((ext_vector_type(2)));

// Code I of the 64-bit window (hi:lo), codes at bit B*I.
template <int B, int I>
__device__ __forceinline__ uint32_t window_code(uint32_t lo, uint32_t hi) {
    constexpr int off = B * I;
    constexpr uint32_t m = (1u << B) - 1u;
    if constexpr (off + B <= 32) return (lo >> off) & m;
    else if constexpr (off >= 32) return (hi >> (off - 32)) & m;
    else return __builtin_amdgcn_alignbit(hi, lo, off) & m;
}

constexpr int kEmbedBlock = 128;  // chunks (threads) per block

template <int B>
__global__ __launch_bounds__(kEmbedBlock) void embed_kernel(const uint32_t *__restrict__ W,
                                                    const uint16_t *__restrict__ scales,
                                                    const uint8_t *__restrict__ zeros,
                                                    int sG, int sg,
                                                    int64_t V, int K, int bpt,
                                                    const int64_t *__restrict__ ids,
                                                    uint16_t *__restrict__ Y) {
    // Block (t, part): bpt blocks of 128 chunks per token (uniform division).
    const int64_t t = blockIdx.x / (unsigned)bpt;
    const int j = (int)(blockIdx.x - t * bpt) * kEmbedBlock + (int)threadIdx.x;
    if (j >= K / 8) return;
    const int64_t id = ids[t];
    u32x4 *dst = reinterpret_cast<u32x4 *>(Y + t * (int64_t)K + 8 * j);
    if (id < 0 || id >= V) {
        *dst = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const int row_words = K / 32 * B;
    const uint32_t *row = W + id * (int64_t)row_words;
    const int byte0 = B * j;
    const int d0 = byte0 >> 2;
    const int last = row_words - 1;
    const uint32_t w0 = row[d0];
    const uint32_t w1 = row[min(d0 + 1, last)];
    const uint32_t sh = 8u * (uint32_t)(byte0 & 3);
    const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, sh);
    uint32_t hi;
    if constexpr (B == 7) {  // 7 bytes from offset 2 or 3 reach a third dword
        const uint32_t w2 = row[min(d0 + 2, last)];
        hi = __builtin_amdgcn_alignbit(w2, w1, sh);
    } else {  // (byte0 & 3) + B <= 8: two dwords hold the chunk
        hi = sh ? (w1 >> sh) : w1;
    }
    const int G = K / kGroup;
    const float s = bf16_to_f32(scales[id * sG + (j >> 4) * sg]);
    const float kOff = zeros ? (float)zeros[id * G + (j >> 4)] : (float)(1 << (B - 1));
    uint32_t c[8];
    c[0] = window_code<B, 0>(lo, hi);
    c[1] = window_code<B, 1>(lo, hi);
    c[2] = window_code<B, 2>(lo, hi);
    c[3] = window_code<B, 3>(lo, hi);
    c[4] = window_code<B, 4>(lo, hi);
    c[5] = window_code<B, 5>(lo, hi);
    c[6] = window_code<B, 6>(lo, hi);
    c[7] = window_code<B, 7>(lo, hi);
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f32x2_e q;
        q.x = ((float)c[2 * p] - kOff) * s;
        q.y = ((float)c[2 * p + 1] - kOff) * s;
        o[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(q, bf16x2_t));
    }
    *dst = u32x4{o[0], o[1], o[2], o[3]};
}

hipError_t launch_embed(const void *W, const uint16_t *scales, const uint8_t *zeros,
                        bool per_channel, int64_t V, int64_t K, int b, const int64_t *ids,
                        int64_t T, uint16_t *Y, hipStream_t stream) {
    const int sG = per_channel ? 1 : (int)(K / kGroup), sg = per_channel ? 0 : 1;
    const int bpt = (int)((K / 8 + kEmbedBlock - 1) / kEmbedBlock);
    const dim3 grid((unsigned)(T * bpt)), block(kEmbedBlock);
    const uint32_t *w = static_cast<const uint32_t *>(W);
    const int k = (int)K;
    switch (b) {
        case 2:
            hipLaunchKernelGGL(embed_kernel<2>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        case 3:
            hipLaunchKernelGGL(embed_kernel<3>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        case 4:
            hipLaunchKernelGGL(embed_kernel<4>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        case 5:
            hipLaunchKernelGGL(embed_kernel<5>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        case 6:
            hipLaunchKernelGGL(embed_kernel<6>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        case 7:
            hipLaunchKernelGGL(embed_kernel<7>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        case 8:
            hipLaunchKernelGGL(embed_kernel<8>, grid, block, 0, stream, w, scales, zeros, sG, sg, V,
                               k, bpt, ids, Y);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wq
