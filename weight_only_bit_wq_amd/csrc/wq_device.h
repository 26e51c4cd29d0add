// wq_device.h -- device-side building blocks shared by the libwq kernels:
// weight-buffer addressing for the two layouts, the in-register bitstream
// unpacker and bf16 helpers.
//
// Bitstream facts used throughout (model card
// "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings: dense layout along
// in_features, ceil(in * bits / 32) words per row):
//   - a group of 128 codes occupies exactly 128*b bits = 16*b bytes = b
//     16-byte chunks, and starts 16-byte aligned inside its row, for every b;
//   - so one lane can own a whole (row, group) with b 128-bit loads, and
//     codes that straddle 32-bit words never straddle lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace wq {

constexpr int kGroup = 128;     // codes per scale group
constexpr int kTileRows = 64;   // rows per tile in the tiled layout (one wave)

__host__ __device__ constexpr int tile_code_bytes(int b) { return b * 1024; }
__host__ __device__ constexpr int tile_bytes(int b) { return b * 1024 + 128; }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Weight addressing.  A "slot" is one (row, group): b chunks of 16 bytes plus
// one bf16 scale.
// ---------------------------------------------------------------------------

// Dense rows as written by wq_pack; scales are a separate [N, G] array.
struct DenseW {
    static constexpr bool kTiled = false;
    const uint8_t *w;
    const uint16_t *s;
    int64_t row_bytes;  // 4 * ceil(K*b/32) == 16 * b * G
    int G;
    int b;
    __device__ const uint4 *chunks(int64_t n, int g) const {
        return reinterpret_cast<const uint4 *>(w + n * row_bytes + (int64_t)g * 16 * b);
    }
    __device__ int64_t chunk_stride() const { return 1; }  // in uint4 units
    __device__ uint16_t scale(int64_t n, int g) const { return s[n * G + g]; }
    // Loop-invariant addressing: slot (n, g) starts at slot0(n) + g *
    // slot_step() bytes; its dword d at + dword_off(d); its scale at
    // scale0(n) + g * scale_step() bytes.
    __device__ const uint8_t *slot0(int64_t n) const { return w + n * row_bytes; }
    __device__ int64_t slot_step() const { return (int64_t)16 * b; }
    __device__ static constexpr int dword_off(int d) { return 4 * d; }
    __device__ const uint8_t *scale0(int64_t n) const {
        return reinterpret_cast<const uint8_t *>(s + n * G);
    }
    __device__ int64_t scale_step() const { return 2; }
};

// Tiled blob written by wq_repack: per (64-row block, group) a tile of b
// planes of 1 KB (plane j: chunk j of each of the 64 rows) + 64 bf16 scales.
struct TiledW {
    static constexpr bool kTiled = true;
    const uint8_t *w;
    int G;
    int b;
    __device__ const uint8_t *tile(int64_t n, int g) const {
        return w + ((n >> 6) * (int64_t)G + g) * (int64_t)tile_bytes(b);
    }
    __device__ const uint4 *chunks(int64_t n, int g) const {
        return reinterpret_cast<const uint4 *>(tile(n, g) + (n & 63) * 16);
    }
    __device__ int64_t chunk_stride() const { return 64; }  // 1 KB in uint4 units
    __device__ uint16_t scale(int64_t n, int g) const {
        return reinterpret_cast<const uint16_t *>(tile(n, g) + tile_code_bytes(b))[n & 63];
    }
    // Loop-invariant addressing (see DenseW).
    __device__ const uint8_t *slot0(int64_t n) const { return tile(n, 0) + (n & 63) * 16; }
    __device__ int64_t slot_step() const { return tile_bytes(b); }
    __device__ static constexpr int dword_off(int d) { return (d >> 2) * 1024 + (d & 3) * 4; }
    __device__ const uint8_t *scale0(int64_t n) const {
        return tile(n, 0) + tile_code_bytes(b) + (n & 63) * 2;
    }
    __device__ int64_t scale_step() const { return tile_bytes(b); }
};

// ---------------------------------------------------------------------------
// In-register unpacker.
//
// A slot's 128 codes sit in 4*B 32-bit words w[].  code_pair<B, P>() returns
// codes 2P and 2P+1 as two 16-bit lanes of one register, (c0 | c1 << 16):
//   1. v_perm_b32 gathers, from the two words that hold them, the byte pair
//      starting at each code's first byte into the low and high halves;
//   2. one packed 16-bit shift drops each half's bit offset inside its byte;
//   3. the caller masks (and can OR a constant in the same instruction).
// Every index is a compile-time constant, so this is 2 VALU ops per pair
// plus the caller's mask, whether or not the codes straddle a word.
// A code's bits [o, o+B) always fit in the 16-bit window starting at byte
// o/8 because B <= 9.
// ---------------------------------------------------------------------------

template <int B, int P>
struct PairSel {
    static constexpr int o0 = 2 * P * B;
    static constexpr int o1 = o0 + B;
    static constexpr int byte0 = o0 >> 3;
    static constexpr int byte1 = o1 >> 3;
    static constexpr int word = byte0 >> 2;          // low word of the window
    static constexpr int base = 4 * word;
    static constexpr uint32_t sel = (uint32_t)(byte0 - base) |
                                    ((uint32_t)(byte0 + 1 - base) << 8) |
                                    ((uint32_t)(byte1 - base) << 16) |
                                    ((uint32_t)(byte1 + 1 - base) << 24);
    static constexpr int sh0 = o0 & 7;
    static constexpr int sh1 = o1 & 7;
    static constexpr bool has_hi = word + 1 < 4 * B;  // else the window's top is padding
    static_assert(byte1 + 1 - base < 8, "pair window exceeds two words");
};

__device__ __forceinline__ uint32_t pk_shr16(uint32_t x, int s0, int s1) {
    u16x2 v = __builtin_bit_cast(u16x2, x);
    u16x2 s = {(unsigned short)s0, (unsigned short)s1};
    return __builtin_bit_cast(uint32_t, (u16x2)(v >> s));
}

// Codes 2P, 2P+1 of the slot, unmasked (garbage above bit B of each half).
template <int B, int P>
__device__ __forceinline__ uint32_t code_pair_raw(const uint32_t *w) {
    using S = PairSel<B, P>;
    const uint32_t lo = w[S::word];
    const uint32_t hi = S::has_hi ? w[S::word + 1] : 0u;
    const uint32_t x = __builtin_amdgcn_perm(hi, lo, S::sel);
    if constexpr (S::sh0 == 0 && S::sh1 == 0) return x;
    return pk_shr16(x, S::sh0, S::sh1);
}

template <int B>
__host__ __device__ constexpr uint32_t pair_mask() {
    return ((1u << B) - 1u) * 0x00010001u;
}

// Codes 2P and 2P+1 as (c0 | c1 << 16).
template <int B, int P>
__device__ __forceinline__ uint32_t code_pair(const uint32_t *w) {
    return code_pair_raw<B, P>(w) & pair_mask<B>();
}

// ---------------------------------------------------------------------------
// Exact signed codes.
//
// The GEMM kernels multiply activations by the signed code q = c - 2^(b-1)
// itself, as an exact bf16 (|q| <= 128 has at most 8 significant bits), and
// apply the group scale once per group in fp32.  So every product a * q is
// exact and the rounding error of a dot product is bounded by the sum of
// |a * w| of its own terms: a row of midpoint codes (zero weights) gives
// exactly zero whatever the activations.  (An operand with a constant offset
// such as 128 + c, removed afterwards, would instead carry rounding error
// proportional to that offset times sum |a|.)
//
// For a b-bit code c, c XOR 2^(b-1) is the b-bit two's complement of q.  A
// run of 32 codes is exactly b 32-bit words, so one XOR per word with the
// pattern of every code's top bit, then one sign-extending bit-field
// extract per code (v_bfe_i32; a code that straddles two words first goes
// through v_alignbit_b32), gives q as an int32; v_cvt_f32_i32 converts it
// exactly and v_cvt_pk_bf16_f32 packs two of them (exact: |q| <= 128).
// For b = 8 the extracts are whole bytes and the compiler folds them into
// the conversions (SDWA byte selects).
// ---------------------------------------------------------------------------

// Top bits of the codes whose top bit lies in word d of a 32-code run.
template <int B>
__host__ __device__ constexpr uint32_t sign_bits(int d) {
    uint32_t p = 0;
    for (int k = 0; k < 32; ++k) {
        const int t = k * B + B - 1 - 32 * d;
        if (t >= 0 && t < 32) p |= 1u << t;
    }
    return p;
}

// XOR the n words of a slot or part of one (starting at word d0 of a
// 32-code run) with the code top bits, in place.
template <int B, int NW>
__device__ __forceinline__ void flip_signs(uint32_t *w, int d0 = 0) {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] ^= sign_bits<B>((d0 + i) % B);
}

// Code K (0..31) of a 32-code run held in B sign-flipped words: q as float.
template <int B, int K>
__device__ __forceinline__ float qcode_f32(const uint32_t *wx) {
    constexpr int o = K * B, d = o >> 5, sh = o & 31;
    int v;
    if constexpr (sh + B <= 32)
        v = __builtin_amdgcn_sbfe((int)wx[d], sh, B);
    else
        v = __builtin_amdgcn_sbfe((int)__builtin_amdgcn_alignbit(wx[d + 1], wx[d], sh), 0, B);
    return (float)v;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats that hold small integers as a bf16 pair (lo, hi); exact.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t f;
    f.x = lo;
    f.y = hi;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Codes 2P, 2P+1 (P = 0..15) of a 32-code run as the bf16 pair (q0, q1).
template <int B, int P>
__device__ __forceinline__ uint32_t qpair(const uint32_t *wx) {
    return pack_bf16x2(qcode_f32<B, 2 * P>(wx), qcode_f32<B, 2 * P + 1>(wx));
}

// With a zero point z (b = 4, 8; words not sign-flipped): (c - z) as float,
// |c - z| <= 255, exact in fp32 and in bf16.
template <int B, int K>
__device__ __forceinline__ float zcode_f32(const uint32_t *w, int z) {
    static_assert(B == 4 || B == 8, "zero points exist for 4 and 8 bits");
    constexpr int o = K * B, d = o >> 5, sh = o & 31;
    return (float)((int)__builtin_amdgcn_ubfe(w[d], sh, B) - z);
}
template <int B, int P>
__device__ __forceinline__ uint32_t zpair(const uint32_t *w, int z) {
    return pack_bf16x2(zcode_f32<B, 2 * P>(w, z), zcode_f32<B, 2 * P + 1>(w, z));
}

// b = 4 with a zero point, a run at a time: the nibbles of word d spread to
// bytes (even codes from the low nibbles into o[2d], odd from the high into
// o[2d + 1]), each byte set to 128 + c, z subtracted from every byte at once
// (no borrow crosses a byte while z <= 128; zero points are below 16 here)
// and the top bits flipped back: int8 c - z in every byte, exact.  About 8
// instructions per 8 codes (mask, set, subtract, flip for each half, and
// one shift), then one sign-extending byte select per code, against an
// extract, a subtract and a conversion per code.
__device__ __forceinline__ void zp4_run(const uint32_t *w, uint32_t *o, int z) {
    const uint32_t zb = (uint32_t)z * 0x01010101u;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        o[2 * d] = (((w[d] & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
        o[2 * d + 1] = ((((w[d] >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
    }
}
// b = 4 without a zero point, a run at a time: each nibble XOR 8 is the
// 4-bit two's complement of q = c - 8; moved to the top of its byte it
// reads as int8 16 q (even codes into o[2d], odd into o[2d + 1], as
// zp4_run).  4 instructions per 8 codes; the 16 is taken out of the group
// scale (operand_scale_inv).
__device__ __forceinline__ void nib4_run(const uint32_t *w, uint32_t *o) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t x = w[d] ^ 0x88888888u;
        o[2 * d] = (x << 4) & 0xF0F0F0F0u;
        o[2 * d + 1] = x & 0xF0F0F0F0u;
    }
}
// Codes 2P, 2P+1 of a run prepared by zp4_run or nib4_run: byte P % 4 of
// o[2 (P / 4)] and of o[2 (P / 4) + 1].
template <int P>
__device__ __forceinline__ uint32_t zp4pair(const uint32_t *o) {
    constexpr int d = P / 4, e = P % 4;
    return pack_bf16x2((float)(int)(int8_t)(uint8_t)(o[2 * d] >> (8 * e)),
                       (float)(int)(int8_t)(uint8_t)(o[2 * d + 1] >> (8 * e)));
}

// Pair P of a run: the symmetric or the zero-point form (w sign-flipped
// only in the symmetric form).
template <int B, int P, bool ZP>
__device__ __forceinline__ uint32_t wpair(const uint32_t *w, int z) {
    if constexpr (ZP) return zpair<B, P>(w, z);
    else return qpair<B, P>(w);
}

// ---------------------------------------------------------------------------
// The int8-ready arrangement of the tiled layout (b = 5, 6, 7).
//
// The repack may store a 32-code run (b words) in any order of its bits, so
// for these widths it stores the signed values v = c XOR 2^(b-1) (b-bit two's
// complement of q = c - 2^(b-1)) such that most codes sit in the top b bits
// of a byte of their own:
//   - codes 0 .. 4b-1: byte k of the run, bits 7 .. 8-b, is v_k; one AND per
//     word then leaves the int8 value q * 2^(8-b) in every byte;
//   - the other 4 (8 - b) codes fill the 8 - b spare low bits of the bytes:
//       b = 6: codes 24 + 4s + e: v bits 5..4, 3..2, 1..0 in bits 1..0 of
//              byte e of words 3s, 3s + 1, 3s + 2;
//       b = 5: codes 20 + 4s + e (s = 0, 1): v bits 4..2 in bits 2..0 of
//              byte e of word s, v bits 1..0 in bits 1..0 of byte e of word
//              3 + s; s = 2: v bits 4..2 in bits 2..0 of byte e of word 2,
//              v bit 1 in bit 2 of byte e of word 3, v bit 0 in bit 2 of
//              byte e of word 4;
//       b = 7: codes 28 + e: v bit i in bit 0 of byte e of word i;
//     a few shifts and bit-field inserts per 4 codes put them at the top of
//     bytes too.
// So a run decodes to 8 words of int8 values q * 2^(8-b), code k in byte
// k % 4 of word k / 4, each converted to fp32 by one v_cvt_f32_i32 with a
// sign-extended byte select: about 2 VALU ops per code instead of about
// 2.8 for the dense stream.  The factor 2^(8-b) is exact and is taken out of
// the group scale (fp32 keeps denormals, so s * 2^-(8-b) is exact too).
// ---------------------------------------------------------------------------
template <int B>
__host__ __device__ constexpr bool int8_ready() { return B >= 5 && B <= 7; }

// (x & m) | (y & ~m): one v_bfi_b32.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t x, uint32_t y) {
    return (x & m) | (y & ~m);
}

// The B words of an arranged run -> 8 words of int8 q * 2^(8-B).
template <int B>
__device__ __forceinline__ void run_int8(const uint32_t *d, uint32_t *o) {
    static_assert(int8_ready<B>(), "arranged runs exist for b = 5, 6, 7");
    constexpr uint32_t top = ((0xFFu << (8 - B)) & 0xFFu) * 0x01010101u;
#pragma unroll
    for (int i = 0; i < B; ++i) o[i] = d[i] & top;
    if constexpr (B == 6) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            o[6 + s] = bfi(0xC0C0C0C0u, d[3 * s] << 6,
                           bfi(0x30303030u, d[3 * s + 1] << 4, d[3 * s + 2] << 2)) & top;
    } else if constexpr (B == 5) {
        o[5] = bfi(0xE0E0E0E0u, d[0] << 5, d[3] << 3) & top;
        o[6] = bfi(0xE0E0E0E0u, d[1] << 5, d[4] << 3) & top;
        o[7] = bfi(0xE0E0E0E0u, d[2] << 5, bfi(0x10101010u, d[3] << 2, d[4] << 1)) & top;
    } else {
        uint32_t r = d[6] & 0x01010101u;
#pragma unroll
        for (int i = 5; i >= 0; --i) r = bfi(0x01010101u, d[i], r << 1);
        o[7] = r << 1;
    }
}

// Arranges 32 signed b-bit values v[k] (low b bits used) into B words, the
// inverse of run_int8 (used by the repack).
template <int B>
__host__ __device__ inline void arrange_run(const uint32_t *v, uint32_t *d) {
    static_assert(int8_ready<B>(), "arranged runs exist for b = 5, 6, 7");
    constexpr uint32_t mask = (1u << B) - 1u;
    for (int i = 0; i < B; ++i) d[i] = 0;
    for (int k = 0; k < 4 * B; ++k) d[k >> 2] |= ((v[k] & mask) << (8 - B)) << (8 * (k & 3));
    for (int e = 0; e < 4; ++e) {
        auto put = [&](int word, int bit, uint32_t bits) { d[word] |= bits << (8 * e + bit); };
        if constexpr (B == 6) {
            for (int s = 0; s < 2; ++s) {
                const uint32_t x = v[24 + 4 * s + e] & mask;
                put(3 * s, 0, (x >> 4) & 3u);
                put(3 * s + 1, 0, (x >> 2) & 3u);
                put(3 * s + 2, 0, x & 3u);
            }
        } else if constexpr (B == 5) {
            for (int s = 0; s < 2; ++s) {
                const uint32_t x = v[20 + 4 * s + e] & mask;
                put(s, 0, (x >> 2) & 7u);
                put(3 + s, 0, x & 3u);
            }
            const uint32_t x = v[28 + e] & mask;
            put(2, 0, (x >> 2) & 7u);
            put(3, 2, (x >> 1) & 1u);
            put(4, 2, x & 1u);
        } else {
            const uint32_t x = v[28 + e] & mask;
            for (int i = 0; i < 7; ++i) put(i, 0, (x >> i) & 1u);
        }
    }
}

// Code K of a decoded run o[] as float: q * 2^(8-B), exact (one
// v_cvt_f32_i32 with a sign-extended byte select).
template <int K>
__device__ __forceinline__ float i8code_f32(const uint32_t *o) {
    return (float)(int)(int8_t)(uint8_t)(o[K >> 2] >> (8 * (K & 3)));
}
template <int P>
__device__ __forceinline__ uint32_t i8pair(const uint32_t *o) {
    return pack_bf16x2(i8code_f32<2 * P>(o), i8code_f32<2 * P + 1>(o));
}

// The factor by which a run's operands exceed q: 2^(8-B) for an arranged
// run (I8) and for b = 4 without zero points (nib4_run), else 1; the group
// scale is multiplied by its inverse (exact: a power of two).
template <int B, bool I8, bool ZP>
__host__ __device__ constexpr float operand_scale_inv() {
    return (I8 || (B == 4 && !ZP)) ? 1.0f / (float)(1 << (8 - B)) : 1.0f;
}

// Whether prep_runs writes 8 int8 words per run into o: arranged runs
// (I8), or b = 4.
template <int B, bool ZP, bool I8>
__host__ __device__ constexpr bool int8_words() { return I8 || B == 4; }

// Prepares the 4 * NQ words of NQ runs (w) for slot_pair: the 8 * NQ int8
// words of arranged runs or of b = 4 runs (with zero point z, or without)
// into o, else sign flips for the dense stream (symmetric) or nothing (b = 8
// with zero points).
template <int B, bool ZP, bool I8, int NQ>
__device__ __forceinline__ void prep_runs(uint32_t *w, uint32_t *o, int z) {
    if constexpr (I8) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) run_int8<B>(w + q * B, o + q * 8);
    } else if constexpr (B == 4) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if constexpr (ZP) zp4_run(w + q * B, o + q * 8, z);
            else nib4_run(w + q * B, o + q * 8);
        }
    } else if constexpr (!ZP) {
        flip_signs<B, NQ * B>(w);
    }
}

// Pair P of the prepared runs (pair P % 16 of run P / 16): from the words
// (w, generic) or from the int8 words (o).
template <int B, int P, bool ZP, bool I8>
__device__ __forceinline__ uint32_t slot_pair(const uint32_t *w, const uint32_t *o, int z) {
    if constexpr (I8) return i8pair<P % 16>(o + (P / 16) * 8);
    else if constexpr (B == 4) return zp4pair<P % 16>(o + (P / 16) * 8);
    else return wpair<B, P % 16, ZP>(w + (P / 16) * B, z);
}

// f(std::integral_constant<int, I>{}) for I = I0 .. N - 1, unrolled.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Load the 4*B words of one slot (B 16-byte chunks, `stride` uint4 apart).
template <int B>
__device__ __forceinline__ void load_slot(const uint4 *p, int64_t stride, uint32_t *w) {
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + j * stride));
        w[4 * j + 0] = v.x;
        w[4 * j + 1] = v.y;
        w[4 * j + 2] = v.z;
        w[4 * j + 3] = v.w;
    }
}

// Wait until this wave's vector-memory stores have completed.  Split-K
// partials are device-scope atomic stores (written through to the
// coherence point); the wave must see them acknowledged before it takes
// its ticket, or the last split could read a partial still in flight.  On
// this architecture vmcnt also counts stores, and a store is counted until
// the coherence point has it.  The "memory" clobber makes the wait a
// compiler barrier as well: relaxed atomics to different addresses may
// otherwise be moved across it.
__device__ __forceinline__ void wait_vm_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Word 3 of a raw buffer resource on this architecture (gfx9 family): 32-bit
// data format, no swizzle or stride; accesses are range-checked against the
// resource's num_records (out of range reads return zero).
constexpr int kBufferRsrcWord3 = 0x00020000;

// s_waitcnt immediate that waits until at most n of this wave's vector-memory
// operations are outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at "no wait").
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt), not for its outstanding global loads, so prefetches stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN): one
// v_cvt_pk_bf16_f32 under the default round-to-nearest-even mode.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over the 64 lanes of a wave (fixed butterfly order: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Wave-uniform sum over the 64 lanes with DPP (no LDS round trips): quad
// swaps, half-row and row mirrors give every lane its 16-lane row sum, two
// row broadcasts carry the rows into lane 63, which is read into an SGPR.
// Fixed order, so the result is deterministic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false);
    return x + __int_as_float(t);
}
__device__ __forceinline__ float wave_sum_uniform(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);  // row_mirror
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---------------------------------------------------------------------------
// Quarter slots.  A group's 128 codes split into 4 quarters of 32 codes; a
// quarter is exactly B 32-bit words (32 * B bits), so dwords [Q*B, Q*B+B) of
// a slot hold quarter Q.  The int8-activation kernel gives a lane a quarter
// of a row and widens it straight into int8 operand registers.
// ---------------------------------------------------------------------------

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

// Dwords [Q*B, Q*B + B) of a slot (its quarter Q: codes 32Q .. 32Q+31) into
// w[0..B), loaded as runs of consecutive dwords within one 16-byte chunk
// (dword d sits at WL::dword_off(d); chunks are 16-byte aligned).
template <class WL, int D, int END>
struct QuarterLoad {
    static constexpr int kRun = ((D | 3) + 1 < END ? (D | 3) + 1 : END) - D;
    __device__ __forceinline__ static void run(const uint8_t *slot, uint32_t *w) {
        const uint8_t *p = slot + WL::dword_off(D);
        if constexpr (kRun == 4) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if constexpr (kRun == 2 && (D & 1) == 0) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
            w[0] = v.x; w[1] = v.y;
        } else {
#pragma unroll
            for (int e = 0; e < kRun; ++e) w[e] = reinterpret_cast<const uint32_t *>(p)[e];
        }
        QuarterLoad<WL, D + kRun, END>::run(slot, w + kRun);
    }
};
template <class WL, int END>
struct QuarterLoad<WL, END, END> {
    __device__ __forceinline__ static void run(const uint8_t *, uint32_t *) {}
};

}  // namespace wq
