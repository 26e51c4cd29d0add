// wq_prefill.hip -- WNA16 prefill path (M > 16): LDS-tiled bf16 MFMA GEMM.
//
// At large batch the layer is compute-bound ("vLLM Quantization", Key points
// and Pitfalls: weight-only gains fade as batch grows), so the product runs
// on the matrix cores (v_mfma_f32_32x32x16_bf16) with fp32 accumulation and
// the codes are dequantized straight into their operand registers.
//
// Exactness.  The B operand holds the signed code q = c - 2^(b-1) itself
// as an exact bf16 (wq_device.h), so the integer codes are never rounded
// and no constant offset is carried through the accumulation.  Each group
// of 128 k is accumulated into its own fp32 block P_g and folded as
// total += s[n,g] * P_g in fp32.  No scale or code is ever rounded to bf16,
// and the rounding error of an output is bounded by the sum of |a * w| of
// its own terms.
//
// Zero points (b = 4 and 8): q = c - z, exact as well (|c - z| <= 255).
//
// Tiling.  Workgroup 256 (m) x 128 (n), 8 waves of 128 x 32 (two per SIMD),
// each as four 32 x 32 MFMA blocks run in two staggered phases.  K runs in
// whole groups of 128: A through LDS (double-buffered, filled by direct
// global -> LDS loads), B from each lane's contiguous half-slot of codes
// straight into operand registers.  Workgroups an XCD runs together share
// an A row block.
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

// LDS tiles are rows of 16-byte chunks (8 bf16 of k), 16 chunks (one group
// of 128 k, 256 bytes) per row; chunk c of row r sits at r*16 + (c ^ (r &
// 15)).  LDS serves a 128-bit read 16 lanes at a time over 64 banks, and
// the 16 consecutive rows such a lane group reads (one chunk each) land on
// 16 distinct 16-byte bank groups; the direct loads write 64 consecutive
// 16-byte slots (four rows) per instruction, conflict free too, with no
// padding.
__device__ __forceinline__ int swz16(int row, int chunk) {
    return row * 16 + (chunk ^ (row & 15));
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// B is unpacked straight into MFMA operand registers and A moved global ->
// LDS by direct loads (global_load_lds_dwordx4): the LDS carries A alone,
// written once per group by the loads and read by the waves.  (Unpacking B
// into LDS for all waves to read, as well, put the LDS traffic at about the
// matrix cores' time.)
//
// Workgroup 256 (m) x 128 (n), 8 waves as 2 (m) x 4 (n), wave (wm, wn) owns
// rows 128 wm .. +128 and columns 32 wn .. +32 as four 32 x 32 blocks i
// (block rows) in one block column.  K order inside a group: k-step j
// (0..7) of v_mfma_f32_32x32x16_bf16 takes, in its lane half h (lanes 32 h
// .. 32 h + 31), the 8 k of chunk 8 h + j; both operands use that order, so
// lane (column n, half h) needs codes 64 h .. 64 h + 63 of row n's group:
// dwords 2 h B .. 2 h B + 2 B - 1 of the slot, one contiguous half-slot,
// loaded with 8-byte loads and unpacked to exact signed bf16 pairs once per
// group.  The A operand of the same k-step is chunk 8 h + j of its LDS row.
//
// Each group runs in two phases of 16 MFMA slots: phase 0 the 8 k-steps of
// block rows 0 and 1, phase 1 those of rows 2 and 3 (two accumulation
// chains each), with the B operand of k-step j unpacked in phase 0 and kept
// for phase 1.  Phase 0 folds rows 2, 3 of the previous group and phase 1
// rows 0, 1 of this one (tot += s * P, two FMAs per slot), so no fold waits
// on the matrix pipe.  A is double-buffered in two LDS objects (256 rows x
// 128 k each), the codes in a second double buffer; at the start of group
// g the waves pass a barrier (group g's A and codes have landed; nobody
// still reads the other buffers), read their half-slots, issue the direct
// loads of group g+1's codes into the other buffers and its scale into a
// register, and run g, issuing group g+1's A into the other buffer one 1 KB
// run per MFMA slot of phase 0 (as one burst at the barrier, the eight
// waves' 64 loads made the kernel about 3% slower).
// GT: NoGroups, or a GroupTable with one entry per m-tile (expert e[i],
// rows [m0[i], m0[i] + me[i]) of A and Y); the grid's m-tiles run the
// entries, each rebasing its rows, weights and zero points.
//
// TM: workgroup rows, 256 (8 waves as above) or 64 for the small m-tiles of
// grouped launches (experts of a few dozen rows): 4 waves of 64 x 32, one
// per SIMD, each running phase 0 only, with a 32 KB A double buffer, so
// that LDS (56 KB at b = 6) leaves room for two workgroups per compute unit
// and their loads overlap each other's matrix work.
template <int B, class WL, bool ZP, class GT, int TM = kPM>
__global__ __launch_bounds__(TM == kPM ? 512 : 256, 2) void prefill_kernel(const uint16_t *__restrict__ A, int M,
                                                      int N, int K, WL wl,
                                                      const uint8_t *__restrict__ zeros,
                                                      uint16_t *__restrict__ Y, int mtiles,
                                                      int ntiles, int splits,
                                                      float *__restrict__ part, int64_t mnp,
                                                      int nfull, int tsplits, const GT gt) {
    static_assert(TM == kPM || TM == 64, "m-tile of 256 or 64 rows");
    constexpr int NW = TM == kPM ? 8 : 4;  // waves
    constexpr bool kSmall = TM != kPM;
    __shared__ u32x4 As0[TM * 16];
    __shared__ u32x4 As1[TM * 16];
    __shared__ u32x4 As2[kSmall ? TM * 16 : 1];  // third A buffer of the 64-row ring
    // Codes of the tile's 128 columns, double-buffered: [buffer][64-row
    // block][plane][row].  (One object: its reads come right after the
    // barrier, before any direct load into it is issued.)
    __shared__ u32x4 Cs[2][kSmall ? 1 : 2 * B * 64];

    const int G = K / kGroup;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = kSmall ? 0 : wave >> 2, wn = wave & 3;
    const int h = lane >> 5;
    const int c32 = lane & 31;

    // Block b runs on XCD b % 8: each XCD gets a contiguous run of logical
    // tiles, n fastest, so the tiles an XCD runs together share A rows.
    // With a uniform K split (splits > 1) the logical index is split-major.
    // With a tail split (tsplits > 1) blocks past nfull run part sp of the K
    // split of tile nfull + (b - nfull) / tsplits, and only the first nfull
    // blocks are remapped.
    const int tiles = mtiles * ntiles;
    const bool tail = tsplits > 1 && (int)blockIdx.x >= nfull;
    int sp, tile, g_lo, g_hi;
    if (tail) {
        const int j = (int)blockIdx.x - nfull;
        tile = nfull + j / tsplits;
        sp = j - (j / tsplits) * tsplits;
        g_lo = (int)(((int64_t)G * sp) / tsplits);
        g_hi = (int)(((int64_t)G * (sp + 1)) / tsplits);
    } else {
        const int total = tsplits > 1 ? nfull : tiles * splits;
        int logical = blockIdx.x;
        if ((total & 7) == 0) logical = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
        sp = logical / tiles;
        tile = logical - sp * tiles;
        g_lo = (int)(((int64_t)G * sp) / splits);
        g_hi = (int)(((int64_t)G * (sp + 1)) / splits);
    }
    const int bm = tile / ntiles;
    const int bn = tile - bm * ntiles;
    int64_t m0 = (int64_t)bm * TM;
    if constexpr (GT::kGrouped) {
        m0 = gt.m0[bm];
        M = (int)(m0 + gt.me[bm]);
        wl.w += (int64_t)gt.e[bm] * gt.expert_bytes;
        if constexpr (ZP) zeros += (int64_t)gt.e[bm] * N * G;
    }
    const int64_t n0 = (int64_t)bn * kPN;

    // Direct loads: wave w fills the 1 KB runs s = w + NW u (u < TM / 4 NW);
    // run s holds rows 4 s .. 4 s + 3, lane l at row 4 s + l / 16, physical
    // chunk l % 16, which is logical chunk (l % 16) ^ (row % 16) (swz16; the
    // row is 4 w + l / 16 modulo 16 for every u).  Rows beyond M read row M-1
    // (their results are dropped).  Byte offsets from the block's column
    // k0, per run, for A (row stride K).
    const int mlim = (int)min((int64_t)M - 1 - m0, (int64_t)TM - 1);
    // A wave whose 128 rows all lie past the tile's last row (a short last
    // tile, or a small expert's tile) computes nothing: it runs its own loop
    // that only takes its part in the workgroup's loads and barriers.
    const bool idle = !kSmall && 128 * wm > mlim;
    // A wave whose last 64 rows (phase 1) are all past the tile's end runs
    // phase 0 only (every wave of a 64-row tile).
    const bool half = kSmall || (!idle && 128 * wm + 64 > mlim);
    const int dma_row0 = 4 * wave + (lane >> 4);
    const int dma_chunk = (lane & 15) ^ (dma_row0 & 15);
    const uint16_t *A_blk = A + m0 * K;
    constexpr int RU = TM / (4 * NW);  // runs per wave
    uint32_t doff[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u)
        doff[u] = (uint32_t)((min(dma_row0 + 4 * NW * u, mlim) * K + 8 * dma_chunk) * 2);
    // Direct loads through a buffer resource on the tile's rows: the lane's
    // offset (under 2^31 bytes: row < 256, K <= 2^22) in a VGPR, the group's
    // column offset in an SGPR, so no per-load 64-bit address arithmetic.
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)A_blk, (short)0, 0x7FFFFFFF, kBufferRsrcWord3);
    auto dma = [&](const uint16_t *, int k0, const uint32_t(&off)[RU], auto bconst)
        __attribute__((always_inline)) {
        constexpr int BUF = decltype(bconst)::value;
        u32x4 *dst = BUF == 0 ? As0 : BUF == 1 ? As1 : As2;
#pragma unroll
        for (int u = 0; u < RU; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                a_rsrc, (__attribute__((address_space(3))) void *)&dst[64 * (wave + NW * u)], 16,
                (int)off[u], 2 * k0, 0, 0);
    };
    // Run u alone (the main loop spreads a group's runs over MFMA slots).
    auto dma_one = [&](int u, int k0, auto bconst) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bconst)::value;
        u32x4 *dst = BUF == 0 ? As0 : BUF == 1 ? As1 : As2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            a_rsrc, (__attribute__((address_space(3))) void *)&dst[64 * (wave + NW * u)], 16,
            (int)doff[u], 2 * k0, 0, 0);
    };

    // Codes: each group's 128 columns x b planes of 16 bytes (2 b runs of
    // 64 lanes, one 64-row block and plane each) go global -> LDS with the
    // same direct loads; wave w issues runs w, w + NW, ...  Lane l of run r
    // (block t = r / b, plane p = r % b) reads chunk p of row n0 + 64 t + l
    // (rows beyond N read row N-1).  The lane's column (32 wn + c32, block
    // t = wn / 2, row rho) and half h then read dword pair i of the half,
    // slot dword d = 2 h B + 2 i, from LDS at coff[i].
    // Codes through a buffer resource based at the tile's first row: every
    // offset is under 2^31 bytes (two 64-row blocks of tiles, or 128 dense
    // rows of at most 4 MB).
    const uint8_t *cbase = reinterpret_cast<const uint8_t *>(wl.chunks(min(n0, (int64_t)N - 1), 0));
    const __amdgpu_buffer_rsrc_t c_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)cbase, (short)0, 0x7FFFFFFF, kBufferRsrcWord3);
    int crow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        crow[t] = (int)(reinterpret_cast<const uint8_t *>(
                            wl.chunks(min(n0 + 64 * t + lane, (int64_t)N - 1), 0)) -
                        cbase);
    const int64_t bstep = wl.slot_step();
    const int cstride = (int)wl.chunk_stride() * 16;
    auto dma_codes = [&](int g, auto bconst) __attribute__((always_inline)) {
        u32x4 *dst = Cs[decltype(bconst)::value];
#pragma unroll
        for (int k = 0; k < (2 * B + NW - 1) / NW; ++k) {
            const int r = wave + NW * k;
            if (r < 2 * B) {
                const int t = r >= B ? 1 : 0, p = r - t * B;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    c_rsrc, (__attribute__((address_space(3))) void *)&dst[64 * r], 16, crow[t],
                    (int)(g * bstep) + p * cstride, 0, 0);
            }
        }
    };
    int coff[B];
    {
        const int c = 32 * wn + c32, t = c >> 6, rho = c & 63;
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int d = 2 * h * B + 2 * i;
            coff[i] = ((t * B + (d >> 2)) * 64 + rho) * 16 + (d & 3) * 4;
        }
    }
    // Even b: the half-slot starts on a 16-byte chunk, read as b / 2 16-byte
    // reads (lanes 16 bytes apart: conflict free; 8-byte reads at that stride
    // put two lanes on each bank).  Odd b: 8-byte reads.
    auto read_codes = [&](auto bconst, uint32_t(&dst)[2 * B]) __attribute__((always_inline)) {
        const uint8_t *src = reinterpret_cast<const uint8_t *>(Cs[decltype(bconst)::value]);
        if constexpr ((B & 1) == 0) {
#pragma unroll
            for (int i = 0; i < B; i += 2) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(src + coff[i]);
                dst[2 * i] = v.x;
                dst[2 * i + 1] = v.y;
                dst[2 * i + 2] = v.z;
                dst[2 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i) {
                const uint2 v = *reinterpret_cast<const uint2 *>(src + coff[i]);
                dst[2 * i] = v.x;
                dst[2 * i + 1] = v.y;
            }
        }
    };
    const int64_t bcol = min(n0 + 32 * wn + c32, (int64_t)N - 1);
    const uint8_t *sptr = wl.scale0(bcol);
    const int64_t sstep = wl.scale_step();
    // Zero points [N, G]: the lane's column, one group ahead like the scale.
    const uint8_t *zrow = ZP ? zeros + bcol * G : nullptr;
    int zop = 0, znext = 0;
    auto load_scale = [&](int g, uint32_t &sc) __attribute__((always_inline)) {
        sc = *reinterpret_cast<const uint16_t *>(sptr + min(g, g_hi - 1) * sstep);
        if constexpr (ZP) znext = zrow[min(g, g_hi - 1)];
    };
    // The lane's half-slot of codes as read (its 2B words are whole 32-code
    // runs), prepared for slot_pair: sign-flipped in place (dense stream,
    // symmetric), as is (zero points), or decoded to int8 words (tiled
    // layout, arranged runs of b = 5, 6, 7).
    constexpr bool I8 = WL::kTiled && int8_ready<B>() && !ZP;
    constexpr float kSInv = operand_scale_inv<B, I8, ZP>();
    uint32_t cint[int8_words<B, ZP, I8>() ? 16 : 1];
    auto flip = [&](uint32_t(&c)[2 * B]) __attribute__((always_inline)) {
        prep_runs<B, ZP, I8, 2>(c, cint, zop);
    };
    // A operand of k-step j: LDS row 128 wm + 64 PH + 32 t + c32 (the last
    // three terms compile-time), chunk (8 h + j) ^ (c32 % 16).
    int aoff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) aoff[j] = (128 * wm + c32) * 16 + ((8 * h + j) ^ (c32 & 15));

    f32x16_t tot[4], P[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            tot[i][r] = 0.0f;
            P[i][r] = 0.0f;
        }
    uint32_t creg[2 * B];
    uint32_t sreg = 0, snext = 0;
    u32x4 bop[8];
    bf16x8_t af[2][2];  // [set][row of the phase]

    // B operand of k-step J: pairs 4 (J % 4) .. +3 of quarter J / 4 of the half.
    auto unpack_pair = [&](auto jconst, auto iconst) __attribute__((always_inline)) {
        constexpr int J = decltype(jconst)::value, I = decltype(iconst)::value;
        bop[J][I] = slot_pair<B, 16 * (J >> 2) + 4 * (J & 3) + I, ZP, I8>(creg, cint, zop);
    };
    auto read_a = [&](auto bconst, int row0, int j, int set) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bconst)::value;
        const u32x4 *src = BUF == 0 ? As0 : BUF == 1 ? As1 : As2;
#pragma unroll
        for (int t = 0; t < 2; ++t)
            af[set][t] = __builtin_bit_cast(bf16x8_t, src[aoff[j] + (row0 + 32 * t) * 16]);
    };
    // The results pass through an empty asm so that the two FMAs stay in
    // their slot: each fold result is next needed a group later, and without
    // it the compiler sinks the whole group's folds into one burst of VALU
    // work next to no MFMA (measured: the kernel ran 50% slower).
    auto fold_slice = [&](int i0, int q, float s) __attribute__((always_inline)) {
        const int i = i0 + (q >> 3), r = 2 * (q & 7);
        float t0 = fmaf(s, P[i][r], tot[i][r]);
        float t1 = fmaf(s, P[i][r + 1], tot[i][r + 1]);
        asm volatile("" : "+v"(t0), "+v"(t1));
        tot[i][r] = t0;
        tot[i][r + 1] = t1;
    };
    // One phase: block rows 2 PH, 2 PH + 1, k-steps 0..7, operands one
    // k-step ahead (k-step 0's already in set 0).  After each MFMA hook(slot)
    // issues a slice of other work; the pair is fenced so the order written
    // is the issue order.  The last k-step reads the next phase's k-step 0
    // (phase 0 only: phase 1's successor follows a barrier).
    auto phase = [&](auto phconst, auto bconst, auto &&hook) __attribute__((always_inline)) {
        constexpr int PH = decltype(phconst)::value;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int set = j & 1;
            if (j + 1 < 8) read_a(bconst, 64 * PH, j + 1, set ^ 1);
            else if (PH == 0 && !kSmall) read_a(bconst, 64, 0, set ^ 1);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x16_t c = P[2 * PH + t];
                if (j == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) c[r] = 0.0f;
                }
                P[2 * PH + t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    af[set][t], __builtin_bit_cast(bf16x8_t, bop[j]), c, 0, 0, 0);
                hook(2 * j + t);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // Phase 0's hook while unpacking: slots 2j, 2j+1 unpack pairs 0,1 and
    // 2,3 of k-step j+1.
    auto unpack_slot = [&](int slot) __attribute__((always_inline)) {
        const int j = (slot >> 1) + 1;
        if (j >= 8) return;
        if ((slot & 1) == 0) {
            switch (j) {
                case 1: unpack_pair(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); break;
                case 2: unpack_pair(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}); break;
                case 3: unpack_pair(std::integral_constant<int, 3>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{}); break;
                case 4: unpack_pair(std::integral_constant<int, 4>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 4>{}, std::integral_constant<int, 1>{}); break;
                case 5: unpack_pair(std::integral_constant<int, 5>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 5>{}, std::integral_constant<int, 1>{}); break;
                case 6: unpack_pair(std::integral_constant<int, 6>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 6>{}, std::integral_constant<int, 1>{}); break;
                default: unpack_pair(std::integral_constant<int, 7>{}, std::integral_constant<int, 0>{}); unpack_pair(std::integral_constant<int, 7>{}, std::integral_constant<int, 1>{}); break;
            }
        } else {
            switch (j) {
                case 1: unpack_pair(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 1>{}, std::integral_constant<int, 3>{}); break;
                case 2: unpack_pair(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{}); break;
                case 3: unpack_pair(std::integral_constant<int, 3>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 3>{}, std::integral_constant<int, 3>{}); break;
                case 4: unpack_pair(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 4>{}, std::integral_constant<int, 3>{}); break;
                case 5: unpack_pair(std::integral_constant<int, 5>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 5>{}, std::integral_constant<int, 3>{}); break;
                case 6: unpack_pair(std::integral_constant<int, 6>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 6>{}, std::integral_constant<int, 3>{}); break;
                default: unpack_pair(std::integral_constant<int, 7>{}, std::integral_constant<int, 2>{}); unpack_pair(std::integral_constant<int, 7>{}, std::integral_constant<int, 3>{}); break;
            }
        }
    };
    auto unpack_k0 = [&]() __attribute__((always_inline)) {
        unpack_pair(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        unpack_pair(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
        unpack_pair(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{});
        unpack_pair(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
    };

    float sq_prev = 0.0f;

    // ---- real groups ----
    // Group g's A in buffer (g - g_lo) & 1.  Prologue: group g_lo's A, codes
    // and scale.
    if constexpr (!kSmall) {
        dma(A_blk, g_lo * kGroup, doff, std::integral_constant<int, 0>{});
        dma_codes(g_lo, std::integral_constant<int, 0>{});
        load_scale(g_lo, snext);
    }
    auto group = [&](int g, auto bconst) __attribute__((always_inline)) {
        constexpr int BUF = decltype(bconst)::value;
        // Group g's A and codes have landed for this wave; after the barrier
        // for every wave, and every wave is done with the other buffers.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        sreg = snext;
        zop = znext;
        read_codes(bconst, creg);
        flip(creg);
        // Group g + 1's A goes out one run per MFMA slot of phase 0, not as
        // one burst at the barrier.
        const int k_next = min(g + 1, g_hi - 1) * kGroup;
        dma_codes(min(g + 1, g_hi - 1), std::integral_constant<int, BUF ^ 1>{});
        load_scale(g + 1, snext);
        unpack_k0();
        read_a(bconst, 0, 0, 0);
        const float sg = bf16_to_f32((uint16_t)sreg) * kSInv;
        phase(std::integral_constant<int, 0>{}, bconst, [&](int slot) {
            fold_slice(2, slot, sq_prev);
            unpack_slot(slot);
            if (slot < RU) dma_one(slot, k_next, std::integral_constant<int, BUF ^ 1>{});
        });
        // Rows 0, 1 finished at phase 0's last slots: their fold starts at
        // slot 2 (32 FMAs over 14 slots) so it does not wait on those MFMAs.
        phase(std::integral_constant<int, 1>{}, bconst, [&](int slot) {
            if (slot >= 2) fold_slice(0, slot - 2, sg);
            if (slot >= 14) fold_slice(0, slot, sg);
        });
        sq_prev = sg;
    };
    int g = g_lo;
    if constexpr (kSmall) {
        // 64-row tile, a three-stage ring: group g's A in LDS buffer
        // (g - g_lo) % 3 and its codes (the lane's half-slot, loaded per lane),
        // scale and zero point in register stage (g - g_lo) % 3, all issued two
        // groups ahead.  The wait before group g leaves the L vector loads each
        // wave issued for group g + 1 in flight (vector loads complete in
        // issue order); the barrier after it also means every wave is done
        // with the buffer group g + 2 then fills (read in group g - 1).
        constexpr int NC = (B & 1) ? B : B / 2;           // code loads per lane
        constexpr int L = RU + NC + 1 + (ZP ? 1 : 0);     // vector loads per group
        static_assert(L < 16, "vmcnt field");
        const uint8_t *cslot = reinterpret_cast<const uint8_t *>(wl.slot0(bcol));
        int goff[NC];
#pragma unroll
        for (int q = 0; q < NC; ++q)
            goff[q] = WL::dword_off(2 * h * B + ((B & 1) ? 2 * q : 4 * q));
        uint32_t cr[3][2 * B];
        uint32_t sr[3], zr[3];
        auto issue = [&](int gi, auto sconst) __attribute__((always_inline)) {
            constexpr int S = decltype(sconst)::value;
            gi = min(gi, g_hi - 1);
            dma(A_blk, gi * kGroup, doff, sconst);
            const uint8_t *src = cslot + gi * bstep;
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                if constexpr ((B & 1) == 0) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(src + goff[q]);
                    cr[S][4 * q] = v.x;
                    cr[S][4 * q + 1] = v.y;
                    cr[S][4 * q + 2] = v.z;
                    cr[S][4 * q + 3] = v.w;
                } else {
                    const uint2 v = *reinterpret_cast<const uint2 *>(src + goff[q]);
                    cr[S][2 * q] = v.x;
                    cr[S][2 * q + 1] = v.y;
                }
            }
            sr[S] = *reinterpret_cast<const uint16_t *>(sptr + gi * sstep);
            if constexpr (ZP) zr[S] = zrow[gi];
        };
        auto ring_group = [&](int gi, auto sconst) __attribute__((always_inline)) {
            constexpr int S = decltype(sconst)::value;
            __builtin_amdgcn_s_waitcnt(0x0F70 | L);  // vmcnt(L)
            // A bare barrier (the memory clobber keeps the compiler from
            // moving LDS accesses across it): __syncthreads()' release fence
            // would wait for every direct load, the next group's too.
            asm volatile("s_barrier" ::: "memory");
#pragma unroll
            for (int i = 0; i < 2 * B; ++i) creg[i] = cr[S][i];
            sreg = sr[S];
            if constexpr (ZP) zop = (int)zr[S];
            flip(creg);
            issue(gi + 2, std::integral_constant<int, (S + 2) % 3>{});
            unpack_k0();
            read_a(sconst, 0, 0, 0);
            const float sg = bf16_to_f32((uint16_t)sreg) * kSInv;
            phase(std::integral_constant<int, 0>{}, sconst, [&](int slot) { unpack_slot(slot); });
#pragma unroll
            for (int q = 0; q < 16; ++q) fold_slice(0, q, sg);
        };
        issue(g_lo, std::integral_constant<int, 0>{});
        issue(g_lo + 1, std::integral_constant<int, 1>{});
        for (; g + 2 < g_hi; g += 3) {
            ring_group(g, std::integral_constant<int, 0>{});
            ring_group(g + 1, std::integral_constant<int, 1>{});
            ring_group(g + 2, std::integral_constant<int, 2>{});
        }
        if (g < g_hi) ring_group(g, std::integral_constant<int, 0>{});
        if (g + 1 < g_hi) ring_group(g + 1, std::integral_constant<int, 1>{});
        g = g_hi;
    }
    if constexpr (!kSmall) if (idle) {
        auto idle_group = [&](int gi, auto bconst) __attribute__((always_inline)) {
            constexpr int BUF = decltype(bconst)::value;
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            dma(A_blk, min(gi + 1, g_hi - 1) * kGroup, doff,
                std::integral_constant<int, BUF ^ 1>{});
            dma_codes(min(gi + 1, g_hi - 1), std::integral_constant<int, BUF ^ 1>{});
        };
        for (; g + 1 < g_hi; g += 2) {
            idle_group(g, std::integral_constant<int, 0>{});
            idle_group(g + 1, std::integral_constant<int, 1>{});
        }
        if (g < g_hi) idle_group(g, std::integral_constant<int, 0>{});
        g = g_hi;
    }
    if constexpr (!kSmall) if (half) {
        // As group(), without phase 1: rows 0, 1 are folded after phase 0,
        // rows 2, 3 are empty.
        auto half_group = [&](int gi, auto bconst) __attribute__((always_inline)) {
            constexpr int BUF = decltype(bconst)::value;
            __builtin_amdgcn_s_waitcnt(0x0F70);
            __syncthreads();
            sreg = snext;
            zop = znext;
            read_codes(bconst, creg);
            flip(creg);
            dma(A_blk, min(gi + 1, g_hi - 1) * kGroup, doff,
                std::integral_constant<int, BUF ^ 1>{});
            dma_codes(min(gi + 1, g_hi - 1), std::integral_constant<int, BUF ^ 1>{});
            load_scale(gi + 1, snext);
            unpack_k0();
            read_a(bconst, 0, 0, 0);
            const float sg = bf16_to_f32((uint16_t)sreg) * kSInv;
            phase(std::integral_constant<int, 0>{}, bconst, [&](int slot) { unpack_slot(slot); });
#pragma unroll
            for (int q = 0; q < 16; ++q) fold_slice(0, q, sg);
        };
        for (; g + 1 < g_hi; g += 2) {
            half_group(g, std::integral_constant<int, 0>{});
            half_group(g + 1, std::integral_constant<int, 1>{});
        }
        if (g < g_hi) half_group(g, std::integral_constant<int, 0>{});
        g = g_hi;
    }
    if constexpr (!kSmall) {
        for (; g + 1 < g_hi; g += 2) {
            group(g, std::integral_constant<int, 0>{});
            group(g + 1, std::integral_constant<int, 1>{});
        }
        if (g < g_hi) group(g, std::integral_constant<int, 0>{});
        // The last group's rows 2, 3.
#pragma unroll
        for (int q = 0; q < 16; ++q) fold_slice(2, q, sq_prev);
    }
    // Drain the (clamped, unused) prefetch of the group after the last.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Output element r of block i: row 8(r/4) + 4h + r%4, column lane%32.
    // A tail part stores its fp32 sums at [part][tail tile][row of the
    // tile][column].
    float *pt = nullptr;
    if (tail) pt = part + ((int64_t)sp * (tiles - nfull) + (tile - nfull)) * (TM * kPN);
    if (!tail && splits == 1 && m0 + TM <= M && n0 + kPN <= N) {
        // A whole tile: each register's 64 values go to two 64-byte row
        // runs; the row offset is wave-uniform, the lane's offset fixed.
        uint16_t *Yw = Y + (m0 + 128 * wm) * N + n0 + 32 * wn;
        const uint32_t lo = (uint32_t)(4 * h) * (uint32_t)N + (uint32_t)c32;
#pragma unroll
        for (int i = 0; i < (kSmall ? 2 : 4); ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                (Yw + (int64_t)(32 * i + 8 * (r >> 2) + (r & 3)) * N)[lo] =
                        f32_to_bf16_rne(tot[i][r]);
        return;
    }
#pragma unroll
    for (int i = 0; i < (kSmall ? 2 : 4); ++i) {
        const int64_t n = n0 + 32 * wn + c32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            if (m < M && n < N) {
                if (pt)
                    pt[(m - m0) * kPN + (n - n0)] = tot[i][r];
                else if (splits == 1)
                    Y[m * N + n] = f32_to_bf16_rne(tot[i][r]);
                else
                    part[(int64_t)sp * mnp + m * N + n] = tot[i][r];
            }
        }
    }
}

// The tail tiles' outputs: thread t takes 4 consecutive columns of one row of
// tail tile t / (TM kPN / 4) and adds the parts' sums in part order.
__global__ __launch_bounds__(256) void prefill_tail_reduce_kernel(
        const float *__restrict__ part, int tsplits, int nfull, int ntail, int ntiles, int tm,
        int M, int N, uint16_t *__restrict__ Y) {
    const int quads = tm * kPN / 4;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int ts = (int)(t / quads);
    if (ts >= ntail) return;
    const int e = (int)(t - (int64_t)ts * quads) * 4;
    const int tile = nfull + ts;
    const int bm = tile / ntiles, bn = tile - (tile / ntiles) * ntiles;
    const int64_t m = (int64_t)bm * tm + e / kPN;
    const int64_t n = (int64_t)bn * kPN + e % kPN;
    if (m >= M || n >= N) return;
    const int64_t stride = (int64_t)ntail * tm * kPN;  // floats from one part to the next
    const float *p = part + (int64_t)ts * tm * kPN + e;
    // All (at most 4) loads before the first add; indices past the last part
    // repeat it and are not added.
    f32x4_t v[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        v[s] = *reinterpret_cast<const f32x4_t *>(p + min(s, tsplits - 1) * stride);
    f32x4_t acc = v[0];
#pragma unroll
    for (int s = 1; s < 4; ++s)
        if (s < tsplits) acc += v[s];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (n + c < N) Y[m * N + n + c] = f32_to_bf16_rne(acc[c]);
}

// Y = bf16(sum over splits of part[s]) in split order (deterministic); four
// consecutive outputs per thread.  Split s's partials start at s * mnp
// (M * N rounded up to 64 floats, so the vector loads stay aligned).
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float *__restrict__ part,
                                                             int splits, int64_t MN, int64_t mnp,
                                                             uint16_t *__restrict__ Y) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= MN) return;
    // Loads in batches of 8 issued before their adds.
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(part + e);
    for (int s0 = 1; s0 < splits; s0 += 8) {
        f32x4_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = *reinterpret_cast<const f32x4_t *>(part + min(s0 + i, splits - 1) * mnp + e);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s0 + i < splits) acc += v[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (e + i < MN) Y[e + i] = f32_to_bf16_rne(acc[i]);
}

// m-tile rows of a plain (not grouped) launch: 64 up to kSmallTileMaxM
// rows, else 256.  Measured, b = 6, 5120 -> 17408 / 17408 -> 5120: M = 17..64
// 32-35 / 44-48 us with 64-row tiles vs 57-58 / 53-56 with 256; M = 96, 128
// 58-61 vs 61-64 both ways; M = 160, 192 within 3% either way; M = 224, 256
// 88-92 vs 85-89.  WQ_PREFILL_TILE_M (64 or 256) forces one.
constexpr int64_t kSmallTileMaxM = 128;
static int prefill_tile_m(int64_t M) {
    static const int forced = [] {
        const char *e = std::getenv("WQ_PREFILL_TILE_M");
        return e ? std::atoi(e) : 0;
    }();
    if (forced == kPM || forced == kPrefillSmallTileM) return forced;
    return M <= kSmallTileMaxM ? kPrefillSmallTileM : kPM;
}

// K splits: when the tiles alone leave compute units idle, split K so that
// tiles x splits is just under the workgroup slots (256 for 256-row tiles,
// one per compute unit; 512 for 64-row tiles, two), at least 8 groups per
// split; between 3/4 and 3/2 of the slots, 2 splits (the second round of
// workgroups would otherwise run nearly empty).  Measured at M = 512:
// 17408 -> 5120 (80 tiles) best at 3 splits, 174 vs 365 us unsplit;
// 5120 -> 17408 (272 tiles) 219 us at 2 splits vs 240 us (from one round
// up, the tail split below replaces this one).
// WQ_PREFILL_SPLITS forces a split count.
static int prefill_splits(int64_t M, int64_t N, int64_t K) {
    const int tm = prefill_tile_m(M);
    const int64_t slots = tm == kPM ? 256 : 512;
    const int64_t tiles = ((M + tm - 1) / tm) * ((N + kPN - 1) / kPN);
    const int G = (int)(K / kGroup);
    static const int forced = [] {
        const char *e = std::getenv("WQ_PREFILL_SPLITS");
        return e ? std::atoi(e) : 0;
    }();
    if (forced > 0) return std::max(1, std::min(forced, G));
    if (tiles >= slots * 3 / 2) return 1;
    if (tiles >= slots * 3 / 4) return G >= 16 ? 2 : 1;
    int s = (int)std::max<int64_t>(1, slots / tiles);
    return std::max(1, std::min(s, G / 8));
}

static int64_t prefill_mnp(int64_t M, int64_t N) { return (M * N + 63) / 64 * 64; }

// Tail balance.  With whole rounds of workgroups and a last round at most a
// quarter full, or at most half full with long tiles (64 groups or more;
// M = 4096 at 17408 -> 5120 is 640 tiles, 2 rounds and 128 tiles of 136
// groups), the last round's tiles are split along K into up to 4 parts of
// at least 8 groups, which fill that round with shorter workgroups; the
// parts store fp32 sums and a second kernel adds them in part order.
// Measured on MI355X, b = 6, 17408 -> 5120: M = 3584 / 4096 / 5120 0.75 /
// 0.76 / 0.97 ms -> 0.67-0.68 / 0.71 / 0.86-0.87; 5120 -> 17408 at M = 4096
// (2176 tiles, 128 of 40 groups in the last round) was no faster split, so
// it is not.  Between one and 1.5 rounds it replaces the uniform 2-way
// split: 5120 -> 17408 at M = 300 and 512 (272 tiles) 134 / 148 -> 106 /
// 117 us, 17408 -> 5120 at M = 1792 (280 tiles) 399 -> 340 us.  The parts of one round hold at most 256 tiles' outputs (32 MiB
// in fp32).  Never with a forced uniform split; WQ_PREFILL_TAIL=0 turns it
// off.
struct PrefillPlan {
    int tm;       // m-tile rows
    int tiles;    // m-tiles x n-tiles
    int splits;   // uniform K split (1: none)
    int full;     // tiles run whole; the others run as tsplits K parts
    int tsplits;  // K parts of a tail tile (1: no tail split)
    int64_t ws_bytes;
};
static PrefillPlan prefill_plan(int64_t M, int64_t N, int64_t K) {
    PrefillPlan p;
    p.tm = prefill_tile_m(M);
    p.tiles = (int)(((M + p.tm - 1) / p.tm) * ((N + kPN - 1) / kPN));
    p.splits = prefill_splits(M, N, K);
    p.full = p.tiles;
    p.tsplits = 1;
    p.ws_bytes = p.splits > 1 ? kWsScratchOffset + p.splits * prefill_mnp(M, N) * 4 : 0;
    static const bool tail_off = [] {
        const char *e = std::getenv("WQ_PREFILL_TAIL");
        return e && std::atoi(e) == 0;
    }();
    static const bool forced = std::getenv("WQ_PREFILL_SPLITS") != nullptr;
    const int slots = p.tm == kPM ? 256 : 512;
    const int G = (int)(K / kGroup);
    const int r = p.tiles % slots;
    // Between one and 1.5 rounds the tail split replaces the uniform one
    // (whose partials cover the whole output).
    const bool sparse = 4 * r <= slots || (2 * r <= slots && G >= 64);
    const bool band = p.splits > 1 && 2 * p.tiles < 3 * slots;
    if (!tail_off && !forced && p.tiles >= slots && r > 0 && (band || (p.splits == 1 && sparse))) {
        const int s = std::min(std::min(slots / r, 4), G / 8);
        const int64_t bytes = kWsScratchOffset + (int64_t)r * s * p.tm * kPN * 4;
        if (s >= 2) {
            p.splits = 1;
            p.full = p.tiles - r;
            p.tsplits = s;
            p.ws_bytes = bytes;
        }
    }
    return p;
}

// Workspace: the shared counter region (unused here), then the fp32 partial
// outputs: uniform K split, split s at s * mnp floats; tail split, part s of
// tail tile t at (s * tail tiles + t) * tm * 128 floats; nothing otherwise.
int64_t prefill_ws_bytes(int64_t M, int64_t N, int64_t K, int) {
    return prefill_plan(M, N, K).ws_bytes;
}

template <int B, bool ZP>
static hipError_t prefill_bz(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                             bool tiled, const uint16_t *scales, const uint8_t *zeros,
                             uint16_t *Y, void *ws, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const PrefillPlan pl = prefill_plan(M, N, K);
    const int splits = pl.splits;
    float *part = pl.ws_bytes > 0 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) +
                                                              kWsScratchOffset)
                                  : nullptr;
    hipError_t e = hipSuccess;
    const int tm = pl.tm;
    const int mtiles = (int)((M + tm - 1) / tm);
    const int ntiles = (int)((N + kPN - 1) / kPN);
    const int ntail = pl.tiles - pl.full;
    const dim3 grid((unsigned)(pl.full * splits + ntail * pl.tsplits));
    auto run = [&](auto wl) {
        typedef decltype(wl) WL;
        if (tm == kPM)
            hipLaunchKernelGGL((prefill_kernel<B, WL, ZP, NoGroups>), grid, dim3(512), 0, stream,
                               A, (int)M, (int)N, (int)K, wl, zeros, Y, mtiles, ntiles,
                               splits, part, prefill_mnp(M, N), pl.full, pl.tsplits, NoGroups{});
        else
            hipLaunchKernelGGL((prefill_kernel<B, WL, ZP, NoGroups, kPrefillSmallTileM>), grid,
                               dim3(256), 0, stream, A, (int)M, (int)N, (int)K, wl, zeros,
                               Y, mtiles, ntiles, splits, part, prefill_mnp(M, N), pl.full,
                               pl.tsplits, NoGroups{});
    };
    if (tiled)
        run(TiledW{static_cast<const uint8_t *>(W), G, B});
    else
        run(DenseW{static_cast<const uint8_t *>(W), scales, (int64_t)16 * B * G, G, B});
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ntail > 0) {
        const int64_t threads = (int64_t)ntail * tm * kPN / 4;
        hipLaunchKernelGGL(prefill_tail_reduce_kernel, dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, stream, part, pl.tsplits, pl.full, ntail, ntiles, tm,
                           (int)M, (int)N, Y);
        return hipGetLastError();
    }
    if (splits == 1) return e;
    const int64_t MN = M * N;
    const int64_t threads = (MN + 3) / 4;
    hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, part, splits, MN, prefill_mnp(M, N), Y);
    return hipGetLastError();
}

template <int B>
static hipError_t prefill_b(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                            bool tiled, const uint16_t *scales, const uint8_t *zeros,
                            uint16_t *Y, void *ws, hipStream_t stream) {
    if (!zeros) return prefill_bz<B, false>(A, M, N, K, W, tiled, scales, nullptr, Y, ws, stream);
    if constexpr (B == 4 || B == 8)  // the widths with an asymmetric form
        return prefill_bz<B, true>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
    return hipErrorInvalidValue;
}

// Grouped prefill: one launch over (table entry, n-tile), tiled layout, no
// K split; no workspace.
template <int B, bool ZP>
static hipError_t prefill_grouped_bz(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                                     const void *W, const uint8_t *zeros, uint16_t *Y,
                                     const GroupTable &gt, int tile_m, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int ntiles = (int)((N + kPN - 1) / kPN);
    TiledW wl{static_cast<const uint8_t *>(W), G, B};
    if (tile_m == kPrefillSmallTileM)
        hipLaunchKernelGGL((prefill_kernel<B, TiledW, ZP, GroupTable, kPrefillSmallTileM>),
                           dim3((unsigned)(gt.n * ntiles)), dim3(256), 0, stream, A, (int)M,
                           (int)N, (int)K, wl, zeros, Y, gt.n, ntiles, 1, (float *)nullptr,
                           (int64_t)0, gt.n * ntiles, 1, gt);
    else if (tile_m == kPrefillTileM)
        hipLaunchKernelGGL((prefill_kernel<B, TiledW, ZP, GroupTable>), dim3((unsigned)(gt.n * ntiles)),
                           dim3(512), 0, stream, A, (int)M, (int)N, (int)K, wl, zeros, Y,
                           gt.n, ntiles, 1, (float *)nullptr, (int64_t)0, gt.n * ntiles, 1, gt);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_prefill_grouped(const uint16_t *A, int64_t M, int64_t N, int64_t K,
                                  const void *W, const uint8_t *zeros, int b, uint16_t *Y,
                                  const GroupTable &gt, int tile_m, hipStream_t stream) {
    if (zeros) {
        if (b == 4) return prefill_grouped_bz<4, true>(A, M, N, K, W, zeros, Y, gt, tile_m, stream);
        if (b == 8) return prefill_grouped_bz<8, true>(A, M, N, K, W, zeros, Y, gt, tile_m, stream);
        return hipErrorInvalidValue;
    }
    switch (b) {
        case 2: return prefill_grouped_bz<2, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
        case 3: return prefill_grouped_bz<3, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
        case 4: return prefill_grouped_bz<4, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
        case 5: return prefill_grouped_bz<5, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
        case 6: return prefill_grouped_bz<6, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
        case 7: return prefill_grouped_bz<7, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
        case 8: return prefill_grouped_bz<8, false>(A, M, N, K, W, nullptr, Y, gt, tile_m, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                          bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                          uint16_t *Y, void *ws, hipStream_t stream) {
    switch (b) {
        case 2: return prefill_b<2>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
        case 3: return prefill_b<3>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
        case 4: return prefill_b<4>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
        case 5: return prefill_b<5>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
        case 6: return prefill_b<6>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
        case 7: return prefill_b<7>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
        case 8: return prefill_b<8>(A, M, N, K, W, tiled, scales, zeros, Y, ws, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
