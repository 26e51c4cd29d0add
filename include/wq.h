/*
 * wq.h -- C ABI of libwq: b-bit weight-only quantized linear layers (WNA16)
 * and the int8-activation variant (W4A8) for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are cited by page title and section):
 *
 *   y[m, n] = sum_k A[m, k] * s[n, k / 128] * (c[n, k] - 2^(b-1))
 *
 *   - A: bf16 activations [M, K] (row-major).
 *   - c: unsigned b-bit weight codes, b in 2..8; the compressed-tensors WNA16
 *     scheme accepts every width from 2 to 8 ("vLLM Can Run INT5-7",
 *     section 1).
 *   - The codes of one output row are stored as a dense little-endian
 *     bitstream along K, ceil(K * b / 32) 32-bit words per row, so 5/6/7-bit
 *     codes straddle word boundaries (model card
 *     "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings).  Code k occupies stream
 *     bits [k*b, k*b + b), least significant bit first.
 *   - Groups are symmetric above four bits (same page, Findings): one bf16
 *     scale s[n, g] per group of 128 input features, no zero point; the
 *     signed weight is c - 2^(b-1).  Scales may be negative (club-3090
 *     discussion #733, "Under the hood").
 *   - The asymmetric form exists for b = 4 and 8 only (same page,
 *     Findings): an optional zero point z[n, g] (uint8 [N, K/128], zeros_d)
 *     makes the signed weight c - z.  A per-channel scale ("vLLM
 *     Quantization", online shorthands: INT8 with one scale per channel) is
 *     group = K, scales [N, 1].
 *   - The result is the plain linear layer on the dequantized weights
 *     ("vLLM Can Run INT5-7", section 2), y = A . W^T, no bias.
 *
 * Life cycle ("vLLM Quantization", How it works: create, repack, run):
 *   wq_pack      host: codes -> dense packed words            (create)
 *   wq_repack    device: dense words + scales -> tiled blob    (repack)
 *   wq_gemm      device: y = A . dequant(W)^T                  (run)
 *   wq_gemm_a8   device: W4A8 run on the same int4 weights and scales
 *
 * Conventions for every entry point:
 *   - Return WQ_OK (0) or a wq_status code; nothing throws or aborts across
 *     this boundary.  wq_status_str() gives the reason in words.  Invalid
 *     requests are refused, never silently computed another way.
 *   - Pointers named *_d are device pointers (hipMalloc'd or torch CUDA
 *     tensors) and must be 16-byte aligned; pointers without the suffix are
 *     host pointers.  The caller allocates and owns every buffer; the library
 *     allocates no device memory.
 *   - `stream` is a hipStream_t (NULL: the default stream).  Device calls are
 *     enqueued on it and return without synchronizing.  A launch failure
 *     returns WQ_ERR_HIP; wq_last_hip_error() gives the hipError_t value
 *     (thread-local).
 *   - bf16 values travel as uint16_t bit patterns.
 *   - Device entry points require a gfx950 device (WQ_ERR_UNSUPPORTED_DEVICE
 *     otherwise), K % 128 == 0, and group == 128 or group == K
 *     (WQ_ERR_BAD_GROUP).  Zero points are NULL (symmetric) or uint8
 *     [N, K/128] with values below 2^b, and only for b = 4 or 8
 *     (WQ_ERR_ZERO_POINTS).
 *   - Sizes are int64_t; M == 0 is a valid no-op; N, K must be > 0.
 *     wq_gemm and wq_gemm_grouped take K <= 2^22 (WQ_ERR_INVALID_ARG above:
 *     their tile offsets are 32-bit).
 */
#ifndef WQ_H
#define WQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_ABI_VERSION 3

typedef enum wq_status {
    WQ_OK = 0,
    WQ_ERR_INVALID_ARG = 1,        /* null pointer, N or K <= 0, M < 0, bad enum */
    WQ_ERR_UNSUPPORTED_BITS = 2,   /* b outside 2..8 */
    WQ_ERR_BAD_GROUP = 3,          /* group not 128 or K, K % 128 != 0, or per-channel
                                      scales (group K) on a GEMM's dense layout */
    WQ_ERR_MISALIGNED = 4,         /* a device pointer is not 16-byte aligned */
    WQ_ERR_CODE_RANGE = 5,         /* wq_pack: a code is >= 2^b (never masked) */
    WQ_ERR_WORKSPACE = 6,          /* workspace missing or smaller than required */
    WQ_ERR_BAD_LAYOUT = 7,         /* unknown layout, or scales given/missing wrongly */
    WQ_ERR_UNSUPPORTED_DEVICE = 8, /* current device is not gfx950 */
    WQ_ERR_HIP = 9,                /* a HIP call or kernel launch failed */
    WQ_ERR_ZERO_POINTS = 10,       /* zero points for a width without an asymmetric form
                                      (b = 4 or 8; b = 4 on the int8-activation path) */
    WQ_ERR_SCRATCH_LIMIT = 11      /* wq_gemm_noalloc: the problem's scratch exceeds
                                      WQ_NOALLOC_SCRATCH_BYTES */
} wq_status;

/* Weight layouts accepted by the device entry points. */
typedef enum wq_layout {
    /* The dense pack-quantized rows exactly as wq_pack writes them:
     * uint32 [N, ceil(K*b/32)], with the scales in a separate bf16 [N, K/128]
     * array passed as scales_d. */
    WQ_LAYOUT_DENSE = 0,
    /* The repacked blob wq_repack writes.  Rows are taken 64 at a time (the
     * last block zero-padded); for each 64-row block and each group g the
     * blob holds one tile of b*1024 + 128 bytes: b planes of 1 KB where plane
     * j holds, for row r of the block, bytes [16j, 16j + 16) of that row's
     * group-g stream (b*16 bytes, 128 codes) at offset 16r, followed by the
     * 64 bf16 scales s[row, g].  Tiles are ordered block-major, then g.
     * Scales live inside the blob, so scales_d must be NULL.
     * For b = 2, 3, 4, 8 the group stream is the dense one.  For b = 5, 6, 7
     * it is rearranged so that it decodes to int8 with masks and shifts:
     * with v_i = c_i XOR 2^(b-1) (the b-bit two's complement of the signed
     * weight c_i - 2^(b-1)), the 16b bytes are 4 runs of 4b bytes, run q
     * holding u_k = v_(32q+k), k < 32.  Byte k < 4b of a run holds u_k in its
     * top b bits; its low 8 - b bits carry u_(4b) .. u_31 (e = 0..3):
     *   b = 7: bit 0 of byte 4i + e is bit i of u_(28+e), i = 0..6;
     *   b = 6: bits 1:0 of bytes 12s + e, 12s + 4 + e, 12s + 8 + e are bits
     *          5:4, 3:2, 1:0 of u_(24+4s+e), s = 0, 1;
     *   b = 5: bits 2:0 of byte 4s + e are bits 4:2 and bits 1:0 of byte
     *          12 + 4s + e are bits 1:0 of u_(20+4s+e), s = 0, 1; bits 2:0
     *          of byte 8 + e are bits 4:2 of u_(28+e), bit 2 of byte 12 + e
     *          its bit 1 and bit 2 of byte 16 + e its bit 0. */
    WQ_LAYOUT_TILED = 1
} wq_layout;

typedef enum wq_op {
    WQ_OP_GEMM = 0,     /* wq_gemm */
    WQ_OP_GEMM_A8 = 1   /* wq_gemm_a8 */
} wq_op;

typedef enum wq_out_dtype {
    WQ_OUT_BF16 = 0,    /* bf16 output, round to nearest even */
    WQ_OUT_F32 = 1      /* fp32 output (wq_gemm_a8 only) */
} wq_out_dtype;

/* WQ_ABI_VERSION of the loaded library. */
int wq_abi_version(void);

/* Static text describing a wq_status value ("unknown status" otherwise):
 * the reason a request was refused, in words (club-3090 discussion #733,
 * "Which slugs": an invalid combination is refused and the reason given;
 * model card "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings: an unsupported
 * width raises instead of computing something else). */
const char *wq_status_str(int status);

/* hipError_t of the last WQ_ERR_HIP returned on this thread (0 if none). */
int wq_last_hip_error(void);

/* 1 if HIP device `device` is a gfx950 the kernels were built for, else 0:
 * the capability gate (model card "Qwen3.8-27B-INT6-Mixed-AutoRound", How
 * to use: the WNA16 kernel declares a minimum device capability and runs
 * only on hardware that meets it; here that is the one architecture the
 * library is built for).  Device entry points run
 * the same check on the current device (WQ_ERR_UNSUPPORTED_DEVICE). */
int wq_device_supported(int device);

/* Packed row length of the dense layout: ceil(K * b / 32) 32-bit words
 * (model card "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings: 960 words for
 * 5120 six-bit codes).  Returns -1 for K < 0 or b outside 1..8. */
int64_t wq_packed_words_per_row(int64_t K, int b);

/* Host.  Pack unsigned codes uint8 [N, K] (each < 2^b) into the dense layout
 * uint32 [N, wq_packed_words_per_row(K, b)].  Rows are independent streams,
 * zero-padded to a whole word.  A code >= 2^b returns WQ_ERR_CODE_RANGE and
 * leaves `packed` unspecified.  Host pointers; no alignment requirement. */
int wq_pack(const uint8_t *codes, int64_t N, int64_t K, int b, int group, uint32_t *packed);

/* Host.  Inverse of wq_pack: packed uint32 [N, ceil(K*b/32)] -> uint8 [N, K]. */
int wq_unpack(const uint32_t *packed, int64_t N, int64_t K, int b, uint8_t *codes);

/* Bytes of a weight buffer in `layout` (dense words only for
 * WQ_LAYOUT_DENSE; the whole blob, scales included, for WQ_LAYOUT_TILED).
 * Returns -1 for invalid arguments. */
int64_t wq_repacked_bytes(int layout, int64_t N, int64_t K, int b, int group);

/* Device.  Repack (the "repack after load" step of "vLLM Quantization", How
 * it works): dense words packed_d uint32 [N, ceil(K*b/32)] and scales_d bf16
 * [N, K/group] -> out_d, wq_repacked_bytes(layout, ...) bytes, in `layout`
 * (only WQ_LAYOUT_TILED is a repack target).  With group = K (per-channel)
 * the row's scale is written into every group of the blob.  Inputs are not
 * modified. */
int wq_repack(const uint32_t *packed_d, const uint16_t *scales_d, int64_t N, int64_t K,
              int b, int group, int layout, void *out_d, void *stream);

/* Device.  Extract the codes of a weight buffer in `layout` into uint8
 * [N, K] with the same in-register unpacker the GEMM kernels use.  Exposed
 * so the unpacker can be checked code for code. */
int wq_unpack_dev(const void *W_d, int layout, int64_t N, int64_t K, int b, int group,
                  uint8_t *codes_d, void *stream);

/* Workspace bytes wq_gemm (op = WQ_OP_GEMM) or wq_gemm_a8 (WQ_OP_GEMM_A8)
 * needs for this problem (0 if none; -1 for invalid arguments).  Every
 * non-empty workspace begins with a region of WQ_WORKSPACE_ZERO_BYTES of
 * split-K counters that must be zero before the first call that uses it;
 * every call leaves that region zero again, whatever the op or shape, so one
 * workspace (sized for the largest call) can serve any sequence of calls
 * ordered on one stream.  The rest is scratch.  Calls that may run
 * concurrently need separate workspaces. */
#define WQ_WORKSPACE_ZERO_BYTES ((int64_t)1 << 16)
int64_t wq_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int b, int group);

/* Device.  WNA16 layer: Y_d bf16 [M, N] = A_d bf16 [M, K] . dequant(W)^T.
 * W_d is in `layout`; scales_d bf16 [N, K/128] for WQ_LAYOUT_DENSE, NULL for
 * WQ_LAYOUT_TILED (whose blob holds them; per-channel scales reach this
 * layer through wq_repack with group = K, the dense layout takes group 128
 * only).  zeros_d: NULL, or uint8 zero points [N, K/128] for b = 4 or 8.
 * Every product multiplies an activation by the exact signed code
 * (c - 2^(b-1), or c - z) as bf16, accumulation is fp32 and the group scale
 * is applied once per group in fp32, so the rounding error of an output is
 * bounded by the sum of |a * w| of its own terms (a row of midpoint codes
 * gives exactly 0); the output is rounded to bf16 (nearest even).
 * ws_d / ws_bytes: see wq_workspace_bytes.  Results are deterministic
 * (fixed reduction order). */
int wq_gemm(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d, int layout,
            const uint16_t *scales_d, const uint8_t *zeros_d, int b, int group, uint16_t *Y_d,
            void *ws_d, int64_t ws_bytes, void *stream);

/* Device.  wq_gemm without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments,
 * results and rounding are those of wq_gemm (the same kernels and plans);
 * the split-K scratch is a static array of WQ_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  A problem
 * whose wq_workspace_bytes(WQ_OP_GEMM, ...) exceeds that size is refused
 * with WQ_ERR_SCRATCH_LIMIT before anything is launched.  All calls on one
 * GPU share its array: calls that may overlap in time on one GPU (different
 * streams, or host threads without ordering) race and must not be issued;
 * calls ordered on one stream are safe.  The first call on a device that
 * needs scratch also enqueues a small kernel that clears its counters. */
#define WQ_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
int wq_gemm_noalloc(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d,
                    int layout, const uint16_t *scales_d, const uint8_t *zeros_d, int b,
                    int group, uint16_t *Y_d, void *stream);

/* Device.  Grouped (mixture-of-experts) WNA16 layer (model card
 * "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings: the dense format has no
 * fused MoE path).  E experts, each a tiled blob (wq_repack output for
 * N x K at b) at W_d + e * expert_bytes (expert_bytes >= that blob's size,
 * a multiple of 16); the rows of A_d bf16 [M, K] are sorted by expert:
 * expert e owns rows [offsets[e], offsets[e+1]) (a host array of E + 1
 * values, offsets[0] = 0, offsets[E] = M, nondecreasing), and Y_d bf16
 * [M, N] row m is row m of A through its expert's layer.  zeros_d: NULL or
 * uint8 [E * N, K/128] (b = 4, 8).  ws_d / ws_bytes: at least
 * wq_grouped_workspace_bytes (the same counter-region rule as wq_gemm).
 * Experts with at most 16 rows run in one decode launch (one table entry per
 * expert, passed as a kernel argument), the others in one prefill launch
 * over their 256-row tiles; experts without rows read nothing. */
int64_t wq_grouped_workspace_bytes(const int64_t *offsets, int64_t E, int64_t N, int64_t K,
                                   int b, int group);
int wq_gemm_grouped(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d,
                    int64_t expert_bytes, const uint8_t *zeros_d, const int64_t *offsets,
                    int64_t E, int b, int group, uint16_t *Y_d, void *ws_d, int64_t ws_bytes,
                    void *stream);

/* Device.  Per-token dynamic int8 activation quantization (club-3090
 * discussion #733, "Under the hood"), fp32 throughout:
 *   sa_d[m] = max_k |A[m,k]| / 127   (IEEE division)
 *   Aq_d[m,k] = clamp(rint(A[m,k] / sa_d[m]), -127, 127)   (ties to even)
 * A row of zeros gives sa = 0 and Aq = 0.  Aq_d int8 [M, K], sa_d fp32 [M]. */
int wq_quant_act_i8(const uint16_t *A_d, int64_t M, int64_t K, int8_t *Aq_d, float *sa_d,
                    void *stream);

/* Device.  Quantized embedding gather on the dense layout (model card
 * "Qwen3.8-27B-INT6-Mixed-AutoRound", Findings: a 5/6/7-bit embed_tokens
 * needs a gather that reads the dense rows, codes straddling words; "vLLM
 * Can Run INT5-7", section 3: the vocabulary tables, 248,320 x 5,120, are
 * worth storing in INT8).  For t in [0, T), with id = ids_d[t]:
 *   Y_d[t, k] = bf16_rne(s[id, k/group] * (c[id, k] - z[id, k/128]))   if 0 <= id < V
 *   Y_d[t, k] = 0                                                       otherwise
 * with z = 2^(b-1) when zeros_d is NULL (ids outside the table give zero
 * rows, as the rows of a vocabulary shard that belong to other shards).
 * W_d: dense packed uint32 [V, ceil(K*b/32)] (what wq_pack writes),
 * scales_d bf16 [V, K/group] (group 128 or K), zeros_d NULL or uint8
 * [V, K/128] (b = 4, 8), ids_d int64 [T], Y_d bf16 [T, K], all device memory
 * owned by the caller.  The product is exact in fp32 and rounded once, so
 * the result is bit-exact.  T = 0 is a no-op. */
int wq_embed(const void *W_d, const uint16_t *scales_d, const uint8_t *zeros_d, int64_t V,
             int64_t K, int b, int group, const int64_t *ids_d, int64_t T, uint16_t *Y_d,
             void *stream);

/* Device.  Int8-activation layer (same page; b = 4 is its W4A8):
 * activations quantized as wq_quant_act_i8 does, b-bit codes widened to
 * int8 without loss (c - 2^(b-1) in [-128, 127]; the page's condition for
 * the widening, met by integer codes of any b <= 8, so b = 8 gives W8A8),
 * int8 products summed exactly in int32 per group of 128, then
 *   Y[m, n] = sa[m] * sum_g s[n, g] * acc_g[m, n]     (fp32)
 * written as bf16 (out_dtype WQ_OUT_BF16) or fp32 (WQ_OUT_F32).  The same
 * packed weights and scales as wq_gemm are used, any b in 2..8.  Zero
 * points (c - z) only for b = 4: at b = 8, c - z can leave the int8 range.
 * The workspace holds Aq and sa. */
int wq_gemm_a8(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d,
               int layout, const uint16_t *scales_d, const uint8_t *zeros_d, int b, int group,
               void *Y_d, int out_dtype, void *ws_d, int64_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
