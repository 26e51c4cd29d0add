// wq_api.hip -- the C ABI declared in include/wq.h: argument validation, the
// host packer/unpacker, sizes, and dispatch to the device kernels.
//
// Every entry point validates before touching memory, returns a wq_status
// and never throws; device work is only enqueued on the caller's stream.
#include "wq.h"
#include "wq_launch.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

namespace {

constexpr int kGroup = 128;
constexpr int kMaxDevices = 64;

thread_local int g_last_hip_error = 0;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return WQ_ERR_HIP;
}

bool valid_bits(int b) { return b >= 2 && b <= 8; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Groups of 128 codes, or one group per row (per-channel scales, group = K).
int check_group(int64_t K, int group) {
    if (K % kGroup != 0 || (group != kGroup && group != K)) return WQ_ERR_BAD_GROUP;
    return WQ_OK;
}

bool per_channel(int64_t K, int group) { return group == K && K != kGroup; }

// Zero points exist for b = 4 and 8 (for b = 4 only on the int8-activation path).
int check_zeros(const uint8_t *zeros, int b, bool a8) {
    if (!zeros) return WQ_OK;
    if (b != 4 && (b != 8 || a8)) return WQ_ERR_ZERO_POINTS;
    if (!aligned16(zeros)) return WQ_ERR_MISALIGNED;
    return WQ_OK;
}

// Shapes the kernels index with 32-bit ints.
bool dims_ok(int64_t M, int64_t N, int64_t K) {
    return M >= 0 && N > 0 && K > 0 && M < (1ll << 31) && N < (1ll << 31) && K < (1ll << 31);
}

// The WNA16 prefill kernel addresses a tile's activation rows with 32-bit
// byte offsets (row * K * 2 with row < 256), which hold for K <= 2^22.
constexpr int64_t kMaxGemmK = 1ll << 22;
bool gemm_dims_ok(int64_t M, int64_t N, int64_t K) { return dims_ok(M, N, K) && K <= kMaxGemmK; }

int query_device(int dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 2;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
}

// The current device must be a gfx950 (result cached per device).
int check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {  // no usable HIP device at all
        g_last_hip_error = (int)e;
        return WQ_ERR_UNSUPPORTED_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return query_device(dev) == 1 ? WQ_OK : WQ_ERR_UNSUPPORTED_DEVICE;
    int st = g_device_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        st = query_device(dev);
        g_device_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? WQ_OK : WQ_ERR_UNSUPPORTED_DEVICE;
}

int64_t words_per_row(int64_t K, int b) { return (K * (int64_t)b + 31) / 32; }

// Run f(row_begin, row_end) over [0, N) on up to 16 host threads.
template <class F>
void parallel_rows(int64_t N, int64_t work_per_row, F f) {
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    int64_t nt = std::min<int64_t>({(int64_t)hw, 16, N});
    if (N * work_per_row < (1 << 20) || nt <= 1) {
        f((int64_t)0, N);
        return;
    }
    std::vector<std::thread> th;
    const int64_t chunk = (N + nt - 1) / nt;
    for (int64_t t = 0; t < nt; ++t) {
        const int64_t r0 = t * chunk, r1 = std::min(N, r0 + chunk);
        if (r0 >= r1) break;
        th.emplace_back([=] { f(r0, r1); });
    }
    for (auto &t : th) t.join();
}

// The WNA16 layer on one weight set: the decode kernel up to kDecodeMaxM
// rows, the prefill kernel above.
hipError_t gemm_dispatch(const uint16_t *A, int64_t M, int64_t N, int64_t K, const void *W,
                         bool tiled, const uint16_t *scales, const uint8_t *zeros, int b,
                         uint16_t *Y, void *ws, hipStream_t stream) {
    if (M <= wq::kDecodeMaxM)
        return wq::launch_decode(A, M, N, K, W, tiled, scales, zeros, b, Y, ws,
                                 wq::decode_plan(M, N, K, b), stream);
    return wq::launch_prefill(A, M, N, K, W, tiled, scales, zeros, b, Y, ws, stream);
}

int64_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int b) {
    if (M == 0) return 0;
    if (M <= wq::kDecodeMaxM) return wq::decode_plan(M, N, K, b).ws_bytes;
    return wq::prefill_ws_bytes(M, N, K, b);
}

// The launches of a grouped call: experts with at most kDecodeMaxM rows go
// into decode tables (one entry per expert), the others into prefill tables
// of 256-row or of 64-row m-tiles (one entry per tile); a table is emitted
// when full or at the end.  emit(is_decode, table, m): for a decode table
// the most rows of its entries, for a prefill table its tile size.
template <class F>
void grouped_tables(const int64_t *off, int64_t E, int64_t N, int64_t expert_bytes, F emit) {
    wq::GroupTable dec{}, pre{}, small{};
    int dec_max = 0;
    dec.per = (int)((N + 63) / 64);
    dec.expert_bytes = pre.expert_bytes = small.expert_bytes = expert_bytes;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t m0 = off[e], me = off[e + 1] - off[e];
        if (me == 0) continue;
        if (me <= wq::kDecodeMaxM) {
            dec.e[dec.n] = (int)e;
            dec.m0[dec.n] = (int)m0;
            dec.me[dec.n] = (int)me;
            dec_max = std::max(dec_max, (int)me);
            if (++dec.n == wq::kMaxGroups) {
                emit(true, dec, dec_max);
                dec.n = 0;
                dec_max = 0;
            }
            continue;
        }
        // 256-row tiles while at least 192 rows remain, then 64-row tiles
        // (a few dozen rows in a 256-row tile leave most of its waves idle).
        for (int64_t r = 0; r < me;) {
            const bool big = me - r >= 192;
            wq::GroupTable &t = big ? pre : small;
            const int tm = big ? wq::kPrefillTileM : wq::kPrefillSmallTileM;
            t.e[t.n] = (int)e;
            t.m0[t.n] = (int)(m0 + r);
            t.me[t.n] = (int)std::min<int64_t>(tm, me - r);
            r += t.me[t.n];
            if (++t.n == wq::kMaxGroups) {
                emit(false, t, tm);
                t.n = 0;
            }
        }
    }
    if (dec.n) emit(true, dec, dec_max);
    if (pre.n) emit(false, pre, wq::kPrefillTileM);
    if (small.n) emit(false, small, wq::kPrefillSmallTileM);
}

// Decode plan of a grouped decode table: the plan for its largest row count
// over the grid's columns, entries * ceil(N/64) blocks of 64, so its row
// blocks (tickets, partial sums, workspace) are exactly the grid's.
wq::DecodePlan grouped_decode_plan(const wq::GroupTable &t, int max_me, int64_t N, int64_t K,
                                   int b) {
    (void)N;
    return wq::decode_plan(max_me, (int64_t)t.n * t.per * 64, K, b, false);
}

int64_t grouped_ws_bytes(const int64_t *off, int64_t E, int64_t N, int64_t K, int b) {
    int64_t need = 0;
    grouped_tables(off, E, N, 0, [&](bool is_dec, const wq::GroupTable &t, int max_me) {
        // Prefill tables need no workspace (no K split).
        if (is_dec) need = std::max(need, grouped_decode_plan(t, max_me, N, K, b).ws_bytes);
    });
    return need;
}

int check_offsets(const int64_t *off, int64_t E, int64_t M) {
    if (!off || E <= 0 || off[0] != 0 || off[E] != M) return WQ_ERR_INVALID_ARG;
    for (int64_t e = 0; e < E; ++e)
        if (off[e + 1] < off[e]) return WQ_ERR_INVALID_ARG;
    return WQ_OK;
}

// The no-allocation entry point's scratch: one array per GPU, owned by the
// library until the process ends.  Its host-side name is not a device
// address; kernels and copies use the address hipGetSymbolAddress gives on
// each device (g_scratch[dev]).  The first WQ_WORKSPACE_ZERO_BYTES are the
// split-K counters, zero at rest: they start zero (static storage), are
// cleared again by a small kernel before the first call on each device and
// after any call whose launch failed, and every completed call leaves them
// zero.
}  // namespace

static __device__ __align__(256) uint8_t scratch[WQ_NOALLOC_SCRATCH_BYTES];

namespace {

struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
    std::atomic<bool> clean{false};
};
ScratchSlot g_scratch[kMaxDevices];

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *__restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The device address of the current device's scratch array (set up once per
// device, with that device current), or an error.
hipError_t scratch_for(int dev, void **ptr) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot &sl = g_scratch[dev];
    std::call_once(sl.once, [&] {
        void *p = nullptr;
        sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (sl.err == hipSuccess) sl.ptr = p;
    });
    *ptr = sl.ptr;
    return sl.err;
}

}  // namespace

extern "C" {

int wq_abi_version(void) { return WQ_ABI_VERSION; }

const char *wq_status_str(int status) {
    switch (status) {
        case WQ_OK: return "ok";
        case WQ_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive N or K, negative M, or unknown enum value)";
        case WQ_ERR_UNSUPPORTED_BITS: return "unsupported bit width: b must be in 2..8";
        case WQ_ERR_BAD_GROUP: return "group must be 128 or K, with K a multiple of 128; per-channel scales (group K) reach a GEMM through wq_repack (tiled layout)";
        case WQ_ERR_MISALIGNED: return "device pointer is not 16-byte aligned";
        case WQ_ERR_CODE_RANGE: return "a code does not fit in b bits (codes are refused, never masked)";
        case WQ_ERR_WORKSPACE: return "workspace missing or smaller than wq_workspace_bytes()";
        case WQ_ERR_BAD_LAYOUT: return "bad layout: unknown value, repack target not TILED, or scales_d given with TILED / missing with DENSE";
        case WQ_ERR_UNSUPPORTED_DEVICE: return "current device is not gfx950 (MI355X)";
        case WQ_ERR_HIP: return "HIP runtime or kernel launch error (see wq_last_hip_error)";
        case WQ_ERR_ZERO_POINTS: return "zero points need b = 4 or 8 (b = 4 on the int8-activation path, where c - z must fit int8)";
        case WQ_ERR_SCRATCH_LIMIT: return "the problem needs more scratch than the static per-GPU array of wq_gemm_noalloc holds (WQ_NOALLOC_SCRATCH_BYTES); call wq_gemm with a workspace";
    }
    return "unknown status";
}

int wq_last_hip_error(void) { return g_last_hip_error; }

int wq_device_supported(int device) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return 0;
    return query_device(device) == 1 ? 1 : 0;
}

int64_t wq_packed_words_per_row(int64_t K, int b) {
    if (K < 0 || b < 1 || b > 8) return -1;
    return words_per_row(K, b);
}

int wq_pack(const uint8_t *codes, int64_t N, int64_t K, int b, int group, uint32_t *packed) {
    if (!codes || !packed || N < 0 || K <= 0) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    const int64_t W = words_per_row(K, b);
    std::atomic<bool> bad{false};
    parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t n = r0; n < r1 && !bad.load(std::memory_order_relaxed); ++n) {
            const uint8_t *src = codes + n * K;
            uint32_t *dst = packed + n * W;
            uint64_t acc = 0;  // pending stream bits, LSB = next bit
            int nbits = 0;
            int64_t wi = 0;
            uint8_t any_high = 0;
            for (int64_t k = 0; k < K; ++k) {
                const uint8_t c = src[k];
                any_high |= (uint8_t)(c >> b);
                acc |= (uint64_t)c << nbits;
                nbits += b;
                if (nbits >= 32) {
                    dst[wi++] = (uint32_t)acc;
                    acc >>= 32;
                    nbits -= 32;
                }
            }
            if (nbits > 0) dst[wi++] = (uint32_t)acc;
            if (any_high) bad.store(true);
        }
    });
    return bad.load() ? WQ_ERR_CODE_RANGE : WQ_OK;
}

int wq_unpack(const uint32_t *packed, int64_t N, int64_t K, int b, uint8_t *codes) {
    if (!codes || !packed || N < 0 || K <= 0) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    const int64_t W = words_per_row(K, b);
    const uint32_t mask = (1u << b) - 1u;
    parallel_rows(N, K, [&](int64_t r0, int64_t r1) {
        for (int64_t n = r0; n < r1; ++n) {
            const uint32_t *src = packed + n * W;
            uint8_t *dst = codes + n * K;
            uint64_t acc = 0;
            int nbits = 0;
            int64_t wi = 0;
            for (int64_t k = 0; k < K; ++k) {
                if (nbits < b) {
                    acc |= (uint64_t)src[wi++] << nbits;
                    nbits += 32;
                }
                dst[k] = (uint8_t)(acc & mask);
                acc >>= b;
                nbits -= b;
            }
        }
    });
    return WQ_OK;
}

int64_t wq_repacked_bytes(int layout, int64_t N, int64_t K, int b, int group) {
    if (N <= 0 || K <= 0 || !valid_bits(b) || check_group(K, group) != WQ_OK) return -1;
    if (layout == WQ_LAYOUT_DENSE) return N * words_per_row(K, b) * 4;
    if (layout == WQ_LAYOUT_TILED) return (N + 63) / 64 * (K / kGroup) * (int64_t)(1024 * b + 128);
    return -1;
}

int wq_repack(const uint32_t *packed_d, const uint16_t *scales_d, int64_t N, int64_t K, int b,
              int group, int layout, void *out_d, void *stream) {
    if (!packed_d || !scales_d || !out_d || !dims_ok(0, N, K)) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (layout != WQ_LAYOUT_TILED) return WQ_ERR_BAD_LAYOUT;
    if (!aligned16(packed_d) || !aligned16(scales_d) || !aligned16(out_d)) return WQ_ERR_MISALIGNED;
    if (int s = check_device()) return s;
    hipError_t e = wq::launch_repack_tiled(packed_d, scales_d, N, K, b, per_channel(K, group),
                                           out_d, (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

int wq_unpack_dev(const void *W_d, int layout, int64_t N, int64_t K, int b, int group,
                  uint8_t *codes_d, void *stream) {
    if (!W_d || !codes_d || !dims_ok(0, N, K)) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (layout != WQ_LAYOUT_DENSE && layout != WQ_LAYOUT_TILED) return WQ_ERR_BAD_LAYOUT;
    if (!aligned16(W_d) || !aligned16(codes_d)) return WQ_ERR_MISALIGNED;
    if (int s = check_device()) return s;
    hipError_t e = wq::launch_unpack(W_d, layout == WQ_LAYOUT_TILED, nullptr, N, K, b, codes_d,
                                     (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

int wq_embed(const void *W_d, const uint16_t *scales_d, const uint8_t *zeros_d, int64_t V,
             int64_t K, int b, int group, const int64_t *ids_d, int64_t T, uint16_t *Y_d,
             void *stream) {
    if (!dims_ok(0, V, K) || T < 0 || T >= (1ll << 31)) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (int s = check_zeros(zeros_d, b, false)) return s;
    if (T * ((K / 8 + 127) / 128) >= (1ll << 32)) return WQ_ERR_INVALID_ARG;  // grid size
    if (T == 0) return WQ_OK;
    if (!W_d || !scales_d || !ids_d || !Y_d) return WQ_ERR_INVALID_ARG;
    if (!aligned16(W_d) || !aligned16(scales_d) || !aligned16(ids_d) || !aligned16(Y_d))
        return WQ_ERR_MISALIGNED;
    if (int s = check_device()) return s;
    hipError_t e = wq::launch_embed(W_d, scales_d, zeros_d, per_channel(K, group), V, K, b, ids_d,
                                    T, Y_d, (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

int64_t wq_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int b, int group) {
    if (!dims_ok(M, N, K) || !valid_bits(b) || check_group(K, group) != WQ_OK) return -1;
    if (op == WQ_OP_GEMM) return K <= kMaxGemmK ? gemm_ws_bytes(M, N, K, b) : -1;
    if (op == WQ_OP_GEMM_A8) return wq::a8_ws_bytes(M, N, K);
    return -1;
}

int wq_gemm(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d, int layout,
            const uint16_t *scales_d, const uint8_t *zeros_d, int b, int group, uint16_t *Y_d,
            void *ws_d, int64_t ws_bytes, void *stream) {
    if (!gemm_dims_ok(M, N, K)) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (layout != WQ_LAYOUT_DENSE && layout != WQ_LAYOUT_TILED) return WQ_ERR_BAD_LAYOUT;
    if ((layout == WQ_LAYOUT_DENSE) != (scales_d != nullptr)) return WQ_ERR_BAD_LAYOUT;
    if (layout == WQ_LAYOUT_DENSE && per_channel(K, group)) return WQ_ERR_BAD_GROUP;
    if (int s = check_zeros(zeros_d, b, false)) return s;
    if (M == 0) return WQ_OK;
    if (!A_d || !W_d || !Y_d) return WQ_ERR_INVALID_ARG;
    if (!aligned16(A_d) || !aligned16(W_d) || !aligned16(Y_d) ||
        (scales_d && !aligned16(scales_d)) || (ws_d && !aligned16(ws_d)))
        return WQ_ERR_MISALIGNED;
    const int64_t need = gemm_ws_bytes(M, N, K, b);
    if (need > 0 && (!ws_d || ws_bytes < need)) return WQ_ERR_WORKSPACE;
    if (int s = check_device()) return s;
    const hipError_t e = gemm_dispatch(A_d, M, N, K, W_d, layout == WQ_LAYOUT_TILED, scales_d,
                                       zeros_d, b, Y_d, ws_d, (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

int wq_gemm_noalloc(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d,
                    int layout, const uint16_t *scales_d, const uint8_t *zeros_d, int b,
                    int group, uint16_t *Y_d, void *stream) {
    if (!gemm_dims_ok(M, N, K)) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (layout != WQ_LAYOUT_DENSE && layout != WQ_LAYOUT_TILED) return WQ_ERR_BAD_LAYOUT;
    if ((layout == WQ_LAYOUT_DENSE) != (scales_d != nullptr)) return WQ_ERR_BAD_LAYOUT;
    if (layout == WQ_LAYOUT_DENSE && per_channel(K, group)) return WQ_ERR_BAD_GROUP;
    if (int s = check_zeros(zeros_d, b, false)) return s;
    if (M == 0) return WQ_OK;
    if (!A_d || !W_d || !Y_d) return WQ_ERR_INVALID_ARG;
    if (!aligned16(A_d) || !aligned16(W_d) || !aligned16(Y_d) ||
        (scales_d && !aligned16(scales_d)))
        return WQ_ERR_MISALIGNED;
    const int64_t need = gemm_ws_bytes(M, N, K, b);
    if (need > WQ_NOALLOC_SCRATCH_BYTES) return WQ_ERR_SCRATCH_LIMIT;
    if (int s = check_device()) return s;
    void *ws = nullptr;
    if (need > 0) {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = scratch_for(dev, &ws);
        if (e != hipSuccess) return hip_fail(e);
        ScratchSlot &sl = g_scratch[dev];
        if (!sl.clean.load(std::memory_order_acquire)) {
            constexpr int words = (int)(WQ_WORKSPACE_ZERO_BYTES / 4);
            hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0,
                               (hipStream_t)stream, static_cast<uint32_t *>(ws), words);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e);
            sl.clean.store(true, std::memory_order_release);
        }
        e = gemm_dispatch(A_d, M, N, K, W_d, layout == WQ_LAYOUT_TILED, scales_d, zeros_d, b,
                          Y_d, ws, (hipStream_t)stream);
        if (e != hipSuccess) {
            sl.clean.store(false, std::memory_order_release);
            return hip_fail(e);
        }
        return WQ_OK;
    }
    const hipError_t e = gemm_dispatch(A_d, M, N, K, W_d, layout == WQ_LAYOUT_TILED, scales_d,
                                       zeros_d, b, Y_d, nullptr, (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

int64_t wq_grouped_workspace_bytes(const int64_t *offsets, int64_t E, int64_t N, int64_t K,
                                   int b, int group) {
    if (!gemm_dims_ok(0, N, K) || !valid_bits(b) || check_group(K, group) != WQ_OK || !offsets ||
        E <= 0)
        return -1;
    const int64_t M = offsets[E];
    if (check_offsets(offsets, E, M) != WQ_OK || M >= (1ll << 31)) return -1;
    return grouped_ws_bytes(offsets, E, N, K, b);
}

int wq_gemm_grouped(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d,
                    int64_t expert_bytes, const uint8_t *zeros_d, const int64_t *offsets,
                    int64_t E, int b, int group, uint16_t *Y_d, void *ws_d, int64_t ws_bytes,
                    void *stream) {
    if (!gemm_dims_ok(M, N, K)) return WQ_ERR_INVALID_ARG;
    if (int s = check_offsets(offsets, E, M)) return s;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (int s = check_zeros(zeros_d, b, false)) return s;
    if (expert_bytes < wq_repacked_bytes(WQ_LAYOUT_TILED, N, K, b, kGroup) || expert_bytes % 16)
        return WQ_ERR_INVALID_ARG;
    if (M == 0) return WQ_OK;
    if (!A_d || !W_d || !Y_d) return WQ_ERR_INVALID_ARG;
    if (!aligned16(A_d) || !aligned16(W_d) || !aligned16(Y_d) || (ws_d && !aligned16(ws_d)))
        return WQ_ERR_MISALIGNED;
    const int64_t need = grouped_ws_bytes(offsets, E, N, K, b);
    if (need > 0 && (!ws_d || ws_bytes < need)) return WQ_ERR_WORKSPACE;
    if (int s = check_device()) return s;
    // One launch per table, in order on the stream (one workspace, used by
    // the decode tables only: each leaves the counter region zero).
    hipError_t err = hipSuccess;
    grouped_tables(offsets, E, N, expert_bytes,
                   [&](bool is_dec, const wq::GroupTable &t, int max_me) {
        if (err != hipSuccess) return;
        if (is_dec) {
            err = wq::launch_decode_grouped(A_d, N, K, W_d, zeros_d, b, Y_d, ws_d,
                                            grouped_decode_plan(t, max_me, N, K, b), t,
                                            (hipStream_t)stream);
        } else {
            err = wq::launch_prefill_grouped(A_d, M, N, K, W_d, zeros_d, b, Y_d, t, max_me,
                                             (hipStream_t)stream);
        }
    });
    return err == hipSuccess ? WQ_OK : hip_fail(err);
}

int wq_quant_act_i8(const uint16_t *A_d, int64_t M, int64_t K, int8_t *Aq_d, float *sa_d,
                    void *stream) {
    if (M < 0 || K <= 0 || M >= (1ll << 31) || K >= (1ll << 31)) return WQ_ERR_INVALID_ARG;
    if (M == 0) return WQ_OK;
    if (!A_d || !Aq_d || !sa_d) return WQ_ERR_INVALID_ARG;
    if (K % 8 != 0) return WQ_ERR_INVALID_ARG;
    if (!aligned16(A_d) || !aligned16(Aq_d) || !aligned16(sa_d)) return WQ_ERR_MISALIGNED;
    if (int s = check_device()) return s;
    hipError_t e = wq::launch_quant_act(A_d, M, K, Aq_d, sa_d, (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

int wq_gemm_a8(const uint16_t *A_d, int64_t M, int64_t N, int64_t K, const void *W_d,
               int layout, const uint16_t *scales_d, const uint8_t *zeros_d, int b, int group,
               void *Y_d, int out_dtype, void *ws_d, int64_t ws_bytes, void *stream) {
    if (!dims_ok(M, N, K)) return WQ_ERR_INVALID_ARG;
    if (!valid_bits(b)) return WQ_ERR_UNSUPPORTED_BITS;
    if (int s = check_group(K, group)) return s;
    if (layout != WQ_LAYOUT_DENSE && layout != WQ_LAYOUT_TILED) return WQ_ERR_BAD_LAYOUT;
    if ((layout == WQ_LAYOUT_DENSE) != (scales_d != nullptr)) return WQ_ERR_BAD_LAYOUT;
    if (layout == WQ_LAYOUT_DENSE && per_channel(K, group)) return WQ_ERR_BAD_GROUP;
    if (int s = check_zeros(zeros_d, b, true)) return s;
    if (out_dtype != WQ_OUT_BF16 && out_dtype != WQ_OUT_F32) return WQ_ERR_INVALID_ARG;
    if (M == 0) return WQ_OK;
    if (!A_d || !W_d || !Y_d) return WQ_ERR_INVALID_ARG;
    if (!aligned16(A_d) || !aligned16(W_d) || !aligned16(Y_d) ||
        (scales_d && !aligned16(scales_d)) || (ws_d && !aligned16(ws_d)))
        return WQ_ERR_MISALIGNED;
    const int64_t need = wq::a8_ws_bytes(M, N, K);
    if (!ws_d || ws_bytes < need) return WQ_ERR_WORKSPACE;
    if (int s = check_device()) return s;
    hipError_t e = wq::launch_gemm_a8(A_d, M, N, K, W_d, layout == WQ_LAYOUT_TILED, scales_d,
                                      zeros_d, b,
                                      Y_d, out_dtype == WQ_OUT_F32, ws_d, (hipStream_t)stream);
    return e == hipSuccess ? WQ_OK : hip_fail(e);
}

}  // extern "C"
