// C ABI of the rtq library: argument validation (host only, before any HIP
// call) and dispatch to the gfx950 kernels. Declarations and the contract of
// each entry point are in rtq.h.
#include <rtq.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "rtq_internal.h"

namespace {

thread_local char g_err[512] = "";

void clear_error() { g_err[0] = '\0'; }

rtq_status fail(rtq_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

rtq_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return RTQ_OK;
    return fail(RTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Largest dimension: kernels form padded row and column indices (up to a
// dimension plus a tile) in 32-bit integers.
constexpr int64_t kMaxDim = (int64_t(1) << 30) - 1;
// Largest element count of one tensor (1 TB of fp32, beyond any device):
// with every dimension below 2^31 the products below cannot overflow, the
// byte ranges of the overlap checks (elements * 4) stay far below 2^63, and
// every kernel grid and tile count derived from a tensor fits 32 bits.
constexpr int64_t kMaxElems = int64_t(1) << 38;

bool math_ok(int32_t m) {
    return m == RTQ_MATH_SPLIT_BF16 || m == RTQ_MATH_FP32_MFMA || m == RTQ_MATH_BF16 || m == RTQ_MATH_SPLIT_F16;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Checks shared by the projection entry points. `name` prefixes messages.
rtq_status check_proj(const char* name, int fmt, const float* x, const void* payload,
                      const void* scale, const float* y, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || M > kMaxDim) return fail(RTQ_ERR_SHAPE, "%s: M=%lld out of range [0, 2^30)", name, (long long)M);
    if (N < 1 || N > kMaxDim) return fail(RTQ_ERR_SHAPE, "%s: N=%lld out of range [1, 2^30)", name, (long long)N);
    if (K < 1 || K > kMaxDim) return fail(RTQ_ERR_SHAPE, "%s: K=%lld out of range [1, 2^30)", name, (long long)K);
    if (M * N > kMaxElems || M * K > kMaxElems || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "%s: M=%lld N=%lld K=%lld exceed 2^38 elements in one tensor", name,
                    (long long)M, (long long)N, (long long)K);
    if (fmt == rtq::kFmtQ4 && K % RTQ_Q4_GROUP != 0)
        return fail(RTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of the int4 group size 32", name, (long long)K);
    if (M == 0) return RTQ_OK;
    if (!x) return fail(RTQ_ERR_NULL, "%s: x is NULL", name);
    if (!payload) return fail(RTQ_ERR_NULL, "%s: payload is NULL", name);
    if (!scale && fmt != rtq::kFmtF8) return fail(RTQ_ERR_NULL, "%s: scale is NULL", name);
    if (!y) return fail(RTQ_ERR_NULL, "%s: y is NULL", name);
    if (!aligned(x, 16)) return fail(RTQ_ERR_ALIGN, "%s: x is not 16-byte aligned", name);
    if (!aligned(y, 16)) return fail(RTQ_ERR_ALIGN, "%s: y is not 16-byte aligned", name);
    if (!aligned(payload, 16)) return fail(RTQ_ERR_ALIGN, "%s: payload is not 16-byte aligned", name);
    if (!aligned(scale, 4)) return fail(RTQ_ERR_ALIGN, "%s: scale is not 4-byte aligned", name);
    const int64_t payload_bytes = fmt == rtq::kFmtQ4 ? N * (K / 2) : N * K;
    const int64_t scale_bytes = fmt == rtq::kFmtQ4 ? N * (K / RTQ_Q4_GROUP) * 4 : fmt == rtq::kFmtQ8 ? N * 4 : 0;
    const Range ry = range_of(y, M * N * 4);
    if (overlaps(ry, range_of(x, M * K * 4)) || overlaps(ry, range_of(payload, payload_bytes)) ||
        overlaps(ry, range_of(scale, scale_bytes)))
        return fail(RTQ_ERR_OVERLAP, "%s: y overlaps an input", name);
    return RTQ_OK;
}

rtq_status check_nk(const char* name, int fmt, const void* a, const void* b, const void* c,
                    int64_t N, int64_t K) {
    if (N < 0 || N > kMaxDim) return fail(RTQ_ERR_SHAPE, "%s: N=%lld out of range [0, 2^30)", name, (long long)N);
    if (K < 1 || K > kMaxDim) return fail(RTQ_ERR_SHAPE, "%s: K=%lld out of range [1, 2^30)", name, (long long)K);
    if (N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "%s: N=%lld K=%lld exceed 2^38 elements", name, (long long)N, (long long)K);
    if (fmt == rtq::kFmtQ4 && K % RTQ_Q4_GROUP != 0)
        return fail(RTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of the int4 group size 32", name, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!a || !b || !c) return fail(RTQ_ERR_NULL, "%s: a pointer argument is NULL", name);
    if (!aligned(a, 16) || !aligned(b, 4) || !aligned(c, 16))
        return fail(RTQ_ERR_ALIGN, "%s: misaligned pointer", name);
    return RTQ_OK;
}

}  // namespace

// Kernel timing: when enabled, every main GEMM launch is bracketed by a pair of
// HIP events recorded on its stream; rtq_timing_read sums their elapsed times.
constexpr int kMaxTimed = 16384;
struct Timing {
    std::mutex mu;
    bool on = false;
    int n = 0;
    int created = 0;
    hipEvent_t begin[kMaxTimed];
    hipEvent_t end[kMaxTimed];
};
Timing g_timing;

namespace rtq {
int timing_begin(hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_timing.mu);
    if (!g_timing.on || g_timing.n >= kMaxTimed) return -1;
    const int i = g_timing.n;
    if (i >= g_timing.created) {
        if (hipEventCreate(&g_timing.begin[i]) != hipSuccess) return -1;
        if (hipEventCreate(&g_timing.end[i]) != hipSuccess) {
            (void)hipEventDestroy(g_timing.begin[i]);
            return -1;
        }
        g_timing.created = i + 1;
    }
    if (hipEventRecord(g_timing.begin[i], stream) != hipSuccess) return -1;
    g_timing.n = i + 1;
    return i;
}

void timing_end(int slot, hipStream_t stream) {
    if (slot < 0) return;
    std::lock_guard<std::mutex> lock(g_timing.mu);
    (void)hipEventRecord(g_timing.end[slot], stream);
}
}  // namespace rtq

extern "C" {

const char* rtq_version(void) { return "rtq 0.1.0 gfx950"; }

rtq_status rtq_timing_enable(int32_t on) {
    clear_error();
    std::lock_guard<std::mutex> lock(g_timing.mu);
    g_timing.on = on != 0;
    g_timing.n = 0;
    return RTQ_OK;
}

rtq_status rtq_timing_read(double* total_ms, int64_t* launches) {
    clear_error();
    if (!total_ms || !launches) return fail(RTQ_ERR_NULL, "rtq_timing_read: NULL output");
    std::lock_guard<std::mutex> lock(g_timing.mu);
    double sum = 0.0;
    for (int i = 0; i < g_timing.n; ++i) {
        hipError_t e = hipEventSynchronize(g_timing.end[i]);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timing.begin[i], g_timing.end[i]);
        if (e != hipSuccess) return fail(RTQ_ERR_HIP, "rtq_timing_read: %s", hipGetErrorString(e));
        sum += ms;
    }
    *total_ms = sum;
    *launches = g_timing.n;
    g_timing.n = 0;
    return RTQ_OK;
}

const char* rtq_last_error(void) { return g_err; }

const char* rtq_status_string(rtq_status s) {
    switch (s) {
        case RTQ_OK: return "ok";
        case RTQ_ERR_NULL: return "null pointer";
        case RTQ_ERR_SHAPE: return "bad shape";
        case RTQ_ERR_ALIGN: return "misaligned pointer";
        case RTQ_ERR_FORMAT: return "unknown format";
        case RTQ_ERR_HIP: return "HIP runtime error";
        case RTQ_ERR_OVERLAP: return "output overlaps an input";
    }
    return "unknown status";
}

rtq_status rtq_gemm_ex(int32_t fmt, const float* x, const void* payload, const void* scale, float* y,
                       int64_t M, int64_t N, int64_t K, int32_t math, void* stream) {
    clear_error();
    const char* name = fmt == RTQ_FMT_Q4 ? "rtq_gemm_q4" : fmt == RTQ_FMT_Q8 ? "rtq_gemm_q8" : "rtq_gemm_f8";
    if (fmt != RTQ_FMT_Q4 && fmt != RTQ_FMT_Q8 && fmt != RTQ_FMT_F8)
        return fail(RTQ_ERR_FORMAT, "rtq_gemm_ex: unknown fmt %d", fmt);
    if (!math_ok(math)) return fail(RTQ_ERR_FORMAT, "%s: unknown arithmetic %d", name, math);
    rtq_status s = check_proj(name, fmt, x, payload, fmt == RTQ_FMT_F8 ? nullptr : scale, y, M, N, K);
    if (s != RTQ_OK || M == 0) return s;
    const rtq::ProjTask t{fmt, static_cast<int>(N), static_cast<int>(K), payload,
                          fmt == RTQ_FMT_F8 ? nullptr : scale, x, y};
    char what[32];
    std::snprintf(what, sizeof(what), "%s launch", name);
    return hip_status(rtq::launch_gemm(t, M, math, static_cast<hipStream_t>(stream)), what);
}

rtq_status rtq_gemm_q4(const float* x, const uint8_t* payload, const uint16_t* pairs, float* y,
                       int64_t M, int64_t N, int64_t K, void* stream) {
    return rtq_gemm_ex(RTQ_FMT_Q4, x, payload, pairs, y, M, N, K, RTQ_MATH_SPLIT_BF16, stream);
}

rtq_status rtq_gemm_q8(const float* x, const int8_t* q, const float* scale, float* y, int64_t M,
                       int64_t N, int64_t K, void* stream) {
    return rtq_gemm_ex(RTQ_FMT_Q8, x, q, scale, y, M, N, K, RTQ_MATH_SPLIT_BF16, stream);
}

rtq_status rtq_gemm_f8(const float* x, const uint8_t* codes, float* y, int64_t M, int64_t N, int64_t K,
                       void* stream) {
    return rtq_gemm_ex(RTQ_FMT_F8, x, codes, nullptr, y, M, N, K, RTQ_MATH_SPLIT_BF16, stream);
}

namespace {

// rtq_block_project / _ex / _noalloc: validation, then the grouped launch and
// the projections the grouped kernels do not take. With no_alloc the split
// path's workspace is the library's fixed scratch array.
// The block projection behind every block entry point: validate, then
// launch with the workspace `mode` names (the library's pool, its scratch
// array, or the caller's `ws` of `ws_bytes`). With size_out set, validate and
// return the workspace bytes the call needs without launching anything.
rtq_status block_project_impl(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math, void* stream,
                              rtq::WsMode mode, void* ws = nullptr, int64_t ws_bytes = 0,
                              int64_t* size_out = nullptr) {
    clear_error();
    if (!math_ok(math)) return fail(RTQ_ERR_FORMAT, "rtq_block_project: unknown arithmetic %d", math);
    if (!blocks) return fail(RTQ_ERR_NULL, "rtq_block_project: blocks is NULL");
    if (n_blocks < 1 || n_blocks > RTQ_MAX_BLOCKS)
        return fail(RTQ_ERR_SHAPE, "rtq_block_project: n_blocks=%d out of range [1, %d]", n_blocks, RTQ_MAX_BLOCKS);
    if (M < 0 || M > kMaxDim) return fail(RTQ_ERR_SHAPE, "rtq_block_project: M=%lld out of range", (long long)M);
    static const char* names[8] = {"wq", "wk", "wv", "wg", "wo", "w1", "w3", "w2"};
    // Per-thread buffers, sized once for the largest call (no stack arrays of
    // this size, no allocation per call).
    thread_local std::vector<rtq::ProjTask> grouped_buf(RTQ_MAX_BLOCKS * 8), single_buf(RTQ_MAX_BLOCKS * 8);
    thread_local std::vector<Range> outs_buf(RTQ_MAX_BLOCKS * 8), ins_buf(RTQ_MAX_BLOCKS * 8 * 4);
    rtq::ProjTask* grouped = grouped_buf.data();
    rtq::ProjTask* single = single_buf.data();
    Range* outs = outs_buf.data();
    Range* ins = ins_buf.data();
    int n_grouped = 0, n_single = 0, n_outs = 0, n_ins = 0;
    for (int b = 0; b < n_blocks; ++b) {
        const rtq_proj* p = &blocks[b].wq;
        for (int j = 0; j < 8; ++j) {
            const rtq_proj& d = p[j];
            if (!d.payload) continue;
            char name[64];
            std::snprintf(name, sizeof(name), "rtq_block_project: block %d %s", b, names[j]);
            if (d.fmt != RTQ_FMT_Q4 && d.fmt != RTQ_FMT_Q8 && d.fmt != RTQ_FMT_F8)
                return fail(RTQ_ERR_FORMAT, "%s: unknown fmt %d", name, d.fmt);
            if (d.reserved != 0) return fail(RTQ_ERR_SHAPE, "%s: reserved field must be 0", name);
            const rtq_status s = check_proj(name, d.fmt, d.x, d.payload, d.scale, d.y, M, d.N, d.K);
            if (s != RTQ_OK) return s;
            if (d.bias && !aligned(d.bias, 4)) return fail(RTQ_ERR_ALIGN, "%s: bias is not 4-byte aligned", name);
            if (M == 0) continue;
            outs[n_outs++] = range_of(d.y, M * int64_t(d.N) * 4);
            const int64_t pb = d.fmt == RTQ_FMT_Q4 ? int64_t(d.N) * (d.K / 2) : int64_t(d.N) * d.K;
            const int64_t sb = d.fmt == RTQ_FMT_Q4 ? int64_t(d.N) * (d.K / 32) * 4
                               : d.fmt == RTQ_FMT_Q8 ? int64_t(d.N) * 4 : 0;
            ins[n_ins++] = range_of(d.x, M * int64_t(d.K) * 4);
            ins[n_ins++] = range_of(d.payload, pb);
            ins[n_ins++] = range_of(d.scale, sb);
            ins[n_ins++] = range_of(d.bias, d.bias ? int64_t(d.N) * 4 : 0);
            const rtq::ProjTask t{d.fmt, d.N, d.K, d.payload, d.scale, d.x, d.y, d.bias};
            if (rtq::grouped_ok(t)) grouped[n_grouped++] = t;
            else single[n_single++] = t;
        }
    }
    // Outputs must be pairwise disjoint and must not overlap any input of any
    // projection: sort the outputs, then check neighbours and binary-search each input.
    std::sort(outs, outs + n_outs, [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (int i = 1; i < n_outs; ++i)
        if (overlaps(outs[i - 1], outs[i]))
            return fail(RTQ_ERR_OVERLAP, "rtq_block_project: two projections write overlapping outputs");
    for (int i = 0; i < n_ins; ++i) {
        const Range r = ins[i];
        // first output whose end lies past the input's start (outputs are disjoint and sorted)
        const Range* it = std::upper_bound(outs, outs + n_outs, r.lo,
                                           [](uintptr_t v, const Range& o) { return v < o.hi; });
        if (it != outs + n_outs && overlaps(*it, r))
            return fail(RTQ_ERR_OVERLAP, "rtq_block_project: an output overlaps a projection's input");
    }
    const int64_t need = M > 0 && n_grouped ? rtq::grouped_workspace_bytes(grouped, n_grouped, M, math) : 0;
    if (need < 0) return fail(RTQ_ERR_SHAPE, "rtq_block_project: too many projections for one call");
    if (size_out) {
        *size_out = need;
        return RTQ_OK;
    }
    if (M == 0) return RTQ_OK;
    if (mode == rtq::kWsScratch && need > rtq::kScratchBytes)
        return fail(RTQ_ERR_SHAPE,
                    "rtq_block_project_noalloc: the call needs %lld bytes of workspace, more than the %lld-byte "
                    "scratch of the allocation-free entry point",
                    (long long)need, (long long)rtq::kScratchBytes);
    if (mode == rtq::kWsCaller) {
        if (need > ws_bytes)
            return fail(RTQ_ERR_SHAPE, "rtq_block_project_ws: the call needs %lld bytes of workspace, %lld given",
                        (long long)need, (long long)ws_bytes);
        if (need > 0 && !ws) return fail(RTQ_ERR_NULL, "rtq_block_project_ws: workspace is NULL");
        if (ws && !aligned(ws, 256)) return fail(RTQ_ERR_ALIGN, "rtq_block_project_ws: workspace is not 256-byte aligned");
        if (ws && need > 0) {
            // the workspace must not overlap any input or output of the call
            const Range w = range_of(ws, need);
            for (int i = 0; i < n_outs; ++i)
                if (overlaps(outs[i], w))
                    return fail(RTQ_ERR_OVERLAP, "rtq_block_project_ws: the workspace overlaps an output");
            for (int i = 0; i < n_ins; ++i)
                if (overlaps(ins[i], w))
                    return fail(RTQ_ERR_OVERLAP, "rtq_block_project_ws: the workspace overlaps an input");
        }
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (n_grouped) {
        const rtq_status s = hip_status(
            rtq::launch_grouped(grouped, n_grouped, M, math, st, mode, static_cast<unsigned char*>(ws), ws_bytes),
            "rtq_block_project launch");
        if (s != RTQ_OK) return s;
    }
    for (int i = 0; i < n_single; ++i) {
        const rtq_status s = hip_status(rtq::launch_gemm(single[i], M, math, st), "rtq_block_project launch");
        if (s != RTQ_OK) return s;
    }
    return RTQ_OK;
}

}  // namespace

rtq_status rtq_block_project(const rtq_block* blocks, int32_t n_blocks, int64_t M, void* stream) {
    return block_project_impl(blocks, n_blocks, M, RTQ_MATH_SPLIT_BF16, stream, rtq::kWsPool);
}

rtq_status rtq_block_project_ex(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math, void* stream) {
    return block_project_impl(blocks, n_blocks, M, math, stream, rtq::kWsPool);
}

rtq_status rtq_block_project_noalloc(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math,
                                     void* stream) {
    return block_project_impl(blocks, n_blocks, M, math, stream, rtq::kWsScratch);
}

rtq_status rtq_block_workspace_bytes(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math,
                                     int64_t* bytes) {
    if (!bytes) {
        clear_error();
        return fail(RTQ_ERR_NULL, "rtq_block_workspace_bytes: bytes is NULL");
    }
    *bytes = 0;
    return block_project_impl(blocks, n_blocks, M, math, nullptr, rtq::kWsCaller, nullptr, 0, bytes);
}

rtq_status rtq_block_project_ws(const rtq_block* blocks, int32_t n_blocks, int64_t M, int32_t math, void* workspace,
                                int64_t workspace_bytes, void* stream) {
    if (workspace_bytes < 0) {
        clear_error();
        return fail(RTQ_ERR_SHAPE, "rtq_block_project_ws: workspace_bytes is negative");
    }
    return block_project_impl(blocks, n_blocks, M, math, stream, rtq::kWsCaller, workspace, workspace_bytes);
}

rtq_status rtq_dequant_q4(const uint8_t* payload, const uint16_t* pairs, float* w, int64_t N, int64_t K,
                          void* stream) {
    clear_error();
    rtq_status s = check_nk("rtq_dequant_q4", rtq::kFmtQ4, payload, pairs, w, N, K);
    if (s != RTQ_OK || N == 0) return s;
    return hip_status(rtq::launch_dequant_q4(payload, pairs, w, N, K, static_cast<hipStream_t>(stream)),
                      "rtq_dequant_q4 launch");
}

rtq_status rtq_dequant_q8(const int8_t* q, const float* scale, float* w, int64_t N, int64_t K, void* stream) {
    clear_error();
    if (N < 0 || N > kMaxDim || K < 1 || K > kMaxDim || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "rtq_dequant_q8: N=%lld K=%lld out of range", (long long)N, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!q || !scale || !w) return fail(RTQ_ERR_NULL, "rtq_dequant_q8: a pointer argument is NULL");
    if (!aligned(scale, 4) || !aligned(w, 4)) return fail(RTQ_ERR_ALIGN, "rtq_dequant_q8: misaligned pointer");
    return hip_status(rtq::launch_dequant_q8(q, scale, w, N, K, static_cast<hipStream_t>(stream)),
                      "rtq_dequant_q8 launch");
}

rtq_status rtq_quantize_q4(const float* w, uint8_t* payload, uint16_t* pairs, int64_t N, int64_t K,
                           void* stream) {
    clear_error();
    rtq_status s = check_nk("rtq_quantize_q4", rtq::kFmtQ4, payload, pairs, w, N, K);
    if (s != RTQ_OK || N == 0) return s;
    return hip_status(rtq::launch_quantize_q4(w, payload, pairs, N, K, static_cast<hipStream_t>(stream)),
                      "rtq_quantize_q4 launch");
}

rtq_status rtq_quantize_q8(const float* w, int8_t* q, float* scale, int64_t N, int64_t K, void* stream) {
    clear_error();
    if (N < 0 || N > kMaxDim || K < 1 || K > kMaxDim || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "rtq_quantize_q8: N=%lld K=%lld out of range", (long long)N, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!w || !q || !scale) return fail(RTQ_ERR_NULL, "rtq_quantize_q8: a pointer argument is NULL");
    if (!aligned(w, 4) || !aligned(scale, 4)) return fail(RTQ_ERR_ALIGN, "rtq_quantize_q8: misaligned pointer");
    return hip_status(rtq::launch_quantize_q8(w, q, scale, N, K, static_cast<hipStream_t>(stream)),
                      "rtq_quantize_q8 launch");
}

rtq_status rtq_dequant_f8(const uint8_t* codes, float* w, int64_t N, int64_t K, void* stream) {
    clear_error();
    if (N < 0 || N > kMaxDim || K < 1 || K > kMaxDim || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "rtq_dequant_f8: N=%lld K=%lld out of range", (long long)N, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!codes || !w) return fail(RTQ_ERR_NULL, "rtq_dequant_f8: a pointer argument is NULL");
    if (!aligned(w, 4)) return fail(RTQ_ERR_ALIGN, "rtq_dequant_f8: misaligned pointer");
    if (overlaps(range_of(w, N * K * 4), range_of(codes, N * K)))
        return fail(RTQ_ERR_OVERLAP, "rtq_dequant_f8: output overlaps the codes");
    return hip_status(rtq::launch_dequant_f8(codes, w, N, K, static_cast<hipStream_t>(stream)),
                      "rtq_dequant_f8 launch");
}

rtq_status rtq_quantize_f8(const float* w, uint8_t* codes, int64_t N, int64_t K, void* stream) {
    clear_error();
    if (N < 0 || N > kMaxDim || K < 1 || K > kMaxDim || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "rtq_quantize_f8: N=%lld K=%lld out of range", (long long)N, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!w || !codes) return fail(RTQ_ERR_NULL, "rtq_quantize_f8: a pointer argument is NULL");
    if (!aligned(w, 4)) return fail(RTQ_ERR_ALIGN, "rtq_quantize_f8: misaligned pointer");
    if (overlaps(range_of(w, N * K * 4), range_of(codes, N * K)))
        return fail(RTQ_ERR_OVERLAP, "rtq_quantize_f8: output overlaps the weights");
    return hip_status(rtq::launch_quantize_f8(w, codes, N, K, static_cast<hipStream_t>(stream)),
                      "rtq_quantize_f8 launch");
}

// ---- diagnostics: measured ceilings ----
rtq_status rtq_diag_stream_read(const void* buf, int64_t bytes, int32_t unroll, int32_t blocks, uint32_t* sink,
                                void* stream) {
    clear_error();
    if (!buf || !sink) return fail(RTQ_ERR_NULL, "rtq_diag_stream_read: a pointer argument is NULL");
    if (bytes < 16 || bytes % 16 != 0 || bytes > (kMaxElems << 2))
        return fail(RTQ_ERR_SHAPE, "rtq_diag_stream_read: bytes=%lld is not a positive multiple of 16", (long long)bytes);
    if (unroll != 4 && unroll != 8 && unroll != 16)
        return fail(RTQ_ERR_SHAPE, "rtq_diag_stream_read: unroll=%d is not 4, 8 or 16", unroll);
    if (blocks < 1 || blocks > (1 << 20)) return fail(RTQ_ERR_SHAPE, "rtq_diag_stream_read: blocks=%d out of range", blocks);
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(RTQ_ERR_ALIGN, "rtq_diag_stream_read: misaligned pointer");
    return hip_status(rtq::launch_stream_read(buf, bytes, unroll, blocks, sink, static_cast<hipStream_t>(stream)),
                      "rtq_diag_stream_read launch");
}

rtq_status rtq_diag_mfma_loop(int32_t kind, int64_t iters, int32_t blocks, float* sink, double* flops, void* stream) {
    clear_error();
    if (kind < 0 || kind > 2) return fail(RTQ_ERR_FORMAT, "rtq_diag_mfma_loop: unknown kind %d", kind);
    if (!sink) return fail(RTQ_ERR_NULL, "rtq_diag_mfma_loop: sink is NULL");
    if (iters < 1 || iters > (int64_t(1) << 31)) return fail(RTQ_ERR_SHAPE, "rtq_diag_mfma_loop: iters out of range");
    if (blocks < 1 || blocks > (1 << 20)) return fail(RTQ_ERR_SHAPE, "rtq_diag_mfma_loop: blocks=%d out of range", blocks);
    if (!aligned(sink, 4)) return fail(RTQ_ERR_ALIGN, "rtq_diag_mfma_loop: misaligned sink");
    if (flops) *flops = double(blocks) * 4.0 * double(iters) * 8.0 * (kind == 2 ? 2.0 * 16 * 16 * 4 : 2.0 * 16 * 16 * 32);
    return hip_status(rtq::launch_mfma_loop(kind, iters, blocks, sink, static_cast<hipStream_t>(stream)),
                      "rtq_diag_mfma_loop launch");
}

// ---- host quantizers: host pointers, no HIP call ----
static int host_threads(int32_t threads) {
    if (threads > 0) return threads < 1024 ? threads : 1024;
    const unsigned hw = std::thread::hardware_concurrency();
    return hw ? static_cast<int>(hw < 1024 ? hw : 1024) : 1;
}

rtq_status rtq_quantize_q4_host(const float* w, uint8_t* payload, uint16_t* pairs, int64_t N, int64_t K,
                                int32_t threads) {
    clear_error();
    rtq_status s = check_nk("rtq_quantize_q4_host", rtq::kFmtQ4, payload, pairs, w, N, K);
    if (s != RTQ_OK || N == 0) return s;
    if (overlaps(range_of(w, N * K * 4), range_of(payload, N * (K / 2))) ||
        overlaps(range_of(w, N * K * 4), range_of(pairs, N * (K / RTQ_Q4_GROUP) * 4)) ||
        overlaps(range_of(payload, N * (K / 2)), range_of(pairs, N * (K / RTQ_Q4_GROUP) * 4)))
        return fail(RTQ_ERR_OVERLAP, "rtq_quantize_q4_host: arrays overlap");
    rtq::quantize_q4_host(w, payload, pairs, N, K, host_threads(threads));
    return RTQ_OK;
}

rtq_status rtq_quantize_q8_host(const float* w, int8_t* q, float* scale, int64_t N, int64_t K, int32_t threads) {
    clear_error();
    if (N < 0 || N > kMaxDim || K < 1 || K > kMaxDim || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "rtq_quantize_q8_host: N=%lld K=%lld out of range", (long long)N, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!w || !q || !scale) return fail(RTQ_ERR_NULL, "rtq_quantize_q8_host: a pointer argument is NULL");
    if (!aligned(w, 4) || !aligned(scale, 4)) return fail(RTQ_ERR_ALIGN, "rtq_quantize_q8_host: misaligned pointer");
    if (overlaps(range_of(w, N * K * 4), range_of(q, N * K)) || overlaps(range_of(w, N * K * 4), range_of(scale, N * 4)) ||
        overlaps(range_of(q, N * K), range_of(scale, N * 4)))
        return fail(RTQ_ERR_OVERLAP, "rtq_quantize_q8_host: arrays overlap");
    rtq::quantize_q8_host(w, q, scale, N, K, host_threads(threads));
    return RTQ_OK;
}

rtq_status rtq_quantize_f8_host(const float* w, uint8_t* codes, int64_t N, int64_t K, int32_t threads) {
    clear_error();
    if (N < 0 || N > kMaxDim || K < 1 || K > kMaxDim || N * K > kMaxElems)
        return fail(RTQ_ERR_SHAPE, "rtq_quantize_f8_host: N=%lld K=%lld out of range", (long long)N, (long long)K);
    if (N == 0) return RTQ_OK;
    if (!w || !codes) return fail(RTQ_ERR_NULL, "rtq_quantize_f8_host: a pointer argument is NULL");
    if (!aligned(w, 4)) return fail(RTQ_ERR_ALIGN, "rtq_quantize_f8_host: misaligned pointer");
    if (overlaps(range_of(w, N * K * 4), range_of(codes, N * K)))
        return fail(RTQ_ERR_OVERLAP, "rtq_quantize_f8_host: output overlaps the weights");
    rtq::quantize_f8_host(w, codes, N, K, host_threads(threads));
    return RTQ_OK;
}

}  // extern "C"
