// Internal launchers of the rtq library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtq {

enum Fmt : int { kFmtQ4 = 1, kFmtQ8 = 2, kFmtF8 = 3 };

hipError_t launch_quantize_q4(const float* w, uint8_t* payload, uint16_t* pairs, int64_t N,
                              int64_t K, hipStream_t stream);
hipError_t launch_quantize_q8(const float* w, int8_t* q, float* scale, int64_t N, int64_t K,
                              hipStream_t stream);
hipError_t launch_dequant_q4(const uint8_t* payload, const uint16_t* pairs, float* w, int64_t N,
                             int64_t K, hipStream_t stream);
hipError_t launch_dequant_q8(const int8_t* q, const float* scale, float* w, int64_t N, int64_t K,
                             hipStream_t stream);
hipError_t launch_quantize_f8(const float* w, uint8_t* codes, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_dequant_f8(const uint8_t* codes, float* w, int64_t N, int64_t K, hipStream_t stream);

// One projection of a grouped launch.
struct ProjTask {
    int fmt;
    int N;
    int K;
    const void* payload;
    const void* scale;
    const float* x;
    float* y;
    const float* bias;      // fp32 [N] or nullptr
};

// Kernel timing marks (rtq_timing_enable): returns a slot or -1 when off.
int timing_begin(hipStream_t stream);
void timing_end(int slot, hipStream_t stream);

// Arithmetic of a GEMM call (the rtq_gemm_ex / rtq_block_project_ex argument).
enum Math : int { kMathSplitBf16 = 0, kMathFp32Mfma = 1, kMathBf16 = 2, kMathSplitF16 = 3 };
// Limbs of the split path for a math mode: 3 (exact bf16 split), 2 (fp16
// split of the row-scaled x) or 1 (bf16 x); 0 = fp32 path.
inline int split_limbs(int mode) {
    return mode == kMathSplitBf16 ? 3 : mode == kMathSplitF16 ? 2 : mode == kMathBf16 ? 1 : 0;
}

// Single projection y[M][N] = x[M][K] . dequant(W)^T in arithmetic `math`.
hipError_t launch_gemm(const ProjTask& task, int64_t M, int math, hipStream_t stream);

// Where the split path's workspace (limb images, K-chunk partials) comes
// from: a stream-ordered allocation from the library's pool, the library's
// fixed scratch array, or a caller's device buffer.
enum WsMode { kWsPool = 0, kWsScratch = 1, kWsCaller = 2 };

// Several projections sharing M, in grouped launches. Every task must satisfy
// grouped_ok(). With kWsCaller the workspace is ws (cap bytes, at least
// grouped_workspace_bytes()).
hipError_t launch_grouped(const ProjTask* tasks, int count, int64_t M, int math, hipStream_t stream,
                          WsMode mode = kWsPool, unsigned char* ws = nullptr, int64_t cap = 0);
bool grouped_ok(const ProjTask& task);
// Workspace bytes launch_grouped needs for these tasks in arithmetic `math`.
int64_t grouped_workspace_bytes(const ProjTask* tasks, int count, int64_t M, int math);

// Split-limb path (gemm_split.hip): every projection of the call, sharing M,
// with NL = 3 bf16 limbs (exact), 2 fp16 limbs of the row-scaled x, or 1 (x
// rounded to bf16). Tasks must satisfy
// split_ok(). Uses a stream-ordered workspace from the library's pool.
bool split_ok(const ProjTask& task);
hipError_t launch_split(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream);
// Workspace bytes launch_split needs for these tasks (0 when they take the
// direct small-M kernel).
int64_t split_workspace_bytes(const ProjTask* tasks, int count, int64_t M, int NL);
// launch_split with the library's fixed per-device scratch array as the
// workspace instead of an allocation (rtq_block_project_noalloc); returns
// hipErrorOutOfMemory, launching nothing, if the call needs more than
// kScratchBytes.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
hipError_t launch_split_scratch(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream);
// launch_split with a caller's workspace of cap bytes (non-null wherever
// split_workspace_bytes() is positive); hipErrorOutOfMemory, launching
// nothing, if it is too small.
hipError_t launch_split_ws(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream,
                           unsigned char* ws, int64_t cap);

// Small-M path of the split arithmetic (gemm_direct.hip): one launch, whole K
// per workgroup, x split in the kernel. direct_fits(): M in 1..32, every K in
// {256, 512, 1024, 2048} and int4 pair arrays 16-byte aligned; the tasks must
// also satisfy split_ok().
bool direct_fits(const ProjTask* tasks, int count, int64_t M);
hipError_t launch_direct(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream);

// Host quantizers (quant.hip): the GPU quantizers' per-group / per-element
// arithmetic run on host memory over `threads` threads; bit-identical results.
void quantize_q4_host(const float* w, uint8_t* payload, uint16_t* pairs, int64_t N, int64_t K, int threads);
void quantize_q8_host(const float* w, int8_t* q, float* scale, int64_t N, int64_t K, int threads);
void quantize_f8_host(const float* w, uint8_t* codes, int64_t N, int64_t K, int threads);

// y += bias (broadcast over the M rows) for every task that has a bias, in
// place, after the GEMM kernels that wrote y (same stream).
hipError_t launch_bias_add(const ProjTask* tasks, int count, int64_t M, hipStream_t stream);

// Diagnostics (diag.hip): measured ceilings.
hipError_t launch_stream_read(const void* buf, int64_t bytes, int unroll, int blocks, uint32_t* sink,
                              hipStream_t stream);
hipError_t launch_mfma_loop(int kind, int64_t iters, int blocks, float* sink, hipStream_t stream);

}  // namespace rtq
