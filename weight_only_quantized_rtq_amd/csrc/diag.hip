// Measured ceilings of the chip, the denominators beside the published peaks:
// a streaming read of a device buffer (how many bytes per second the HBM
// delivers to plain coalesced 16-byte loads) and back-to-back matrix
// instructions (how many flops per second the matrix cores issue at the
// clock they run under load). Neither touches the projection path.
#include "rtq_internal.h"
#include "split_device.h"

namespace rtq {

namespace {

// Each lane keeps U 16-byte loads in flight; a wave's load covers 1 KB of
// consecutive bytes and the grid strides over the buffer. The words are
// folded with XOR and stored only if the fold hits a value no buffer the
// caller passes produces in practice, so the loads stay live and nothing is
// written.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16, uint32_t* sink) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Eight independent accumulators per wave, each updated by one matrix
// instruction per iteration (no dependence between consecutive issues).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* sink) {
    const uint32_t t = threadIdx.x + 1u;
    u32x4 a, b;
    a[0] = t * 0x00010001u; a[1] = a[0] ^ 0x3c003c00u; a[2] = a[0] + 7u; a[3] = a[1] - 3u;
    b[0] = a[3]; b[1] = a[2]; b[2] = a[1]; b[3] = a[0];
    const float fa = __builtin_bit_cast(float, t | 0x3c000000u), fb = 1.0f / fa;
    floatx4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (KIND == 0) acc[j] = mfma_f16(a, b, acc[j]);
            else if constexpr (KIND == 1) acc[j] = mfma_bf16(a, b, acc[j]);
            else acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa, fb, acc[j], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (s == 1234567.0f) sink[0] = s;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, int unroll, int blocks, uint32_t* sink,
                              hipStream_t stream) {
    const u32x4* p = static_cast<const u32x4*>(buf);
    const int64_t n16 = bytes / 16;
    switch (unroll) {
        case 4: stream_read_kernel<4><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
        case 8: stream_read_kernel<8><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
        case 16: stream_read_kernel<16><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mfma_loop(int kind, int64_t iters, int blocks, float* sink, hipStream_t stream) {
    switch (kind) {
        case 0: mfma_loop_kernel<0><<<blocks, 256, 0, stream>>>(iters, sink); break;
        case 1: mfma_loop_kernel<1><<<blocks, 256, 0, stream>>>(iters, sink); break;
        case 2: mfma_loop_kernel<2><<<blocks, 256, 0, stream>>>(iters, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rtq
