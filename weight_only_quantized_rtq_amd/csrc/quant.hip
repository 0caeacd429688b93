// Quantizers and element-wise dequantizers for the two weight formats.
//
// int4 (RT-J int4 model card, "Quantization format"): groups of 32 along K,
// two codes per byte with the low nibble at the even index, one fp16
// (scale, min) pair per group, W = code * scale + min; group ranges from a
// min-MSE clip search over the shrink factors 1.00 .. 0.80.
// int8 (RT-J int8 model card, "Quantization format"): one symmetric fp32
// scale per output row, scale = max|row| / 127, W = q * scale.
#include <algorithm>
#include <cmath>
#include <thread>
#include <vector>

#include "rtq_device.h"
#include "rtq_internal.h"

namespace rtq {

namespace {

constexpr int kGroup = 32;

// ---------------------------------------------------------------------------
// int4 quantizer: one thread per 32-group (on the GPU; the host quantizer runs
// the same function per group). All decisions in fp64 with every operation
// rounded on its own (no contraction), so the codes and pairs are a
// deterministic function of the fp32 input, the same on both sides.
// ---------------------------------------------------------------------------
__host__ __device__ inline void quantize_q4_group(const float* __restrict__ w, uint8_t* __restrict__ payload,
                                                  uint32_t* __restrict__ pairs, int64_t gid,
                                                  int64_t groups_per_row, int64_t K) {
#pragma clang fp contract(off)
    const int64_t row = gid / groups_per_row;
    const int64_t grp = gid - row * groups_per_row;
    const float4* src = reinterpret_cast<const float4*>(w + row * K + grp * kGroup);

    double v[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup / 4; ++i) {
        const float4 f = src[i];
        v[4 * i + 0] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
    double wmin = v[0], wmax = v[0];
#pragma unroll
    for (int k = 1; k < kGroup; ++k) {
        wmin = fmin(wmin, v[k]);
        wmax = fmax(wmax, v[k]);
    }

    const double alphas[5] = {1.00, 0.95, 0.90, 0.85, 0.80};
    double best_err = 0.0;
    uint32_t best_pair = 0;
    uint32_t best_codes[4] = {0, 0, 0, 0};
#pragma unroll
    for (int a = 0; a < 5; ++a) {
        const double lo = alphas[a] * wmin;
        const double hi = alphas[a] * wmax;
        const uint32_t s16 = double_to_half_bits((hi - lo) / 15.0);
        const uint32_t m16 = double_to_half_bits(lo);
        const double s = half_bits_value(s16);
        const double m = half_bits_value(m16);
        double err = 0.0;
        uint32_t codes[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
            double q = 0.0;
            if (s > 0.0) {
                q = __builtin_rint((v[k] - m) / s);
                q = fmin(fmax(q, 0.0), 15.0);
            }
            const double recon = q * s + m;
            const double d = recon - v[k];
            const double sq = d * d;
            err = err + sq;
            codes[k / 8] |= static_cast<uint32_t>(q) << (4 * (k % 8));
        }
        if (a == 0 || err < best_err) {
            best_err = err;
            best_pair = s16 | (m16 << 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) best_codes[i] = codes[i];
        }
    }
    uint4 out;
    out.x = best_codes[0];
    out.y = best_codes[1];
    out.z = best_codes[2];
    out.w = best_codes[3];
    *reinterpret_cast<uint4*>(payload + row * (K / 2) + grp * (kGroup / 2)) = out;
    pairs[gid] = best_pair;
}

__global__ __launch_bounds__(256) void quantize_q4_kernel(const float* __restrict__ w,
                                                          uint8_t* __restrict__ payload,
                                                          uint32_t* __restrict__ pairs,
                                                          int64_t n_groups, int64_t groups_per_row,
                                                          int64_t K) {
    for (int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; gid < n_groups;
         gid += static_cast<int64_t>(gridDim.x) * blockDim.x)
        quantize_q4_group(w, payload, pairs, gid, groups_per_row, K);
}

// ---------------------------------------------------------------------------
// int8 quantizer: one 256-thread workgroup per row (the host quantizer runs
// the same per-element arithmetic).
// ---------------------------------------------------------------------------
// Row scale from the row's largest magnitude: max|row| / 127, rounded to fp32.
__host__ __device__ inline float q8_scale_of(float amax) {
    return static_cast<float>(static_cast<double>(amax) / 127.0);
}

// Code of one weight: rint(w / scale) in fp64, half to even, clamped to
// -127..127; 0 for a zero scale.
__host__ __device__ inline int8_t q8_code(float w, double scd) {
    double r = 0.0;
    if (scd > 0.0) {
        r = __builtin_rint(static_cast<double>(w) / scd);
        r = fmin(fmax(r, -127.0), 127.0);
    }
    return static_cast<int8_t>(r);
}

__global__ __launch_bounds__(256) void quantize_q8_kernel(const float* __restrict__ w,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale, int64_t K) {
    const int64_t row = blockIdx.x;
    const float* src = w + row * K;
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) amax = fmaxf(amax, fabsf(src[k]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    const float sc = q8_scale_of(amax);
    if (threadIdx.x == 0) scale[row] = sc;
    const double scd = sc;
    int8_t* dst = q + row * K;
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) dst[k] = q8_code(src[k], scd);
}

// ---------------------------------------------------------------------------
// Element-wise dequantizers (same arithmetic as the GEMM's staging step).
// ---------------------------------------------------------------------------
// One thread per 8 codes (one 32-bit word of payload).
__global__ __launch_bounds__(256) void dequant_q4_kernel(const uint32_t* __restrict__ payload,
                                                         const uint32_t* __restrict__ pairs,
                                                         float* __restrict__ w, int64_t n_words,
                                                         int64_t words_per_row, int64_t K) {
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n_words;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t row = t / words_per_row;
        const int64_t word = t - row * words_per_row;       // covers k = 8*word .. 8*word+7
        const uint32_t bits = payload[t];
        const uint32_t pr = pairs[row * (K / kGroup) + (word * 8) / kGroup];
        const float s = half_bits_to_float(pr & 0xffffu);
        const float m = half_bits_to_float(pr >> 16);
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(static_cast<float>(nibble(bits, i)), s, m);
        float4* dst = reinterpret_cast<float4*>(w + row * K + word * 8);
        dst[0] = make_float4(o[0], o[1], o[2], o[3]);
        dst[1] = make_float4(o[4], o[5], o[6], o[7]);
    }
}

__global__ __launch_bounds__(256) void dequant_q8_kernel(const int8_t* __restrict__ q,
                                                         const float* __restrict__ scale,
                                                         float* __restrict__ w, int64_t total, int64_t K) {
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x)
        w[t] = static_cast<float>(q[t]) * scale[t / K];
}

// Grid of an element-wise kernel (every one loops grid-stride): enough
// workgroups to cover n items once, at most 2^20.
inline unsigned blocks_for(int64_t n, int per) {
    const int64_t b = (n + per - 1) / per;
    return static_cast<unsigned>(b < (int64_t(1) << 20) ? (b > 0 ? b : 1) : (int64_t(1) << 20));
}

// FP8 E4M3 codes of fp32 weights, as a cast to PyTorch's float8_e4m3fn gives
// them (FP8 model card, "FP8 Format"): the nearest point of the E4M3 grid,
// ties to the even code, NaN (0x7F with the input's sign) past 448 and for
// infinities and NaN. With e the binary exponent of |w|, clamped below at -6
// (the smallest normal exponent), |w| * 2^(3-e) lies in [0, 16) and is exact;
// its rounding to an integer is the mantissa (plus 8 for normal values), so
// code = 8 * (e + 6) + rint(|w| * 2^(3-e)), and a rounding up to 16 carries
// into the exponent field by itself.
__host__ __device__ inline uint8_t f8_code(float w) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, w);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t mag = bits & 0x7fffffffu;
    uint32_t code = 0x7fu;                                       // infinity or NaN
    if (mag < 0x7f800000u) {
        const int eb = static_cast<int>(mag >> 23) - 127;
        const int e = eb > -6 ? eb : -6;
        const int q = static_cast<int>(rintf(ldexpf(__builtin_bit_cast(float, mag), 3 - e)));
        const int c = 8 * (e + 6) + q;
        code = c > 0x7e ? 0x7fu : static_cast<uint32_t>(c);
    }
    return static_cast<uint8_t>(sign | code);
}

__global__ __launch_bounds__(256) void quantize_f8_kernel(const float* __restrict__ w,
                                                          uint8_t* __restrict__ codes, int64_t total) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256)
        codes[i] = f8_code(w[i]);
}

// Host: rows [0, N) split into contiguous ranges over `threads` threads (the
// calling thread takes the first range).
template <class F>
void for_rows(int64_t N, int threads, F&& fn) {
    const int64_t t = std::max<int64_t>(1, std::min<int64_t>(threads, N));
    const int64_t per = (N + t - 1) / t;
    std::vector<std::thread> pool;
    for (int64_t i = 1; i < t; ++i) {
        const int64_t b = i * per, e = std::min(N, b + per);
        if (b < e) pool.emplace_back([&fn, b, e] { fn(b, e); });
    }
    fn(0, std::min(N, per));
    for (auto& th : pool) th.join();
}

__global__ __launch_bounds__(256) void dequant_f8_kernel(const uint8_t* __restrict__ codes,
                                                         float* __restrict__ w, int64_t total) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256)
        w[i] = f8_to_float(codes[i]);
}

}  // namespace

hipError_t launch_quantize_q4(const float* w, uint8_t* payload, uint16_t* pairs, int64_t N,
                              int64_t K, hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t n_groups = N * G;
    quantize_q4_kernel<<<blocks_for(n_groups, 256), 256, 0, stream>>>(
        w, payload, reinterpret_cast<uint32_t*>(pairs), n_groups, G, K);
    return hipGetLastError();
}

hipError_t launch_quantize_q8(const float* w, int8_t* q, float* scale, int64_t N, int64_t K,
                              hipStream_t stream) {
    quantize_q8_kernel<<<static_cast<unsigned>(N), 256, 0, stream>>>(w, q, scale, K);
    return hipGetLastError();
}

void quantize_q4_host(const float* w, uint8_t* payload, uint16_t* pairs, int64_t N, int64_t K, int threads) {
    const int64_t G = K / kGroup;
    uint32_t* pr = reinterpret_cast<uint32_t*>(pairs);
    for_rows(N, threads, [&](int64_t r0, int64_t r1) {
        for (int64_t gid = r0 * G; gid < r1 * G; ++gid) quantize_q4_group(w, payload, pr, gid, G, K);
    });
}

void quantize_q8_host(const float* w, int8_t* q, float* scale, int64_t N, int64_t K, int threads) {
    for_rows(N, threads, [&](int64_t r0, int64_t r1) {
        for (int64_t row = r0; row < r1; ++row) {
            const float* src = w + row * K;
            float amax = 0.0f;
            for (int64_t k = 0; k < K; ++k) amax = std::fmax(amax, std::fabs(src[k]));
            const float sc = q8_scale_of(amax);
            scale[row] = sc;
            for (int64_t k = 0; k < K; ++k) q[row * K + k] = q8_code(src[k], sc);
        }
    });
}

void quantize_f8_host(const float* w, uint8_t* codes, int64_t N, int64_t K, int threads) {
    for_rows(N, threads, [&](int64_t r0, int64_t r1) {
        for (int64_t i = r0 * K; i < r1 * K; ++i) codes[i] = f8_code(w[i]);
    });
}

hipError_t launch_dequant_q4(const uint8_t* payload, const uint16_t* pairs, float* w, int64_t N,
                             int64_t K, hipStream_t stream) {
    const int64_t words_per_row = K / 8;
    const int64_t n_words = N * words_per_row;
    dequant_q4_kernel<<<blocks_for(n_words, 256), 256, 0, stream>>>(
        reinterpret_cast<const uint32_t*>(payload), reinterpret_cast<const uint32_t*>(pairs), w,
        n_words, words_per_row, K);
    return hipGetLastError();
}

hipError_t launch_dequant_q8(const int8_t* q, const float* scale, float* w, int64_t N, int64_t K,
                             hipStream_t stream) {
    const int64_t total = N * K;
    dequant_q8_kernel<<<blocks_for(total, 256), 256, 0, stream>>>(q, scale, w, total, K);
    return hipGetLastError();
}

}  // namespace rtq

namespace rtq {

hipError_t launch_quantize_f8(const float* w, uint8_t* codes, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t total = N * K;
    quantize_f8_kernel<<<blocks_for(total, 256), 256, 0, stream>>>(w, codes, total);
    return hipGetLastError();
}

hipError_t launch_dequant_f8(const uint8_t* codes, float* w, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t total = N * K;
    dequant_f8_kernel<<<blocks_for(total, 256), 256, 0, stream>>>(codes, w, total);
    return hipGetLastError();
}

}  // namespace rtq
