// Device-side helpers shared by the gfx950 kernels of the rtq library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtq {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// fp16 bit pattern -> its exact fp64 value, from the bits alone (used by the
// quantizers, which also run on the host): (1024 + f) * 2^(e - 25) for normal
// codes, f * 2^-24 for subnormal ones.
__host__ __device__ inline double half_bits_value(uint32_t h) {
    const uint32_t e = (h >> 10) & 0x1fu, f = h & 0x3ffu;
    double v;
    if (e == 0x1fu) {
        v = f ? __builtin_nan("") : __builtin_inf();
    } else {
        const uint32_t mant = e ? (f | 0x400u) : f;
        const int pw = e ? static_cast<int>(e) - 25 : -24;        // in [-24, 5]: a normal fp64 power of two
        v = static_cast<double>(mant) * __builtin_bit_cast(double, static_cast<uint64_t>(1023 + pw) << 52);
    }
    return (h & 0x8000u) ? -v : v;
}

// fp64 -> fp16 bit pattern, round to nearest, ties to even, directly from the
// fp64 value (no intermediate fp32 rounding). Subnormal fp16 results are kept;
// magnitudes that round above 65504 become infinity.
__host__ __device__ inline uint32_t double_to_half_bits(double d) {
    const uint64_t b = __builtin_bit_cast(uint64_t, d);
    const uint32_t sign = static_cast<uint32_t>(b >> 63) << 15;
    const int exp = static_cast<int>((b >> 52) & 0x7ff);
    const uint64_t frac = b & ((1ull << 52) - 1);
    if (exp == 0x7ff) return sign | 0x7c00u | (frac ? 0x200u : 0u);   // inf / nan
    if (exp == 0) return sign;                                        // fp64 zero or subnormal
    const int e = exp - 1023;                                         // value in [2^e, 2^(e+1))
    if (e >= 16) return sign | 0x7c00u;
    const uint64_t sig = frac | (1ull << 52);
    int shift;
    uint32_t base;
    if (e >= -14) {            // normal fp16 range: keep 11 significant bits
        shift = 42;
        base = static_cast<uint32_t>(e + 15) << 10;
    } else {                   // fp16 subnormal: units of 2^-24
        shift = 42 + (-14 - e);
        base = 0;
        if (shift > 53) return sign;                                  // below half the smallest subnormal
    }
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    uint32_t h;
    if (base) h = base + static_cast<uint32_t>(q) - 1024u;   // q in [1024, 2048]; 2048 carries into the exponent
    else h = static_cast<uint32_t>(q);                        // q in [0, 1024]; 1024 is the smallest normal
    return sign | h;
}

// Segment lookup for kernels whose workgroups are numbered segment by segment
// (projection by projection, input by input): segment j starts at item
// begin[j] (begin[0] = 0, nondecreasing) and the launch has `count` segments;
// coarse[c] = begin[c * kSegStride] for the slots below count. Returns the
// segment that holds item w: the coarse table picks the run of kSegStride
// slots, then that run picks the segment. Both sums are unrolled and
// branch-free, so each level is one round of independent argument loads; the
// level results pass through an empty asm statement, which makes them opaque
// values, so the loads that depend on them are addressed as base plus a
// sign-extended index.
constexpr int kSegStride = 8;
__host__ __device__ constexpr int seg_coarse_slots(int slots) { return (slots + kSegStride - 1) / kSegStride; }
__host__ __device__ constexpr int seg_begin_slots(int slots) { return slots + kSegStride - 1; }

// begin[] carries kSegStride - 1 slots of padding past the last segment slot,
// so the second level reads one whole run without clamping.
template <int SLOTS, int NC, class T>
__device__ __forceinline__ int segment_of(const T (&begin)[SLOTS], const T (&coarse)[NC], int count, int w) {
    static_assert(NC == seg_coarse_slots(SLOTS - (kSegStride - 1)), "coarse table size");
    int c = 0;
#pragma unroll
    for (int j = 1; j < NC; ++j)
        c += static_cast<int>(j * kSegStride < count) & static_cast<int>(static_cast<int>(coarse[j]) <= w);
    c = __builtin_amdgcn_readfirstlane(c);
    asm volatile("" : "+s"(c));
    const int base = c * kSegStride;
    int i = base;
    const T* run = begin + base;
#pragma unroll
    for (int j = 1; j < kSegStride; ++j)
        i += static_cast<int>(base + j < count) & static_cast<int>(static_cast<int>(run[j]) <= w);
    i = __builtin_amdgcn_readfirstlane(i);
    asm volatile("" : "+s"(i));
    return i;
}

// Host side: fills the coarse table of segment_of from begin[0 .. count).
template <int SLOTS, int NC, class T>
inline void seg_fill_coarse(const T (&begin)[SLOTS], T (&coarse)[NC], int count) {
    for (int c = 0; c < NC; ++c) coarse[c] = c * kSegStride < count ? begin[c * kSegStride] : begin[0];
}

// FP8 E4M3 ("fn": bias 7, subnormals, S.1111.111 = NaN) code -> fp32, exact,
// through the hardware conversion (the byte in bits 0..7).
__device__ __forceinline__ float f8_to_float(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8(code, 0); }

// The value of a one-byte weight code: int8 for the int8 format, E4M3 for FP8.
template <int FMT>
__device__ __forceinline__ float code8_value(uint32_t byte) {
    if constexpr (FMT == 3) return f8_to_float(byte & 0xffu);
    else return static_cast<float>(static_cast<int8_t>(byte & 0xffu));
}

// Low nibble = even index.
__device__ __forceinline__ uint32_t nibble(uint32_t word, int idx) {
    return (word >> (4 * idx)) & 0xFu;
}

}  // namespace rtq
