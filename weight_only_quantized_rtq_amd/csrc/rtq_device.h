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

__device__ __forceinline__ double half_bits_to_double(uint32_t bits16) {
    return static_cast<double>(half_bits_to_float(bits16));
}

// fp64 -> fp16 bit pattern, round to nearest, ties to even, directly from the
// fp64 value (no intermediate fp32 rounding). Subnormal fp16 results are kept;
// magnitudes that round above 65504 become infinity.
__device__ __forceinline__ uint32_t double_to_half_bits(double d) {
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
// begin[j] (begin[0] = 0, nondecreasing) and the launch has `count` segments.
// Returns the segment that holds item w: the number of segments j >= 1 that
// start at or before w. The sum is unrolled over the slots and branch-free, so
// the argument loads have fixed offsets and none waits for another. The result
// is then passed through an empty asm statement, which makes it an opaque
// value: descriptor loads indexed by it are addressed as base plus the
// sign-extended index.
template <int SLOTS, class T>
__device__ __forceinline__ int segment_of(const T (&begin)[SLOTS], int count, int w) {
    int i = 0;
#pragma unroll
    for (int j = 1; j < SLOTS; ++j) i += static_cast<int>(j < count) & static_cast<int>(static_cast<int>(begin[j]) <= w);
    i = __builtin_amdgcn_readfirstlane(i);
    asm volatile("" : "+s"(i));
    return i;
}

// Low nibble = even index.
__device__ __forceinline__ uint32_t nibble(uint32_t word, int idx) {
    return (word >> (4 * idx)) & 0xFu;
}

}  // namespace rtq
