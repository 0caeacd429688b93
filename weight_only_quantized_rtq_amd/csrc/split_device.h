// Device helpers of the split-limb kernels (gemm_split.hip, gemm_direct.hip):
// the exact three-limb split of fp32 activations into bf16 and the two-limb
// fp16 split, weight code to bf16 / fp16 conversions, the bf16 and fp16
// MFMAs, the swizzled 16 x 32 operand layout in LDS and the XCD-aware
// workgroup order.
#pragma once

#include "rtq_device.h"

namespace rtq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// Exact three-limb split of two fp32 values into packed bf16x2 words (element
// a in the low half, b in the high half).
__device__ __forceinline__ void split2(float a, float b, uint32_t& h, uint32_t& mid, uint32_t& lo) {
    const uint32_t ha = fbits(a) & 0xffff0000u, hb = fbits(b) & 0xffff0000u;
    const float ra = a - bitsf(ha), rb = b - bitsf(hb);
    const uint32_t ma = fbits(ra) & 0xffff0000u, mb = fbits(rb) & 0xffff0000u;
    const float sa = ra - bitsf(ma), sb = rb - bitsf(mb);
    h = (ha >> 16) | hb;
    mid = (ma >> 16) | mb;
    lo = (fbits(sa) >> 16) | (fbits(sb) & 0xffff0000u);
}

// Value of the lane N places further along its 16-lane row (DPP row_ror:N).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    static_assert(N >= 1 && N <= 15, "rotation");
    return bitsf(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(fbits(v)), 0x120 + N, 0xf, 0xf, true)));
}

// Byte k of a word -> fp32 (v_cvt_f32_ubyte{k}: exact).
__device__ __forceinline__ float ubyte0(uint32_t x) { float r; asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x)); return r; }
__device__ __forceinline__ float ubyte1(uint32_t x) { float r; asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x)); return r; }
__device__ __forceinline__ float ubyte2(uint32_t x) { float r; asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x)); return r; }
__device__ __forceinline__ float ubyte3(uint32_t x) { float r; asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x)); return r; }

// High halves of two fp32 (bf16 truncation of exact small integers) -> one bf16x2 word.
__device__ __forceinline__ uint32_t pack_hi(float even, float odd) {
    return __builtin_amdgcn_perm(fbits(odd), fbits(even), 0x07060302u);
}

// 8 int4 codes (one payload word, low nibble first) -> 8 bf16 (exact integers).
__device__ __forceinline__ u32x4 codes4_to_bf16(uint32_t w) {
    const uint32_t lo = w & 0x0f0f0f0fu;           // codes 0,2,4,6 in bytes 0..3
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;    // codes 1,3,5,7
    u32x4 r;
    r[0] = pack_hi(ubyte0(lo), ubyte0(hi));
    r[1] = pack_hi(ubyte1(lo), ubyte1(hi));
    r[2] = pack_hi(ubyte2(lo), ubyte2(hi));
    r[3] = pack_hi(ubyte3(lo), ubyte3(hi));
    return r;
}

// 8 int8 codes (two words) -> 8 bf16 (exact integers).
__device__ __forceinline__ u32x4 codes8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = d < 2 ? w0 : w1;
        const int sh = 16 * (d & 1);
        const float e = static_cast<float>(static_cast<int8_t>((w >> sh) & 0xffu));
        const float o = static_cast<float>(static_cast<int8_t>((w >> (sh + 8)) & 0xffu));
        r[d] = pack_hi(e, o);
    }
    return r;
}

// 8 FP8 E4M3 codes (two words, low byte first) -> 8 bf16, exactly: an E4M3
// value has at most 4 significant bits and lies within the bf16 exponent
// range, so the high half of its fp32 form is the value.
__device__ __forceinline__ u32x4 codes8f_to_bf16(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), true);
    u32x4 r;
    r[0] = pack_hi(a[0], a[1]);
    r[1] = pack_hi(b[0], b[1]);
    r[2] = pack_hi(c[0], c[1]);
    r[3] = pack_hi(d[0], d[1]);
    return r;
}

// fp16 forms for the two-limb fp16 split (NL = 2). A word 0x64XX is the fp16
// value 1024 + XX (the 10-bit mantissa holds XX exactly), so placing a code
// byte under 0x64 and subtracting a constant in fp16 gives the code's value
// exactly: the difference is a small integer, representable without rounding.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t f16x2_sub(uint32_t w, _Float16 c) {
    const f16x2 r = __builtin_bit_cast(f16x2, w) - f16x2{c, c};
    return __builtin_bit_cast(uint32_t, r);
}

// 8 int4 codes (one payload word, low nibble first) -> 8 fp16 (exact integers).
__device__ __forceinline__ u32x4 codes4_to_f16(uint32_t w) {
    const uint32_t lo = w & 0x0f0f0f0fu;                           // codes 0,2,4,6
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;                    // codes 1,3,5,7
    const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u); // bytes: codes 0,1,2,3
    const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u); // codes 4,5,6,7
    constexpr uint32_t k64 = 0x64646464u;
    u32x4 r;
    r[0] = f16x2_sub(__builtin_amdgcn_perm(k64, a, 0x04010400u), 1024.0f16);
    r[1] = f16x2_sub(__builtin_amdgcn_perm(k64, a, 0x04030402u), 1024.0f16);
    r[2] = f16x2_sub(__builtin_amdgcn_perm(k64, b, 0x04010400u), 1024.0f16);
    r[3] = f16x2_sub(__builtin_amdgcn_perm(k64, b, 0x04030402u), 1024.0f16);
    return r;
}

// 8 int8 codes (two words) -> 8 fp16 (exact integers): the byte b + 128 under
// 0x64 is 1152 + b, less 1152.
__device__ __forceinline__ u32x4 codes8_to_f16(uint32_t w0, uint32_t w1) {
    const uint32_t t0 = w0 ^ 0x80808080u, t1 = w1 ^ 0x80808080u;
    constexpr uint32_t k64 = 0x64646464u;
    u32x4 r;
    r[0] = f16x2_sub(__builtin_amdgcn_perm(k64, t0, 0x04010400u), 1152.0f16);
    r[1] = f16x2_sub(__builtin_amdgcn_perm(k64, t0, 0x04030402u), 1152.0f16);
    r[2] = f16x2_sub(__builtin_amdgcn_perm(k64, t1, 0x04010400u), 1152.0f16);
    r[3] = f16x2_sub(__builtin_amdgcn_perm(k64, t1, 0x04030402u), 1152.0f16);
    return r;
}

// 8 FP8 E4M3 codes -> 8 fp16, exactly: an E4M3 value has at most 4
// significant bits and lies inside the fp16 range (subnormals included), so
// the rounding of the fp32 -> fp16 conversion never acts.
__device__ __forceinline__ u32x4 codes8f_to_f16(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), true);
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a[0], a[1]));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(b[0], b[1]));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(c[0], c[1]));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(d[0], d[1]));
    return r;
}

// The same conversions in the two-limb k order: word j of the result holds
// the codes of k = j (low half) and k = j + 4 (high half), so an operand's
// eight k of a lane run 0, 4, 1, 5, 2, 6, 3, 7. The limb image of the
// two-limb arithmetic stores x in that order (prep_kernel<2>). For int4 the
// nibbles of k and k + 4 sit 16 bits apart in the payload word, so one
// and-or puts both under the fp16 exponent byte 0x64: 1024 + c for the low
// nibble of a byte, 1024 + 16c for the high nibble (then (t/16) - 64 in one
// fp16 fma, exact: t/16 = 64 + c).
__device__ __forceinline__ uint32_t f16x2_fma(uint32_t w, _Float16 m, _Float16 c) {
    const f16x2 r = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, w), f16x2{m, m}, f16x2{c, c});
    return __builtin_bit_cast(uint32_t, r);
}

// (w & mask) | e in one v_and_or_b32 (the compiler splits it when both
// constants are literals); e is passed in a VGPR, the mask in an SGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t e) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(e));
    return r;
}

__device__ __forceinline__ u32x4 codes4_to_f16_k04(uint32_t w) {
    const uint32_t e = 0x64006400u;
    const uint32_t t = w >> 8;
    u32x4 r;
    r[0] = f16x2_sub(and_or(w, 0x000f000fu, e), 1024.0f16);                   // k 0, 4
    r[1] = f16x2_fma(and_or(w, 0x00f000f0u, e), 0.0625f16, -64.0f16);         // k 1, 5
    r[2] = f16x2_sub(and_or(t, 0x000f000fu, e), 1024.0f16);                   // k 2, 6
    r[3] = f16x2_fma(and_or(t, 0x00f000f0u, e), 0.0625f16, -64.0f16);         // k 3, 7
    return r;
}

// 8 int8 codes (bytes 0..3 of w0, 4..7 of w1) -> fp16 in the k order 0, 4, 1, 5, ...
__device__ __forceinline__ u32x4 codes8_to_f16_k04(uint32_t w0, uint32_t w1) {
    const uint32_t t0 = w0 ^ 0x80808080u, t1 = w1 ^ 0x80808080u;
    const uint32_t lo = __builtin_amdgcn_perm(t1, t0, 0x05010400u);    // bytes: k 0, 4, 1, 5
    const uint32_t hi = __builtin_amdgcn_perm(t1, t0, 0x07030602u);    // k 2, 6, 3, 7
    constexpr uint32_t k64 = 0x64646464u;
    u32x4 r;
    r[0] = f16x2_sub(__builtin_amdgcn_perm(k64, lo, 0x04010400u), 1152.0f16);
    r[1] = f16x2_sub(__builtin_amdgcn_perm(k64, lo, 0x04030402u), 1152.0f16);
    r[2] = f16x2_sub(__builtin_amdgcn_perm(k64, hi, 0x04010400u), 1152.0f16);
    r[3] = f16x2_sub(__builtin_amdgcn_perm(k64, hi, 0x04030402u), 1152.0f16);
    return r;
}

// 8 FP8 E4M3 codes -> fp16 in the k order 0, 4, 1, 5, ... (exact, as above).
__device__ __forceinline__ u32x4 codes8f_to_f16_k04(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), false);   // k 0, 1
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), true);    // k 2, 3
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), false);   // k 4, 5
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), true);    // k 6, 7
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a[0], c[0]));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a[1], c[1]));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(b[0], d[0]));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(b[1], d[1]));
    return r;
}

__device__ __forceinline__ floatx4 mfma_f16(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}

// Two-limb fp16 split of two fp32 values already scaled into the fp16 range:
// h = nearest fp16 of v (ties to even), l = nearest fp16 of v - h (the
// difference is exact in fp32). Packed words, a in the low half.
__device__ __forceinline__ void split_f16x2(float a, float b, uint32_t& h, uint32_t& l) {
    const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
    const _Float16 la = static_cast<_Float16>(a - static_cast<float>(ha));
    const _Float16 lb = static_cast<_Float16>(b - static_cast<float>(hb));
    h = __builtin_bit_cast(uint32_t, f16x2{ha, hb});
    l = __builtin_bit_cast(uint32_t, f16x2{la, lb});
}

__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// Nearest bf16 of two fp32 values (ties to even), packed: a low, b high.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// 16 rows x 32 k of bf16 (1 KB, MFMA operand order): row r (0..15), 16-byte
// chunk c (k = 8c..8c+7) sits at (r*4 + (c ^ ((r>>2)&3))) * 16. The XOR keeps
// the 16-byte reads of one MFMA operand free of LDS bank conflicts.
__device__ __forceinline__ int swz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Workgroup w of a G-workgroup launch -> the item it runs, so that each XCD
// (the hardware deals workgroups round-robin over 8 XCDs) gets one contiguous
// range of items and the items that share inputs share that XCD's L2.
__device__ __forceinline__ int xcd_remap_split(int w, int G) {
    const int q = G / 8, r = G % 8;
    const int xcd = w % 8, local = w / 8;
    const int start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return start + local;
}

}  // namespace rtq
