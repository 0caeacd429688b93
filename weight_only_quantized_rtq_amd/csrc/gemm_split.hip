// Dequant-in-GEMM on the bf16 matrix cores with exact fp32 products.
//
// y[M][N] = x[M][K] . W^T with W in its packed int4 / int8 form (RT-J int4 and
// int8 model cards, section "Quantization format"), dequantized inside the
// GEMM as the cards' opening paragraphs describe.
//
// Arithmetic. Every fp32 activation is split, exactly, into three bf16 limbs:
//   x1 = x with the low 16 bits of its encoding cleared  (top 8 significant bits)
//   r  = x - x1                                           (exact, <= 16 bits)
//   x2 = r with the low 16 bits cleared, x3 = r - x2      (x3 has <= 8 bits: exact in bf16)
// so x == x1 + x2 + x3. The int4 codes (0..15) and int8 codes (-127..127) are
// exact in bf16, so every product code * limb is exact in fp32, and
// v_mfma_f32_16x16x32_bf16 accumulates them in fp32: the per-group code sum
// P_g[m][o] = sum_{k in g} code[o][k] * x[m][k] is an fp32 dot product of the
// exact values. One MFMA covers exactly one 32-wide int4 group, so
//   int4: y = sum_g ( scale_g[o] * P_g + min_g[o] * X_g[m] ),  X_g[m] = sum_{k in g} x[m][k]
//   int8: y = scale[o] * sum_k q[o][k] * x[m][k]
// which is W = code*scale + min (int4) and W = q*scale (int8) by
// distributivity. The two fp32 multiply-adds per group run on the VALU.
//
// Data movement. A workgroup stages its x rows once per group into LDS as the
// three bf16 planes plus the group sums X_g (shared by all its waves); each wave
// streams its own packed weight columns from global memory straight into
// registers in MFMA operand layout (4 bytes of int4 codes or 8 bytes of int8
// codes per lane per group), so the packed payload is read once per row tile.
#include "rtq_device.h"
#include "rtq_internal.h"

namespace rtq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXS = 40;   // limb-plane row stride in bf16 (80 bytes: conflict-free b128 reads)

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

__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

struct SplitArgs {
    const float* x;
    const void* payload;
    const void* scale;
    float* y;
    int M, N, K;
};

// LDS: two stages of 3 limb planes [BM][kXS] bf16, then a ring of the last 8
// groups' sums X_g [8][BM] fp32 (read by the deferred min term).
constexpr int kRing = 8;
template <int BM>
struct StageLayout {
    static constexpr int PLANE = BM * kXS * 2;                     // bytes
    static constexpr int BYTES = 3 * PLANE;
    static constexpr int RING = 2 * BYTES;                         // offset of the X ring
    static constexpr int TOTAL = 2 * BYTES + kRing * BM * 4;
};

// One BM x (WN*TN*16) tile (this workgroup's rows m0.., columns n0..) over the
// whole K. Waves are laid out WM x WN; each owns TM x TN 16x16 output tiles.
template <int FMT, int WM, int WN, int TM, int TN>
__device__ __forceinline__ void split_tile(const SplitArgs& a, int m0, int n0, unsigned char* smem) {
    constexpr int BM = WM * TM * 16;
    constexpr int NT = WM * WN * 64;
    using L = StageLayout<BM>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int li = lane & 15;
    const int lc = lane >> 4;
    const int M = a.M, N = a.N, K = a.K;
    const int G = K / 32;

    // ---- x staging: thread -> (row, 16 consecutive k of the group) ----
    const int srow = tid >> 1;
    const int shalf = tid & 1;
    const bool stager = srow < BM;
    const float* xsrc = a.x + static_cast<int64_t>(min(m0 + min(srow, BM - 1), M - 1)) * K + 16 * shalf;
    auto stage_load = [&](int g, float4 (&xr)[4]) {
        if (stager) {
            const float4* p = reinterpret_cast<const float4*>(xsrc + g * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[i] = p[i];
        }
    };
    auto stage_store = [&](int buf, int g, const float4 (&xr)[4]) {
        if (stager) {
            unsigned char* base = smem + buf * L::BYTES;
            const float v[16] = {xr[0].x, xr[0].y, xr[0].z, xr[0].w, xr[1].x, xr[1].y, xr[1].z, xr[1].w,
                                 xr[2].x, xr[2].y, xr[2].z, xr[2].w, xr[3].x, xr[3].y, xr[3].z, xr[3].w};
            uint32_t hw[8], mw[8], lw[8];
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                split2(v[2 * j], v[2 * j + 1], hw[j], mw[j], lw[j]);
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) sum += v[j];
            const int off = (srow * kXS + 16 * shalf) * 2;
            uint4* ph = reinterpret_cast<uint4*>(base + 0 * L::PLANE + off);
            uint4* pm = reinterpret_cast<uint4*>(base + 1 * L::PLANE + off);
            uint4* pl = reinterpret_cast<uint4*>(base + 2 * L::PLANE + off);
            ph[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            ph[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
            pm[0] = make_uint4(mw[0], mw[1], mw[2], mw[3]);
            pm[1] = make_uint4(mw[4], mw[5], mw[6], mw[7]);
            pl[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            pl[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
            // group sum: first 16 + last 16, the same order in both threads
            const float other = __shfl_xor(sum, 1, 64);
            const float gsum = shalf ? other + sum : sum + other;
            if (shalf == 0) reinterpret_cast<float*>(smem + L::RING)[(g & (kRing - 1)) * BM + srow] = gsum;
        }
    };

    // ---- weights: lane (li, lc) of column tile tn holds row n0 + wn*TN*16 + tn*16 + li,
    //      k = 8*lc .. 8*lc+7 of the group ----
    const unsigned char* wrow[TN];
    const uint32_t* prow[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int col = min(n0 + wn * TN * 16 + tn * 16 + li, N - 1);
        if constexpr (FMT == kFmtQ4) {
            wrow[tn] = static_cast<const unsigned char*>(a.payload) + static_cast<int64_t>(col) * (K / 2) + 4 * lc;
            prow[tn] = static_cast<const uint32_t*>(a.scale) + static_cast<int64_t>(col) * G;
        } else {
            wrow[tn] = static_cast<const unsigned char*>(a.payload) + static_cast<int64_t>(col) * K + 8 * lc;
            prow[tn] = nullptr;
        }
    }
    auto w_load = [&](int g, uint32_t (&wq)[TN][2], uint32_t (&wp)[TN]) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if constexpr (FMT == kFmtQ4) {
                wq[tn][0] = *reinterpret_cast<const uint32_t*>(wrow[tn] + g * 16);
                wq[tn][1] = 0;
                wp[tn] = prow[tn][g];
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(wrow[tn] + g * 32);
                wq[tn][0] = v.x;
                wq[tn][1] = v.y;
                wp[tn] = 0;
            }
        }
    };

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // int4 min term, deferred: lane group c keeps min_g of group 4b+c for its
    // columns; every 4 groups one fp32 MFMA 16x16x4 adds sum_g X_g[row] * min_g[col].
    float mreg[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) mreg[tn] = 0.0f;

    auto compute = [&](int buf, int g, const uint32_t (&cq)[TN][2], const uint32_t (&cp)[TN]) {
        const unsigned char* base = smem + buf * L::BYTES;
        u32x4 b[TN];
        float s[TN];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if constexpr (FMT == kFmtQ4) {
                b[tn] = codes4_to_bf16(cq[tn][0]);
                s[tn] = half_bits_to_float(cp[tn] & 0xffffu);
                const float mn = half_bits_to_float(cp[tn] >> 16);
                mreg[tn] = lc == (g & 3) ? mn : mreg[tn];
            } else {
                b[tn] = codes8_to_bf16(cq[tn][0], cq[tn][1]);
            }
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int r = wm * TM * 16 + tm * 16;
            const int off = ((r + li) * kXS + 8 * lc) * 2;
            const u32x4 xh = *reinterpret_cast<const u32x4*>(base + 0 * L::PLANE + off);
            const u32x4 xm = *reinterpret_cast<const u32x4*>(base + 1 * L::PLANE + off);
            const u32x4 xl = *reinterpret_cast<const u32x4*>(base + 2 * L::PLANE + off);
            if constexpr (FMT == kFmtQ4) {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    floatx4 p = mfma_bf16(xl, b[tn], floatx4{0.f, 0.f, 0.f, 0.f});
                    p = mfma_bf16(xm, b[tn], p);
                    p = mfma_bf16(xh, b[tn], p);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[tm][tn][e] = fmaf(s[tn], p[e], acc[tm][tn][e]);
                }
            } else {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    acc[tm][tn] = mfma_bf16(xl, b[tn], acc[tm][tn]);
                    acc[tm][tn] = mfma_bf16(xm, b[tn], acc[tm][tn]);
                    acc[tm][tn] = mfma_bf16(xh, b[tn], acc[tm][tn]);
                }
            }
        }
    };
    // After group g: if it closes a block of 4 (or is the last), add the block's min term.
    auto min_flush = [&](int g) {
        if constexpr (FMT == kFmtQ4) {
            if ((g & 3) != 3 && g != G - 1) return;
            const int gc = (g & ~3) + lc;                 // this lane group's group
            const bool live = gc <= g;
            const float* ring = reinterpret_cast<const float*>(smem + L::RING) + (gc & (kRing - 1)) * BM;
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const float xv = live ? ring[wm * TM * 16 + tm * 16 + li] : 0.0f;
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, mreg[tn], acc[tm][tn], 0, 0, 0);
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) mreg[tn] = 0.0f;
        }
    };

    // ---- main loop: one 32-wide group per stage, double-buffered LDS; global
    //      loads run two groups ahead through two register slots (the loop is
    //      unrolled by two so the slots are fixed registers) ----
    float4 xr0[4], xr1[4];
    uint32_t wq0[TN][2], wq1[TN][2], wp0[TN], wp1[TN];
    stage_load(0, xr0);
    w_load(0, wq0, wp0);
    if (G > 1) {
        stage_load(1, xr1);
        w_load(1, wq1, wp1);
    }
    stage_store(0, 0, xr0);
    __syncthreads();
    for (int g = 0; g < G; g += 2) {
        {
            uint32_t cq[TN][2], cp[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) { cq[tn][0] = wq0[tn][0]; cq[tn][1] = wq0[tn][1]; cp[tn] = wp0[tn]; }
            if (g + 2 < G) {
                stage_load(g + 2, xr0);
                w_load(g + 2, wq0, wp0);
            }
            compute(0, g, cq, cp);
            min_flush(g);
            if (g + 1 < G) stage_store(1, g + 1, xr1);
            __syncthreads();
        }
        if (g + 1 >= G) break;
        __builtin_amdgcn_sched_barrier(0);
        {
            uint32_t cq[TN][2], cp[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) { cq[tn][0] = wq1[tn][0]; cq[tn][1] = wq1[tn][1]; cp[tn] = wp1[tn]; }
            if (g + 3 < G) {
                stage_load(g + 3, xr1);
                w_load(g + 3, wq1, wp1);
            }
            compute(1, g + 1, cq, cp);
            min_flush(g + 1);
            if (g + 2 < G) stage_store(0, g + 2, xr0);
            __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- epilogue: lane holds D[4*lc + e][li] of each 16x16 tile ----
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int col = n0 + wn * TN * 16 + tn * 16 + li;
        if (col >= N) continue;
        float sc = 1.0f;
        if constexpr (FMT == kFmtQ8) sc = static_cast<const float*>(a.scale)[col];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * TM * 16 + tm * 16 + 4 * lc + e;
                if (row < M) {
                    float v = acc[tm][tn][e];
                    if constexpr (FMT == kFmtQ8) v *= sc;
                    a.y[static_cast<int64_t>(row) * N + col] = v;
                }
            }
        }
    }
}

__device__ __forceinline__ int xcd_remap_split(int w, int G) {
    const int q = G / 8, r = G % 8;
    const int xcd = w % 8, local = w / 8;
    const int start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return start + local;
}

// Large M: 128 x 128 tiles, 2 x 2 waves of 64 x 64.
constexpr int kLWM = 2, kLWN = 2, kLTM = 4, kLTN = 4;
constexpr int kLBM = kLWM * kLTM * 16;
constexpr int kLBN = kLWN * kLTN * 16;

template <int FMT>
__global__ __launch_bounds__(256) void split_gemm_kernel(SplitArgs a, int tiles_n) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[StageLayout<kLBM>::TOTAL];
    const int w = xcd_remap_split(blockIdx.x, gridDim.x);
    split_tile<FMT, kLWM, kLWN, kLTM, kLTN>(a, (w / tiles_n) * kLBM, (w % tiles_n) * kLBN, smem);
}

// Small M (<= 80): one row tile of TM*16 rows; 4 waves side by side along N,
// each with TN column tiles, TN chosen per projection so that TN*K is about
// constant (long-K projections get narrower tiles and more workgroups).
constexpr int kMaxSplitGrouped = 96;
constexpr int kMaxSplitInputs = 48;

struct SplitGroupArgs {
    int count;
    int M;
    int n_inputs;
    int total;
    const float* xs[kMaxSplitInputs];
    int xk[kMaxSplitInputs];
    const void* payload[kMaxSplitGrouped];
    const void* scale[kMaxSplitGrouped];
    float* y[kMaxSplitGrouped];
    int n[kMaxSplitGrouped];
    int tile_begin[kMaxSplitGrouped];
    uint8_t x_idx[kMaxSplitGrouped];
    uint8_t fmt[kMaxSplitGrouped];
};
static_assert(sizeof(SplitGroupArgs) <= 4096, "kernel arguments must stay within 4 KiB");

__host__ __device__ inline int split_tn(int K) {
    return K >= 2048 ? 1 : (K >= 1024 ? 2 : 4);
}

template <int TM, int TN>
__device__ __forceinline__ void grouped_dispatch(const SplitArgs& a, int fmt, int n0, unsigned char* smem) {
    if (fmt == kFmtQ4)
        split_tile<kFmtQ4, 1, 4, TM, TN>(a, 0, n0, smem);
    else
        split_tile<kFmtQ8, 1, 4, TM, TN>(a, 0, n0, smem);
}

template <int TM>
__global__ __launch_bounds__(256) void split_grouped_kernel(SplitGroupArgs g) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[StageLayout<TM * 16>::TOTAL];
    const int w = blockIdx.x;
    int i = 0;
    while (i + 1 < g.count && g.tile_begin[i + 1] <= w) ++i;
    const int xi = g.x_idx[i];
    const int K = g.xk[xi];
    const SplitArgs a{g.xs[xi], g.payload[i], g.scale[i], g.y[i], g.M, g.n[i], K};
    const int tn = split_tn(K);
    const int n0 = (w - g.tile_begin[i]) * 4 * tn * 16;
    if (tn == 1)
        grouped_dispatch<TM, 1>(a, g.fmt[i], n0, smem);
    else if (tn == 2)
        grouped_dispatch<TM, 2>(a, g.fmt[i], n0, smem);
    else
        grouped_dispatch<TM, 4>(a, g.fmt[i], n0, smem);
}

}  // namespace

bool split_ok(const ProjTask& t) {
    return t.K % 32 == 0 && (reinterpret_cast<uintptr_t>(t.x) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(t.payload) & 15) == 0;
}

hipError_t launch_split_gemm(const ProjTask& t, int64_t M, hipStream_t stream) {
    const SplitArgs a{t.x, t.payload, t.scale, t.y, static_cast<int>(M), t.N, t.K};
    const int tn = (t.N + kLBN - 1) / kLBN;
    const int tm = static_cast<int>((M + kLBM - 1) / kLBM);
    if (t.fmt == kFmtQ4)
        split_gemm_kernel<kFmtQ4><<<tm * tn, 256, 0, stream>>>(a, tn);
    else
        split_gemm_kernel<kFmtQ8><<<tm * tn, 256, 0, stream>>>(a, tn);
    return hipGetLastError();
}

hipError_t launch_split_grouped(const ProjTask* tasks, int count, int64_t M, hipStream_t stream) {
    int order[8 * 64];
    for (int i = 0; i < count; ++i) order[i] = i;
    for (int i = 1; i < count; ++i) {                 // stable insertion sort, K descending
        const int v = order[i];
        int j = i - 1;
        while (j >= 0 && tasks[order[j]].K < tasks[v].K) {
            order[j + 1] = order[j];
            --j;
        }
        order[j + 1] = v;
    }
    int done = 0;
    while (done < count) {
        SplitGroupArgs g{};
        g.M = static_cast<int>(M);
        int tiles = 0;
        while (done < count && g.count < kMaxSplitGrouped) {
            const ProjTask& t = tasks[order[done]];
            int xi = -1;
            for (int k = 0; k < g.n_inputs; ++k)
                if (g.xs[k] == t.x && g.xk[k] == t.K) xi = k;
            if (xi < 0) {
                if (g.n_inputs == kMaxSplitInputs) break;
                xi = g.n_inputs++;
                g.xs[xi] = t.x;
                g.xk[xi] = t.K;
            }
            const int c = g.count++;
            g.payload[c] = t.payload;
            g.scale[c] = t.scale;
            g.y[c] = t.y;
            g.n[c] = t.N;
            g.tile_begin[c] = tiles;
            g.x_idx[c] = static_cast<uint8_t>(xi);
            g.fmt[c] = static_cast<uint8_t>(t.fmt);
            const int bn = 4 * split_tn(t.K) * 16;
            tiles += (t.N + bn - 1) / bn;
            ++done;
        }
        g.total = tiles;
        switch (static_cast<int>((M + 15) / 16)) {
            case 1: split_grouped_kernel<1><<<tiles, 256, 0, stream>>>(g); break;
            case 2: split_grouped_kernel<2><<<tiles, 256, 0, stream>>>(g); break;
            case 3: split_grouped_kernel<3><<<tiles, 256, 0, stream>>>(g); break;
            case 4: split_grouped_kernel<4><<<tiles, 256, 0, stream>>>(g); break;
            default: split_grouped_kernel<5><<<tiles, 256, 0, stream>>>(g); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace rtq
