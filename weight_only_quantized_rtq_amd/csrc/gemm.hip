// Dequant-in-GEMM kernels: y[M][N] = x[M][K] . W^T with W kept packed in HBM.
//
// The packed weights are streamed once per output tile, unpacked and
// dequantized in registers while the tile is staged into LDS (int4: code*s+m
// with the group's fp16 pair; int8: code*scale[row], the single-rounded fp32
// product, so no sum is formed before the scale and the range is that of an
// fp32 GEMM; FP8: the E4M3 value), and the contraction runs on the fp32 MFMA
// (v_mfma_f32_16x16x4_f32) with fp32 accumulators. The formats are those of
// the RT-J int4 / int8 model cards, section "Quantization format", and of the
// FP8 card, section "FP8 Format"; the dequantize-inside-the-GEMM design is the
// one their opening paragraphs describe. These kernels write x . W^T; a bias
// is added afterwards by the finish pass (launch_bias_add).
#include <vector>

#include "rtq_device.h"
#include "rtq_internal.h"

namespace rtq {

namespace {

constexpr int kBK = 32;        // K step: one int4 group
constexpr int kLD = kBK + 4;   // LDS row stride in floats (pad keeps b128 reads conflict-free)
constexpr int kMaxGrouped = 96;

struct TileArgs {
    const float* x;
    const void* payload;
    const void* scale;
    float* y;
    int M, N, K;
};

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles sharing an x row-block share an L2.
__device__ __forceinline__ int xcd_remap(int w, int G) {
    const int q = G / 8, r = G % 8;
    const int xcd = w % 8, local = w / 8;
    const int start = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return start + local;
}

template <int WM, int WN, int TM, int TN>
struct TileShape {
    static constexpr int NT = WM * WN * 64;
    static constexpr int BM = WM * TM * 16;
    static constexpr int BN = WN * TN * 16;
    static constexpr int XV = BM * (kBK / 4);              // float4 loads per x tile
    static constexpr int XPT = (XV + NT - 1) / NT;
    static constexpr int SMEM = 2 * (BM + BN) * kLD;       // floats, double buffered
    static_assert(BN * kBK == NT * 16, "each thread stages 16 weights of the W tile");
};

// One BM x BN output tile over the whole K range.
// SAFE: per-element bounds on K (int8 with K % 32 != 0 or unaligned rows).
template <int FMT, int WM, int WN, int TM, int TN, bool SAFE>
__device__ __forceinline__ void gemm_tile(const TileArgs& a, int mt, int nt, float* smem) {
    using S = TileShape<WM, WN, TM, TN>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int m0 = mt * S::BM;
    const int n0 = nt * S::BN;
    const int M = a.M, N = a.N, K = a.K;
    const int KT = (K + kBK - 1) / kBK;

    float* xs[2] = {smem, smem + S::BM * kLD};
    float* ws[2] = {smem + 2 * S::BM * kLD, smem + 2 * S::BM * kLD + S::BN * kLD};

    // Staging registers.
    float4 xr[S::XPT];
    const int wr = tid >> 1;        // W tile row staged by this thread
    const int wh = tid & 1;         // which 16 of the 32 k
    const int wrow = n0 + wr;
    // int8 row scale of the staged W row (multiplied into every code)
    const float wscale = FMT == kFmtQ8 && wrow < N ? static_cast<const float*>(a.scale)[wrow] : 1.0f;
    uint2 q4bits = make_uint2(0, 0);
    uint32_t q4pair = 0;
    uint4 q8bits = make_uint4(0, 0, 0, 0);
    float wsafe[16];

    const float* __restrict__ x = a.x;

    auto load = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < S::XPT; ++i) {
            const int idx = tid + i * S::NT;
            if (idx < S::XV) {
                const int r = idx >> 3;
                const int c = idx & 7;
                const int row = m0 + r;
                const int k = k0 + 4 * c;
                if constexpr (SAFE) {
                    const float* p = x + static_cast<int64_t>(row) * K;
                    const bool rv = row < M;
                    xr[i].x = (rv && k + 0 < K) ? p[k + 0] : 0.0f;
                    xr[i].y = (rv && k + 1 < K) ? p[k + 1] : 0.0f;
                    xr[i].z = (rv && k + 2 < K) ? p[k + 2] : 0.0f;
                    xr[i].w = (rv && k + 3 < K) ? p[k + 3] : 0.0f;
                } else {
                    xr[i] = row < M ? *reinterpret_cast<const float4*>(x + static_cast<int64_t>(row) * K + k)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
        if constexpr (FMT == kFmtQ4) {
            if (wrow < N) {
                const uint8_t* p = static_cast<const uint8_t*>(a.payload) +
                                   static_cast<int64_t>(wrow) * (K / 2) + kt * (kBK / 2) + wh * 8;
                q4bits = *reinterpret_cast<const uint2*>(p);
                q4pair = static_cast<const uint32_t*>(a.scale)[static_cast<int64_t>(wrow) * (K / kBK) + kt];
            } else {
                q4bits = make_uint2(0, 0);
                q4pair = 0;
            }
        } else {
            const int8_t* p = static_cast<const int8_t*>(a.payload) + static_cast<int64_t>(wrow) * K;
            const int kb = k0 + wh * 16;
            if constexpr (SAFE) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    wsafe[j] = (wrow < N && kb + j < K) ? code8_value<FMT>(static_cast<uint8_t>(p[kb + j])) : 0.0f;
            } else {
                q8bits = wrow < N ? *reinterpret_cast<const uint4*>(p + kb) : make_uint4(0, 0, 0, 0);
            }
        }
    };

    auto commit = [&](int buf) {
        float* xd = xs[buf];
#pragma unroll
        for (int i = 0; i < S::XPT; ++i) {
            const int idx = tid + i * S::NT;
            if (idx < S::XV) {
                const int r = idx >> 3;
                const int c = idx & 7;
                *reinterpret_cast<float4*>(xd + r * kLD + 4 * c) = xr[i];
            }
        }
        float wv[16];
        if constexpr (FMT == kFmtQ4) {
            const float s = half_bits_to_float(q4pair & 0xffffu);
            const float m = half_bits_to_float(q4pair >> 16);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                wv[j] = fmaf(static_cast<float>(nibble(q4bits.x, j)), s, m);
                wv[8 + j] = fmaf(static_cast<float>(nibble(q4bits.y, j)), s, m);
            }
        } else if constexpr (SAFE) {
#pragma unroll
            for (int j = 0; j < 16; ++j) wv[j] = FMT == kFmtQ8 ? wsafe[j] * wscale : wsafe[j];
        } else {
            const uint32_t words[4] = {q8bits.x, q8bits.y, q8bits.z, q8bits.w};
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float c = code8_value<FMT>(words[j >> 2] >> (8 * (j & 3)));
                wv[j] = FMT == kFmtQ8 ? c * wscale : c;
            }
        }
        float* wd = ws[buf] + wr * kLD + wh * 16;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4*>(wd + 4 * j) = make_float4(wv[4 * j], wv[4 * j + 1], wv[4 * j + 2], wv[4 * j + 3]);
    };

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // MFMA 16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16]. The four
    // lane groups c = l/16 take the physical k = 8c + kk at step kk, the same
    // permutation for x and W, so each lane reads 8 consecutive k from LDS.
    const int li = lane & 15;
    const int kq = (lane >> 4) * 8;
    auto compute = [&](int buf) {
        const float* xsrc = xs[buf];
        const float* wsrc = ws[buf];
        float xa[TM][8];
        float wb[TN][8];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const float* p = xsrc + (wm * TM * 16 + tm * 16 + li) * kLD + kq;
            const float4 v0 = *reinterpret_cast<const float4*>(p);
            const float4 v1 = *reinterpret_cast<const float4*>(p + 4);
            xa[tm][0] = v0.x; xa[tm][1] = v0.y; xa[tm][2] = v0.z; xa[tm][3] = v0.w;
            xa[tm][4] = v1.x; xa[tm][5] = v1.y; xa[tm][6] = v1.z; xa[tm][7] = v1.w;
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const float* p = wsrc + (wn * TN * 16 + tn * 16 + li) * kLD + kq;
            const float4 v0 = *reinterpret_cast<const float4*>(p);
            const float4 v1 = *reinterpret_cast<const float4*>(p + 4);
            wb[tn][0] = v0.x; wb[tn][1] = v0.y; wb[tn][2] = v0.z; wb[tn][3] = v0.w;
            wb[tn][4] = v1.x; wb[tn][5] = v1.y; wb[tn][6] = v1.z; wb[tn][7] = v1.w;
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[tm][kk], wb[tn][kk], acc[tm][tn], 0, 0, 0);
    };

    load(0);
    commit(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) load(kt + 1);
        compute(kt & 1);
        if (more) commit((kt + 1) & 1);
        __syncthreads();
    }

    // Epilogue. Lane l holds D[4*(l/16) + r][l%16] of each 16x16 tile.
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int col = n0 + wn * TN * 16 + tn * 16 + li;
        if (col >= N) continue;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * TM * 16 + tm * 16 + 4 * (lane >> 4) + r;
                if (row < M) {
                    a.y[static_cast<int64_t>(row) * N + col] = acc[tm][tn][r];
                }
            }
        }
    }
}

template <int FMT, int WM, int WN, int TM, int TN, bool SAFE>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(TileArgs a, int tiles_n, int remap) {
    __shared__ __attribute__((aligned(16))) float smem[TileShape<WM, WN, TM, TN>::SMEM];
    int w = blockIdx.x;
    if (remap) w = xcd_remap(w, gridDim.x);
    gemm_tile<FMT, WM, WN, TM, TN, SAFE>(a, w / tiles_n, w % tiles_n, smem);
}

// ---------------------------------------------------------------------------
// Small-M streaming kernel (M <= 80). Every wave owns all TM*16 rows and TN*16
// output columns over one K chunk and loads both operands straight from global
// memory into registers, in MFMA operand layout: no LDS staging and no barrier
// in the main loop. The packed weights are read exactly once.
//
// K is walked in blocks of 128 (four int4 groups). In a block, lane group
// c = l/16 owns group 4b+c: at MFMA step t (0..31) it supplies k = 32(4b+c)+t,
// for x (A operand) and W (B operand) alike. So each lane fetches one 16-byte
// run of packed codes and one (scale, min) pair per column tile per block and
// dequantizes with its own group's pair, and each x row is read as 32
// consecutive floats per lane.
//
// A workgroup is 4 waves: 4/KS column slices x KS K-chunks. With KS > 1 the
// chunk partials are summed through LDS in a fixed order (deterministic).
// ---------------------------------------------------------------------------
constexpr int kStreamTN = 4;

template <int FMT, int TM, int TN>
__device__ __forceinline__ void stream_tile(const TileArgs& a, int slice, int n_slices, int ks, int chunk,
                                            float* red) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15;
    const int lc = lane >> 4;
    const int M = a.M, N = a.N, K = a.K;
    const int G = K / 32;                          // 32-wide groups along K
    const int g_lo = chunk * G / ks;
    const int g_hi = (chunk + 1) * G / ks;
    const bool valid = slice < n_slices;
    const int n0 = slice * TN * 16;

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (valid) {
        // Out-of-range rows/columns read a clamped in-bounds row (their results
        // are never stored); groups past the chunk read a clamped group of the
        // same row and contribute zero through a zeroed weight. No load is
        // predicated, so the loop body has no branches.
        const float* xp[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int row = min(tm * 16 + li, M - 1);
            xp[tm] = a.x + static_cast<int64_t>(row) * K;
        }
        const uint8_t* wp[TN];
        const uint32_t* pp[TN];
        float qsc[TN];                          // int8 row scale of the lane's W row
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int col = min(n0 + tn * 16 + li, N - 1);
            qsc[tn] = FMT == kFmtQ8 ? static_cast<const float*>(a.scale)[col] : 1.0f;
            if constexpr (FMT == kFmtQ4) {
                wp[tn] = static_cast<const uint8_t*>(a.payload) + static_cast<int64_t>(col) * (K / 2);
                pp[tn] = static_cast<const uint32_t*>(a.scale) + static_cast<int64_t>(col) * G;
            } else {
                wp[tn] = reinterpret_cast<const uint8_t*>(static_cast<const int8_t*>(a.payload) + static_cast<int64_t>(col) * K);
                pp[tn] = nullptr;
            }
        }

        // Weight registers for one 128-k block: int4 -> 4 dwords + pair; int8 -> 8 dwords.
        constexpr int WD = FMT == kFmtQ4 ? 4 : 8;
        uint32_t wcur[TN][WD], wnxt[TN][WD];
        uint32_t pcur[TN], pnxt[TN];

        auto load_w = [&](int gblk, uint32_t (&wd)[TN][WD], uint32_t (&pr)[TN]) {
            const int g = gblk + lc;
            const bool live = g < g_hi;
            const int gc = live ? g : g_hi - 1;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                if constexpr (FMT == kFmtQ4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(wp[tn] + gc * 16);
                    const uint32_t p = pp[tn][gc];
                    wd[tn][0] = v.x; wd[tn][1] = v.y; wd[tn][2] = v.z; wd[tn][3] = v.w;
                    pr[tn] = live ? p : 0u;           // (scale, min) = (0, 0): contributes 0
                } else {
                    const uint4* q = reinterpret_cast<const uint4*>(wp[tn] + gc * 32);
                    const uint4 v0 = q[0];
                    const uint4 v1 = q[1];
                    wd[tn][0] = live ? v0.x : 0u; wd[tn][1] = live ? v0.y : 0u;
                    wd[tn][2] = live ? v0.z : 0u; wd[tn][3] = live ? v0.w : 0u;
                    wd[tn][4] = live ? v1.x : 0u; wd[tn][5] = live ? v1.y : 0u;
                    wd[tn][6] = live ? v1.z : 0u; wd[tn][7] = live ? v1.w : 0u;
                    pr[tn] = 0;
                }
            }
        };
        // x for steps 8u..8u+7 of the block starting at group gblk.
        auto load_x = [&](int gblk, int u, float (&xa)[TM][8]) {
            const int g = min(gblk + lc, g_hi - 1);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const float4* p = reinterpret_cast<const float4*>(xp[tm] + g * 32 + 8 * u);
                const float4 v0 = p[0];
                const float4 v1 = p[1];
                xa[tm][0] = v0.x; xa[tm][1] = v0.y; xa[tm][2] = v0.z; xa[tm][3] = v0.w;
                xa[tm][4] = v1.x; xa[tm][5] = v1.y; xa[tm][6] = v1.z; xa[tm][7] = v1.w;
            }
        };
        auto compute = [&](int u, const float (&xa)[TM][8], const uint32_t (&wd)[TN][WD], const uint32_t (&pr)[TN]) {
            float s[TN], m[TN];
            if constexpr (FMT == kFmtQ4) {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    s[tn] = half_bits_to_float(pr[tn] & 0xffffu);
                    m[tn] = half_bits_to_float(pr[tn] >> 16);
                }
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int step = 8 * u + t;      // 0..31 within the group
                float b[TN];
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    if constexpr (FMT == kFmtQ4) {
                        b[tn] = fmaf(static_cast<float>(nibble(wd[tn][step >> 3], step & 7)), s[tn], m[tn]);
                    } else if constexpr (FMT == kFmtQ8) {
                        b[tn] = code8_value<FMT>(wd[tn][step >> 2] >> (8 * (step & 3))) * qsc[tn];
                    } else {
                        b[tn] = code8_value<FMT>(wd[tn][step >> 2] >> (8 * (step & 3)));
                    }
                }
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[tm][t], b[tn], acc[tm][tn], 0, 0, 0);
            }
        };

        float xa0[TM][8], xa1[TM][8];
        load_w(g_lo, wcur, pcur);
        load_x(g_lo, 0, xa0);
        for (int gb = g_lo; gb < g_hi; gb += 4) {
            // Prefetch the next block unconditionally (clamped past the end).
            load_w(gb + 4, wnxt, pnxt);
            load_x(gb, 1, xa1);
            compute(0, xa0, wcur, pcur);
            load_x(gb, 2, xa0);
            compute(1, xa1, wcur, pcur);
            load_x(gb, 3, xa1);
            compute(2, xa0, wcur, pcur);
            load_x(gb + 4, 0, xa0);
            compute(3, xa1, wcur, pcur);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                for (int i = 0; i < WD; ++i) wcur[tn][i] = wnxt[tn][i];
                pcur[tn] = pnxt[tn];
            }
        }
    }

    if (ks > 1) {
        // Chunk partials -> LDS, then chunk 0 adds chunks 1..ks-1 in order.
        constexpr int R = TM * TN * 4;
        if (chunk != 0) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[(wave * R + (tm * TN + tn) * 4 + r) * 64 + lane] = acc[tm][tn][r];
        }
        __syncthreads();
        if (chunk != 0) return;
        for (int c = 1; c < ks; ++c) {
            const int src = wave + c;         // waves of one slice are consecutive
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[tm][tn][r] += red[(src * R + (tm * TN + tn) * 4 + r) * 64 + lane];
        }
    }
    if (!valid) return;

#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int col = n0 + tn * 16 + li;
        if (col >= N) continue;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = tm * 16 + 4 * lc + r;
                if (row < M) {
                    a.y[static_cast<int64_t>(row) * N + col] = acc[tm][tn][r];
                }
            }
        }
    }
}

// Number of K chunks for a projection: about 512 of K per wave, at most 4.
__host__ __device__ inline int stream_ks(int K) {
    const int G = K / 32;
    return G >= 64 ? 4 : (G >= 32 ? 2 : 1);
}

// Kernel arguments of a grouped launch, laid out as arrays so that the 96
// projections of a 12-block RT-J pass fit in one launch under the 4 KiB
// kernel-argument budget. Inputs are deduplicated into a small table (the
// projections of a block share four of them).
constexpr int kMaxInputs = 48;

struct GroupArgs {
    int count;                        // projections in this launch
    int M;
    int n_inputs;
    int total_tiles;
    const float* xs[kMaxInputs];
    int xk[kMaxInputs];               // K of each input
    const void* payload[kMaxGrouped];
    const void* scale[kMaxGrouped];
    float* y[kMaxGrouped];
    int n[kMaxGrouped];
    int tile_begin[seg_begin_slots(kMaxGrouped)];
    int tile_coarse[seg_coarse_slots(kMaxGrouped)];
    uint8_t x_idx[kMaxGrouped];
    uint8_t fmt[kMaxGrouped];
};
static_assert(sizeof(GroupArgs) <= 4096, "kernel arguments must stay within 4 KiB");

template <int TM>
__global__ __launch_bounds__(256) void grouped_stream_kernel(GroupArgs g) {
    __shared__ __attribute__((aligned(16))) float red[4 * TM * kStreamTN * 4 * 64];
    const int w = blockIdx.x;
    const int i = segment_of(g.tile_begin, g.tile_coarse, g.count, w);
    const int xi = g.x_idx[i];
    const int N = g.n[i];
    const int K = g.xk[xi];
    const int ks = stream_ks(K);
    const int per_wg = 4 / ks;                                  // column slices per workgroup
    const int n_slices = (N + kStreamTN * 16 - 1) / (kStreamTN * 16);
    const int wave = threadIdx.x >> 6;
    const int slice = (w - g.tile_begin[i]) * per_wg + wave / ks;
    const int chunk = wave % ks;
    const TileArgs a{g.xs[xi], g.payload[i], g.scale[i], g.y[i], g.M, N, K};
    if (g.fmt[i] == kFmtQ4)
        stream_tile<kFmtQ4, TM, kStreamTN>(a, slice, n_slices, ks, chunk, red);
    else if (g.fmt[i] == kFmtQ8)
        stream_tile<kFmtQ8, TM, kStreamTN>(a, slice, n_slices, ks, chunk, red);
    else
        stream_tile<kFmtF8, TM, kStreamTN>(a, slice, n_slices, ks, chunk, red);
}

template <int FMT, bool SAFE>
hipError_t launch_one_untimed(const TileArgs& a, hipStream_t stream);

// Tile configurations: small M keeps all rows in one tile and splits N over
// four waves; large M uses 128x128 tiles on a 2x2 wave grid.
using Small = TileShape<1, 4, 5, 2>;
using Large = TileShape<2, 2, 4, 4>;
constexpr int kSmallMaxM = Small::BM;

template <int FMT, bool SAFE>
hipError_t launch_one(const TileArgs& a, hipStream_t stream) {
    const int mark = timing_begin(stream);
    const hipError_t e = launch_one_untimed<FMT, SAFE>(a, stream);
    timing_end(mark, stream);
    return e;
}

template <int FMT, bool SAFE>
hipError_t launch_one_untimed(const TileArgs& a, hipStream_t stream) {
    if (a.M <= kSmallMaxM) {
        const int tn = (a.N + Small::BN - 1) / Small::BN;
        const int tm = (a.M + Small::BM - 1) / Small::BM;
        gemm_kernel<FMT, 1, 4, 5, 2, SAFE><<<tm * tn, Small::NT, 0, stream>>>(a, tn, 0);
    } else {
        const int tn = (a.N + Large::BN - 1) / Large::BN;
        const int tm = static_cast<int>((int64_t(a.M) + Large::BM - 1) / Large::BM);
        gemm_kernel<FMT, 2, 2, 4, 4, SAFE><<<tm * tn, Large::NT, 0, stream>>>(a, tn, 1);
    }
    return hipGetLastError();
}

}  // namespace

bool grouped_ok(const ProjTask& t) {
    // Vector loads need whole 32-wide K steps and 16-byte aligned rows.
    return t.K % kBK == 0 && (reinterpret_cast<uintptr_t>(t.x) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(t.payload) & 15) == 0;
}

hipError_t launch_gemm(const ProjTask& t, int64_t M, int math, hipStream_t stream) {
    const TileArgs a{t.x, t.payload, t.scale, t.y, static_cast<int>(M), t.N, t.K};
    const bool safe = !grouped_ok(t);
    const int nl = split_limbs(math);
    if (!safe && nl && split_ok(t)) return launch_split(&t, 1, M, nl, stream);
    if (!safe && M <= kSmallMaxM) return launch_grouped(&t, 1, M, kMathFp32Mfma, stream);
    hipError_t e;
    if (t.fmt == kFmtQ4) e = launch_one<kFmtQ4, false>(a, stream);
    else if (t.fmt == kFmtQ8) e = safe ? launch_one<kFmtQ8, true>(a, stream) : launch_one<kFmtQ8, false>(a, stream);
    else e = safe ? launch_one<kFmtF8, true>(a, stream) : launch_one<kFmtF8, false>(a, stream);
    if (e == hipSuccess && t.bias) e = launch_bias_add(&t, 1, M, stream);
    return e;
}

namespace {

hipError_t launch_grouped_fp32(const ProjTask* tasks, int count, int64_t M, hipStream_t stream) {
    if (M > kSmallMaxM) {
        // Many row tiles: every projection alone already fills the GPU; one
        // launch each keeps the XCD-contiguous tile order. Biases are left
        // to the caller (launch_grouped_fp32_bias).
        for (int i = 0; i < count; ++i) {
            ProjTask t = tasks[i];
            t.bias = nullptr;
            const hipError_t e = launch_gemm(t, M, kMathFp32Mfma, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // Small M: all projections in one launch (or as few as the argument
    // budget allows), longest K first so the long tiles start early.
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
        GroupArgs g{};
        g.M = static_cast<int>(M);
        int tiles = 0;
        while (done < count && g.count < kMaxGrouped) {
            const ProjTask& t = tasks[order[done]];
            int xi = -1;
            for (int k = 0; k < g.n_inputs; ++k)
                if (g.xs[k] == t.x && g.xk[k] == t.K) xi = k;
            if (xi < 0) {
                if (g.n_inputs == kMaxInputs) break;
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
            const int ks = stream_ks(t.K);
            const int n_slices = (t.N + kStreamTN * 16 - 1) / (kStreamTN * 16);
            tiles += (n_slices + 4 / ks - 1) / (4 / ks);
            ++done;
        }
        g.total_tiles = tiles;
        seg_fill_coarse(g.tile_begin, g.tile_coarse, g.count);
        const int tm = static_cast<int>((M + 15) / 16);
        const int mark = timing_begin(stream);
        switch (tm) {
            case 1: grouped_stream_kernel<1><<<tiles, 256, 0, stream>>>(g); break;
            case 2: grouped_stream_kernel<2><<<tiles, 256, 0, stream>>>(g); break;
            case 3: grouped_stream_kernel<3><<<tiles, 256, 0, stream>>>(g); break;
            case 4: grouped_stream_kernel<4><<<tiles, 256, 0, stream>>>(g); break;
            default: grouped_stream_kernel<5><<<tiles, 256, 0, stream>>>(g); break;
        }
        timing_end(mark, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_grouped_fp32_bias(const ProjTask* tasks, int count, int64_t M, hipStream_t stream) {
    // The fp32 grouped kernels write y; the biases follow in one pass.
    const hipError_t e = launch_grouped_fp32(tasks, count, M, stream);
    return e == hipSuccess ? launch_bias_add(tasks, count, M, stream) : e;
}

int64_t grouped_workspace_bytes(const ProjTask* tasks, int count, int64_t M, int math) {
    const int nl = split_limbs(math);
    if (!nl) return 0;
    thread_local std::vector<ProjTask> split_buf(8 * 64);
    if (count > static_cast<int>(split_buf.size())) return -1;
    int n_split = 0;
    for (int i = 0; i < count; ++i)
        if (split_ok(tasks[i])) split_buf[n_split++] = tasks[i];
    return split_workspace_bytes(split_buf.data(), n_split, M, nl);
}

hipError_t launch_grouped(const ProjTask* tasks, int count, int64_t M, int math, hipStream_t stream, WsMode mode,
                          unsigned char* ws, int64_t cap) {
    const int nl = split_limbs(math);
    if (!nl) return launch_grouped_fp32_bias(tasks, count, M, stream);
    // Split path for every task it takes; the rest (weights past 32-bit
    // offsets) run on the fp32 kernels.
    thread_local std::vector<ProjTask> split_buf(8 * 64), rest_buf(8 * 64);
    if (count > static_cast<int>(split_buf.size())) return hipErrorInvalidValue;
    ProjTask* split = split_buf.data();
    ProjTask* rest = rest_buf.data();
    int n_split = 0, n_rest = 0;
    for (int i = 0; i < count; ++i) {
        if (split_ok(tasks[i])) split[n_split++] = tasks[i];
        else rest[n_rest++] = tasks[i];
    }
    if (n_split) {
        const hipError_t e = mode == kWsScratch ? launch_split_scratch(split, n_split, M, nl, stream)
                             : mode == kWsCaller ? launch_split_ws(split, n_split, M, nl, stream, ws, cap)
                                                 : launch_split(split, n_split, M, nl, stream);
        if (e != hipSuccess) return e;
    }
    return n_rest ? launch_grouped_fp32_bias(rest, n_rest, M, stream) : hipSuccess;
}

}  // namespace rtq
