// Small-M projections (M <= 32) in one launch, without a pre-pass or K chunks.
//
// y[M][N] = x[M][K] . W^T for every projection of a call, W packed as int4,
// int8 or FP8 (RT-J model cards, section "Quantization format"; RT-J FP8 card,
// section "FP8 Format"), with the arithmetic of the split-limb path: x split
// exactly into bf16 limbs (three, or one bf16-rounded limb), weight codes exact
// in bf16, v_mfma_f32_16x16x32_bf16 accumulating in fp32, the int4 scale as one
// fp32 FMA per output and group and the int4 min term on the fp32 matrix cores.
//
// One workgroup (4 waves) covers 64 * tn output columns of one projection over
// the whole K, and its TM row tiles (TM = 1 or 2: 16 rows each, rows >= M
// zero). tn = 4, 2, 1 for K = 512, 1024, 2048 (256 also takes 4), so every wave
// streams the same number of weight bytes whatever the projection.
//  - x: the workgroup builds its x stages itself from the fp32 activation, one
//    phase of PG groups at a time (PG = 8 for one row tile, 4 for two, 24 KB
//    of limbs either way), into a double-buffered LDS area, one barrier per
//    phase. Thread (h, j, kp) takes k = 2kp, 2kp+1 of group j of the phase for
//    the rows h, h + RS, h + 2RS, ... below M, splits (or rounds) them, writes
//    the limbs in MFMA operand order and sums the group over its 16 lanes with
//    DPP row rotations (the int4 min term needs X_g). Rows >= M stay zero.
//  - weights: each wave loads its own rows into registers in blocks of 4
//    groups, 16 bytes per lane and load, a few blocks ahead (direct_db) in a
//    statically indexed ring. int4: lane lc loads group 4b + lc of its row whole, plus
//    that group's (scale, min) word; the 4 lanes of a row exchange words
//    through a private LDS area of the wave (word w of group j goes to lane w,
//    which feeds it to the MFMA of group j). int8/FP8: lane lc loads bytes
//    16lc.. and 64 + 16lc.. of the block and the MFMAs contract k in that
//    order; x is read from the matching places, so no exchange is needed.
//  - the codes of a group are converted to bf16 once and serve all TM row tiles.
// The K loop is unrolled completely (K fixed per instantiation), so the
// compiler tracks every load and waits only for the group it uses; the x reads
// of the next row tile or group are issued before the MFMAs of the current one.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "rtq_internal.h"
#include "split_device.h"

namespace rtq {

namespace {

constexpr int kDirectMaxTM = 2;             // 32 rows
constexpr int kDirectMaxProj = 96;          // projections per launch (argument block)
constexpr int kDirectMaxInputs = 48;        // distinct activations per launch
constexpr int kDirectMaxTiles = 1 << 30;    // workgroups per launch
constexpr int kSumSlots = 16;               // ring of group sums X_g (4 blocks)

// Row tiles for M rows.
__host__ __device__ constexpr int direct_tm(int M) { return M <= 16 ? 1 : 2; }
// Groups per x phase.
__host__ __device__ constexpr int direct_pg(int TM) { return TM == 1 ? 8 : 4; }
// Column tiles of 16 per wave: 4, 2, 1 for K <= 512, 1024, 2048, so every wave
// streams about the same weight bytes.
__host__ __device__ constexpr int direct_tn(int K) { return K <= 512 ? 4 : K <= 1024 ? 2 : 1; }
// Weight blocks (4 groups) in flight per wave: about the same bytes at every tn.
__host__ __device__ constexpr int direct_db(int TN) { return TN >= 4 ? 1 : 4 / TN; }
// K values with an instantiation.
__host__ __device__ constexpr bool direct_k(int K) { return K == 256 || K == 512 || K == 1024 || K == 2048; }

// f(std::integral_constant<int, i>) for i = B .. E-1, expanded at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int NL, int TM>
struct DirectLds {
    static constexpr int PG = direct_pg(TM);
    static constexpr int GBYTES = TM * NL * 1024;       // one group: TM row tiles x NL limbs of 1 KB
    static constexpr int XBUF = PG * GBYTES;            // one phase
    static constexpr int SUMS = kSumSlots * 16 * TM * 4;
    static constexpr int XTOTAL = 2 * XBUF + SUMS;
    // per-wave int4 staging: 16 rows of 4 x 16 bytes of codes (+ 16 bytes of
    // padding); two areas, used by alternate column tiles
    static constexpr int STG_ROW = 80;
    static constexpr int STG_TILE = 16 * STG_ROW;
    static constexpr int STG_AREAS = 2;
    static constexpr int STG = STG_AREAS * STG_TILE;
    // per-wave int4 (scale, min) words of every column tile for the whole K,
    // rows padded by 16 bytes: at most 4 tiles x 16 rows x (16 + 4) words
    // (tn * K / 32 is at most 64 words per row)
    static constexpr int PAIRS = 4 * 16 * 80;
    static constexpr int TOTAL = XTOTAL + 4 * STG + 4 * PAIRS;
};

template <int FMT, int TN, int NL, int G, int TM>
__device__ __forceinline__ void direct_tile(const float* __restrict__ x, const void* payload_v, const void* scale_v,
                                            float* __restrict__ y, int M, int N, int n0, unsigned char* smem) {
    using L = DirectLds<NL, TM>;
    constexpr int PG = L::PG;
    static_assert(G % PG == 0 && G % 4 == 0, "whole phases and whole blocks");
    constexpr int NPH = G / PG;
    constexpr int K = G * 32;
    constexpr int LPG = PG == 8 ? 3 : 2;
    constexpr int RS = 256 / (16 * PG);                 // rows staged side by side
    constexpr int NR = 16 * TM / RS;                    // rows per thread at most
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lc = lane >> 4;

    // ---- x stages ----
    const int kp = tid & 15;                            // k pair 2kp, 2kp+1 (one DPP row of 16 lanes)
    const int xj = (tid >> 4) & (PG - 1);               // group of the phase
    const int xh = tid >> (4 + LPG);                    // first row
    const int nrows = M > xh ? (M - xh + RS - 1) / RS : 0;
    const float* xcol = x + xh * static_cast<int64_t>(K) + xj * 32 + 2 * kp;
    float2 xr[NR];
    auto x_load = [&](int ph) {
#pragma unroll
        for (int t = 0; t < NR; ++t)
            if (t < nrows)
                xr[t] = *reinterpret_cast<const float2*>(xcol + static_cast<int64_t>(RS * t) * K + ph * (PG * 32));
    };
    auto x_convert = [&](int ph) {
        unsigned char* buf = smem + (ph & 1) * L::XBUF + xj * L::GBYTES + (kp & 3) * 4;
        float* sums = reinterpret_cast<float*>(smem + 2 * L::XBUF) + ((ph * PG + xj) % kSumSlots) * (16 * TM);
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            if (t >= nrows) break;
            const int r = xh + RS * t;
            float v0 = xr[t].x, v1 = xr[t].y;
            unsigned char* blk = buf + (r >> 4) * (NL * 1024) + swz(r & 15, kp >> 2) * 16;
            if constexpr (NL == 3) {
                uint32_t h, m, l;
                split2(v0, v1, h, m, l);
                *reinterpret_cast<uint32_t*>(blk) = h;
                *reinterpret_cast<uint32_t*>(blk + 1024) = m;
                *reinterpret_cast<uint32_t*>(blk + 2048) = l;
            } else {
                const uint32_t h = bf16x2_rne(v0, v1);
                *reinterpret_cast<uint32_t*>(blk) = h;
                v0 = bitsf(h << 16);                        // the sum is over the rounded values
                v1 = bitsf(h & 0xffff0000u);
            }
            // sum over the 16 lanes of the (row, group) (one DPP row); lane kp = 0 holds it
            float sum = v0 + v1;
            sum += row_ror<8>(sum);
            sum += row_ror<4>(sum);
            sum += row_ror<2>(sum);
            sum += row_ror<1>(sum);
            if (kp == 0) sums[r] = sum;
        }
    };
    auto lds_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xc07f);             // this wave's LDS writes done (lgkmcnt(0))
        __builtin_amdgcn_s_barrier();
    };

    // ---- weights: lane (li, lc) of tile tn holds column n0 + wave*TN*16 + tn*16 + li ----
    // Addressed as the (uniform) base plus a 32-bit byte offset per tile: the
    // path takes weights below 2^32 bytes (N*K < 2^32).
    const unsigned char* payload = static_cast<const unsigned char*>(payload_v);
    const unsigned char* pairs = static_cast<const unsigned char*>(scale_v);
    uint32_t woff[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const uint32_t col = static_cast<uint32_t>(min(n0 + wave * TN * 16 + tn * 16 + li, N - 1));
        if constexpr (FMT == kFmtQ4) woff[tn] = col * (K / 2) + 16 * lc;
        else woff[tn] = col * K + 16 * lc;
    }
    constexpr int NB = G / 4;                                    // blocks of 4 groups
    constexpr int CW = FMT == kFmtQ4 ? 4 : 8;                    // code words per lane and block
    constexpr int DB = direct_db(TN) < NB ? direct_db(TN) : NB;   // blocks in flight
    uint32_t bc[DB][TN][CW], bp[DB][TN];
    auto b_issue = [&](int b, uint32_t (&c)[TN][CW], uint32_t (&pr)[TN]) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if constexpr (FMT == kFmtQ4) {
                const uint4 v = *reinterpret_cast<const uint4*>(payload + woff[tn] + b * 64);
                c[tn][0] = v.x; c[tn][1] = v.y; c[tn][2] = v.z; c[tn][3] = v.w;
                pr[tn] = 0;
            } else {
                const uint4 v0 = *reinterpret_cast<const uint4*>(payload + woff[tn] + b * 128);
                const uint4 v1 = *reinterpret_cast<const uint4*>(payload + woff[tn] + b * 128 + 64);
                c[tn][0] = v0.x; c[tn][1] = v0.y; c[tn][2] = v0.z; c[tn][3] = v0.w;
                c[tn][4] = v1.x; c[tn][5] = v1.y; c[tn][6] = v1.z; c[tn][7] = v1.w;
                pr[tn] = 0;
            }
        }
    };
    // int4 (scale, min) words: every column tile's rows for the whole K, read
    // once in contiguous 16-byte pieces (a tile's rows are consecutive in the
    // pair array) into this wave's area, row r of tile tn at
    // tn * 16 * PROW + r * PROW (PROW = 4G + 16 bytes); b_stage reads the
    // block's four words of its row from there.
    constexpr int PROW = 4 * G + 16;
    static_assert(TN * 16 * PROW <= L::PAIRS, "pair area");
    unsigned char* pair_area = smem + L::XTOTAL + 4 * L::STG + wave * L::PAIRS;
    const unsigned char* pair_row = pair_area + li * PROW;
    constexpr int PTILE = 16 * 4 * G;                          // bytes of a tile's 16 rows of words
    constexpr int PIECES = FMT == kFmtQ4 ? (PTILE + 1023) / 1024 : 0;   // 16-byte loads per lane and tile
    uint4 pv[TN][PIECES > 0 ? PIECES : 1];
    auto pairs_issue = [&]() {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int col0 = n0 + wave * TN * 16 + tn * 16;
#pragma unroll
            for (int i = 0; i < PIECES; ++i) {
                // byte of the tile's block; lanes past it (K = 256) load the
                // first piece again, so that no branch surrounds the load (a
                // load under a branch kept the pieces in scratch memory)
                const int o0 = i * 1024 + lane * 16;
                const int o = o0 < PTILE ? o0 : o0 - PTILE;
                const int r = o / (4 * G), w = o - r * (4 * G);
                const uint32_t row = static_cast<uint32_t>(min(col0 + r, N - 1));
                pv[tn][i] = *reinterpret_cast<const uint4*>(pairs + row * (4u * G) + w);
            }
        }
    };
    auto pairs_store = [&]() {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int i = 0; i < PIECES; ++i) {
                const int o = i * 1024 + lane * 16;
                if (o < PTILE) {
                    const int r = o / (4 * G), w = o - r * (4 * G);
                    *reinterpret_cast<uint4*>(pair_area + tn * (16 * PROW) + r * PROW + w) = pv[tn][i];
                }
            }
    };

    // Operand words of the block's 4 MFMAs (wq[tn][j] for group 4b + j) and, for
    // int4, its (scale, min) words. A staging area is rewritten (two tiles or a
    // block later) only after this wave's reads of it: one wave's LDS operations
    // run in order, so no barrier is needed.
    unsigned char* stg = smem + L::XTOTAL + wave * L::STG + li * L::STG_ROW;
    auto b_stage = [&](int b, const uint32_t (&c)[TN][CW], const uint32_t (&pr)[TN], uint32_t (&wq)[TN][4][2],
                       uint32_t (&pq)[TN][4]) {
        (void)pr;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if constexpr (FMT == kFmtQ4) {
                unsigned char* t = stg + (tn % L::STG_AREAS) * L::STG_TILE;
#pragma unroll
                for (int w = 0; w < 4; ++w) *reinterpret_cast<uint32_t*>(t + w * 16 + lc * 4) = c[tn][w];
                const u32x4 r = *reinterpret_cast<const u32x4*>(t + lc * 16);
                const u32x4 q = *reinterpret_cast<const u32x4*>(pair_row + tn * (16 * PROW) + b * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wq[tn][j][0] = r[j];
                    wq[tn][j][1] = 0;
                    pq[tn][j] = q[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wq[tn][j][0] = c[tn][2 * j];
                    wq[tn][j][1] = c[tn][2 * j + 1];
                    pq[tn][j] = 0;
                }
            }
        }
    };

    // int8/FP8 accumulate every group into their tile's accumulator; narrow waves
    // with one row tile spread the groups over NA accumulators so consecutive
    // MFMAs do not wait on each other, and add them up at the end (with two row
    // tiles the MFMAs of a group already alternate between accumulators).
    constexpr int NA = FMT == kFmtQ4 || TM > 1 ? 1 : 4 / TN;
    floatx4 acc[TM][TN][NA];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int a = 0; a < NA; ++a) acc[tm][tn][a] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mreg[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) mreg[tn] = 0.0f;
    const int aoff = swz(li, lc) * 16;
    // int8/FP8: the k of lane lc in the MFMA j of a block lie in group 2(j >> 1) + (lc >> 1)
    // of the block, at lane place 2(lc & 1) + (j & 1)
    int aoff8[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) aoff8[h] = (lc >> 1) * L::GBYTES + swz(li, 2 * (lc & 1) + h) * 16;

    // x limbs (high, mid, low) of row tile tm of group g
    auto x_read = [&](int g, int tm, u32x4 (&xv)[NL]) {
        const int ph = g / PG;
        const unsigned char* blk;
        if constexpr (FMT == kFmtQ4)
            blk = smem + (ph & 1) * L::XBUF + (g % PG) * L::GBYTES + tm * (NL * 1024) + aoff;
        else
            blk = smem + (ph & 1) * L::XBUF + ((g & ~1) % PG) * L::GBYTES + tm * (NL * 1024) + aoff8[g & 1];
#pragma unroll
        for (int l = 0; l < NL; ++l) xv[l] = *reinterpret_cast<const u32x4*>(blk + l * 1024);
    };
    // Group g, row tile tm. The first row tile converts the group's codes of
    // each column tile into bop (next to its MFMAs, so the conversions overlap
    // them) and reads the int4 scale and min; later row tiles reuse them.
    auto compute_tm = [&](int g, int tm, const u32x4 (&xv)[NL], const uint32_t (&wq)[TN][4][2],
                          const uint32_t (&pq)[TN][4], u32x4 (&bop)[TN], float (&sc)[TN]) {
        const int jb = g & 3;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if (tm == 0) {
                if constexpr (FMT == kFmtQ4) {
                    bop[tn] = codes4_to_bf16(wq[tn][jb][0]);
                    sc[tn] = half_bits_to_float(pq[tn][jb] & 0xffffu);
                    const float mn = half_bits_to_float(pq[tn][jb] >> 16);
                    mreg[tn] = lc == jb ? mn : mreg[tn];
                } else {
                    if constexpr (FMT == kFmtF8) bop[tn] = codes8f_to_bf16(wq[tn][jb][0], wq[tn][jb][1]);
                    else bop[tn] = codes8_to_bf16(wq[tn][jb][0], wq[tn][jb][1]);
                    sc[tn] = 1.0f;
                }
            }
            if constexpr (FMT == kFmtQ4) {
                floatx4 p = floatx4{0.f, 0.f, 0.f, 0.f};
                if constexpr (NL == 3) {
                    p = mfma_bf16(xv[2], bop[tn], p);
                    p = mfma_bf16(xv[1], bop[tn], p);
                }
                p = mfma_bf16(xv[0], bop[tn], p);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[tm][tn][0][e] = fmaf(sc[tn], p[e], acc[tm][tn][0][e]);
            } else {
                floatx4& a = acc[tm][tn][g % NA];
                if constexpr (NL == 3) {
                    a = mfma_bf16(xv[2], bop[tn], a);
                    a = mfma_bf16(xv[1], bop[tn], a);
                }
                a = mfma_bf16(xv[0], bop[tn], a);
            }
        }
    };

    // ---- prologue: zero both x areas and the sums (rows >= M stay zero), load
    //      phase 0 of x and the int4 pair words, start the weights, stage both ----
    {
        uint4* z = reinterpret_cast<uint4*>(smem);
        for (int t = tid; t < L::XTOTAL / 16; t += 256) z[t] = make_uint4(0u, 0u, 0u, 0u);
    }
    lds_barrier();
    x_load(0);
    pairs_issue();
#pragma unroll
    for (int b = 0; b < DB; ++b) b_issue(b, bc[b], bp[b]);
    pairs_store();
    x_convert(0);
    lds_barrier();
    u32x4 xcur[NL];
    x_read(0, 0, xcur);
    uint32_t wq[TN][4][2], pq[TN][4];

    // ---- main loop, unrolled over the groups at compile time (static_for: a
    //      #pragma unroll gives up on the longest K). Block b (groups 4b..4b+3)
    //      sits in ring slot b % DB, refilled with block b + DB once its codes are
    //      in operand order. The x of phase p + 1 is loaded when phase p starts
    //      and staged when it ends. ----
    static_for<0, G>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int ph = g / PG;
        constexpr int jb = g & 3;
        if (g % PG == 0 && ph + 1 < NPH) x_load(ph + 1);
        if (jb == 0) {
            constexpr int b = g / 4;
            b_stage(b, bc[b % DB], bp[b % DB], wq, pq);
            if (b + DB < NB) b_issue(b + DB, bc[b % DB], bp[b % DB]);
        }
        u32x4 bop[TN];
        float sc[TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            // read ahead: the next row tile, or the first of the next group in this phase
            const bool ahead = tm + 1 < TM || (g + 1) % PG != 0;
            u32x4 xnext[NL];
            if (ahead) x_read(tm + 1 < TM ? g : g + 1, tm + 1 < TM ? tm + 1 : 0, xnext);
            __builtin_amdgcn_sched_barrier(0);           // keep the reads ahead of these MFMAs
            compute_tm(g, tm, xcur, wq, pq, bop, sc);
            if (ahead) {
#pragma unroll
                for (int l = 0; l < NL; ++l) xcur[l] = xnext[l];
            }
        }
        // int4 min term of the block that g closes: sum over its 4 groups of X_g[row] * min_g[col]
        if constexpr (FMT == kFmtQ4) {
            if (jb == 3) {
                const float* sums = reinterpret_cast<const float*>(smem + 2 * L::XBUF);
                const float* srow = sums + (((g & ~3) + lc) % kSumSlots) * (16 * TM) + li;
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    const float xs = srow[16 * tm];
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        acc[tm][tn][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs, mreg[tn], acc[tm][tn][0], 0, 0, 0);
                }
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) mreg[tn] = 0.0f;
            }
        }
        if (g % PG == PG - 1) {
            if (ph + 1 < NPH) x_convert(ph + 1);
            lds_barrier();
            if (ph + 1 < NPH) x_read(g + 1, 0, xcur);   // first group of the next phase
        }
    });

    // ---- epilogue: lane holds D[4*lc + e][li] of each 16x16 tile ----
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int col = n0 + wave * TN * 16 + tn * 16 + li;
        if (col >= N) continue;
        float s = 1.0f;
        if constexpr (FMT == kFmtQ8) s = static_cast<const float*>(scale_v)[col];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int a = 1; a < NA; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[tm][tn][0][e] += acc[tm][tn][a][e];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * tm + 4 * lc + e;
                if (row < M) {
                    float v = acc[tm][tn][0][e];
                    if constexpr (FMT == kFmtQ8) v *= s;
                    y[static_cast<int64_t>(row) * N + col] = v;
                }
            }
        }
    }
}

// One projection of a direct launch: 32 bytes, read with one scalar load.
// Packed to 4-byte alignment (the pointers stay pointers, so the compiler
// still knows they address global memory).
struct __attribute__((packed, aligned(4))) DirectProj {
    const void* payload;
    const void* scale;
    float* y;
    int n;
    uint32_t k_fmt_x;                   // K | format << 16 | input index << 24
};
static_assert(sizeof(DirectProj) == 32, "direct descriptor layout");

struct DirectArgs {
    int count;
    int M;
    int tiles;                          // workgroups of the launch
    int pad;
    int tile_begin[seg_begin_slots(kDirectMaxProj)];    // first workgroup of each projection
    int tile_coarse[seg_coarse_slots(kDirectMaxProj)];
    const float* xs[kDirectMaxInputs];
    DirectProj proj[kDirectMaxProj];
};
static_assert(sizeof(DirectArgs) <= 4096, "kernel arguments must stay within 4 KiB");

template <int FMT, int NL, int TM>
__device__ __forceinline__ void direct_dispatch_k(int K, const float* x, const void* p, const void* s, float* y,
                                                  int M, int N, int n0, unsigned char* smem) {
    if (K == 512) direct_tile<FMT, direct_tn(512), NL, 16, TM>(x, p, s, y, M, N, n0, smem);
    else if (K == 2048) direct_tile<FMT, direct_tn(2048), NL, 64, TM>(x, p, s, y, M, N, n0, smem);
    else if (K == 1024) direct_tile<FMT, direct_tn(1024), NL, 32, TM>(x, p, s, y, M, N, n0, smem);
    else direct_tile<FMT, direct_tn(256), NL, 8, TM>(x, p, s, y, M, N, n0, smem);
}

template <int TM, int NL>
__global__ __launch_bounds__(256) void direct_kernel(DirectArgs g) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[DirectLds<NL, TM>::TOTAL];
    // Argument loads in four rounds: the header with the coarse table, the
    // run of the fine table it points at (which also holds the projection's
    // first workgroup), the projection's descriptor, its input pointer. Each
    // empty asm takes a round's values as scalar operands, so the compiler
    // issues that round's loads before its one wait (scalar loads return out
    // of order: any use waits for all of them).
    constexpr int NC = seg_coarse_slots(kDirectMaxProj);
    static_assert(NC == 12, "the round-one operand list below names twelve coarse slots");
    const int count = g.count, tiles = g.tiles, M = g.M;
    int coarse[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) coarse[j] = g.tile_coarse[j];
    asm volatile("" ::"s"(count), "s"(tiles), "s"(M), "s"(coarse[0]), "s"(coarse[1]), "s"(coarse[2]), "s"(coarse[3]),
                 "s"(coarse[4]), "s"(coarse[5]), "s"(coarse[6]), "s"(coarse[7]), "s"(coarse[8]), "s"(coarse[9]),
                 "s"(coarse[10]), "s"(coarse[11]));
    const int w = xcd_remap_split(blockIdx.x, tiles);
    int c = 0;
#pragma unroll
    for (int j = 1; j < NC; ++j) c += static_cast<int>(j * kSegStride < count) & static_cast<int>(coarse[j] <= w);
    c = __builtin_amdgcn_readfirstlane(c);
    asm volatile("" : "+s"(c));
    const int base = c * kSegStride;
    int run[kSegStride];
#pragma unroll
    for (int j = 0; j < kSegStride; ++j) run[j] = g.tile_begin[base + j];
    int i = base, begin = run[0];
#pragma unroll
    for (int j = 1; j < kSegStride; ++j) {
        const bool in = base + j < count && run[j] <= w;
        i += static_cast<int>(in);
        begin = in ? run[j] : begin;
    }
    i = __builtin_amdgcn_readfirstlane(i);
    asm volatile("" : "+s"(i));
    const DirectProj d = g.proj[i];
    const void* payload = d.payload;
    const void* scale = d.scale;
    float* y = d.y;
    const int N = d.n;
    const uint32_t kfx = d.k_fmt_x;
    asm volatile("" ::"s"(payload), "s"(scale), "s"(y), "s"(N), "s"(kfx));
    const int K = static_cast<int>(kfx & 0xffffu);
    const int fmt = static_cast<int>((kfx >> 16) & 0xffu);
    const float* x = g.xs[kfx >> 24];
    const int n0 = (w - begin) * direct_tn(K) * 64;
    if (fmt == kFmtQ4)
        direct_dispatch_k<kFmtQ4, NL, TM>(K, x, payload, scale, y, M, N, n0, smem);
    else if (fmt == kFmtQ8)
        direct_dispatch_k<kFmtQ8, NL, TM>(K, x, payload, scale, y, M, N, n0, smem);
    else
        direct_dispatch_k<kFmtF8, NL, TM>(K, x, payload, scale, y, M, N, n0, smem);
}

template <int NL>
void launch_direct_tm(int tm, int tiles, const DirectArgs& g, hipStream_t stream) {
    if (tm == 1)
        direct_kernel<1, NL><<<tiles, 256, 0, stream>>>(g);
    else
        direct_kernel<2, NL><<<tiles, 256, 0, stream>>>(g);
}

}  // namespace

bool direct_fits(const ProjTask* tasks, int count, int64_t M) {
    if (M < 1 || M > 16 * kDirectMaxTM) return false;
    for (int i = 0; i < count; ++i) {
        if (!direct_k(tasks[i].K)) return false;
        // int4 (scale, min) words are read 16 bytes at a time
        if (tasks[i].fmt == kFmtQ4 && (reinterpret_cast<uintptr_t>(tasks[i].scale) & 15) != 0) return false;
    }
    return true;
}

// Every projection in as few launches as the argument block allows (96
// projections, 48 distinct inputs), then the biases in one finish pass.
hipError_t launch_direct(const ProjTask* tasks, int count, int64_t M64, int NL, hipStream_t stream) {
    if ((NL != 1 && NL != 3) || !direct_fits(tasks, count, M64)) return hipErrorInvalidValue;
    const int M = static_cast<int>(M64);
    const int tm = direct_tm(M);
    // Workgroups with the most work per wave (K * tn) first, so the longest
    // ones are not left for the end of the launch.
    thread_local std::vector<int> order;
    order.resize(count);
    for (int i = 0; i < count; ++i) order[i] = i;
    auto work = [&](int i) { return tasks[i].K * direct_tn(tasks[i].K); };
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return work(a) > work(b); });
    int done = 0;
    while (done < count) {
        DirectArgs g{};
        g.M = M;
        int tiles = 0, n_in = 0;
        while (done < count && g.count < kDirectMaxProj) {
            const ProjTask& t = tasks[order[done]];
            const int cols = 64 * direct_tn(t.K);
            const int t_tiles = (t.N + cols - 1) / cols;
            if (tiles + t_tiles > kDirectMaxTiles) break;
            int xi = -1;
            for (int k = 0; k < n_in; ++k)
                if (g.xs[k] == t.x) xi = k;
            if (xi < 0) {
                if (n_in == kDirectMaxInputs) break;
                xi = n_in++;
                g.xs[xi] = t.x;
            }
            const int c = g.count++;
            DirectProj& d = g.proj[c];
            d.payload = t.payload;
            d.scale = t.scale;
            d.y = t.y;
            d.n = t.N;
            d.k_fmt_x = static_cast<uint32_t>(t.K) | static_cast<uint32_t>(t.fmt) << 16 | static_cast<uint32_t>(xi) << 24;
            g.tile_begin[c] = tiles;
            tiles += t_tiles;
            ++done;
        }
        if (g.count == 0) return hipErrorInvalidValue;   // one projection alone exceeds a launch
        seg_fill_coarse(g.tile_begin, g.tile_coarse, g.count);
        g.tiles = tiles;
        const int mark = timing_begin(stream);
        if (NL == 1)
            launch_direct_tm<1>(tm, tiles, g, stream);
        else
            launch_direct_tm<3>(tm, tiles, g, stream);
        timing_end(mark, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_bias_add(tasks, count, M64, stream);
}

}  // namespace rtq
