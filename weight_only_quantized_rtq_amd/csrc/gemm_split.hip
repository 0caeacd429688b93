// Dequant-in-GEMM on the bf16 matrix cores with exact fp32 products.
//
// y[M][N] = x[M][K] . W^T (+ bias) with W in its packed int4 / int8 form (RT-J
// int4 and int8 model cards, section "Quantization format") or as FP8 E4M3
// codes (RT-J FP8 card, section "FP8 Format"), dequantized inside the GEMM as
// the cards' opening paragraphs describe.
//
// Row scale. Every row of x is first scaled by the power of two 2^e that puts
// its largest magnitude in [2^14, 2^15) (exact for every value that stays a
// normal fp32 number), and every output row is scaled back by 2^-e (exact)
// after the int8 scale, before the bias. The code sums below therefore stay
// far inside the fp32 range whatever the magnitude of the row. "x" below is
// the scaled row.
//
// Arithmetic. Every fp32 activation is split, exactly, into three bf16 limbs:
//   x1 = x with the low 16 bits of its encoding cleared  (top 8 significant bits)
//   r  = x - x1                                           (exact, <= 16 bits)
//   x2 = r with the low 16 bits cleared, x3 = r - x2      (x3 has <= 8 bits: exact in bf16)
// so x == x1 + x2 + x3. The int4 codes (0..15), int8 codes (-127..127) and
// E4M3 values are exact in bf16, so every product code * limb is exact in
// fp32, and v_mfma_f32_16x16x32_bf16 accumulates them in fp32: the per-group
// code sum P_g[m][o] = sum_{k in g} code[o][k] * x[m][k] is an fp32 dot product
// of the exact values. One MFMA covers exactly one 32-wide int4 group, so
//   int4: y = sum_g scale_g[o] * P_g  +  sum_g min_g[o] * X_g[m],   X_g[m] = sum_{k in g} x[m][k]
//   int8: y = scale[o] * sum_k q[o][k] * x[m][k]
//   FP8:  y = sum_k w[o][k] * x[m][k]
// which is W = code*scale + min (int4) and W = q*scale (int8) by
// distributivity. The scale term is one fp32 FMA per output per group on the
// VALU; the min term is a K/32-long contraction run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32, four groups per instruction).
//
// bf16 activations (one limb). The same kernels with NL = 1 take x rounded to
// the nearest bf16 (ties to even) as their only limb: one MFMA per group and
// tile instead of three, y = bf16(x) . W^T with the same exact weight side and
// fp32 accumulation; the group sums X_g are those of the rounded values.
//
// Two fp16 limbs (NL = 2). Each scaled value v (largest magnitude of the row
// in [2^14, 2^15), inside the fp16 range) is split as h = fp16(v),
// l = fp16(v - h) (both roundings to nearest). h + l holds v to
// 22 significant bits (relative error <= 2^-22 per element, plus an absolute
// 2^-25 in the scaled units for elements far below the row's largest). Codes
// are exact in fp16, products of code and limb exact in fp32, and
// v_mfma_f32_16x16x32_f16 accumulates two limb products per group and tile
// instead of three. X_g are the sums of the scaled values.
//
// Data movement.
//  1. A pre-pass (prep_kernel) scales and splits every distinct activation
//     once into a limb image in a device workspace: NL limb planes in MFMA
//     operand order, with an XOR swizzle that makes the LDS reads
//     conflict-free, plus X_g and the row exponents.
//  2. The GEMM copies each 32-wide group of its row block from that image into
//     an LDS ring with global_load_lds_dwordx4 (direct to LDS: no registers, no
//     VALU), ahead of the compute, one barrier per group.
//  3. Weights. Small M (split_grouped_kernel, every projection of the call in
//     one launch; calls with M <= 32 whose every K is 256, 512, 1024 or 2048
//     run gemm_direct.hip instead): each wave copies its rows as 16-byte (row, group) records
//     into a private LDS ring, two groups per copy, a chunk ahead; K is cut into
//     chunks of at most 16 groups, and finish_kernel sums the chunks' partials
//     in order (and adds biases). Large M (split_gemm_kernel, 128 x 128 tiles):
//     each wave loads its codes into registers one group ahead, from L2.
//  4. Workgroup ids are remapped so that each XCD runs a contiguous range of
//     tiles: the tiles that share an activation image share that XCD's L2.
#include <mutex>
#include <type_traits>

#include "rtq_internal.h"
#include "split_device.h"

namespace rtq {

namespace {

// ---------------------------------------------------------------------------
// Limb image of one activation x [M][K] with NL limbs (G = K/32 groups, RB row
// blocks of 16, RB*16 >= M; rows >= M are zero):
//   block (g, rb) of NL KB at byte ((g*RB + rb)*NL + limb) * 1024; with NL = 3
//   limb 0 = x1 (high), 1 = x2, 2 = x3, with NL = 1 the bf16-rounded x, with
//   NL = 2 the fp16 limbs h, l of the scaled row; inside a limb, row r (0..15)
//   and 16-byte chunk c (k = 8c..8c+7 of the group) sit at
//   (r*4 + (c ^ ((r>>2)&3))) * 16; a chunk holds its eight k in order, except
//   with NL = 2, where it holds k = 8c + 0, 4, 1, 5, 2, 6, 3, 7 (the order in
//   which the two-limb code conversions produce the weights);
//   then the group sums X[g][row] (fp32, RB*16 rows per group);
//   then the row exponents e[row] (int32, RB*16 rows): row `row` of x was
//   scaled by 2^e[row] before the split.
// For a fixed group the RB blocks are contiguous, so a row block of BM rows is
// one contiguous run of BM/16 * NL KB.
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t image_plane_bytes(int G, int RB, int NL) { return int64_t(G) * RB * 1024 * NL; }
__host__ __device__ inline int64_t image_exp_offset(int G, int RB, int NL) {
    return image_plane_bytes(G, RB, NL) + int64_t(G) * RB * 16 * 4;
}
__host__ __device__ inline int64_t image_bytes(int G, int RB, int NL) {
    return image_exp_offset(G, RB, NL) + int64_t(RB) * 16 * 4;
}

constexpr int kMaxImages = 48;
struct PrepArgs {
    int M;                              // rows of every image of the launch
    int RB;                             // their 16-row blocks
    const float* x[kMaxImages];
    unsigned char* img[kMaxImages];
    int K[kMaxImages];
};
static_assert(sizeof(PrepArgs) <= 4096, "kernel arguments must stay within 4 KiB");

// One wave per row: the row's scale needs its largest magnitude first. Lane L
// takes k = 512*j + 8L .. 8L+7 of every 512-wide piece j (group 16j + L/4,
// chunk L%4); the row maximum is a wave reduction. With max|x[row][:]| =
// f * 2^E, f in [0.5, 1), the exponent is e = 15 - E (e = 15 for a zero row),
// so the scaled row's largest magnitude lies in [2^14, 2^15). Every scaled
// value v = x * 2^e (exact while v stays a normal fp32 number) is then
//   NL = 3: split exactly into three bf16 limbs (split2);
//   NL = 2: split into two fp16 limbs h = fp16(v), l = fp16(v - h);
//   NL = 1: rounded to the nearest bf16;
// and the group sums X_g are sums of the scaled values (of the rounded ones
// with NL = 1), each formed as ((v0+v1)+(v2+v3))+((v4+v5)+(v6+v7)) per chunk,
// then chunks (0+1)+(2+3). Rows of K <= 512*kPrepHold stay in registers
// between the two passes; longer rows are read again.
constexpr int kPrepHold = 4;
// Grid: (RB * 4, images); blockIdx.y is the image, blockIdx.x its four rows.
template <int NL>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs p) {
    const int i = blockIdx.y;
    const int M = p.M, K = p.K[i], RB = p.RB;
    const int G = K / 32;
    const int row = static_cast<int>(blockIdx.x) * 4 + static_cast<int>(threadIdx.x >> 6);   // < RB * 16
    const int lane = threadIdx.x & 63;
    const int c = lane & 3;
    const int r = row & 15, rb = row >> 4;
    const bool live = row < M;
    const float* src = p.x[i] + static_cast<int64_t>(live ? row : 0) * K + 8 * lane;
    const int pieces = (K + 511) / 512;
    auto load = [&](int j, float (&v)[8]) {
        if (live && 512 * j + 8 * lane < K) {
            const float4* q = reinterpret_cast<const float4*>(src + 512 * j);
            const float4 a = q[0], bb = q[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = bb.x; v[5] = bb.y; v[6] = bb.z; v[7] = bb.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
    };
    float hold[kPrepHold][8];
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < kPrepHold; ++j) {
        load(j, hold[j]);                                        // past the row: zeros
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(hold[j][e]));
    }
    for (int j = kPrepHold; j < pieces; ++j) {
        float v[8];
        load(j, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
    }
    // Row maximum without the LDS crossbar: DPP rotations inside each row of
    // 16 lanes, then the four rows' results read as scalars.
    mx = fmaxf(mx, row_ror<8>(mx));
    mx = fmaxf(mx, row_ror<4>(mx));
    mx = fmaxf(mx, row_ror<2>(mx));
    mx = fmaxf(mx, row_ror<1>(mx));
    auto lane_f = [](float v, int l) {
        return bitsf(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(fbits(v)), l)));
    };
    mx = fmaxf(fmaxf(lane_f(mx, 0), lane_f(mx, 16)), fmaxf(lane_f(mx, 32), lane_f(mx, 48)));
    int E = 0;
    (void)frexpf(mx, &E);
    const int ex = 15 - E;

    unsigned char* img = p.img[i];
    float* X = reinterpret_cast<float*>(img + image_plane_bytes(G, RB, NL));
    auto emit = [&](int j, float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ldexpf(v[e], ex);
        uint32_t h[4], m[4], l[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (NL == 3) {
                split2(v[2 * q], v[2 * q + 1], h[q], m[q], l[q]);
            } else if constexpr (NL == 2) {
                split_f16x2(v[q], v[q + 4], h[q], l[q]);          // k order 0, 4, 1, 5, ...
            } else {
                h[q] = bf16x2_rne(v[2 * q], v[2 * q + 1]);
                v[2 * q] = bitsf(h[q] << 16);               // the group sum is over the rounded values
                v[2 * q + 1] = bitsf(h[q] & 0xffff0000u);
            }
        }
        float s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        // partner lanes c ^ 1, then c ^ 2, inside each quad (DPP quad_perm)
        const float s1 = bitsf(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(fbits(s)), 0xb1, 0xf, 0xf, true)));
        s = (c & 1) ? s1 + s : s + s1;
        const float s2 = bitsf(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(fbits(s)), 0x4e, 0xf, 0xf, true)));
        s = (c & 2) ? s2 + s : s + s2;
        const int g = 16 * j + (lane >> 2);
        if (g < G) {
            unsigned char* blk = img + (static_cast<int64_t>(g) * RB + rb) * (NL * 1024) + swz(r, c) * 16;
            *reinterpret_cast<uint4*>(blk) = make_uint4(h[0], h[1], h[2], h[3]);
            if constexpr (NL == 3) {
                *reinterpret_cast<uint4*>(blk + 1024) = make_uint4(m[0], m[1], m[2], m[3]);
                *reinterpret_cast<uint4*>(blk + 2048) = make_uint4(l[0], l[1], l[2], l[3]);
            } else if constexpr (NL == 2) {
                *reinterpret_cast<uint4*>(blk + 1024) = make_uint4(l[0], l[1], l[2], l[3]);
            }
            if (c == 0) X[static_cast<int64_t>(g) * RB * 16 + row] = s;
        }
    };
#pragma unroll
    for (int j = 0; j < kPrepHold; ++j)
        if (j < pieces) emit(j, hold[j]);
    for (int j = kPrepHold; j < pieces; ++j) {
        float v[8];
        load(j, v);
        emit(j, v);
    }
    if (lane == 0) reinterpret_cast<int*>(img + image_exp_offset(G, RB, NL))[row] = ex;
}

// ---------------------------------------------------------------------------
// GEMM on the limb image.
// ---------------------------------------------------------------------------
struct SplitArgs {
    const unsigned char* img;     // limb image of x
    const void* payload;
    const void* scale;
    float* y;                     // output (or this K chunk's partial), [M][N]
    int M, N, K, RB;
    int g_lo, g_cnt;              // groups [g_lo, g_lo + g_cnt) of K
    const float* bias;            // fp32 [N] added in the epilogue, or nullptr
};

constexpr int kStages = 2;        // LDS ring depth (loads run one group ahead)
constexpr int kRing = 8;          // group sums kept for the deferred min term
constexpr int kChunk = 2;         // steps per weight chunk when the weights stream through LDS

// LDS map of a workgroup: x stages, group-sum ring and, when the weights
// stream through LDS (WL > 0), WL + 1 weight-chunk slots per wave. A chunk
// holds the wave's TN*16 rows for kChunk steps: int4 as 16-byte code records
// (one per row and group) plus 4-byte (scale, min) records, int8 as two
// 16-byte halves per row and group (TN * 1024 bytes either way). With the
// weights in LDS the x stages run XL steps ahead (XL + 1 stages).
template <int BM, int TN = 1, int XL = 0, int WL = 0, int NL = 3, int NW = 4>
struct Lds {
    static constexpr int NSTAGE = WL > 0 ? XL + 1 : kStages;      // x stages
    static constexpr int NWSLOT = WL + 1;                         // weight-chunk slots per wave
    static constexpr int STAGE = (BM / 16) * NL * 1024;
    static constexpr int XRING = NSTAGE * STAGE;
    // Group-sum slot: even waves copy rows 0..63, odd waves rows
    // XSLOT-64 .. XSLOT-1 (the same rows several times, identical bytes).
    static constexpr int XSLOT = BM <= 96 ? 96 : 128;
    static constexpr int WRING = XRING + kRing * XSLOT * 4;
    static constexpr int WCHUNK = TN * 1024;
    // the tile's row exponents, copied in 64-row pieces before the first stage
    static constexpr int EXPS = WRING + (WL > 0 ? NWSLOT * NW * WCHUNK : 0);
    static constexpr int NEXP = (BM + 63) / 64;
    static constexpr int TOTAL = EXPS + NEXP * 256;
    static constexpr int COPIES = (BM / 16) * NL;                  // 1 KB copies per stage
    static constexpr int PER_WAVE = (COPIES + NW - 1) / NW;
    static_assert(BM <= XSLOT, "group-sum slot holds every row of the tile");
    static_assert(NEXP <= NW, "one exponent copy per wave at most");
};

// f(std::integral_constant<int, i>) for i = B .. E-1, expanded at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

// Wait until at most n (uniform, 0 <= n) vector-memory operations are in
// flight; n above MAXN waits for MAXN.
template <int MAXN>
__device__ __forceinline__ void wait_vm_upto(int n) {
    if constexpr (MAXN == 0) {
        wait_vm<0>();
    } else {
        if (n >= MAXN) wait_vm<MAXN>();
        else wait_vm_upto<MAXN - 1>(n);
    }
}

__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// DMA schedule of the x stages and weight chunks when the weights stream
// through LDS (XL, WL >= 1): NX ops per x stage and NWC per weight chunk (per
// wave); stage s lands in slot s % (XL + 1), chunk c (steps 2c, 2c + 1) in slot
// c % (WL + 1).
//  - Before the loop every slot is free: stages 0..XL and chunks 0..WL are
//    issued in the order of the step that first needs them (a chunk before the
//    stage of the same step).
//  - Iteration j >= 1 issues stage j + XL after its barrier, then, for even
//    j >= 2, chunk j/2 + WL: the earliest iteration whose barrier follows
//    every wave's last read of the slot's previous occupant.
//  - At the top of iteration i a wave waits until at most allowed(i, GS) of
//    its ops are in flight: the ops issued after step i's stage and chunk
//    (loads complete in order). A chunk issued one step ahead of the step
//    before it is needed therefore stays in flight across that step.
// verify() replays the schedule for every chunk length up to 48 with an
// in-order completion model and checks that what each step reads has landed,
// that allowed() leaves exactly the ops issued after it in flight (no stricter
// wait), that each slot holds what its step reads, that no slot is refilled
// before the barrier after its last read, and that nothing is left in flight
// at the end.
template <int XL, int WL, int NX, int NWC>
struct DmaSchedule {
    __host__ __device__ static constexpr int stage_iter(int s) { return s <= XL ? -1 : s - XL; }
    __host__ __device__ static constexpr int chunk_iter(int c) { return c <= WL ? -1 : 2 * c - 2 * WL; }
    // position in the issue order
    __host__ __device__ static constexpr int stage_key(int s) { return s <= XL ? 2 * s + 1 : 4096 + 2 * (s - XL); }
    __host__ __device__ static constexpr int chunk_key(int c) { return c <= WL ? 4 * c : 4096 + 2 * (2 * c - 2 * WL) + 1; }
    static constexpr int kMax = XL * NX + (WL + 1) * NWC;
    static constexpr int kPrologue = XL > 2 * WL ? XL : 2 * WL;     // last step the prologue serves
    // before the loop, for need = 0..kPrologue: chunk need/2, then stage need
    __host__ __device__ static constexpr bool pro_chunk(int need, int GS) { return (need & 1) == 0 && need / 2 <= WL && need < GS; }
    __host__ __device__ static constexpr bool pro_stage(int need, int GS) { return need <= XL && need < GS; }
    // after the barrier of iteration i: stage i + XL, then chunk i/2 + WL
    __host__ __device__ static constexpr bool it_stage(int i, int GS) { return i >= 1 && i + XL < GS; }
    __host__ __device__ static constexpr bool it_chunk(int i, int GS) { return i >= 2 && (i & 1) == 0 && i + 2 * WL < GS; }
    // Away from both ends (steps kSteadyLo .. steady_hi(GS) - 1) the count
    // depends on the parity of i only, and every step issues its stage (and,
    // when even, its chunk): the loop runs those steps in pairs with these
    // constants (verify() checks them against allowed() and it_*()).
    static constexpr int kSteadyLo = kPrologue + 1;
    __host__ __device__ static constexpr int steady_hi(int GS) { return GS - kPrologue - 1; }
    __host__ __device__ static constexpr bool steady_at(int i, int GS) { return i >= kSteadyLo && i < steady_hi(GS); }
    static constexpr int steady(int parity) { return allowed(2 * kPrologue + 2 + parity, 1 << 20); }
    // The first kSteadyLo steps (the head) take allowed(h, kBig) once GS >= kBig.
    static constexpr int kBig = 2 * kPrologue + 3;
    // Past the head, a step r steps before the last takes tail(r, parity): the
    // count depends only on r and the parity of the step. At most kTail steps
    // follow the steady pairs.
    static constexpr int kTail = kPrologue + 2;
    static constexpr int tail(int r, int parity) { return allowed(2 * kPrologue + 2 + parity, 2 * kPrologue + 3 + parity + r); }
    __host__ __device__ static constexpr int allowed(int i, int GS) {
        const int need = stage_key(i) > chunk_key(i / 2) ? stage_key(i) : chunk_key(i / 2);
        int n = 0;
        for (int s = i + 1; s <= i + XL; ++s)
            if (s < GS && stage_iter(s) <= i - 1 && stage_key(s) > need) n += NX;
        for (int c = i / 2 + 1; c <= i / 2 + WL + 1; ++c)
            if (2 * c < GS && chunk_iter(c) <= i - 1 && chunk_key(c) > need) n += NWC;
        return n;
    }
    static constexpr bool verify() {
        if (!(XL >= 1 && WL >= 1 && XL <= 2 * WL)) return false;
        constexpr int kMaxGS = 48;
        constexpr int kCap = (kMaxGS + XL + 1) * NX + (kMaxGS / 2 + WL + 2) * NWC;
        for (int GS = 1; GS <= kMaxGS; ++GS) {
            int kind[kCap] = {}, idx[kCap] = {};   // unit ops in issue order: 0 stage, 1 chunk
            int issued = 0, landed = 0;
            int sslot[XL + 1], cslot[WL + 1];
            for (int k = 0; k <= XL; ++k) sslot[k] = -1;
            for (int k = 0; k <= WL; ++k) cslot[k] = -1;
            bool ok = true;
            auto issue = [&](int kd, int ix, int step) {   // step: barrier already passed (-1: none)
                if (kd == 0) {
                    const int occ = sslot[ix % (XL + 1)];
                    if (occ >= 0 && occ > step - 1) ok = false;            // read at step occ
                    sslot[ix % (XL + 1)] = ix;
                    for (int u = 0; u < NX; ++u) { kind[issued] = 0; idx[issued++] = ix; }
                } else {
                    const int occ = cslot[ix % (WL + 1)];
                    if (occ >= 0 && 2 * occ + 1 > step - 1) ok = false;    // read at steps 2occ, 2occ+1
                    cslot[ix % (WL + 1)] = ix;
                    for (int u = 0; u < NWC; ++u) { kind[issued] = 1; idx[issued++] = ix; }
                }
            };
            for (int need = 0; need <= kPrologue; ++need) {
                if (pro_chunk(need, GS)) issue(1, need / 2, -1);
                if (pro_stage(need, GS)) issue(0, need, -1);
            }
            for (int i = 0; i < GS; ++i) {
                const int a = allowed(i, GS);
                if (a < 0 || a > kMax) return false;
                if (issued - a > landed) landed = issued - a;
                bool have_s = false, have_c = false;
                int last = -1;
                for (int u = 0; u < issued; ++u) {
                    const bool mine = (kind[u] == 0 && idx[u] == i) || (kind[u] == 1 && idx[u] == i / 2);
                    if (mine && u >= landed) return false;                 // step i's data in flight
                    if (mine) last = u;
                    if (mine && kind[u] == 0) have_s = true;
                    if (mine && kind[u] == 1) have_c = true;
                }
                if (!have_s || !have_c) return false;
                if (a != issued - (last + 1)) return false;                // no stricter wait than needed
                if (steady_at(i, GS) && a != steady(i & 1)) return false;
                if (steady_at(i, GS) && !(it_stage(i, GS) && it_chunk(i, GS) == ((i & 1) == 0))) return false;
                if (i < kSteadyLo && GS >= kBig && a != allowed(i, kBig)) return false;
                if (i >= kSteadyLo) {                                      // closed forms of the tail
                    const int r = GS - 1 - i;
                    if (a != tail(r, i & 1)) return false;
                    if (it_stage(i, GS) != (r >= XL)) return false;
                    if (it_chunk(i, GS) != ((i & 1) == 0 && r >= 2 * WL)) return false;
                }
                if (sslot[i % (XL + 1)] != i || cslot[(i / 2) % (WL + 1)] != i / 2) return false;
                if (it_stage(i, GS)) issue(0, i + XL, i);
                if (it_chunk(i, GS)) issue(1, i / 2 + WL, i);
                if (!ok) return false;
            }
            if (allowed(GS - 1, GS) != 0 || landed != issued) return false;   // nothing left in flight
        }
        return true;
    }
};

// One BM x (WN*TN*16) tile (rows m0.., columns n0..) over the whole K. The
// workgroup's 4 or 8 waves are laid out WM x WN; each owns TM x TN 16x16 output
// tiles.
//
// K order: the tile walks the groups starting at group `rot` (cyclically), so
// the column tiles that share a row block (rot = their column-tile index) read
// different groups at any moment and, after the first group, find the limb
// image already in L2 instead of all missing on the same lines together.
// Iteration i is called step i below; the group it processes is (rot + i) % G.
//
// Weights: with WL == 0 each wave loads its codes and pairs into registers one
// step ahead (enough when they come from L2), and the x stages run one step
// ahead; with WL > 0 the weights are copied by DMA into a per-wave LDS ring WL
// chunks ahead (for weights streamed from HBM) and the x stages XL steps ahead.
//
// STREAM_Y: store y with nontemporal stores. The large-M tiles write hundreds
// of MB per launch that nothing in the launch reads again; kept in L2 they
// only evict the limb images that the other column tiles still read. The
// grouped kernel's K-chunk partials are read by the finish pass right after,
// so it keeps ordinary stores.
template <int FMT, int WM, int WN, int TM, int TN, int XL, int WL, int NL, bool STREAM_Y = false>
__device__ __forceinline__ void split_tile(const SplitArgs& a, int m0, int n0, int rot, unsigned char* smem) {
    constexpr int BM = WM * TM * 16;
    constexpr int NW = WM * WN;                                   // waves of the workgroup
    using L = Lds<BM, TN, XL, WL, NL, NW>;
    static_assert(NL >= 1 && NL <= 3, "limbs");
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(WL == 0 || (XL >= 1 && XL <= 2 * WL && WL <= 3), "prefetch leads");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The wave index is uniform: made explicit so that everything derived
    // from it (LDS destinations, copy indices) stays in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int li = lane & 15;
    const int lc = lane >> 4;
    const int M = a.M, N = a.N, K = a.K, RB = a.RB;
    const int G = K / 32;                                 // groups of the whole row (image, pairs)
    const int GS = a.g_cnt;                               // steps: groups of this K chunk
    const int rb0 = m0 / 16;

    // ---- async stage copies: 1 KB per wave instruction, all waves issue the same count.
    //      Every copy is a uniform base plus a fixed per-lane byte offset. ----
    const unsigned char* xsum = a.img + image_plane_bytes(G, RB, NL);
    const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
    const uint32_t xrow4 = static_cast<uint32_t>(min(m0 + (wave & 1) * (L::XSLOT - 64) + lane, RB * 16 - 1)) * 4u;
    auto group_of = [&](int i) { const int g = rot + i; return a.g_lo + (g >= GS ? g - GS : g); };
    auto stage_copy = [&](int i) {
        const int g = group_of(i);
        const unsigned char* src = a.img + (static_cast<int64_t>(g) * RB + rb0) * (NL * 1024);
        unsigned char* dst = smem + (i % L::NSTAGE) * L::STAGE;
#pragma unroll
        for (int j = 0; j < L::PER_WAVE; ++j) {
            // Every wave issues the same count; padding copies repeat the last
            // copy exactly (same source, same destination, same bytes).
            const int c = wave * L::PER_WAVE + j;
            const int cpy = c < L::COPIES ? c : L::COPIES - 1;
            dma16(src + cpy * 1024 + lane16, dst + cpy * 1024);
        }
        unsigned char* xdst = smem + L::XRING + ((i % kRing) * L::XSLOT + (wave & 1) * (L::XSLOT - 64)) * 4;
        dma4(xsum + static_cast<int64_t>(g) * RB * 16 * 4 + xrow4, xdst);
    };

    // ---- weights: lane (li, lc) of column tile tn holds row n0 + wn*TN*16 + tn*16 + li,
    //      k = 8*lc .. 8*lc+7 of the group ----
    // Weight addresses are the uniform payload / pair base plus 32-bit per-lane
    // byte offsets (the payload of a split projection is below 4 GiB).
    const unsigned char* payload = static_cast<const unsigned char*>(a.payload);
    const unsigned char* pairs = static_cast<const unsigned char*>(a.scale);
    uint32_t wvoff[TN], pvoff[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const uint32_t col = static_cast<uint32_t>(min(n0 + wn * TN * 16 + tn * 16 + li, N - 1));
        if constexpr (FMT == kFmtQ4) {
            wvoff[tn] = col * static_cast<uint32_t>(K / 2) + 4u * lc;
            pvoff[tn] = col * static_cast<uint32_t>(G) * 4u;
        } else {
            wvoff[tn] = col * static_cast<uint32_t>(K) + 8u * lc;
            pvoff[tn] = 0;
        }
    }
    auto w_load = [&](int i, uint32_t (&wq)[TN][2], uint32_t (&wp)[TN]) {
        const int g = group_of(i);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if constexpr (FMT == kFmtQ4) {
                wq[tn][0] = *reinterpret_cast<const uint32_t*>(payload + (wvoff[tn] + g * 16u));
                wq[tn][1] = 0;
                wp[tn] = *reinterpret_cast<const uint32_t*>(pairs + (pvoff[tn] + g * 4u));
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(payload + (wvoff[tn] + g * 32u));
                wq[tn][0] = v.x;
                wq[tn][1] = v.y;
                wp[tn] = 0;
            }
        }
    };

    // Weight chunks (WL > 0): chunk c holds the weights of steps kChunk*c and
    // kChunk*c + 1 for this wave's TN*16 rows, in slot c % (WL + 1). Each lane copies
    // whole 16-byte records (int4: the 32 codes of one row and group; int8:
    // half of them), so one instruction covers 64 (row, group) records.
    // Record order is swizzled so that the per-step reads are bank-spread:
    //   int4 codes: record row*2 + (h ^ (row>>3 & 1)), pairs: row*2 + h (4 B);
    //   int8: record row*4 + ((2h + half) ^ (row>>2 & 3)),
    // with h the step within the chunk and row = tn*16 + li.
    unsigned char* wring = smem + L::WRING + wave * L::WCHUNK;
    const int wrow0 = n0 + wn * TN * 16;
    // Per lane and chunk instruction j: the record's row offset (fixed) and
    // which of the chunk's two steps it belongs to.
    constexpr int NCI = WL > 0 ? (FMT == kFmtQ4 ? TN / 2 : TN) : 1;
    uint32_t cvoff[NCI], cpoff[NCI];
    bool csec[NCI], psec[NCI];
#pragma unroll
    for (int j = 0; j < NCI; ++j) {
        const int rec = j * 64 + lane;
        if constexpr (FMT == kFmtQ4) {
            const int row = rec >> 1;
            const uint32_t col = static_cast<uint32_t>(min(wrow0 + row, N - 1));
            csec[j] = ((rec & 1) ^ ((row >> 3) & 1)) != 0;
            psec[j] = (rec & 1) != 0;
            cvoff[j] = col * static_cast<uint32_t>(K / 2);
            cpoff[j] = col * static_cast<uint32_t>(G) * 4u;
        } else {
            const int row = rec >> 2;
            const int sub = (rec & 3) ^ ((row >> 2) & 3);
            const uint32_t col = static_cast<uint32_t>(min(wrow0 + row, N - 1));
            csec[j] = (sub >> 1) != 0;
            psec[j] = false;
            cvoff[j] = col * static_cast<uint32_t>(K) + static_cast<uint32_t>(sub & 1) * 16u;
            cpoff[j] = 0;
        }
    }
    auto w_chunk_issue = [&](int c) {
        if constexpr (WL > 0) {
            unsigned char* slot = wring + (c % L::NWSLOT) * NW * L::WCHUNK;
            const int s0 = kChunk * c;
            const int g0 = group_of(s0);                          // s0 < GS
            const int g1 = group_of(min(s0 + 1, GS - 1));
            if constexpr (FMT == kFmtQ4) {
#pragma unroll
                for (int j = 0; j < TN / 2; ++j)
                    dma16(payload + (cvoff[j] + static_cast<uint32_t>(csec[j] ? g1 : g0) * 16u), slot + j * 1024);
#pragma unroll
                for (int j = 0; j < TN / 2; ++j)
                    dma4(pairs + (cpoff[j] + static_cast<uint32_t>(psec[j] ? g1 : g0) * 4u), slot + TN * 512 + j * 256);
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    dma16(payload + (cvoff[j] + static_cast<uint32_t>(csec[j] ? g1 : g0) * 32u), slot + j * 1024);
            }
        }
    };
    auto w_read = [&](int i, uint32_t (&wq)[TN][2], uint32_t (&wp)[TN]) {
        const unsigned char* slot = wring + ((i / kChunk) % L::NWSLOT) * NW * L::WCHUNK;
        const int h = i % kChunk;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int row = tn * 16 + li;
            if constexpr (FMT == kFmtQ4) {
                const int rec = row * 2 + (h ^ ((row >> 3) & 1));
                wq[tn][0] = *reinterpret_cast<const uint32_t*>(slot + rec * 16 + 4 * lc);
                wq[tn][1] = 0;
                wp[tn] = *reinterpret_cast<const uint32_t*>(slot + TN * 512 + (row * 2 + h) * 4);
            } else {
                const int rec = row * 4 + ((2 * h + (lc >> 1)) ^ ((row >> 2) & 3));
                const uint2 v = *reinterpret_cast<const uint2*>(slot + rec * 16 + 8 * (lc & 1));
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

    const int aoff = swz(li, lc) * 16;                                  // this lane's A chunk in a limb
    auto compute = [&](int i, const uint32_t (&cq)[TN][2], const uint32_t (&cp)[TN]) {
        const unsigned char* base = smem + (i % L::NSTAGE) * L::STAGE;
        u32x4 b[TN];
        float s[TN];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            if constexpr (FMT == kFmtQ4) {
                b[tn] = NL == 2 ? codes4_to_f16_k04(cq[tn][0]) : codes4_to_bf16(cq[tn][0]);
                s[tn] = half_bits_to_float(cp[tn] & 0xffffu);
                const float mn = half_bits_to_float(cp[tn] >> 16);
                mreg[tn] = lc == (i & 3) ? mn : mreg[tn];
            } else if constexpr (FMT == kFmtF8) {
                b[tn] = NL == 2 ? codes8f_to_f16_k04(cq[tn][0], cq[tn][1]) : codes8f_to_bf16(cq[tn][0], cq[tn][1]);
            } else {
                b[tn] = NL == 2 ? codes8_to_f16_k04(cq[tn][0], cq[tn][1]) : codes8_to_bf16(cq[tn][0], cq[tn][1]);
            }
        }
        // the limb products, smallest limb first
        auto mma = [](const u32x4& x, const u32x4& w, floatx4 c) {
            if constexpr (NL == 2) return mfma_f16(x, w, c);
            else return mfma_bf16(x, w, c);
        };
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const unsigned char* blk = base + (wm * TM + tm) * (NL * 1024) + aoff;
            u32x4 xl[NL];
#pragma unroll
            for (int l = 0; l < NL; ++l) xl[l] = *reinterpret_cast<const u32x4*>(blk + l * 1024);
            if constexpr (FMT == kFmtQ4) {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    floatx4 p = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int l = NL - 1; l >= 0; --l) p = mma(xl[l], b[tn], p);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[tm][tn][e] = fmaf(s[tn], p[e], acc[tm][tn][e]);
                }
            } else {
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                    for (int l = NL - 1; l >= 0; --l) acc[tm][tn] = mma(xl[l], b[tn], acc[tm][tn]);
            }
        }
    };
    // After step i: if it closes a block of 4 steps (or is the last), add the block's min term.
    auto min_flush = [&](int i) {
        if constexpr (FMT == kFmtQ4) {
            if ((i & 3) != 3 && i != GS - 1) return;
            const int ic = (i & ~3) + lc;                 // this lane group's step
            const bool live = ic <= i;
            const float* ring = reinterpret_cast<const float*>(smem + L::XRING) + (ic % kRing) * L::XSLOT;
            // every row tile's sums read first (one wait for all), then zeroed
            // for a lane group past the last step (its slot holds no sum of this tile)
            float xv[TM];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) xv[tm] = ring[wm * TM * 16 + tm * 16 + li];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                const float xs = live ? xv[tm] : 0.0f;
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs, mreg[tn], acc[tm][tn], 0, 0, 0);
            }
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) mreg[tn] = 0.0f;
        }
    };

    // ---- main loop: while step i computes, later steps stream into the other
    //      LDS stages and weight slots. A stage or slot is refilled only after
    //      the barrier that follows every wave's last read of it. ----
    uint32_t wq[TN][2], wp[TN], cq[TN][2], cp[TN];
    // The epilogue's operands are fetched before any stage: the tile's row
    // exponents by DMA into LDS (waves 0 .. NEXP-1, 64 rows each), this wave's
    // int8 scales into registers. These are the oldest loads of the wave, so
    // the first step's wait covers them without changing the schedule's
    // in-flight counts below, and the first barrier publishes the exponents
    // to every wave. (Biases, rare, are read in the epilogue.)
    if (wave < L::NEXP) {
        const int* exps = reinterpret_cast<const int*>(a.img + image_exp_offset(G, RB, NL));
        dma4(exps + min(m0 + wave * 64 + lane, RB * 16 - 1), smem + L::EXPS + wave * 256);
    }
    float escale[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        if constexpr (FMT == kFmtQ8)
            escale[tn] = static_cast<const float*>(a.scale)[min(n0 + wn * TN * 16 + tn * 16 + li, N - 1)];
        else
            escale[tn] = 1.0f;
    }
    // With WL > 0 the x stages and weight chunks follow DmaSchedule (above).
    constexpr int NX = L::PER_WAVE + 1;
    constexpr int NWC = TN;
    static_assert(WL == 0 || (kChunk == 2 && TN % 2 == 0), "weight-chunk schedule");
    using Sched = DmaSchedule<XL, WL, NX, NWC>;
    static_assert(WL == 0 || Sched::verify(), "x-stage / weight-chunk DMA schedule");
    if constexpr (WL == 0) {
        stage_copy(0);
        w_load(0, wq, wp);
    } else {
#pragma unroll
        for (int need = 0; need <= Sched::kPrologue; ++need) {
            if (Sched::pro_chunk(need, GS)) w_chunk_issue(need / 2);
            if (Sched::pro_stage(need, GS)) stage_copy(need);
        }
    }
    // Barrier without a memory fence: the LDS data of step i came in by DMA
    // and is complete after the wait before it (in every wave, after the
    // barrier); nothing else writes LDS, and a fence would also wait for later
    // steps.
    if constexpr (WL == 0) {
        for (int i = 0; i < GS; ++i) {
            wait_vm<0>();                                 // this wave's part of step i has landed
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                cq[tn][0] = wq[tn][0];
                cq[tn][1] = wq[tn][1];
                cp[tn] = wp[tn];
            }
            if (i + 1 < GS) {
                stage_copy(i + 1);
                w_load(i + 1, wq, wp);
            }
            __builtin_amdgcn_sched_barrier(0);
            compute(i, cq, cp);
            min_flush(i);
        }
    } else {
        // Step i after its wait: barrier, this step's weights from LDS, the
        // stage / chunk the schedule issues here, the arithmetic.
        auto step = [&](int i, bool issue_stage, bool issue_chunk) {
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            w_read(i, cq, cp);
            if (issue_stage) stage_copy(i + XL);
            if (issue_chunk) w_chunk_issue(i / 2 + WL);
            __builtin_amdgcn_sched_barrier(0);
            compute(i, cq, cp);
            min_flush(i);
        };
        // The head (steps 0 .. kSteadyLo - 1, unrolled) and the tail (at most
        // kTail steps, unrolled by their distance r from the last) take their
        // waits as constants; only a call with fewer than kBig steps evaluates
        // allowed() in the head. The steady steps run in pairs of known parity.
        static_for<0, Sched::kSteadyLo>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if (h < GS) {
                if (GS >= Sched::kBig) wait_vm<Sched::allowed(h, Sched::kBig)>();
                else wait_vm_upto<Sched::kMax>(Sched::allowed(h, GS));
                step(h, Sched::it_stage(h, GS), Sched::it_chunk(h, GS));
            }
        });
        constexpr int P0 = Sched::kSteadyLo & 1;          // parity of the first step of each pair
        int i = Sched::kSteadyLo;
        for (; i + 1 < Sched::steady_hi(GS); i += 2) {
            wait_vm<Sched::steady(P0)>();
            step(i, true, P0 == 0);
            wait_vm<Sched::steady(1 - P0)>();
            step(i + 1, true, P0 == 1);
        }
        static_for<0, Sched::kTail>([&](auto rc) {
            constexpr int r = Sched::kTail - 1 - decltype(rc)::value;
            const int j = GS - 1 - r;
            if (j >= i) {
                if (j & 1) wait_vm<Sched::tail(r, 1)>();
                else wait_vm<Sched::tail(r, 0)>();
                step(j, r >= XL, (j & 1) == 0 && r >= 2 * WL);
            }
        });
    }

    // ---- epilogue: lane holds D[4*lc + e][li] of each 16x16 tile. Each row
    //      is scaled back by 2^-e[row] (exact) after the int8 scale and before
    //      the bias. ----
    int rexp[TM][4];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int4 v = *reinterpret_cast<const int4*>(smem + L::EXPS + (wm * TM * 16 + tm * 16 + 4 * lc) * 4);
        rexp[tm][0] = -v.x;
        rexp[tm][1] = -v.y;
        rexp[tm][2] = -v.z;
        rexp[tm][3] = -v.w;
    }
    // the int8 scale first: the code sum of a row scaled far down would
    // overflow if scaled back before it
    // (The call's bias test is taken once, below: a select per store would
    // cost two instructions.)
    auto value = [&](auto bias_tag, int tm, int tn, int e, float bv) {
        float v = acc[tm][tn][e];
        if constexpr (FMT == kFmtQ8) v *= escale[tn];
        v = ldexpf(v, rexp[tm][e]);
        if constexpr (decltype(bias_tag)::value) v += bv;
        return v;
    };
    auto put = [](float* dst, float v) {
        if constexpr (STREAM_Y) __builtin_nontemporal_store(v, dst);
        else *dst = v;
    };
    // A tile whose rows all lie below M, in an output of less than 2^32
    // bytes (every tile of the small-M launches, all but the last row block
    // of the large-M ones), stores without row checks, addressed as the base
    // plus a 32-bit byte offset per row.
    auto store = [&](auto bias_tag) {
        constexpr int BN = WN * TN * 16;
        if (m0 + BM <= M && n0 + BN <= N && static_cast<int64_t>(M) * N < (int64_t(1) << 30)) {
            // Whole tile inside the output: no checks at all, and each row's
            // pieces from the wave's column tiles go out back to back, so a
            // nontemporal line is complete before it leaves.
            unsigned char* ybytes = reinterpret_cast<unsigned char*>(a.y);
            const uint32_t rstride = static_cast<uint32_t>(N) * 4u;
            const int col0 = n0 + wn * TN * 16 + li;
            float bv[TN];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                bv[tn] = 0.0f;
                if constexpr (decltype(bias_tag)::value) bv[tn] = a.bias[col0 + tn * 16];
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
                uint32_t off = static_cast<uint32_t>(m0 + wm * TM * 16 + tm * 16 + 4 * lc) * rstride +
                               static_cast<uint32_t>(col0) * 4u;
#pragma unroll
                for (int e = 0; e < 4; ++e, off += rstride)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        put(reinterpret_cast<float*>(ybytes + off + tn * 64), value(bias_tag, tm, tn, e, bv[tn]));
            }
            return;
        }
        if (m0 + BM <= M && static_cast<int64_t>(M) * N < (int64_t(1) << 30)) {
            unsigned char* ybytes = reinterpret_cast<unsigned char*>(a.y);
            const uint32_t rstride = static_cast<uint32_t>(N) * 4u;
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int col = n0 + wn * TN * 16 + tn * 16 + li;
                if (col >= N) continue;
                float bv = 0.0f;
                if constexpr (decltype(bias_tag)::value) bv = a.bias[col];
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    uint32_t off = static_cast<uint32_t>(m0 + wm * TM * 16 + tm * 16 + 4 * lc) * rstride +
                                   static_cast<uint32_t>(col) * 4u;
#pragma unroll
                    for (int e = 0; e < 4; ++e, off += rstride)
                        put(reinterpret_cast<float*>(ybytes + off), value(bias_tag, tm, tn, e, bv));
                }
            }
            return;
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int col = n0 + wn * TN * 16 + tn * 16 + li;
            if (col >= N) continue;
            float bv = 0.0f;
            if constexpr (decltype(bias_tag)::value) bv = a.bias[col];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = m0 + wm * TM * 16 + tm * 16 + 4 * lc + e;
                    if (row < M) put(a.y + static_cast<int64_t>(row) * N + col, value(bias_tag, tm, tn, e, bv));
                }
            }
        }
    };
    if (a.bias) store(std::true_type{});
    else store(std::false_type{});
}

// Large M: 128 x 128 tiles, 4 waves side by side along N, each 128 rows x 32 columns.
constexpr int kLWM = 1, kLWN = 4, kLTM = 8, kLTN = 2;
constexpr int kLBM = kLWM * kLTM * 16;
constexpr int kLBN = kLWN * kLTN * 16;
// Prefetch leads of the large-M kernel per limb count. One or two limbs: the
// x stages run a step ahead and the weights stream through a per-wave LDS ring
// a chunk ahead, and three workgroups still fit a CU (with one limb the LDS
// would admit four, but the kernel's registers hold it to three: at 128 VGPRs
// it spills).
// Three limbs (24 KB stages) keep the registers-one-step-ahead schedule, which
// fits three workgroups where the LDS ring would leave two.
template <int NL> struct LargeLead { static constexpr int XL = NL == 3 ? 0 : 1, WL = NL == 3 ? 0 : 1; };

template <int FMT, int NL>
__global__ __launch_bounds__(256) void split_gemm_kernel(SplitArgs a, int tiles_n) {
    constexpr int XL = LargeLead<NL>::XL, WL = LargeLead<NL>::WL;
    using L = Lds<kLBM, WL ? kLTN : 1, XL, WL, NL>;
    static_assert(L::TOTAL * (NL == 1 ? 4 : 3) <= 160 * 1024, "three workgroups per CU (four with one limb)");
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
    const int w = xcd_remap_split(blockIdx.x, gridDim.x);
    const int nt = w % tiles_n;
    split_tile<FMT, kLWM, kLWN, kLTM, kLTN, XL, WL, NL, true>(a, (w / tiles_n) * kLBM, nt * kLBN, nt % a.g_cnt, smem);
}

// Small M (<= 80): one row block of TM*16 rows and 256 columns per workgroup,
// every projection of the call in one launch.
constexpr int kMaxSplitGrouped = 96;

// One projection of a grouped launch: 36 bytes, so the kernel reads all of it
// with two scalar loads. Packed to 4-byte alignment (the pointers stay
// pointers, so the compiler still knows they address global memory).
struct __attribute__((packed, aligned(4))) GroupedProj {
    const void* payload;                // packed weights (int4 payload / int8 / FP8 codes)
    const void* scale;                  // int4 (scale, min) pairs or int8 row scales
    float* y;                           // output, or the partial buffer [ks][M][N] when K spans ks > 1 chunks
    uint32_t img_off;                   // byte offset of the projection's limb image in the workspace
    uint32_t n_fmt;                     // N | format << 30 (a split projection has N < 2^27)
    int k;
};
static_assert(sizeof(GroupedProj) == 36, "grouped descriptor layout");

struct SplitGroupArgs {
    int count;
    int M;
    int RB;
    int chunk_groups;                       // K chunk length in groups (split_chunks)
    int tiles;                              // workgroups of the launch
    int pad;
    const unsigned char* ws;                // workspace holding the limb images
    int tile_begin[seg_begin_slots(kMaxSplitGrouped)];   // first workgroup of each projection
    int tile_coarse[seg_coarse_slots(kMaxSplitGrouped)];
    GroupedProj proj[kMaxSplitGrouped];
};
static_assert(sizeof(SplitGroupArgs) <= 4096, "kernel arguments must stay within 4 KiB");

// Small M: column tiles of 256 and K chunks of at most 16 groups (512 of K),
// so every workgroup does about the same work.
constexpr int kSmallBN = 256;
// The 256 columns are spread over kSmallWaves waves side by side, kSmallTN
// column tiles each: eight waves halve each wave's work per K step, and a K
// step's time is mostly the latency of one wave's instruction chain.
constexpr int kSmallWaves = 8;
constexpr int kSmallTN = kSmallBN / (16 * kSmallWaves);
constexpr int kMaxGroupedTiles = 1 << 30;   // workgroups of one grouped launch
// Prefetch leads of the small-M kernel: x stages XL steps ahead, weight chunks
// (streamed from HBM) WL chunks ahead, per limb count. With eight waves per
// workgroup one step of x lead is enough (two measured 1-3 % slower).
template <int NL> struct SmallLead { static constexpr int XL = 1, WL = 1; };
// K chunks of at most kChunkGroups groups, or shorter (down to kMinChunkGroups)
// when a call has too few workgroups to fill the GPU and runs the finish pass
// anyway (a projection with K above 16 groups, or a bias): a small call (one
// block) then walks its K in parallel chunks at no extra launch. A call that
// would need the finish pass only for shorter chunks keeps them long: there
// the extra launch costs more host time than the shorter K walk saves.
constexpr int kChunkGroups = 16;
constexpr int kMinChunkGroups = 4;
constexpr int kFillTiles = 256;             // one workgroup per CU
__host__ __device__ inline int split_chunks(int K, int chunk_groups) {
    const int G = K / 32;
    return (G + chunk_groups - 1) / chunk_groups;
}

template <int TM, int NL>
__global__ __launch_bounds__(64 * kSmallWaves, 4) void split_grouped_kernel(SplitGroupArgs g) {
    constexpr int XL = SmallLead<NL>::XL, WL = SmallLead<NL>::WL;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Lds<TM * 16, kSmallTN, XL, WL, NL, kSmallWaves>::TOTAL];
    // Find this workgroup's projection: tiles are numbered projection by
    // projection, (column block, K chunk) within one. Consecutive tiles go to
    // one XCD, so the column tiles that read the same activation image share
    // that XCD's L2 instead of each fetching the image from memory.
    // Argument loads in three dependent steps: the header with the coarse
    // table, the run of the fine table the coarse table points at (which also
    // holds the projection's first workgroup), and the projection's descriptor
    // (which the compiler reads in two rounds: four rounds in all). The
    // launch's size comes with the arguments, not from the dispatch packet.
    constexpr int NC = seg_coarse_slots(kMaxSplitGrouped);
    static_assert(NC == 12, "the round-one operand list below names twelve coarse slots");
    const int count = g.count, tiles = g.tiles;
    const int M = g.M, RB = g.RB, chunk_groups = g.chunk_groups;
    const unsigned char* ws = g.ws;
    int coarse[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) coarse[j] = g.tile_coarse[j];
    // Each empty asm below takes the round's values as scalar operands, so
    // the compiler issues all of that round's loads before its one wait
    // (scalar loads return out of order: any use waits for all of them).
    asm volatile("" ::"s"(count), "s"(tiles), "s"(M), "s"(RB), "s"(chunk_groups), "s"(ws), "s"(coarse[0]), "s"(coarse[1]), "s"(coarse[2]), "s"(coarse[3]),
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
    const GroupedProj d = g.proj[i];
    const int K = d.k;
    const uint32_t n_fmt = d.n_fmt;
    const uint32_t img_off = d.img_off;
    const void* payload = d.payload;
    const void* scale = d.scale;
    float* y0 = d.y;
    asm volatile("" ::"s"(K), "s"(n_fmt), "s"(img_off), "s"(payload), "s"(scale), "s"(y0));
    const int N = static_cast<int>(n_fmt & 0x3fffffffu);
    const int fmt = static_cast<int>(n_fmt >> 30);
    const int G = K / 32;
    const int ks = split_chunks(K, chunk_groups);
    const int local = w - begin;
    const int cb = local / ks, kc = local % ks;
    const int g_lo = kc * G / ks, g_hi = (kc + 1) * G / ks;
    float* y = y0 + static_cast<int64_t>(ks > 1 ? kc : 0) * M * N;
    // Biases of grouped projections are added by finish_kernel.
    const SplitArgs a{ws + img_off, payload, scale, y, M, N, K, RB, g_lo, g_hi - g_lo, nullptr};
    const int rot = cb % (g_hi - g_lo);
    if (fmt == kFmtQ4)
        split_tile<kFmtQ4, 1, kSmallWaves, TM, kSmallTN, XL, WL, NL>(a, 0, cb * kSmallBN, rot, smem);
    else if (fmt == kFmtQ8)
        split_tile<kFmtQ8, 1, kSmallWaves, TM, kSmallTN, XL, WL, NL>(a, 0, cb * kSmallBN, rot, smem);
    else
        split_tile<kFmtF8, 1, kSmallWaves, TM, kSmallTN, XL, WL, NL>(a, 0, cb * kSmallBN, rot, smem);
}

// Finishes projections after their GEMM launch: sums the K-chunk partials in
// chunk order and adds the bias, y = (P_0 + ... + P_{ks-1}) + bias. With
// ks == 1 the single "partial" is y itself and the bias is added in place.
constexpr int kMaxFinish = 96;
struct FinishArgs {
    int count;
    int pad;
    const float* part[kMaxFinish];  // chunk c of entry i at part[i] + c * elems[i]
    float* y[kMaxFinish];
    const float* bias[kMaxFinish];  // fp32 [n] or nullptr
    int64_t elems[kMaxFinish];      // M * n
    int ks[kMaxFinish];
    int n[kMaxFinish];
};
static_assert(sizeof(FinishArgs) <= 4096, "kernel arguments must stay within 4 KiB");

__global__ __launch_bounds__(256) void finish_kernel(FinishArgs r) {
    const int i = blockIdx.y;
    const int64_t n = r.elems[i];
    const int N = r.n[i];
    const float* bias = r.bias[i];
    const int64_t stride = int64_t(gridDim.x) * 256;
    int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    int col = static_cast<int>(e % N);                 // column of element e, kept in step with e
    const int col_step = static_cast<int>(stride % N);
    for (; e < n; e += stride) {
        float s = r.part[i][e];
        for (int c = 1; c < r.ks[i]; ++c) s += r.part[i][c * n + e];
        if (bias) s += bias[col];
        r.y[i][e] = s;
        col += col_step;
        if (col >= N) col -= N;
    }
}

// Adds one projection to a finish launch; returns the blocks it asks for.
int finish_entry(FinishArgs& r, const float* part, float* y, const float* bias, int64_t elems, int ks, int N) {
    const int c = r.count++;
    r.part[c] = part;
    r.y[c] = y;
    r.bias[c] = bias;
    r.elems[c] = elems;
    r.ks[c] = ks;
    r.n[c] = N;
    const int64_t need = (elems + 255) / 256;
    return need < 1024 ? static_cast<int>(need) : 1024;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct Input {
    const float* x;
    int K;
    int64_t offset;     // of its image in the workspace
};

hipError_t run_prep(const Input* in, int n_in, unsigned char* ws, int M, int RB, int NL, hipStream_t stream) {
    int done = 0;
    while (done < n_in) {
        PrepArgs p{};
        p.M = M;
        p.RB = RB;
        int count = 0;
        while (done < n_in && count < kMaxImages) {
            const Input& u = in[done++];
            p.x[count] = u.x;
            p.img[count] = ws + u.offset;
            p.K[count] = u.K;
            ++count;
        }
        const dim3 grid(RB * 4, count);                     // one wave per row
        if (NL == 1)
            prep_kernel<1><<<grid, 256, 0, stream>>>(p);
        else if (NL == 2)
            prep_kernel<2><<<grid, 256, 0, stream>>>(p);
        else
            prep_kernel<3><<<grid, 256, 0, stream>>>(p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The library's own stream-ordered memory pool of a device, created on first
// use and kept for the process; it keeps freed memory (release threshold at
// the maximum), so steady-state calls are served from the pool without a
// driver allocation. The device's default pool is left as it is.
hipError_t library_pool(int device, hipMemPool_t* out) {
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    if (device < 0 || device >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[device]) {
        hipMemPoolProps props{};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = device;
        hipMemPool_t pool = nullptr;
        hipError_t e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = ~0ull;
        e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(pool);
            return e;
        }
        pools[device] = pool;
    }
    *out = pools[device];
    return hipSuccess;
}

}  // namespace

bool split_ok(const ProjTask& t) {
    // K in whole groups, 16-byte aligned rows, and weights addressable by
    // 32-bit offsets from their base (N*K below 2^32).
    return t.K % 32 == 0 && (reinterpret_cast<uintptr_t>(t.x) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(t.payload) & 15) == 0 && int64_t(t.N) * t.K < (int64_t(1) << 32);
}

template <int NL>
void launch_grouped_tm(int tm, int tiles, const SplitGroupArgs& g, hipStream_t stream) {
    switch (tm) {
        case 1: split_grouped_kernel<1, NL><<<tiles, 64 * kSmallWaves, 0, stream>>>(g); break;
        case 2: split_grouped_kernel<2, NL><<<tiles, 64 * kSmallWaves, 0, stream>>>(g); break;
        case 3: split_grouped_kernel<3, NL><<<tiles, 64 * kSmallWaves, 0, stream>>>(g); break;
        case 4: split_grouped_kernel<4, NL><<<tiles, 64 * kSmallWaves, 0, stream>>>(g); break;
        default: split_grouped_kernel<5, NL><<<tiles, 64 * kSmallWaves, 0, stream>>>(g); break;
    }
}

template <int NL>
void launch_large(int fmt, int blocks, const SplitArgs& a, int tn, hipStream_t stream) {
    if (fmt == kFmtQ4)
        split_gemm_kernel<kFmtQ4, NL><<<blocks, 256, 0, stream>>>(a, tn);
    else if (fmt == kFmtQ8)
        split_gemm_kernel<kFmtQ8, NL><<<blocks, 256, 0, stream>>>(a, tn);
    else
        split_gemm_kernel<kFmtF8, NL><<<blocks, 256, 0, stream>>>(a, tn);
}

namespace {

// Workspace layout of a split call (no direct kernel): one limb image per
// distinct (x, K), then the K-chunk partials of the grouped launch.
struct SplitPlan {
    bool small = false;     // grouped small-M launch (else one tiled launch per projection)
    int RB = 0;             // 16-row blocks of every image
    int chunk_groups = kChunkGroups;   // K chunk length of the grouped launch
    int n_in = 0;
    Input inputs[8 * 64];
    int img_of[8 * 64];
    int64_t part_off[8 * 64];
    int64_t ws_bytes = 0;
};

void plan_split(const ProjTask* tasks, int count, int M, int NL, SplitPlan& p) {
    const int tm_small = static_cast<int>((int64_t(M) + 15) / 16);
    // The grouped small-M launch addresses the limb images by 32-bit offsets;
    // a call whose images would not fit (enormous K) takes the tiled path.
    p.small = M <= 80;
    for (;;) {
        p.RB = p.small ? tm_small : static_cast<int>((int64_t(M) + kLBM - 1) / kLBM) * (kLBM / 16);
        // Distinct inputs (pointer, K).
        p.n_in = 0;
        p.ws_bytes = 0;
        for (int i = 0; i < count; ++i) {
            int found = -1;
            for (int j = 0; j < p.n_in; ++j)
                if (p.inputs[j].x == tasks[i].x && p.inputs[j].K == tasks[i].K) found = j;
            if (found < 0) {
                found = p.n_in++;
                p.inputs[found] = Input{tasks[i].x, tasks[i].K, p.ws_bytes};
                p.ws_bytes += (image_bytes(tasks[i].K / 32, p.RB, NL) + 255) / 256 * 256;
            }
            p.img_of[i] = found;
        }
        if (!p.small || p.ws_bytes <= int64_t(UINT32_MAX)) break;
        p.small = false;
    }
    // Shorter K chunks while the grouped launch would leave CUs idle.
    p.chunk_groups = kChunkGroups;
    bool finishes = false;
    for (int i = 0; i < count; ++i)
        finishes = finishes || split_chunks(tasks[i].K, kChunkGroups) > 1 || tasks[i].bias != nullptr;
    if (p.small && finishes) {
        for (;;) {
            int64_t tiles = 0;
            for (int i = 0; i < count; ++i)
                tiles += int64_t(tasks[i].N + kSmallBN - 1) / kSmallBN * split_chunks(tasks[i].K, p.chunk_groups);
            if (tiles >= kFillTiles || p.chunk_groups <= kMinChunkGroups) break;
            p.chunk_groups /= 2;
        }
    }
    for (int i = 0; i < count; ++i) {
        p.part_off[i] = -1;
        const int ks = split_chunks(tasks[i].K, p.chunk_groups);
        if (p.small && ks > 1) {
            p.part_off[i] = p.ws_bytes;
            p.ws_bytes += (int64_t(ks) * M * tasks[i].N * 4 + 255) / 256 * 256;
        }
    }
}

}  // namespace

int64_t split_workspace_bytes(const ProjTask* tasks, int count, int64_t M, int NL) {
    if (count == 0 || direct_fits(tasks, count, M)) return 0;
    thread_local SplitPlan plan;
    plan_split(tasks, count, static_cast<int>(M), NL, plan);
    return plan.ws_bytes;
}

namespace {

// All projections (sharing M) of this call: split every distinct input once into
// a workspace, run the GEMMs. The workspace is ext_ws (ext_cap bytes) when
// given, else a stream-ordered allocation from the library's pool, returned
// at the end. NL = 3: exact three-limb split; NL = 2: two fp16 limbs of the
// row-scaled x; NL = 1: x rounded to bf16. The direct small-M kernel splits x
// itself and has no row scale: with NL = 2 it runs the exact three-limb split.
hipError_t split_impl(const ProjTask* tasks, int count, int64_t M64, int NL, hipStream_t stream,
                      unsigned char* ext_ws, int64_t ext_cap) {
    if (NL < 1 || NL > 3) return hipErrorInvalidValue;
    const int M = static_cast<int>(M64);
    if (direct_fits(tasks, count, M)) return launch_direct(tasks, count, M, NL == 2 ? 3 : NL, stream);
    const int tm_small = static_cast<int>((int64_t(M) + 15) / 16);
    thread_local SplitPlan plan;
    plan_split(tasks, count, M, NL, plan);
    const bool small = plan.small;
    const int RB = plan.RB;
    const Input* inputs = plan.inputs;
    const int* img_of = plan.img_of;
    const int64_t* part_off = plan.part_off;
    const int64_t ws_bytes = plan.ws_bytes;
    void* ws = ext_ws;
    hipError_t e = hipSuccess;
    if (ext_ws) {
        if (ws_bytes > ext_cap) return hipErrorOutOfMemory;
    } else {
        int device = 0;
        e = hipGetDevice(&device);
        hipMemPool_t pool = nullptr;
        if (e == hipSuccess) e = library_pool(device, &pool);
        if (e == hipSuccess) e = hipMallocFromPoolAsync(&ws, static_cast<size_t>(ws_bytes), pool, stream);
        if (e != hipSuccess) return e;
    }
    unsigned char* wsb = static_cast<unsigned char*>(ws);
    e = run_prep(inputs, plan.n_in, wsb, M, RB, NL, stream);

    if (e == hipSuccess && small) {
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
        FinishArgs red{};
        int red_blocks = 0;
        while (e == hipSuccess && done < count) {
            SplitGroupArgs g{};
            g.M = M;
            g.RB = RB;
            g.chunk_groups = plan.chunk_groups;
            g.ws = wsb;
            int tiles = 0;
            while (done < count && g.count < kMaxSplitGrouped &&
                   tiles + (tasks[order[done]].N + kSmallBN - 1) / kSmallBN *
                                   split_chunks(tasks[order[done]].K, plan.chunk_groups) <=
                       kMaxGroupedTiles) {
                const int ti = order[done++];
                const ProjTask& t = tasks[ti];
                const int c = g.count++;
                const int ks = split_chunks(t.K, plan.chunk_groups);
                GroupedProj& d = g.proj[c];
                d.payload = t.payload;
                d.scale = t.scale;
                d.y = ks > 1 ? reinterpret_cast<float*>(wsb + part_off[ti]) : t.y;
                d.img_off = static_cast<uint32_t>(inputs[img_of[ti]].offset);
                d.n_fmt = static_cast<uint32_t>(t.N) | static_cast<uint32_t>(t.fmt) << 30;
                d.k = t.K;
                g.tile_begin[c] = tiles;
                tiles += (t.N + kSmallBN - 1) / kSmallBN * ks;
                if (ks > 1 || t.bias) {
                    const float* part = ks > 1 ? reinterpret_cast<const float*>(wsb + part_off[ti]) : t.y;
                    const int nb = finish_entry(red, part, t.y, t.bias, int64_t(M) * t.N, ks, t.N);
                    red_blocks = red_blocks > nb ? red_blocks : nb;
                }
            }
            seg_fill_coarse(g.tile_begin, g.tile_coarse, g.count);
            g.tiles = tiles;
            const int mark = timing_begin(stream);
            if (NL == 1)
                launch_grouped_tm<1>(tm_small, tiles, g, stream);
            else if (NL == 2)
                launch_grouped_tm<2>(tm_small, tiles, g, stream);
            else
                launch_grouped_tm<3>(tm_small, tiles, g, stream);
            timing_end(mark, stream);
            e = hipGetLastError();
            if (e == hipSuccess && red.count) {
                finish_kernel<<<dim3(red_blocks, red.count), 256, 0, stream>>>(red);
                e = hipGetLastError();
                red = FinishArgs{};
                red_blocks = 0;
            }
        }
    } else if (e == hipSuccess) {
        for (int i = 0; i < count && e == hipSuccess; ++i) {
            const ProjTask& t = tasks[i];
            const SplitArgs a{wsb + inputs[img_of[i]].offset, t.payload, t.scale, t.y, M, t.N, t.K, RB, 0, t.K / 32,
                              t.bias};
            const int tn = (t.N + kLBN - 1) / kLBN;
            const int tmb = static_cast<int>((int64_t(M) + kLBM - 1) / kLBM);
            const int mark = timing_begin(stream);
            if (NL == 1)
                launch_large<1>(t.fmt, tmb * tn, a, tn, stream);
            else if (NL == 2)
                launch_large<2>(t.fmt, tmb * tn, a, tn, stream);
            else
                launch_large<3>(t.fmt, tmb * tn, a, tn, stream);
            timing_end(mark, stream);
            e = hipGetLastError();
        }
    }
    if (ext_ws) return e;
    const hipError_t f = hipFreeAsync(ws, stream);
    return e != hipSuccess ? e : f;
}

}  // namespace

hipError_t launch_split(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream) {
    return split_impl(tasks, count, M, NL, stream, nullptr, 0);
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is `scratch`, a fixed device array of
// the library (one copy per device, each GPU the library runs on holding it
// for the life of the process). Host code never passes the array's name to a
// kernel: its device address is resolved once per device, with that device
// current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(unsigned char** out) {
    static std::mutex mu;
    static unsigned char* addr[64] = {};
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return e;
    if (device < 0 || device >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[device] = static_cast<unsigned char*>(p);
    }
    *out = addr[device];
    return hipSuccess;
}

hipError_t launch_split_scratch(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream) {
    unsigned char* ws = nullptr;
    if (split_workspace_bytes(tasks, count, M, NL) > 0) {
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) return e;
    }
    return split_impl(tasks, count, M, NL, stream, ws, kScratchBytes);
}

hipError_t launch_split_ws(const ProjTask* tasks, int count, int64_t M, int NL, hipStream_t stream,
                           unsigned char* ws, int64_t cap) {
    if (!ws && split_workspace_bytes(tasks, count, M, NL) > 0) return hipErrorInvalidValue;
    return split_impl(tasks, count, M, NL, stream, ws, cap);
}

hipError_t launch_bias_add(const ProjTask* tasks, int count, int64_t M, hipStream_t stream) {
    FinishArgs r{};
    int blocks = 0;
    for (int i = 0; i <= count; ++i) {
        if (r.count == kMaxFinish || (i == count && r.count)) {
            finish_kernel<<<dim3(blocks, r.count), 256, 0, stream>>>(r);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            r = FinishArgs{};
            blocks = 0;
        }
        if (i == count || !tasks[i].bias) continue;
        const ProjTask& t = tasks[i];
        const int nb = finish_entry(r, t.y, t.y, t.bias, M * t.N, 1, t.N);
        blocks = blocks > nb ? blocks : nb;
    }
    return hipSuccess;
}

}  // namespace rtq
