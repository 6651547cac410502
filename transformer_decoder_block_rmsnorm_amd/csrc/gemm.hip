// Weight GEMMs of the decoder block: y = x W with W stored [in, out]
// (tirogla "Transformer block", Code: weights are kept [in, out] and applied
// as y = x W).
//
// bf16 (large M): MFMA 32x32x16 tiles with fp32 accumulation.  Operands go
// from global memory straight into LDS through a ring of k stages; the A
// fragments are plain 16-byte LDS reads, the weight fragments come from the
// N-contiguous weight tile through the gfx950 transpose read
// ds_read_b64_tr_b16, so no operand is transposed in registers.  Small M
// (decode) goes to the split-K weight-streaming kernel in skinny.hip.
//
// Fused epilogues (epilogue.h): RoPE + KV-cache scatter for the fused QKV
// projection, residual add for Wo and W2, SiLU(gate) * up for the fused
// gate-up projection (W1 and W3 tiles interleaved in 32-column blocks), fp32
// store for the LM head.
//
// fp32: a plain LDS-tiled VALU GEMM with the same epilogues (the fp32 storage
// path serves small shapes; it is launch-latency bound).
#include <algorithm>

#include "epilogue.h"
#include "kernels.h"

namespace tfb {

// Where the columns of the B operand come from.
//  SRC_ONE:    a single [K, N] matrix.
//  SRC_CONCAT: up to three matrices side by side (Wq | Wk | Wv); a column
//              tile never straddles two of them.
//  SRC_DUAL:   W1 and W3 interleaved in 32-column blocks (gate-up); the
//              logical output has N/2 columns.
enum SrcKind { SRC_ONE = 0, SRC_CONCAT = 1, SRC_DUAL = 2 };

// Most k ranges a tile of the split-K tail is divided into.
constexpr int kMaxSplitK = 4;

struct GemmArgs {
    const void *A;
    int64_t lda;
    int M, K;
    int N;              // B columns in this launch (DUAL: 2 * logical width)
    const void *w[3];
    int w_cols[3];      // columns (= leading dimension) of each matrix
    int tiles_m, tiles_n, group_m;
    // split-K tail: workgroups [0, full_tiles) compute whole tiles; the
    // remaining tiles are each computed by `splits` workgroups over equal
    // k ranges, which write fp32 partials to `part`, and a fix-up kernel adds
    // them in a fixed order and applies the epilogue
    int full_tiles, splits;
    float *part;        // [tiles - full_tiles][splits][BM][BN]
    // A folded RMSNorm (rss non-null): the A rows are bf16(x * gain), and
    // rss [M][rss_n] holds partial sums of x^2 over column tiles of x, added
    // here in order; the products of row m are scaled by
    // 1 / sqrt(sum / rss_d + rss_eps) before the epilogue.
    const float *rss;
    int rss_n, rss_d;
    float rss_eps;
};

// Workgroups are dealt to the 8 XCDs round robin.  xcd_remap gives each XCD a
// contiguous run of n consecutive logical indices (n a multiple of 8), so the
// tiles resident on one XCD share A and B panels in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    return (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3);
}

// Tile index -> (tm, tn): runs of `group_m` row panels, column-major inside
// a run, so consecutive tiles reuse the same weight columns.
__device__ __forceinline__ void tile_coords(const GemmArgs &g, int L, int &tm, int &tn) {
    const int per_group = g.group_m * g.tiles_n;
    const int grp = L / per_group;
    const int first_m = grp * g.group_m;
    const int gm = min(g.tiles_m - first_m, g.group_m);
    const int r = L - grp * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// Work of workgroup `bid`: its tile and, for the split tail, its k split
// (-1: the whole k range).  Whole tiles come first in launch order.
__device__ __forceinline__ void wg_work(const GemmArgs &g, int bid, int &tile, int &split) {
    if (bid < g.full_tiles) {
        tile = xcd_remap(bid, g.full_tiles);
        split = -1;
    } else {
        const int n_split = (g.tiles_m * g.tiles_n - g.full_tiles) * g.splits;
        const int j = xcd_remap(bid - g.full_tiles, n_split);
        tile = g.full_tiles + j / g.splits;
        split = j % g.splits;
    }
}

// ---------------------------------------------------------------------------
// bf16 GEMM: operands go from global memory straight into LDS
// (global_load_lds_dwordx4: lane i of an instruction writes the i-th 16-byte
// slot of a 1 KB block), through a ring of NST stages of BK = 32, so up to
// three k steps of loads are in flight while one is multiplied.  Each lane
// fetches the global chunk that belongs in its slot, which lays the tiles out
// already swizzled: A rows (64 bytes, k contiguous) with
// chunk ^ ((row >> 2) & 3), B rows (N contiguous) with 32-byte granules
// ^ swz_tr(row), so the transpose reads of one 16-lane group fall in
// different banks.  The waits are explicit: before a stage is used,
// s_waitcnt vmcnt leaves only the younger stages outstanding, then a barrier
// makes every wave's slots visible.  The MFMAs of one 16-wide k half run
// while the fragments of the next half are read from LDS.
// ---------------------------------------------------------------------------
// NORM: a folded RMSNorm.  0 none; NORM_SCALE: A holds bf16(x * gain) and
// g.rss the row sums (the row scale is applied to the products); NORM_FOLD
// (RESID): the epilogue folds the next norm (ep.nu).  Separate instances, so
// the plain kernels carry none of the extra registers.
enum NormKind { NORM_NONE = 0, NORM_SCALE = 1, NORM_FOLD = 2 };
template <int BM, int BN, int WM, int WN, int SRC, int EPI, int NORM>
__global__ __launch_bounds__(WM *WN * 64) void gemm_bf16_dma_kernel(GemmArgs g, EpiParams ep) {
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int BKD = 32, NST = 4;  // ring stages of BKD k each
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int A_INS = BM * BKD * 2 / 1024 / NW;   // 1 KB A blocks per wave per stage
    constexpr int B_INS = BKD * BN * 2 / 1024 / NW;
    constexpr int A_ELEMS = BM * BKD, STAGE = BM * BKD + BKD * BN;  // elements
    static_assert(A_INS * NW * 1024 == BM * BKD * 2 && B_INS * NW * 1024 == BKD * BN * 2, "tiles split in 1 KB blocks");
    static_assert(BN / 16 >= 8, "granule swizzle needs 8 granules per row");
    static_assert(SRC != SRC_DUAL || TN % 2 == 0, "dual source needs gate/up tile pairs");
    static_assert(NW * 32 * (WTN + 4) * 4 <= NST * STAGE * 2, "epilogue staging must fit");
    static_assert((32 * (EPI == EPI_SWIGLU ? WTN / 2 : WTN) / 8) % 64 == 0, "whole 8-column segments per lane");

    __shared__ __attribute__((aligned(1024))) bf16_t lds[NST * STAGE];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t *)lds;  // LDS byte address of the ring

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int tile, split, tm, tn;
    wg_work(g, blockIdx.x, tile, split);
    tile_coords(g, tile, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // k steps of this workgroup
    const int KT_all = g.K / BKD;
    const int kt0 = split < 0 ? 0 : (split * KT_all) / g.splits;
    const int kt1 = split < 0 ? KT_all : ((split + 1) * KT_all) / g.splits;

    // ---- per-lane source of each 1 KB block this wave fills
    const bf16_t *A = (const bf16_t *)g.A;
    const bf16_t *a_src[A_INS];
#pragma unroll
    for (int j = 0; j < A_INS; ++j) {
        const int slot = (wave * A_INS + j) * 64 + lane;
        const int row = slot >> 2, p = slot & 3, c = p ^ ((row >> 2) & 3);
        a_src[j] = A + (int64_t)min(m0 + row, g.M - 1) * g.lda + 8 * c + kt0 * BKD;
    }
    const bf16_t *b_src[B_INS];
    int b_ld[B_INS];
#pragma unroll
    for (int j = 0; j < B_INS; ++j) {
        const int slot = (wave * B_INS + j) * 64 + lane;
        const int k = slot / (BN / 8), p = slot % (BN / 8);
        const int gsw = (p >> 1) ^ swz_tr(k);
        const int cglob = n0 + 16 * gsw + 8 * (p & 1);
        const bf16_t *base;
        int ld, col;
        if constexpr (SRC == SRC_ONE) {
            base = (const bf16_t *)g.w[0]; ld = g.w_cols[0]; col = cglob;
        } else if constexpr (SRC == SRC_CONCAT) {
            int sidx = 0, c2 = cglob;
            if (c2 >= g.w_cols[0]) { c2 -= g.w_cols[0]; sidx = 1; if (c2 >= g.w_cols[1]) { c2 -= g.w_cols[1]; sidx = 2; } }
            if (sidx == 2 && c2 >= g.w_cols[2]) c2 = g.w_cols[2] - 8;  // ragged tail: a valid, unused column
            // selects rather than an index into the argument arrays, which
            // the compiler would load per lane from memory
            base = (const bf16_t *)(sidx == 0 ? g.w[0] : (sidx == 1 ? g.w[1] : g.w[2]));
            ld = sidx == 0 ? g.w_cols[0] : (sidx == 1 ? g.w_cols[1] : g.w_cols[2]);
            col = c2;
        } else {
            const int sidx = (cglob >> 5) & 1;
            base = (const bf16_t *)(sidx ? g.w[1] : g.w[0]);
            ld = sidx ? g.w_cols[1] : g.w_cols[0];
            col = 32 * (cglob >> 6) + (cglob & 31);
        }
        if (col >= ld) col = ld - 8;  // ragged tail: a valid column whose outputs are never stored
        b_ld[j] = ld;
        b_src[j] = base + (int64_t)(k + kt0 * BKD) * ld + col;
    }
    auto issue = [&](int kt, int stage) {
        // LDS byte address of this wave's first block in the stage (wave-uniform)
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_base + stage * STAGE * 2 + wave * A_INS * 1024);
        const uint32_t stb = __builtin_amdgcn_readfirstlane(lds_base + stage * STAGE * 2 + A_ELEMS * 2 +
                                                            wave * B_INS * 1024);
#pragma unroll
        for (int j = 0; j < A_INS; ++j) dma16(a_src[j] + kt * BKD, st + j * 1024);
#pragma unroll
        for (int j = 0; j < B_INS; ++j) dma16(b_src[j] + (int64_t)kt * BKD * b_ld[j], stb + j * 1024);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int KT = kt1 - kt0;
    const int lr = lane & 31, lh = lane >> 5;
    const int q = lane >> 4, sl = lane & 15;
    const int b_row = (q >> 1) * 8 + (sl >> 2);
    const int b_in = (sl & 3) * 4;
    constexpr int PER = A_INS + B_INS;  // vmem instructions per stage per thread

    static_assert(BKD == 32 && NST >= 3 && NST <= 6, "the pipeline below is written for two 16-wide k halves");
    // Fragments of one 16-wide k half of a stage.
    auto read_frags = [&](const bf16_t *As, int ks, bf16x8 (&af)[TM], bf16x8 (&bfr)[TN]) {
        const bf16_t *Bs = As + A_ELEMS;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int gran = (wn * WTN + j * 32) / 16 + (q & 1);
            const int r0 = ks * 16 + b_row, r1 = r0 + 4;
            const u32x2 lo = lds_read_tr16(Bs + r0 * BN + ((gran ^ swz_tr(r0)) * 16) + b_in);
            const u32x2 hi = lds_read_tr16(Bs + r1 * BN + ((gran ^ swz_tr(r1)) * 16) + b_in);
            bfr[j] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
        const int ch = ks * 2 + lh;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + lr;
            af[i] = as_bf16x8(*(const u32x4 *)(As + row * BKD + ((ch ^ ((row >> 2) & 3)) * 8)));
        }
    };
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];  // fragments of k halves 0 and 1
    // The first MFMA of a k half (its operands are complete), then the rest.
    auto first_product = [&](const bf16x8 (&af)[TM], const bf16x8 (&bfr)[TN]) {
        acc[0][0] = mfma32(af[0], bfr[0], acc[0][0]);
    };
    auto other_products = [&](const bf16x8 (&af)[TM], const bf16x8 (&bfr)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                if (i | j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    };
    // k half 0 of stage kt: its MFMAs run while half 1's fragments are read.
    auto half0 = [&](const bf16_t *As) {
        first_product(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(As, 1, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        other_products(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // k half 1 of stage kt: its MFMAs run while half 0 of the next stage is read.
    auto half1 = [&](const bf16_t *An) {
        first_product(fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(An, 0, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        other_products(fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's reads of stage kt are done
        asm volatile("s_barrier" ::: "memory");  // every wave: stage kt+1 landed, stage kt read
    };
    auto slot = [&](int kt) { return (const bf16_t *)(lds + (kt % NST) * STAGE); };

    // Folded norm: the partial sums of the tile's rows are one contiguous
    // block of BM * rss_n floats; thread t loads half of row t / 2 (the
    // halves of a row sit in adjacent lanes), with 16-byte loads when the
    // halves are whole 16-byte groups, so the loads coalesce.  They are
    // issued right before the operand stream starts (the empty asm keeps
    // them after the setup above) and added after the main loop, whose last
    // wait has drained every load.  Indexes are clamped into the row, so the
    // loads are unconditional and issue together.
    constexpr int RS_MAX = kRowSsMaxParts / 2;
    static_assert(NT == 2 * BM, "two threads per tile row");
    __shared__ float rs_scale[BM];
    const int rs_row = tid >> 1, rs_half = tid & 1;
    f32x4 rsv[RS_MAX / 4];
    int rs_cnt = 0;
    if constexpr (NORM == NORM_SCALE) {
        asm volatile("" ::: "memory");
        const int per = (g.rss_n + 1) / 2, j0 = rs_half * per;
        rs_cnt = min(per, g.rss_n - j0);
        const float *row = g.rss + (int64_t)min(m0 + rs_row, g.M - 1) * g.rss_n;
        if (g.rss_n % 8 == 0) {
#pragma unroll
            for (int q = 0; q < RS_MAX / 4; ++q)
                rsv[q] = *(const f32x4 *)(row + j0 + min(4 * q, per - 4));
        } else {
#pragma unroll
            for (int q = 0; q < RS_MAX / 4; ++q)
#pragma unroll
                for (int k = 0; k < 4; ++k) rsv[q][k] = row[min(j0 + 4 * q + k, g.rss_n - 1)];
        }
    }
    // Software pipeline at half-stage granularity: the LDS reads of the next
    // k half are in flight while the MFMAs of the current one run, so LDS and
    // matrix cores work at the same time instead of in turn after each
    // barrier.  Stage s lives in ring slot s % NST; all NST slots are filled
    // ahead, and a slot is refilled right after the barrier that follows the
    // last read of its stage.
#pragma unroll
    for (int st = 0; st < NST; ++st)
        if (st < KT) issue(st, st);
    // waits until at most n of this wave's stage loads are still in flight
    auto wait_stages = [&](int n) {
        switch (n) {
            case 0: wait_vmcnt<0>(); break;
            case 1: wait_vmcnt<PER>(); break;
            case 2: wait_vmcnt<2 * PER>(); break;
            case 3: wait_vmcnt<3 * PER>(); break;
            case 4: wait_vmcnt<4 * PER>(); break;
            default: wait_vmcnt<5 * PER>(); break;
        }
    };
    wait_stages(min(NST - 1, KT - 1));
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");  // stage 0 visible to every wave
    read_frags(slot(0), 0, fa0, fb0);
    int kt = 0;
    for (; kt + NST - 1 < KT; ++kt) {
        // steady state: the loads of stages kt+2 .. kt+NST-1 may stay in flight
        half0(slot(kt));
        wait_vmcnt<(NST - 2) * PER>();
        sync();
        if (kt + NST < KT) issue(kt + NST, kt % NST);
        half1(slot(kt + 1));
    }
    for (; kt + 1 < KT; ++kt) {
        half0(slot(kt));
        wait_stages(KT - 2 - kt);
        sync();
        half1(slot(kt + 1));
    }
    half0(slot(KT - 1));
    first_product(fa1, fb1);
    other_products(fa1, fb1);
    wait_vmcnt<0>();
    if constexpr (NORM == NORM_SCALE) {
        // each half in order, then the two halves (adjacent lanes); 1/rms of
        // the row by the same expression as a standalone RMSNorm
        // (the empty asm keeps the additions here, after the loop, rather
        // than next to the loads, where they would wait for each load)
        float part = 0.0f;
#pragma unroll
        for (int q = 0; q < RS_MAX / 4; ++q) {
            asm volatile("" : "+v"(rsv[q]));
#pragma unroll
            for (int k = 0; k < 4; ++k) part += 4 * q + k < rs_cnt ? rsv[q][k] : 0.0f;
        }
        const float other = __shfl_xor(part, 1);
        const float sum = rs_half ? other + part : part + other;
        if (!rs_half) rs_scale[rs_row] = 1.0f / sqrtf(sum / (float)g.rss_d + g.rss_eps);
    }
    __syncthreads();  // every wave is done with the ring before it is reused for staging
    if constexpr (NORM == NORM_SCALE) {
        // every product of a row is scaled by its 1/rms
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 sv = *(const f32x4 *)(rs_scale + wm * WTM + i * 32 + 8 * q4 + 4 * lh);
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j][4 * q4 + k] *= sv[k];
            }
    }

    // Epilogue, one 32-row slab of the wave tile at a time: the accumulators
    // go through LDS (row stride SW floats) so that each lane then holds 8
    // consecutive columns of one row and the stores are 16 bytes wide.
    // SwiGLU is applied before staging: the gate (j even) and up (j + 1)
    // values of one output sit in the same register of the same lane.
    constexpr int UW = (EPI == EPI_SWIGLU) ? WTN / 2 : WTN;  // output columns of the wave
    constexpr int SW = WTN + 4;                               // staging row stride (floats)
    float *stage = (float *)lds + wave * (32 * SW);
    // 16-byte chunk pair of lane segment sg: segments 4..7 of a 64-wide row
    // read their two chunks in the other order, so the eight lanes of one
    // row fall in distinct banks.
    auto read8 = [&](const float *src, int sg, float (&v)[8]) {
        const int f = (sg >> 2) & 1;
        const f32x4 a = *(const f32x4 *)(src + 4 * f), b = *(const f32x4 *)(src + 4 * (1 - f));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[4 * f + k] = a[k];
            v[4 * (1 - f) + k] = b[k];
        }
    };
    constexpr int SEGS = UW / 8;         // 8-column segments per row
    constexpr int NG = 32 * SEGS / 64;   // segments per lane in one slab
    const int c0 = (EPI == EPI_SWIGLU) ? tn * (BN / 2) + wn * UW : n0 + wn * WTN;
    // A tile wholly inside the output takes the fast path: every group of
    // the lane is whole, with its column fixed and its rows increasing.  The
    // SwiGLU epilogue reads nothing and stays on the general path, which
    // measured slightly faster for it.
    const bool whole = EPI != EPI_SWIGLU && split < 0 && ep.vec8 && m0 + BM <= ep.M && n0 + BN <= ep.N;
    // A folded RMSNorm of the output (RESID with ep.nu): each group's sum of
    // y^2 is added over the lanes of its row (a fixed butterfly), each wave
    // leaves its rows' sums in LDS past the staging area, and after the
    // epilogue the WN sums of a row are added in wave order.  A lane's
    // columns are the same in every group, so it widens its gains once.
    const bool fold = NORM == NORM_FOLD && split < 0;
    static_assert((NW * 32 * SW + WN * BM) * 4 <= NST * STAGE * 2, "row sums fit past the staging area");
    float *ssl = (float *)lds + NW * 32 * SW;  // [WN][BM]
    float gn[8] = {};
    if constexpr (NORM == NORM_FOLD)
        if (fold && c0 + 8 * (lane % SEGS) < ep.N) load_bf16x8(ep.ng + c0 + 8 * (lane % SEGS), gn);  // in the row
    auto fold_group = [&](int row_local, int m, int c, const float (&y)[8]) {
        float ss = epi_norm8(ep, m, c, y, gn);
#pragma unroll
        for (int o = SEGS / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        if (lane % SEGS == 0) ssl[wn * BM + row_local] = ss;
    };
    if (whole) {
        EpiLane L;
        const int rbase = m0 + wm * WTM + lane / SEGS;  // the lane's first row; rows step by 64 / SEGS
        epi_lane_init<EPI>(ep, c0 + 8 * (lane % SEGS), rbase, L);
        constexpr int RSTEP = 64 / SEGS;
        EpiPre pre[NG];
        EpiLane Ln = L;
        auto load_lane_slab = [&](int i, EpiPre (&pp)[NG], EpiLane &cur) {
#pragma unroll
            for (int r = 0; r < NG; ++r) {
                epi_lane_seek<EPI>(ep, rbase + i * 32 + r * RSTEP, cur);
                epi_load8_lane<EPI>(ep, cur, pp[r]);
            }
        };
        load_lane_slab(0, pre, Ln);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) stage[(8 * (v >> 2) + 4 * lh + (v & 3)) * SW + j * 32 + lr] = acc[i][j][v];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            EpiPre nxt[NG];
            if (i + 1 < TM) load_lane_slab(i + 1, nxt, Ln);
#pragma unroll
            for (int r = 0; r < NG; ++r) {
                const int rl = r * RSTEP + lane / SEGS, sg = lane % SEGS;
                float v8[8];
                read8(stage + rl * SW + 8 * sg, sg, v8);
                epi_lane_seek<EPI>(ep, rbase + i * 32 + r * RSTEP, L);
                if constexpr (EPI == EPI_RESID) {
                    float y8[8];
                    epi_store8_lane<EPI>(ep, L, v8, pre[r], y8);
                    if (fold) fold_group(wm * WTM + i * 32 + rl, L.m, L.c, y8);
                } else {
                    epi_store8_lane<EPI>(ep, L, v8, pre[r]);
                }
            }
            if (i + 1 < TM)
#pragma unroll
                for (int r = 0; r < NG; ++r) pre[r] = nxt[r];
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        // Edge tiles and split-K partials: each group checks its own bounds.
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row0 = m0 + wm * WTM + i * 32;
            if (split >= 0 || EPI != EPI_SWIGLU) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) stage[(8 * (v >> 2) + 4 * lh + (v & 3)) * SW + j * 32 + lr] = acc[i][j][v];
            } else {
#pragma unroll
                for (int jp = 0; jp < TN / 2; ++jp)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        stage[(8 * (v >> 2) + 4 * lh + (v & 3)) * SW + jp * 32 + lr] =
                            silu_f(acc[i][2 * jp][v]) * acc[i][2 * jp + 1][v];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (split >= 0) {
                // split tail: raw fp32 partial of this k range, tile-local layout
                float *dst = g.part + ((int64_t)(tile - g.full_tiles) * g.splits + split) * (BM * BN) +
                             (wm * WTM + i * 32) * BN + wn * WTN;
#pragma unroll
                for (int r = 0; r < 32 * WTN / 4 / 64; ++r) {
                    const int p = r * 64 + lane, rl = p / (WTN / 4), c4 = p % (WTN / 4);
                    *(f32x4 *)(dst + rl * BN + 4 * c4) = *(const f32x4 *)(stage + rl * SW + 4 * c4);
                }
            } else {
#pragma unroll
                for (int r = 0; r < NG; ++r) {
                    const int p = r * 64 + lane, rl = p / SEGS, sg = p % SEGS;
                    float v8[8];
                    read8(stage + rl * SW + 8 * sg, sg, v8);
                    if constexpr (EPI == EPI_RESID) {
                        float y8[8];
                        epi_store8<EPI>(ep, row0 + rl, c0 + 8 * sg, v8, y8);
                        if (fold) fold_group(wm * WTM + i * 32 + rl, row0 + rl, c0 + 8 * sg, y8);
                    } else {
                        epi_store8<EPI>(ep, row0 + rl, c0 + 8 * sg, v8);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    if (fold) {
        __syncthreads();
        for (int row = tid; row < BM; row += NT) {
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < WN; ++w) sum += ssl[w * BM + row];
            if (m0 + row < ep.M) ep.nss[(int64_t)(m0 + row) * ep.nss_n + tn] = sum;
        }
    }
}

// fp32 storage: 64x64 output tile per 256 threads, 16-wide k steps in LDS,
// each thread computes a 4 (rows) x 4 (columns) patch.  SWIGLU computes the
// gate and up dot products of each logical column side by side.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, EpiParams ep) {
    constexpr int TMt = 64, TNt = 64, TK = 16;
    __shared__ float As[TK][TMt + 4];
    __shared__ float Bs[2][TK][TNt + 4];
    const int tid = threadIdx.x;
    const int m0 = blockIdx.y * TMt, n0 = blockIdx.x * TNt;  // logical columns
    const int tr = tid / 16, tc = tid % 16;
    const float *A = (const float *)g.A;
    constexpr int NSRC = (EPI == EPI_SWIGLU) ? 2 : 1;
    float acc[NSRC][4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += TK) {
        for (int e = tid; e < TMt * TK; e += 256) {
            int r = e / TK, kk = e % TK;
            int gr = m0 + r, gk = k0 + kk;
            As[kk][r] = (gr < g.M && gk < g.K) ? A[(int64_t)gr * g.lda + gk] : 0.0f;
        }
        for (int s = 0; s < NSRC; ++s)
            for (int e = tid; e < TK * TNt; e += 256) {
                int kk = e / TNt, c = e % TNt;
                int gc = n0 + c, gk = k0 + kk;
                float v = 0.0f;
                if (gk < g.K) {
                    // (selects rather than indexes into the argument arrays)
                    if (EPI == EPI_SWIGLU) {
                        const int ldw = s ? g.w_cols[1] : g.w_cols[0];
                        if (gc < ldw) v = ((const float *)(s ? g.w[1] : g.w[0]))[(int64_t)gk * ldw + gc];
                    } else {
                        int src = 0, cc = gc;
                        if (g.w[1] && cc >= g.w_cols[0]) {
                            cc -= g.w_cols[0];
                            src = 1;
                            if (g.w[2] && cc >= g.w_cols[1]) {
                                cc -= g.w_cols[1];
                                src = 2;
                            }
                        }
                        const int ldw = src == 0 ? g.w_cols[0] : (src == 1 ? g.w_cols[1] : g.w_cols[2]);
                        const float *wm = (const float *)(src == 0 ? g.w[0] : (src == 1 ? g.w[1] : g.w[2]));
                        if (cc < ldw) v = wm[(int64_t)gk * ldw + cc];
                    }
                }
                Bs[s][kk][c] = v;
            }
        __syncthreads();
        for (int kk = 0; kk < TK; ++kk) {
            float a[4];
            for (int i = 0; i < 4; ++i) a[i] = As[kk][tr * 4 + i];
            for (int s = 0; s < NSRC; ++s)
                for (int j = 0; j < 4; ++j) {
                    float b = Bs[s][kk][tc * 4 + j];
                    for (int i = 0; i < 4; ++i) acc[s][i][j] += a[i] * b;
                }
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        int row = m0 + tr * 4 + i;
        for (int j = 0; j < 4; j += 2) {
            int col = n0 + tc * 4 + j;
            if constexpr (EPI == EPI_SWIGLU) {
                epi_store_swiglu<float>(ep, row, col, acc[0][i][j], acc[1][i][j]);
                epi_store_swiglu<float>(ep, row, col + 1, acc[0][i][j + 1], acc[1][i][j + 1]);
            } else {
                epi_store_pair<EPI, float>(ep, row, col, acc[0][i][j], acc[0][i][j + 1]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Split tail: add the k-split partials of one tile in a fixed order (so the
// result does not depend on which workgroup finished first) and apply the
// epilogue.  One thread per 4 tile-local columns of a row.
template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_split_fixup_kernel(GemmArgs g, EpiParams ep) {
    // SwiGLU: 4 gate columns (and their up columns) per thread; otherwise 8
    // columns, stored through the 16-byte epilogue
    constexpr int EPT = EPI == EPI_SWIGLU ? 4 : 8;
    const int pt = blockIdx.y;
    const int e = (blockIdx.x * 256 + threadIdx.x) * EPT;
    if (e >= BM * BN) return;
    int tm, tn;
    tile_coords(g, g.full_tiles + pt, tm, tn);
    const int row = e / BN, col = e % BN;
    if constexpr (EPI == EPI_SWIGLU) {
        if ((col & 63) >= 32) return;  // up columns are read by the gate's thread
    }
    // every split's partial is loaded before any is added (at most
    // kMaxSplitK; a loop over the run-time count would wait for each load in
    // turn), then they are summed in split order
    const float *src = g.part + (int64_t)pt * g.splits * (BM * BN) + row * BN + col;
    const int o2 = EPI == EPI_SWIGLU ? 32 : 4;  // second vector: the up columns, or columns 4..7
    f32x4 pa[kMaxSplitK], pb[kMaxSplitK];
#pragma unroll
    for (int s = 0; s < kMaxSplitK; ++s) {
        if (s < g.splits) {
            pa[s] = *(const f32x4 *)(src + (int64_t)s * (BM * BN));
            pb[s] = *(const f32x4 *)(src + (int64_t)s * (BM * BN) + o2);
        } else {
            pa[s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            pb[s] = pa[s];
        }
    }
    f32x4 v = pa[0], u = pb[0];
#pragma unroll
    for (int s = 1; s < kMaxSplitK; ++s) {
        if (s < g.splits) {
            v += pa[s];
            u += pb[s];
        }
    }
    const int m = tm * BM + row;
    if constexpr (EPI == EPI_SWIGLU) {
        const int lc = tn * (BN / 2) + (col >> 6) * 32 + (col & 31);
#pragma unroll
        for (int k = 0; k < 4; ++k) epi_store_swiglu<bf16_t>(ep, m, lc + k, v[k], u[k]);
    } else {
        const float v8[8] = {v[0], v[1], v[2], v[3], u[0], u[1], u[2], u[3]};
        if constexpr (EPI == EPI_RESID) {
            if (ep.nu) {
                // folded norm: the BN / 8 threads of a row are consecutive
                // lanes; their sums of y^2 are added by a fixed butterfly
                const int c = tn * BN + col;
                float y8[8], gn[8] = {};
                epi_store8<EPI>(ep, m, c, v8, y8);
                if (c < ep.N) load_bf16x8(ep.ng + c, gn);  // a group past the row's end reads no gains
                float ss = epi_norm8(ep, m, c, y8, gn);
#pragma unroll
                for (int o = BN / 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
                if (col == 0 && m < ep.M) ep.nss[(int64_t)m * ep.nss_n + tn] = ss;
                return;
            }
        }
        epi_store8<EPI>(ep, m, tn * BN + col, v8);
    }
}

// Split-K plan for the last, partial round of tiles: with `rem` tiles left
// over after whole rounds on `cus` compute units, split each of them `splits`
// ways so that rem * splits <= cus (at least 8 k steps per split, at most 4).
struct SplitPlan {
    int full_tiles, splits;
    size_t part_bytes;
};
static SplitPlan plan_split(int tiles, int k_steps, int cus, int tile_elems) {
    SplitPlan p{tiles, 1, 0};
    const int rem = tiles % cus;
    if (rem == 0) return p;
    int s = std::min(std::min(cus / rem, k_steps / 8), kMaxSplitK);
    if (s < 2) return p;
    p.full_tiles = tiles - rem;
    p.splits = s;
    p.part_bytes = (size_t)rem * s * tile_elems * sizeof(float);
    return p;
}

template <int BM, int BN, int WM, int WN, int SRC, int EPI>
static hipError_t launch_dma(GemmArgs g, EpiParams ep, void *part, size_t part_bytes, hipStream_t s) {
    g.tiles_m = (g.M + BM - 1) / BM;
    g.tiles_n = (g.N + BN - 1) / BN;
    g.group_m = 8;
    if (ep.nu) {  // a folded norm: one partial sum of squares per row and column tile
        if (EPI != EPI_RESID || !ep.vec8 || ep.N % 8 || g.tiles_n > kRowSsMaxParts) return hipErrorInvalidValue;
        ep.nss_n = g.tiles_n;
    }
    if (g.rss && (g.rss_n < 1 || g.rss_n > kRowSsMaxParts)) return hipErrorInvalidValue;
    const int tiles = g.tiles_m * g.tiles_n;
    SplitPlan sp = plan_split(tiles, g.K / 32, device_cus(), BM * BN);
    if (!part || sp.part_bytes > part_bytes) sp = SplitPlan{tiles, 1, 0};
    g.full_tiles = sp.full_tiles;
    g.splits = sp.splits;
    g.part = (float *)part;
    const int blocks = sp.full_tiles + (tiles - sp.full_tiles) * sp.splits;
    if constexpr (EPI == EPI_RESID) {
        if (ep.nu)
            hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, SRC, EPI, NORM_FOLD>), dim3(blocks),
                               dim3(WM * WN * 64), 0, s, g, ep);
        else
            hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, SRC, EPI, NORM_NONE>), dim3(blocks),
                               dim3(WM * WN * 64), 0, s, g, ep);
    } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_QKV) {
        if (g.rss)
            hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, SRC, EPI, NORM_SCALE>), dim3(blocks),
                               dim3(WM * WN * 64), 0, s, g, ep);
        else
            hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, SRC, EPI, NORM_NONE>), dim3(blocks),
                               dim3(WM * WN * 64), 0, s, g, ep);
    } else {
        if (g.rss) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, WM, WN, SRC, EPI, NORM_NONE>), dim3(blocks),
                           dim3(WM * WN * 64), 0, s, g, ep);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sp.splits == 1) return e;
    dim3 fg((BM * BN / (EPI == EPI_SWIGLU ? 4 : 8) + 255) / 256, tiles - sp.full_tiles);
    hipLaunchKernelGGL((gemm_split_fixup_kernel<BM, BN, EPI>), fg, dim3(256), 0, s, g, ep);
    return hipGetLastError();
}

// Tile shape of a large-M bf16 GEMM (8 waves unless noted):
//  T_256:     256x256, a partial last round of tiles split along k;
//  T_256x128: 256x128, which needs no split partials and no fix-up pass but
//             moves 1.5x the operand bytes per flop;
//  T_128:     128x128 on 4 waves, when fewer than half the compute units
//             would get a 256x256 tile.
// Between the first two, when 256x256 tiles leave a partial last round: a
// cost model in units of one 256x256 k step, with constants measured on the
// 7B block (K = 11008): a 256x128 k step costs 0.63 units plus 7 units of
// epilogue per round, and the split tail costs 0.77 units per MB of fp32
// partials written and re-read.  (It picks 256x128 for the 7B Wo, one round
// of 256x128 tiles, and a split tail for the 7B and the 32-layer model's
// fused QKV; measured on MI355X in one process, the 7B block step took 0.919
// ms that way against 0.944 ms with the QKV on three rounds of 256x128
// tiles, and the model's QKV 215 against 231 us.)
enum TilePlan { T_256 = 0, T_256x128 = 1, T_128 = 2 };
static TilePlan plan_tiles(int M, int N_virtual, int K) {
    const int cus = device_cus();
    const int tm = (M + 255) / 256, kt = K / 32;
    const int t256 = tm * ((N_virtual + 255) / 256), t128 = tm * ((N_virtual + 127) / 128);
    if (t256 * 2 < cus) return T_128;
    if (t256 % cus == 0) return T_256;
    const SplitPlan sp = plan_split(t256, kt, cus, 256 * 256);
    double c256 = (double)(t256 / cus) * kt;
    if (sp.splits > 1) c256 += (double)kt / sp.splits + 0.77 * sp.part_bytes / (1 << 20);
    else if (t256 % cus) c256 += kt;
    const double c128 = (double)((t128 + cus - 1) / cus) * (0.63 * kt + 7.0);
    return c128 < c256 ? T_256x128 : T_256;
}

int gemm_fold_parts(int M, int N, int K) {
    if (M <= kSkinnyMaxM || N % 8) return 0;
    const int bn = plan_tiles(M, N, K) == T_256 ? 256 : 128;
    const int parts = (N + bn - 1) / bn;
    return parts <= kRowSsMaxParts ? parts : 0;
}

size_t gemm_split_bytes(int M, int N_virtual, int K) {
    if (M <= kSkinnyMaxM || plan_tiles(M, N_virtual, K) != T_256) return 0;
    const int tiles = ((M + 255) / 256) * ((N_virtual + 255) / 256);
    return plan_split(tiles, K / 32, device_cus(), 256 * 256).part_bytes;
}

template <int SRC, int EPI>
static hipError_t launch_planned(const GemmArgs &g, const EpiParams &ep, void *part, size_t pb, hipStream_t s) {
    switch (plan_tiles(g.M, g.N, g.K)) {
        case T_256: return launch_dma<256, 256, 2, 4, SRC, EPI>(g, ep, part, pb, s);
        case T_256x128:
            // the gate-up pairing needs two 32-column blocks per wave
            if constexpr (SRC == SRC_DUAL) return launch_dma<256, 128, 4, 2, SRC, EPI>(g, ep, nullptr, 0, s);
            else return launch_dma<256, 128, 2, 4, SRC, EPI>(g, ep, nullptr, 0, s);
        default: return launch_dma<128, 128, 2, 2, SRC, EPI>(g, ep, nullptr, 0, s);
    }
}

hipError_t gemm_launch(const GemmCall &c, hipStream_t s) {
    GemmArgs g{};
    g.A = c.A;
    g.lda = c.lda;
    g.M = c.M;
    g.K = c.K;
    for (int i = 0; i < 3; ++i) { g.w[i] = c.w[i]; g.w_cols[i] = c.w_cols[i]; }
    g.rss = c.row_ss;
    g.rss_n = c.row_ss_n;
    g.rss_d = c.K;
    g.rss_eps = c.row_ss_eps;
    EpiParams ep = c.ep;
    ep.ng = nullptr;
    ep.nu = nullptr;
    ep.nss = nullptr;
    if (c.norm_ss) {  // fold the next RMSNorm (large-M path only)
        if (c.dtype != TFB_BF16 || c.M <= kSkinnyMaxM || c.epi != EPI_RESID || !c.norm_g || !c.norm_out)
            return hipErrorInvalidValue;
        ep.ng = (const bf16_t *)c.norm_g;
        ep.nu = (bf16_t *)c.norm_out;
        ep.ldu = c.ep.N;
        ep.nss = c.norm_ss;
    }
    if (c.row_ss && (c.dtype != TFB_BF16 || c.M <= kSkinnyMaxM)) return hipErrorInvalidValue;
    // 16-byte epilogue accesses need every 8-column group to start 16-byte
    // aligned: leading dimensions in elements, and whole groups inside one head
    switch (c.epi) {
        case EPI_SWIGLU: ep.vec8 = ep.ldo % 8 == 0; break;
        case EPI_RESID: ep.vec8 = ep.ldr % (ep.res_f32 ? 4 : 8) == 0 && ep.ldo % (ep.out_f32 ? 4 : 8) == 0; break;
        case EPI_F32: ep.vec8 = ep.ldo % 4 == 0; break;
        case EPI_QKV: ep.vec8 = ep.dh % 8 == 0; break;
        default: ep.vec8 = 0;
    }
    if (c.dtype == TFB_F32) {
        g.N = c.ep.N;
        dim3 grid((c.ep.N + 63) / 64, (c.M + 63) / 64);
        switch (c.epi) {
            case EPI_QKV: hipLaunchKernelGGL(gemm_f32_kernel<EPI_QKV>, grid, dim3(256), 0, s, g, ep); break;
            case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, dim3(256), 0, s, g, ep); break;
            case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, g, ep); break;
            case EPI_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_F32>, grid, dim3(256), 0, s, g, ep); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (c.M <= kSkinnyMaxM && c.scratch) return skinny_gemm_launch(c, c.scratch, c.scratch_bytes, s);
    void *part = c.split_scratch;
    const size_t pb = c.split_bytes;
    switch (c.epi) {
        case EPI_QKV:
            g.N = c.w_cols[0] + c.w_cols[1] + c.w_cols[2];
            return launch_planned<SRC_CONCAT, EPI_QKV>(g, ep, part, pb, s);
        case EPI_RESID:
            g.N = c.w_cols[0];
            return launch_planned<SRC_ONE, EPI_RESID>(g, ep, part, pb, s);
        case EPI_SWIGLU:
            g.N = 2 * c.w_cols[0];
            return launch_planned<SRC_DUAL, EPI_SWIGLU>(g, ep, part, pb, s);
        case EPI_F32:
            g.N = c.w_cols[0];
            return launch_planned<SRC_ONE, EPI_F32>(g, ep, part, pb, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tfb
