// Skinny weight GEMMs of the decode step: y = x W with few rows (M = number
// of sequences, at most 64) and W [K, N] streamed from HBM exactly once.
// Page short names: [TIR] tirogla "Transformer block", [PID] pidoku "The
// Transformer" (6. Under the hood: a decode step reads every weight once and
// is bandwidth bound).
//
// Work unit = one 4-wave workgroup: a BN-column block of W (BN = 64 or 128)
// times a range of k, split only as far as needed to give every compute unit
// a workgroup.  Stages of SK k rows of the weight block, plus the same SK
// columns of the rows of x the MFMA row tiles cover (16 per tile, rows past M
// clamped; SK = 128 when a 64-row stage of those rows would not split into
// whole 1 KB blocks per wave), go from global memory straight
// into a ring of LDS stages (global_load_lds_dwordx4), so the loads in flight
// cost no registers and the ring keeps several stages of HBM reads
// outstanding.  The weights, read once, take the nontemporal policy; the
// rows of x, which every column block reads again, take the plain one and
// stay in L2 (streamed like the weights, they were fetched again from
// beyond L2, and each GEMM of a 64-row decode step took 3.5-4.5 us longer).  Each wave owns BN/4 output columns: its weight fragments come
// from the transpose read ds_read_b64_tr_b16 on the N-contiguous weight rows
// (32-byte granules swizzled by row), the x fragments are 16-byte reads
// (chunks swizzled by row), and the products run on MFMA 16x16x32.  Each
// workgroup writes an fp32 partial [split][M][N]; a second kernel adds the
// splits in a fixed order and applies the fused epilogue (RoPE + KV append,
// residual, SwiGLU, fp32 store), so the result is deterministic.  The
// gate-up GEMM in a single k range skips that pass: W1 and W3 are
// interleaved in 16-column groups, so each wave holds the gate and the up
// value of the same outputs and writes SiLU(gate) * up itself.
#include <algorithm>

#include "epilogue.h"
#include "kernels.h"

namespace tfb {

struct SkinnyArgs {
    const bf16_t *x;  // [M, K]
    int64_t ldx;
    int M, K, N;      // N = columns of the virtual B
    int splits;       // k ranges per column block
    const bf16_t *w[3];
    int w_cols[3];
    int src;          // 0: one matrix, 1: concat (wq|wk|wv), 2: w1 and w3 interleaved in 16-column groups
    float *part;      // [splits][M][N]
    bf16_t *act;      // src 2 with one k range: SiLU(gate) * up written here directly, row stride ld_act
    int64_t ld_act;
    AttnChunks ac;    // XC kernels: x is the merge of these decode attention partials
};

// XC kernels: the k range of a workgroup is at most this many columns, so its
// whole activation slice sits in LDS beside a weight-only ring.
constexpr int kSkinnyXcMaxK = 512;

// Column c of the virtual B -> (matrix, column).  Concat: matrices side by
// side.  Dual: w1 and w3 interleaved in 16-column groups (virtual columns
// 32 g .. 32 g + 15 are w1 columns 16 g .., the next 16 the same w3 columns),
// so one wave's two 16-column tiles hold the gate and the up value of the same
// outputs.  Every matrix width is a multiple of 64, so an 8-column chunk never
// straddles two matrices or groups.
// The matrix is chosen among wave-uniform copies of the argument arrays
// (readfirstlane): indexing the arrays with a per-lane value, or selecting
// between their elements, makes the compiler load them per lane from the
// argument memory and wait for those loads before the first weight DMA.
__device__ __forceinline__ const bf16_t *b_column(const SkinnyArgs &a, int c, int &ld) {
    const int wc0 = uniform_i32(a.w_cols[0]), wc1 = uniform_i32(a.w_cols[1]), wc2 = uniform_i32(a.w_cols[2]);
    const bf16_t *w0 = (const bf16_t *)uniform_ptr(a.w[0]), *w1 = (const bf16_t *)uniform_ptr(a.w[1]),
                 *w2 = (const bf16_t *)uniform_ptr(a.w[2]);
    int s = 0;
    if (a.src == 2) {
        s = (c >> 4) & 1;
        c = 16 * (c >> 5) + (c & 15);
    } else if (a.src != 0) {
        if (w1 && c >= wc0) {
            c -= wc0;
            s = 1;
            if (w2 && c >= wc1) {
                c -= wc1;
                s = 2;
            }
        }
    }
    ld = s == 0 ? wc0 : (s == 1 ? wc1 : wc2);
    const bf16_t *base = s == 0 ? w0 : (s == 1 ? w1 : w2);
    return base + min(c, ld - 8);
}

// 32-byte granule swizzle of a weight row in LDS: the four rows one 16-lane
// group of a transpose read touches fall in distinct bank groups.
template <int BN>
__device__ __forceinline__ int skinny_gswz(int row) {
    if constexpr (BN >= 128) return swz_tr(row);
    else return row & 3;
}

template <int BN, int SK, int MT, bool XC>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs a) {
    // SK: k rows per stage.  XC: x is not loaded but built in LDS, once, from
    // the decode attention's chunk partials (a.ac), for the whole k range.
    constexpr int WST = SK * BN;               // weight elements per stage
    constexpr int XST = 16 * MT * SK;          // x elements per stage (the rows of the MT row tiles)
    constexpr int STAGE = XC ? WST : WST + XST;
    constexpr int XFULL = XC ? 16 * MT * kSkinnyXcMaxK : 0;  // XC: the activation slice
    constexpr int RING = 144 * 1024 - XFULL * 2;
    constexpr int NST = RING / (STAGE * 2) < 16 ? RING / (STAGE * 2) : 16;  // ring stages
    constexpr int WBLK = WST * 2 / 1024, XBLK = XC ? 0 : XST * 2 / 1024;  // 1 KB blocks
    constexpr int PW = WBLK / 4, PX = XBLK / 4, PER = PW + PX;   // DMAs per wave per stage
    constexpr int WRPB = 1024 / (BN * 2);      // weight rows per 1 KB block
    constexpr int CPR = BN / 8;                // 16-byte chunks per weight row
    constexpr int NC = BN / 64;                // 16-column tiles per wave
    constexpr int XCH = SK / 8;                // 16-byte chunks per x row
    constexpr int XRPL = XCH >= 8 ? 1 : 8 / XCH;  // x rows per 128 bytes (at least one)
    static_assert(PW * 4 == WBLK && PX * 4 == XBLK && WRPB >= 1, "stage splits into 1 KB blocks per wave");
    static_assert(NST >= 3 && (SK == 32 || SK == 64 || SK == 128), "ring depth and x row layout");
    static_assert(!XC || MT == 1, "the activation slice is one 16-row tile");
    __shared__ __attribute__((aligned(1024))) bf16_t lds[NST * STAGE + XFULL];
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t *)lds;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_cb = a.N / BN;
    const int cb = (int)blockIdx.x % n_cb, sp = (int)blockIdx.x / n_cb;
    const int c0 = cb * BN;
    const int n_st_all = a.K / SK;
    const int st_lo = sp * n_st_all / a.splits, st_hi = (sp + 1) * n_st_all / a.splits;
    const int n_st = st_hi - st_lo;

    // per-lane DMA sources (stage 0 of this range; later stages step by SK rows)
    const bf16_t *wsrc[PW];
    int wld[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int row = (wave * PW + i) * WRPB + lane / CPR, p = lane % CPR;
        const int col = c0 + 16 * ((p >> 1) ^ skinny_gswz<BN>(row)) + 8 * (p & 1);
        int ld;
        const bf16_t *base = b_column(a, col, ld);
        wld[i] = ld;
        wsrc[i] = base + (int64_t)(st_lo * SK + row) * ld;
    }
    const bf16_t *xsrc[PX > 0 ? PX : 1];
#pragma unroll
    for (int i = 0; i < PX; ++i) {
        // x rows of 2 SK bytes; chunk XOR (row / XRPL) keeps the 16-lane fragment reads conflict free
        const int row = (wave * PX + i) * (64 / XCH) + lane / XCH, p = lane % XCH;  // row < 16 MT
        xsrc[i] = a.x + (int64_t)min(row, a.M - 1) * a.ldx + st_lo * SK + 8 * (p ^ ((row / XRPL) & (XCH - 1)));
    }
    auto issue = [&](int st, int slot) {
        const uint32_t wb = __builtin_amdgcn_readfirstlane(lds_base + slot * STAGE * 2 + wave * PW * 1024);
        const uint32_t xb = __builtin_amdgcn_readfirstlane(lds_base + slot * STAGE * 2 + WST * 2 + wave * PX * 1024);
#pragma unroll
        for (int i = 0; i < PW; ++i) dma16_stream(wsrc[i] + (int64_t)st * SK * wld[i], wb + i * 1024);
#pragma unroll
        for (int i = 0; i < PX; ++i) dma16(xsrc[i] + st * SK, xb + i * 1024);
    };
    auto wait_stages = [&](int n) {  // at most n later stages of this wave still in flight
        static_assert((NST - 2) * PER < 64, "vmcnt range");
#define TFB_WAIT_CASE(k) \
    case k:                                   \
        wait_vmcnt<(k <= NST - 2 ? k : 0) * PER>(); \
        break;
        switch (n) {
            TFB_WAIT_CASE(1) TFB_WAIT_CASE(2) TFB_WAIT_CASE(3) TFB_WAIT_CASE(4) TFB_WAIT_CASE(5)
            TFB_WAIT_CASE(6) TFB_WAIT_CASE(7) TFB_WAIT_CASE(8) TFB_WAIT_CASE(9) TFB_WAIT_CASE(10)
            TFB_WAIT_CASE(11) TFB_WAIT_CASE(12) TFB_WAIT_CASE(13) TFB_WAIT_CASE(14)
            default: wait_vmcnt<0>(); break;
        }
#undef TFB_WAIT_CASE
    };
    f32x4 acc[MT][NC];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NC; ++t) acc[mt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // fragment geometry: 16-lane group g4 holds k 8 g4 .. 8 g4 + 7 of a 32-k step
    const int g4 = lane >> 4, ln = lane & 15;
    const int b_row = 8 * g4 + (ln >> 2), b_in = 4 * (ln & 3);
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < n_st) issue(s, s);
    bf16_t *const xfull = lds + NST * STAGE;
    if constexpr (XC) {
        // The activation slice, while the first weight stages load: row b,
        // columns st_lo*SK .. of att, merged from the chunk partials as the
        // merge pass does it (max, then the weighted sums in chunk order, one
        // division), rounded to bf16 and laid out per stage as the DMA would
        // have put it.  Rows past M repeat row M-1.
        const AttnChunks &ac = a.ac;
        const int kr = n_st * SK, groups = kr / 8;
        for (int it = tid; it < a.M * groups; it += 256) {
            const int b = it / groups, gq = it % groups;
            const int c0 = st_lo * SK + 8 * gq, h = c0 / ac.dh, e0 = c0 % ac.dh;
            const int pos = ac.pos[b];
            const int n_keys = ac.kvm.ring ? pos + 1 : min(pos + 1, ac.kvm.pos0 + ac.kvm.t_max);
            const int n_range = ac.window > 0 ? min(n_keys, ac.window) : n_keys;
            const int n_ch = min((n_range + ac.chunk_keys - 1) / ac.chunk_keys, ac.max_chunks);
            const float *base = ac.part + ((int64_t)b * ac.H + h) * ac.max_chunks * (ac.dh + 4);
            float M = -INFINITY, L = 0.0f, O[8] = {};
            if (n_ch <= 16) {
                float pm[16], pl[16];
                f32x4 pa[16], pb[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const float *p = base + c * (ac.dh + 4);
                    const bool in = c < n_ch;
                    pm[c] = in ? p[0] : -INFINITY;
                    pl[c] = in ? p[1] : 0.0f;
                    pa[c] = in ? *(const f32x4 *)(p + 4 + e0) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    pb[c] = in ? *(const f32x4 *)(p + 8 + e0) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
#pragma unroll
                for (int c = 0; c < 16; ++c) M = fmaxf(M, pm[c]);
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    if (c < n_ch) {
                        const float sc = __builtin_amdgcn_exp2f(pm[c] - M);
                        L += sc * pl[c];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            O[i] += sc * pa[c][i];
                            O[i + 4] += sc * pb[c][i];
                        }
                    }
                }
            } else {
                for (int c = 0; c < n_ch; ++c) M = fmaxf(M, base[c * (ac.dh + 4)]);
                for (int c = 0; c < n_ch; ++c) {
                    const float *p = base + c * (ac.dh + 4);
                    const float sc = __builtin_amdgcn_exp2f(p[0] - M);
                    L += sc * p[1];
#pragma unroll
                    for (int i = 0; i < 8; ++i) O[i] += sc * p[4 + e0 + i];
                }
            }
            const float inv = 1.0f / L;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = O[i] * inv;
            const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                             pack_bf16x2(v[6], v[7])};
            const int sl = (8 * gq) / SK, ch = ((8 * gq) % SK) / 8;
            for (int r = b; r < 16 * MT; r += (b == a.M - 1 ? 1 : 16 * MT)) {
                *(u32x4 *)(xfull + sl * XST + r * SK + 8 * (ch ^ ((r / XRPL) & (XCH - 1)))) = w;
            }
            if (cb == 0) *(u32x4 *)((bf16_t *)ac.att_out + (int64_t)b * ac.H * ac.dh + c0) = w;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's slice writes are done (the loop's first barrier publishes them)
    }
    for (int st = 0; st < n_st; ++st) {
        wait_stages(min(NST - 2, n_st - 1 - st));  // stage st landed
        asm volatile("s_barrier" ::: "memory");    // every wave's did; stage st-1's slot is free
        if (st + NST - 1 < n_st) issue(st + NST - 1, (st + NST - 1) % NST);
        const bf16_t *Ws = lds + (st % NST) * STAGE, *Xs = XC ? xfull + st * XST : Ws + WST;
#pragma unroll
        for (int ks = 0; ks < SK / 32; ++ks) {
            bf16x8 bf[NC], af[MT];
#pragma unroll
            for (int t = 0; t < NC; ++t) {
                const int gran = (wave * (BN / 4) + 16 * t) / 16;
                const int r0 = 32 * ks + b_row, r1 = r0 + 4;
                const u32x2 lo = lds_read_tr16(Ws + r0 * BN + ((gran ^ skinny_gswz<BN>(r0)) * 16) + b_in);
                const u32x2 hi = lds_read_tr16(Ws + r1 * BN + ((gran ^ skinny_gswz<BN>(r1)) * 16) + b_in);
                bf[t] = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = 16 * mt + ln, ch = 4 * ks + g4;
                af[mt] = as_bf16x8(*(const u32x4 *)(Xs + row * SK + 8 * (ch ^ ((row / XRPL) & (XCH - 1)))));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int t = 0; t < NC; ++t) acc[mt][t] = mfma16(af[mt], bf[t], acc[mt][t]);
        }
    }
    if (a.act) {
        // gate-up with one k range: tile 0 holds the gate and tile 1 the up
        // value of output column 16 * (group) + ln, rows 16 mt + 4 g4 + v
        static_assert(NC == 2 || BN != 128, "gate/up tile pair per wave");
        if constexpr (NC == 2) {
            const int lc = (c0 + wave * (BN / 4)) / 2 + ln;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = 16 * mt + 4 * g4 + v;
                    if (m < a.M) a.act[(int64_t)m * a.ld_act + lc] = f32_to_bf16(silu_f(acc[mt][0][v]) * acc[mt][1][v]);
                }
        }
        return;
    }
    // partial: rows 16 mt + 4 g4 + v, column c0 + wave * BN/4 + 16 t + ln
    float *dst = a.part + (int64_t)sp * a.M * a.N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 16 * mt + 4 * g4 + v;
            if (m >= a.M) continue;
#pragma unroll
            for (int t = 0; t < NC; ++t) dst[(int64_t)m * a.N + c0 + wave * (BN / 4) + 16 * t + ln] = acc[mt][t][v];
        }
}

// The reduce passes load every K-slice of their columns before adding them
// (in slice order, so the sums are the same): with the slice count known
// only at run time, a plain loop would wait for each slice's load in turn.
constexpr int kSkinnyMaxSplits = 16;

// Sum the K-slices in order and apply the epilogue.  One thread per pair of
// logical output columns.
template <int EPI>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float *part, int slices, int M, int N, int n_out,
                                                            EpiParams ep) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int pairs = n_out / 2;
    if (idx >= (int64_t)M * pairs) return;
    const int m = (int)(idx / pairs), c = 2 * (int)(idx % pairs);
    const int64_t stride = (int64_t)M * N;
    if constexpr (EPI == EPI_SWIGLU) {
        // output column c: gate at virtual column 32 (c / 16) + c % 16, up 16 later
        const float *p = part + (int64_t)m * N + 32 * (c >> 4) + (c & 15);
        float2 gv[kSkinnyMaxSplits], uv[kSkinnyMaxSplits];
#pragma unroll
        for (int s = 0; s < kSkinnyMaxSplits; ++s)
            if (s < slices) {
                gv[s] = *(const float2 *)(p + s * stride);
                uv[s] = *(const float2 *)(p + s * stride + 16);
            }
        float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
#pragma unroll
        for (int s = 0; s < kSkinnyMaxSplits; ++s)
            if (s < slices) {
                g0 += gv[s].x; g1 += gv[s].y; u0 += uv[s].x; u1 += uv[s].y;
            }
        epi_store_swiglu<bf16_t>(ep, m, c, g0, u0);
        epi_store_swiglu<bf16_t>(ep, m, c + 1, g1, u1);
    } else {
        const float *p = part + (int64_t)m * N + c;
        float2 pv[kSkinnyMaxSplits];
#pragma unroll
        for (int s = 0; s < kSkinnyMaxSplits; ++s)
            if (s < slices) pv[s] = *(const float2 *)(p + s * stride);
        float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
        for (int s = 0; s < kSkinnyMaxSplits; ++s)
            if (s < slices) {
                v0 += pv[s].x;
                v1 += pv[s].y;
            }
        epi_store_pair<EPI, bf16_t>(ep, m, c, v0, v1);
    }
}

// Reduce + residual + RMSNorm of one row per workgroup (EPI_RESID with a
// norm): out = res + sum of the k-range partials in order (stored in out's
// storage type), then the stored row is normalised, as the separate norm
// kernel would read it back, and written to norm_out in bf16
// ([TIR] Code, rms_norm: y = x / sqrt(mean(x^2) + eps) * g).
template <int IT, int NT>
__global__ __launch_bounds__(NT) void skinny_reduce_norm_kernel(const float *part, int slices, int M, int N,
                                                                EpiParams ep, const bf16_t *g, bf16_t *hn, float eps) {
    const int m = blockIdx.x, tid = threadIdx.x;
    if (m >= M) return;
    const int64_t stride = (int64_t)M * N;
    float v[IT][8];
    float ss = 0.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int c = (it * NT + tid) * 8;
        if (c >= N) continue;
        const float *p = part + (int64_t)m * N + c;
        f32x4 pa[kSkinnyMaxSplits], pb[kSkinnyMaxSplits];
#pragma unroll
        for (int s = 0; s < kSkinnyMaxSplits; ++s)
            if (s < slices) {
                pa[s] = *(const f32x4 *)(p + s * stride);
                pb[s] = *(const f32x4 *)(p + s * stride + 4);
            }
        f32x4 a = pa[0], b = pb[0];
#pragma unroll
        for (int s = 1; s < kSkinnyMaxSplits; ++s)
            if (s < slices) {
                a += pa[s];
                b += pb[s];
            }
        float r[8];
        if (ep.res_f32) {
            const float *rr = (const float *)ep.res + (int64_t)m * ep.ldr + c;
            const f32x4 x0 = *(const f32x4 *)rr, x1 = *(const f32x4 *)(rr + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) { r[k] = x0[k]; r[k + 4] = x1[k]; }
        } else {
            load_bf16x8((const bf16_t *)ep.res + (int64_t)m * ep.ldr + c, r);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) { v[it][k] = r[k] + a[k]; v[it][k + 4] = r[k + 4] + b[k]; }
        if (ep.out_f32) {
            float *o = (float *)ep.out + (int64_t)m * ep.ldo + c;
            *(f32x4 *)o = f32x4{v[it][0], v[it][1], v[it][2], v[it][3]};
            *(f32x4 *)(o + 4) = f32x4{v[it][4], v[it][5], v[it][6], v[it][7]};
        } else {
            store_bf16x8((bf16_t *)ep.out + (int64_t)m * ep.ldo + c, v[it]);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[it][k] = bf16_to_f32(f32_to_bf16(v[it][k]));  // the stored value
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += v[it][k] * v[it][k];
    }
    __shared__ float red[NT / 64];
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    ss = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) ss += red[w];
    const float rs = 1.0f / sqrtf(ss / (float)N + eps);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int c = (it * NT + tid) * 8;
        if (c >= N) continue;
        float gv[8], o[8];
        load_bf16x8(g + c, gv);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = v[it][k] * rs * gv[k];
        store_bf16x8(hn + (int64_t)m * N + c, o);
    }
}

// Column block width and k splits of a skinny GEMM: 128-column blocks when N
// allows (each workgroup also streams its x slice, 64/BN of its weight bytes),
// then k is split so that the workgroups come close to one per compute unit
// without exceeding it.
// Stage depth by row tiles: the x part of a stage (16 MT rows of SK k) must
// split into whole 1 KB blocks over the four waves.
constexpr int skinny_sk(int mt) { return (mt == 1 || mt == 3) ? 128 : 64; }
// Row tiles a launch uses: one more than M needs when K does not take
// 128-deep stages (the extra tile holds clamped copies of the last row).
static int skinny_mt(int M, int K) {
    int mt = (M + 15) / 16;
    if ((mt == 1 || mt == 3) && K % 128) ++mt;
    return mt;
}

static void skinny_plan(int M, int K, int N, int &bn, int &splits) {
    bn = N % 128 == 0 ? 128 : 64;
    const int n_cb = N / bn;
    splits = std::max(1, std::min(device_cus() / n_cb, K / skinny_sk(skinny_mt(M, K))));
    splits = std::min(splits, kSkinnyMaxSplits);
}

size_t skinny_part_bytes(int M, int K, int N) {
    int bn, splits;
    skinny_plan(M, K, N, bn, splits);
    return (size_t)splits * M * N * sizeof(float);
}

bool skinny_takes_attn_chunks(int M, int K, int N) {
    if (M < 1 || M > kSkinnyMaxM || K % 64 || N % 64 || skinny_mt(M, K) != 1) return false;
    int bn, splits;
    skinny_plan(M, K, N, bn, splits);
    const int n_st = K / skinny_sk(1);
    return (n_st + splits - 1) / splits * skinny_sk(1) <= kSkinnyXcMaxK;  // the longest k range of a workgroup
}

template <int BN>
static void skinny_launch_bn(const SkinnyArgs &a, int blocks, hipStream_t s, bool xc) {
    if (xc) {  // one 16-row tile (checked by skinny_takes_attn_chunks)
        hipLaunchKernelGGL((skinny_gemm_kernel<BN, skinny_sk(1), 1, true>), dim3(blocks), dim3(256), 0, s, a);
        return;
    }
    switch (skinny_mt(a.M, a.K)) {
        case 1: hipLaunchKernelGGL((skinny_gemm_kernel<BN, skinny_sk(1), 1, false>), dim3(blocks), dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((skinny_gemm_kernel<BN, skinny_sk(2), 2, false>), dim3(blocks), dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((skinny_gemm_kernel<BN, skinny_sk(3), 3, false>), dim3(blocks), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((skinny_gemm_kernel<BN, skinny_sk(4), 4, false>), dim3(blocks), dim3(256), 0, s, a); break;
    }
}

hipError_t skinny_gemm_launch(const GemmCall &c, void *part, size_t part_bytes, hipStream_t s) {
    SkinnyArgs a{};
    a.x = (const bf16_t *)c.A;
    a.ldx = c.lda;
    a.M = c.M;
    a.K = c.K;
    int n_out = c.ep.N;
    for (int i = 0; i < 3; ++i) { a.w[i] = (const bf16_t *)c.w[i]; a.w_cols[i] = c.w_cols[i]; }
    if (c.epi == EPI_QKV) { a.src = 1; a.N = c.w_cols[0] + c.w_cols[1] + c.w_cols[2]; }
    else if (c.epi == EPI_SWIGLU) { a.src = 2; a.N = 2 * c.w_cols[0]; a.w[2] = nullptr; }
    else { a.src = 0; a.N = c.w_cols[0]; a.w[1] = a.w[2] = nullptr; }
    // the stage and block layout needs whole 64-row stages and 64-column
    // blocks, 16-byte aligned rows of x, and every matrix a multiple of 64 wide
    if (a.M < 1 || a.M > 64 || a.K % 64 || a.N % 64 || a.ldx % 8) return hipErrorInvalidValue;
    // x from the decode attention's chunk partials: one 16-row tile, short
    // k ranges, a plain residual GEMM over the head outputs (K = H * dh)
    const bool xc = c.attn_chunks != nullptr;
    if (xc) {
        const AttnChunks &ac = *c.attn_chunks;
        if (c.epi != EPI_RESID || !skinny_takes_attn_chunks(a.M, a.K, a.N) || a.K != ac.H * ac.dh || ac.dh % 8 ||
            !ac.part || !ac.pos || !ac.att_out || ac.chunk_keys < 1 || ac.max_chunks < 1)
            return hipErrorInvalidValue;
        a.ac = ac;
    }
    for (int i = 0; i < 3; ++i)
        if (a.w[i] && a.w_cols[i] % 64) return hipErrorInvalidValue;
    int bn;
    skinny_plan(a.M, a.K, a.N, bn, a.splits);
    if (a.splits > kSkinnyMaxSplits) return hipErrorInvalidValue;  // the reduce passes hold at most this many
    if ((size_t)a.splits * a.M * a.N * sizeof(float) > part_bytes) return hipErrorInvalidValue;
    a.part = (float *)part;
    // gate-up in one k range: the kernel applies SiLU(gate) * up itself
    const bool direct = c.epi == EPI_SWIGLU && a.splits == 1 && bn == 128;
    if (direct) {
        a.act = (bf16_t *)c.ep.out;
        a.ld_act = c.ep.ldo;
    }
    const int blocks = (a.N / bn) * a.splits;
    if (bn == 128) skinny_launch_bn<128>(a, blocks, s, xc);
    else skinny_launch_bn<64>(a, blocks, s, xc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    if (c.epi == EPI_QKV && c.qkv_deferred_splits) {  // the decode attention kernel reduces them
        *c.qkv_deferred_splits = a.splits;
        return hipSuccess;
    }
    if (c.norm_g) {
        // the caller skips its own norm launch, so a norm that cannot be fused is an error
        if (c.epi != EPI_RESID || n_out > kSkinnyNormMaxN || n_out % 8 || !c.norm_out) return hipErrorInvalidValue;
        // one workgroup per row (a decode batch has few rows): 8 columns per
        // thread, so that each thread's slice loads go out in one round
        const dim3 ng(a.M);
        if (n_out <= 2048)
            hipLaunchKernelGGL((skinny_reduce_norm_kernel<1, 256>), ng, dim3(256), 0, s, a.part, a.splits, a.M, a.N,
                               c.ep, (const bf16_t *)c.norm_g, (bf16_t *)c.norm_out, c.norm_eps);
        else if (n_out <= 4096)
            hipLaunchKernelGGL((skinny_reduce_norm_kernel<1, 512>), ng, dim3(512), 0, s, a.part, a.splits, a.M, a.N,
                               c.ep, (const bf16_t *)c.norm_g, (bf16_t *)c.norm_out, c.norm_eps);
        else
            hipLaunchKernelGGL((skinny_reduce_norm_kernel<2, 512>), ng, dim3(512), 0, s, a.part, a.splits, a.M, a.N,
                               c.ep, (const bf16_t *)c.norm_g, (bf16_t *)c.norm_out, c.norm_eps);
        return hipGetLastError();
    }
    const int64_t threads = (int64_t)a.M * (n_out / 2);
    dim3 rg((unsigned)((threads + 255) / 256));
    switch (c.epi) {
        case EPI_QKV: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_QKV>, rg, dim3(256), 0, s, a.part, a.splits, a.M, a.N, n_out, c.ep); break;
        case EPI_RESID: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_RESID>, rg, dim3(256), 0, s, a.part, a.splits, a.M, a.N, n_out, c.ep); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_SWIGLU>, rg, dim3(256), 0, s, a.part, a.splits, a.M, a.N, n_out, c.ep); break;
        case EPI_F32: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_F32>, rg, dim3(256), 0, s, a.part, a.splits, a.M, a.N, n_out, c.ep); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tfb
