// Skinny weight GEMMs of the decode step: y = x W with few rows (M = number
// of sequences, at most 64) and W [K, N] streamed from HBM exactly once.
// Page short names: [TIR] tirogla "Transformer block", [PID] pidoku "The
// Transformer" (6. Under the hood: a decode step reads every weight once and
// is bandwidth bound).
//
// Work unit = one wave: a 128-column block of W times a K-slice.  Per 32-row
// k step a lane loads 8 rows x 16 bytes of W (lanes l and l+16k read whole
// 256-byte row segments, so each load instruction covers 4 full rows) with
// the nontemporal hint, transposes the 8x8 block in registers and feeds it as
// the B operand of eight MFMA 16x16x32 (output column n of MFMA c is
// 8n + c of the block).  x fragments (the A operand) come through L1/L2.
// Several k steps are in flight per wave.  Each wave writes an fp32 partial
// [slice][M][N]; a second kernel adds the slices in a fixed order and applies
// the fused epilogue (RoPE + KV append, residual, SwiGLU, fp32 store), so the
// result is deterministic.
#include <algorithm>

#include "epilogue.h"
#include "kernels.h"

namespace tfb {

struct SkinnyArgs {
    const bf16_t *x;  // [M, K]
    int64_t ldx;
    int M, K, N;      // N = columns of the virtual B
    int slices, ks;   // K-slices and rows per slice (multiple of 32)
    const bf16_t *w[3];
    int w_cols[3];
    int src;          // 0: one matrix, 1: concat (wq|wk|wv), 2: two matrices side by side (w1|w3)
    float *part;      // [slices][M][N]
};

// Column c of the virtual B -> (matrix, column).  Concat: matrices side by
// side; dual: w1 columns then w3 columns.
__device__ __forceinline__ const bf16_t *b_column(const SkinnyArgs &a, int c, int &ld, bool &ok) {
    int s = 0;
    if (a.src != 0) {
        while (s < 2 && a.w[s + 1] && c >= a.w_cols[s]) { c -= a.w_cols[s]; ++s; }
    }
    ld = a.w_cols[s];
    ok = c < ld;
    return a.w[s] + (ok ? c : 0);
}

template <int MT, int UNROLL>
__global__ __launch_bounds__(64) void skinny_gemm_kernel(SkinnyArgs a) {
    // one wave per workgroup, so the tasks spread over every CU
    const int lane = threadIdx.x & 63;
    const int ln = lane & 15, g4 = lane >> 4;
    const int n_cb = (a.N + 127) / 128;
    const int task = blockIdx.x;
    if (task >= n_cb * a.slices) return;  // no barriers in this kernel
    const int cb = task % n_cb, sl = task / n_cb;
    const int c0 = cb * 128;
    const int k_lo = sl * a.ks, k_hi = min(a.K, k_lo + a.ks);

    int ld;
    bool col_ok;
    const bf16_t *wcol = b_column(a, c0 + 8 * ln, ld, col_ok);

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[mt][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int k0 = k_lo; k0 < k_hi; k0 += 32 * UNROLL) {
        u32x4 wr[UNROLL][8];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = k0 + 32 * u + 8 * g4;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int k = kb + r;
                wr[u][r] = (col_ok && k < k_hi) ? ld_stream(wcol + (int64_t)k * ld) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = k0 + 32 * u + 8 * g4;
            bf16x8 af[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int m = 16 * mt + ln;
                u32x4 v = {0, 0, 0, 0};
                if (m < a.M && kb < k_hi) v = *(const u32x4 *)(a.x + (int64_t)m * a.ldx + kb);
                af[mt] = as_bf16x8(v);
            }
            u32x4 wt[8];
            transpose8x8_bf16(wr[u], wt);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][c] = mfma16(af[mt], as_bf16x8(wt[c]), acc[mt][c]);
        }
    }
    // partial: rows 16mt + 4*g4 + v, columns c0 + 8*ln + c (c = 0..7)
    const int col = c0 + 8 * ln;
    if (col >= a.N) return;
    float *dst = a.part + (int64_t)sl * a.M * a.N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 16 * mt + 4 * g4 + v;
            if (m >= a.M) continue;
            float *p = dst + (int64_t)m * a.N + col;
            *(f32x4 *)p = f32x4{acc[mt][0][v], acc[mt][1][v], acc[mt][2][v], acc[mt][3][v]};
            *(f32x4 *)(p + 4) = f32x4{acc[mt][4][v], acc[mt][5][v], acc[mt][6][v], acc[mt][7][v]};
        }
}

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
        // gate columns [0, n_out), up columns [n_out, 2 n_out)
        float g0 = 0.0f, g1 = 0.0f, u0 = 0.0f, u1 = 0.0f;
        const float *p = part + (int64_t)m * N + c;
        for (int s = 0; s < slices; ++s) {
            const float2 gv = *(const float2 *)(p + s * stride);
            const float2 uv = *(const float2 *)(p + s * stride + n_out);
            g0 += gv.x; g1 += gv.y; u0 += uv.x; u1 += uv.y;
        }
        epi_store_swiglu<bf16_t>(ep, m, c, g0, u0);
        epi_store_swiglu<bf16_t>(ep, m, c + 1, g1, u1);
    } else {
        float v0 = 0.0f, v1 = 0.0f;
        const float *p = part + (int64_t)m * N + c;
        for (int s = 0; s < slices; ++s) {
            const float2 v = *(const float2 *)(p + s * stride);
            v0 += v.x;
            v1 += v.y;
        }
        epi_store_pair<EPI, bf16_t>(ep, m, c, v0, v1);
    }
}

// Splits of K for a skinny GEMM: enough waves to keep many loads in flight,
// while the fp32 partials stay below half of the weight bytes.
static void skinny_split(int M, int K, int N, int &slices, int &ks) {
    const int n_cb = (N + 127) / 128;
    const int mpad = ((M + 15) / 16) * 16;
    int s_cap = (K * 2) / (2 * 4 * mpad);       // partial bytes <= weight bytes / 2
    int s_want = (2048 + n_cb - 1) / n_cb;      // ~2048 waves
    int s = std::max(1, std::min(s_cap, s_want));
    s = std::min(s, K / 32);
    ks = ((K + s - 1) / s + 31) / 32 * 32;
    slices = (K + ks - 1) / ks;
}

size_t skinny_part_bytes(int M, int K, int N) {
    int slices, ks;
    skinny_split(M, K, N, slices, ks);
    return (size_t)slices * M * N * sizeof(float);
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
    skinny_split(a.M, a.K, a.N, a.slices, a.ks);
    if ((size_t)a.slices * a.M * a.N * sizeof(float) > part_bytes || a.M > 64) return hipErrorInvalidValue;
    a.part = (float *)part;
    const int n_cb = (a.N + 127) / 128;
    const int waves = n_cb * a.slices;
    dim3 grid(waves);
    const int mt = (a.M + 15) / 16;
    switch (mt) {
        case 1: hipLaunchKernelGGL((skinny_gemm_kernel<1, 4>), grid, dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((skinny_gemm_kernel<2, 4>), grid, dim3(64), 0, s, a); break;
        case 3: hipLaunchKernelGGL((skinny_gemm_kernel<3, 2>), grid, dim3(64), 0, s, a); break;
        default: hipLaunchKernelGGL((skinny_gemm_kernel<4, 2>), grid, dim3(64), 0, s, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)a.M * (n_out / 2);
    dim3 rg((unsigned)((threads + 255) / 256));
    switch (c.epi) {
        case EPI_QKV: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_QKV>, rg, dim3(256), 0, s, a.part, a.slices, a.M, a.N, n_out, c.ep); break;
        case EPI_RESID: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_RESID>, rg, dim3(256), 0, s, a.part, a.slices, a.M, a.N, n_out, c.ep); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_SWIGLU>, rg, dim3(256), 0, s, a.part, a.slices, a.M, a.N, n_out, c.ep); break;
        case EPI_F32: hipLaunchKernelGGL(skinny_reduce_kernel<EPI_F32>, rg, dim3(256), 0, s, a.part, a.slices, a.M, a.N, n_out, c.ep); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tfb
