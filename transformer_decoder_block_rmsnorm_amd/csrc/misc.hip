// Small kernels of the decoder-block path: RMSNorm, RoPE table, KV append,
// embedding gather, last-row gather, greedy argmax, position updates.
// Page short names: [TIR] tirogla "Transformer block", [PID] pidoku "The
// Transformer".
#include <atomic>

#include <type_traits>

#include "kernels.h"

namespace tfb {

int device_cus() {
    static std::atomic<int> cache[64];  // zero-initialised: not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// RMSNorm ([TIR] Code, rms_norm; [PID] Tiny example, rmsnorm): one wave per
// row, fp32 sum of squares reduced across the wave, y = x * r * g.
// Vector path (bf16 output): each lane owns NCH 16-byte chunks of the row
// (chunk i of lane l holds elements 64 EPC i + EPC l ..), loads them all at
// once, keeps them in registers for the reduction and the scaled write, so a
// row is read from memory once.  Other widths or fp32 output: a plain
// two-pass loop.
template <typename Tin, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(const Tin *x, int64_t ldx, const bf16_t *g, bf16_t *y,
                                                          int64_t ldy, int rows, float eps) {
    constexpr int EPC = 16 / sizeof(Tin);  // elements per 16-byte chunk
    constexpr int D = 64 * EPC * NCH;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const Tin *xr = x + (int64_t)row * ldx;
    u32x4 v[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) v[i] = *(const u32x4 *)(xr + 64 * EPC * i + EPC * lane);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if constexpr (EPC == 8) {
                const float a = bf16_lo(v[i][w]), b = bf16_hi(v[i][w]);
                ss += a * a + b * b;
            } else {
                const float a = __uint_as_float(v[i][w]);
                ss += a * a;
            }
        }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    bf16_t *yr = y + (int64_t)row * ldy;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = 64 * EPC * i + EPC * lane;
        if constexpr (EPC == 8) {
            const u32x4 gv = *(const u32x4 *)(g + c);
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                o[w] = pack_bf16x2(bf16_lo(v[i][w]) * r * bf16_lo(gv[w]), bf16_hi(v[i][w]) * r * bf16_hi(gv[w]));
            *(u32x4 *)(yr + c) = o;
        } else {
            const u32x2 gv = *(const u32x2 *)(g + c);
            u32x2 o;
            o[0] = pack_bf16x2(__uint_as_float(v[i][0]) * r * bf16_lo(gv[0]), __uint_as_float(v[i][1]) * r * bf16_hi(gv[0]));
            o[1] = pack_bf16x2(__uint_as_float(v[i][2]) * r * bf16_lo(gv[1]), __uint_as_float(v[i][3]) * r * bf16_hi(gv[1]));
            *(u32x2 *)(yr + c) = o;
        }
    }
}

template <typename Tin, typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const Tin *x, int64_t ldx, const T *g, T *y, int64_t ldy,
                                                      int rows, int d, float eps) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const Tin *xr = x + (int64_t)row * ldx;
    T *yr = y + (int64_t)row * ldy;
    float ss = 0.0f;
    for (int c = lane; c < d; c += 64) {
        const float a = Elem<Tin>::load(xr, c);
        ss += a * a;
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < d; c += 64) Elem<T>::store(yr, c, Elem<Tin>::load(xr, c) * r * Elem<T>::load(g, c));
}

template <typename Tin>
static bool rmsnorm_vec_launch(dim3 grid, const Tin *x, int64_t ldx, const bf16_t *g, bf16_t *y, int64_t ldy,
                               int rows, int d, float eps, hipStream_t s) {
    constexpr int EPC = 16 / sizeof(Tin);
    if (d % (64 * EPC) || ldx % EPC || ldy % 8) return false;
    switch (d / (64 * EPC)) {
        case 1: hipLaunchKernelGGL((rmsnorm_vec_kernel<Tin, 1>), grid, dim3(256), 0, s, x, ldx, g, y, ldy, rows, eps); return true;
        case 2: hipLaunchKernelGGL((rmsnorm_vec_kernel<Tin, 2>), grid, dim3(256), 0, s, x, ldx, g, y, ldy, rows, eps); return true;
        case 4: hipLaunchKernelGGL((rmsnorm_vec_kernel<Tin, 4>), grid, dim3(256), 0, s, x, ldx, g, y, ldy, rows, eps); return true;
        case 8: hipLaunchKernelGGL((rmsnorm_vec_kernel<Tin, 8>), grid, dim3(256), 0, s, x, ldx, g, y, ldy, rows, eps); return true;
        case 16: hipLaunchKernelGGL((rmsnorm_vec_kernel<Tin, 16>), grid, dim3(256), 0, s, x, ldx, g, y, ldy, rows, eps); return true;
        default: return false;
    }
}

hipError_t rmsnorm_launch(int dtype, const void *x, int64_t ldx, const void *g, void *y, int64_t ldy, int rows, int d,
                          float eps, hipStream_t s, bool x_f32) {
    dim3 grid((rows + 3) / 4);
    if (dtype == TFB_BF16 && !x_f32) {
        if (!rmsnorm_vec_launch<bf16_t>(grid, (const bf16_t *)x, ldx, (const bf16_t *)g, (bf16_t *)y, ldy, rows, d, eps, s))
            hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, (const bf16_t *)x, ldx,
                               (const bf16_t *)g, (bf16_t *)y, ldy, rows, d, eps);
    } else if (dtype == TFB_BF16) {
        if (!rmsnorm_vec_launch<float>(grid, (const float *)x, ldx, (const bf16_t *)g, (bf16_t *)y, ldy, rows, d, eps, s))
            hipLaunchKernelGGL((rmsnorm_kernel<float, bf16_t>), grid, dim3(256), 0, s, (const float *)x, ldx,
                               (const bf16_t *)g, (bf16_t *)y, ldy, rows, d, eps);
    } else {
        hipLaunchKernelGGL((rmsnorm_kernel<float, float>), grid, dim3(256), 0, s, (const float *)x, ldx,
                           (const float *)g, (float *)y, ldy, rows, d, eps);
    }
    return hipGetLastError();
}

// RoPE table ([TIR] Implementation notes: a [T_max, dh/2] cos/sin table;
// frequencies base^(-2i/dh) over interleaved pairs).  fp64 angle, fp32 values.
__global__ void rope_table_kernel(int t_max, int dh, double base, float *table) {
    const int half = dh / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)t_max * half) return;
    const int t = (int)(idx / half), i = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)i / (double)dh);
    const double a = (double)t * theta;
    table[2 * idx] = (float)cos(a);
    table[2 * idx + 1] = (float)sin(a);
}

hipError_t rope_table_launch(int t_max, int dh, double base, float *table, hipStream_t s) {
    const int64_t n = (int64_t)t_max * (dh / 2);
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, t_max, dh, base, table);
    return hipGetLastError();
}

// KV append ([TIR] How it works, KV cache): [B, n, Hkv, dh] -> cache rows
// start[b] + t (or their ring slots).  One thread per pair of elements (dh is even, so a pair never
// straddles a row and every pair is 4- or 8-byte aligned); positions the
// cache has no slot for are skipped.
template <typename T>
__global__ void kv_append_kernel(T *kc, T *vc, const T *kn, const T *vn, const int32_t *start, int B, int n_new,
                                 int Hkv, int dh, KvMap kvm) {
    typedef typename std::conditional<sizeof(T) == 2, uint32_t, u32x2>::type Pair;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per_row = dh / 2;
    const int64_t total = (int64_t)B * n_new * Hkv * per_row;
    if (idx >= total) return;
    const int e2 = (int)(idx % per_row);
    int64_t r = idx / per_row;
    const int g = (int)(r % Hkv);
    r /= Hkv;
    const int t = (int)(r % n_new);
    const int b = (int)(r / n_new);
    const int p = start[b] + t;
    if (!kv_has(kvm, p)) return;
    const int64_t src = (((int64_t)b * n_new + t) * Hkv + g) * dh + e2 * 2;
    const int64_t dst = kv_row(kvm, b, Hkv, g, p) * dh + e2 * 2;
    *(Pair *)(kc + dst) = *(const Pair *)(kn + src);
    *(Pair *)(vc + dst) = *(const Pair *)(vn + src);
}

hipError_t kv_append_launch(int dtype, void *kc, void *vc, const void *k_new, const void *v_new, const int32_t *start,
                            int B, int n_new, int Hkv, int dh, const KvMap &kvm, hipStream_t s) {
    const int64_t total = (int64_t)B * n_new * Hkv * (dh / 2);
    dim3 grid((unsigned)((total + 255) / 256));
    if (dtype == TFB_BF16)
        hipLaunchKernelGGL(kv_append_kernel<bf16_t>, grid, dim3(256), 0, s, (bf16_t *)kc, (bf16_t *)vc,
                           (const bf16_t *)k_new, (const bf16_t *)v_new, start, B, n_new, Hkv, dh, kvm);
    else
        hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, (float *)kc, (float *)vc,
                           (const float *)k_new, (const float *)v_new, start, B, n_new, Hkv, dh, kvm);
    return hipGetLastError();
}

// Copy the keys and values of positions p_lo .. p_lo+n-1 of every sequence
// and KV head between two caches with different row maps (a bounded window
// cache and the contiguous staging copy a prefill works in).  16-byte chunks;
// a position either map has no slot for is skipped.
__global__ void kv_copy_kernel(const uint8_t *sk, const uint8_t *sv, KvMap sm, uint8_t *dk, uint8_t *dv, KvMap dm,
                               int B, int Hkv, int row_bytes, int p_lo, int n) {
    const int chunks = row_bytes / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)B * Hkv * n * chunks) return;
    const int c = (int)(idx % chunks);
    int64_t r = idx / chunks;
    const int p = p_lo + (int)(r % n);
    r /= n;
    const int g = (int)(r % Hkv), b = (int)(r / Hkv);
    if (!kv_has(sm, p) || !kv_has(dm, p)) return;
    const int64_t so = kv_row(sm, b, Hkv, g, p) * row_bytes + c * 16, d = kv_row(dm, b, Hkv, g, p) * row_bytes + c * 16;
    *(u32x4 *)(dk + d) = *(const u32x4 *)(sk + so);
    *(u32x4 *)(dv + d) = *(const u32x4 *)(sv + so);
}

hipError_t kv_copy_launch(int dtype, const void *sk, const void *sv, const KvMap &sm, void *dk, void *dv,
                          const KvMap &dm, int B, int Hkv, int dh, int p_lo, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int row_bytes = dh * (dtype == TFB_BF16 ? 2 : 4);
    if (row_bytes % 16) return hipErrorInvalidValue;
    const int64_t total = (int64_t)B * Hkv * n * (row_bytes / 16);
    hipLaunchKernelGGL(kv_copy_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, (const uint8_t *)sk,
                       (const uint8_t *)sv, sm, (uint8_t *)dk, (uint8_t *)dv, dm, B, Hkv, row_bytes, p_lo, n);
    return hipGetLastError();
}

// Embedding gather ([PID] Tiny example, forward: x[s] = Embed[id]); 16-byte
// chunks; an id outside [0, vocab) yields a zero row.
__global__ void embed_kernel(const int32_t *ids, const uint8_t *table, uint8_t *x, int64_t rows, int row_bytes,
                             int vocab) {
    const int chunks = row_bytes / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * chunks) return;
    const int64_t r = idx / chunks;
    const int c = (int)(idx % chunks);
    const int id = ids[r];
    u32x4 v = {0, 0, 0, 0};
    if (id >= 0 && id < vocab) v = *(const u32x4 *)(table + (int64_t)id * row_bytes + c * 16);
    *(u32x4 *)(x + r * row_bytes + c * 16) = v;
}

hipError_t embed_launch(int dtype, const int32_t *ids, const void *table, void *x, int64_t rows, int d, int vocab,
                        hipStream_t s) {
    const int row_bytes = d * (dtype == TFB_BF16 ? 2 : 4);
    const int64_t n = rows * (row_bytes / 16);
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids,
                       (const uint8_t *)table, (uint8_t *)x, rows, row_bytes, vocab);
    return hipGetLastError();
}

__global__ void gather_last_kernel(const uint8_t *x, uint8_t *y, int B, int T, int row_bytes) {
    const int chunks = row_bytes / 16;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)B * chunks) return;
    const int b = (int)(idx / chunks), c = (int)(idx % chunks);
    *(u32x4 *)(y + (int64_t)b * row_bytes + c * 16) =
        *(const u32x4 *)(x + ((int64_t)b * T + T - 1) * row_bytes + c * 16);
}

hipError_t gather_last_launch(int dtype, const void *x, void *y, int B, int T, int d, hipStream_t s) {
    const int row_bytes = d * (dtype == TFB_BF16 ? 2 : 4);
    const int64_t n = (int64_t)B * (row_bytes / 16);
    hipLaunchKernelGGL(gather_last_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)x, (uint8_t *)y, B, T, row_bytes);
    return hipGetLastError();
}

// Greedy next token: argmax of each row, lowest index among equal maxima.
// One 1024-thread workgroup per row (a decode batch has few rows): 16-byte
// loads, unrolled so that a thread's loads are in flight together; each
// thread visits its elements in increasing index order and keeps the first
// maximum, then the threads' (value, index) pairs are merged, preferring the
// lower index on equal values.
__device__ __forceinline__ void argmax_merge(float &bv, int &bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}
__global__ __launch_bounds__(1024) void argmax_kernel(const float *logits, int64_t ld, int n, int32_t *out) {
    const float *row = logits + (int64_t)blockIdx.x * ld;
    const int tid = threadIdx.x;
    float best = -INFINITY;
    int idx = 0x7FFFFFFF;
    if ((ld % 4) == 0 && ((uintptr_t)logits % 16) == 0) {
        const int n4 = n / 4;
#pragma unroll 8
        for (int i = tid; i < n4; i += 1024) {
            const f32x4 v = *(const f32x4 *)(row + 4 * i);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (v[k] > best) { best = v[k]; idx = 4 * i + k; }
        }
        for (int j = 4 * n4 + tid; j < n; j += 1024) {  // tail: indices above every vector element
            const float v = row[j];
            if (v > best) { best = v; idx = j; }
        }
    } else {
        for (int j = tid; j < n; j += 1024) {
            const float v = row[j];
            if (v > best) { best = v; idx = j; }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        argmax_merge(best, idx, __shfl_xor(best, o, 64), __shfl_xor(idx, o, 64));
    __shared__ float sv[16];
    __shared__ int si[16];
    if ((tid & 63) == 0) { sv[tid >> 6] = best; si[tid >> 6] = idx; }
    __syncthreads();
    if (tid < 64) {
        best = tid < 16 ? sv[tid] : -INFINITY;
        idx = tid < 16 ? si[tid] : 0x7FFFFFFF;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1)
            argmax_merge(best, idx, __shfl_xor(best, o, 64), __shfl_xor(idx, o, 64));
        if (tid == 0) out[blockIdx.x] = idx == 0x7FFFFFFF ? 0 : idx;
    }
}

hipError_t argmax_launch(const float *logits, int64_t ld, int rows, int n, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(1024), 0, s, logits, ld, n, out);
    return hipGetLastError();
}

__global__ void add_scalar_kernel(int32_t *v, int n, int32_t add) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) v[i] += add;
}
__global__ void fill_i32_kernel(int32_t *v, int n, int32_t value) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) v[i] = value;
}

hipError_t add_scalar_launch(int32_t *v, int n, int32_t add, hipStream_t s) {
    hipLaunchKernelGGL(add_scalar_kernel, dim3((n + 255) / 256), dim3(256), 0, s, v, n, add);
    return hipGetLastError();
}
hipError_t fill_i32_launch(int32_t *v, int n, int32_t value, hipStream_t s) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, v, n, value);
    return hipGetLastError();
}

}  // namespace tfb
