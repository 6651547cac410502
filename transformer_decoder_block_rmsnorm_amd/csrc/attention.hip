// Causal grouped-query attention over the KV cache.
// Page short names: [TIR] tirogla "Transformer block", [MSA] msaqlain "AI
// engineering: transformers", [GEN] thegeniusblogs "The Transformer
// Architecture".
//
// The query of token t of sequence b sits at absolute position
// p = pos[b] (decode) or start + t (prefill) and attends cache rows 0..p
// (causal, key j <= query i: [TIR] How it works step 2; [MSA] 5.1).  Query
// head h reads KV head h / (H / Hkv): consecutive query heads share a KV head
// ([TIR] Code, the GQA index in Block::forward).  Softmax in fp32 with a running maximum ([TIR]
// Implementation notes; [MSA] 1.3).
#include "kernels.h"

namespace tfb {

// One wave per (b, h, t): lanes take 64 keys at a time, online softmax over
// the chunks, each lane accumulates dh/64 output dimensions.  Serves the fp32
// storage path and decode.
template <typename T>
__global__ __launch_bounds__(256) void attn_rowwise_kernel(AttnCall a) {
    __shared__ float qs[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + wave;
    const int64_t total = (int64_t)a.B * a.H * a.T;
    const bool valid = w < total;
    int t = 0, h = 0, b = 0;
    if (valid) {
        t = (int)(w % a.T);
        h = (int)((w / a.T) % a.H);
        b = (int)(w / ((int64_t)a.T * a.H));
    }
    const T *q = (const T *)a.q + (((int64_t)b * a.H + h) * a.T + t) * a.dh;
    for (int e = lane; e < a.dh; e += 64) qs[wave][e] = valid ? Elem<T>::load(q, e) : 0.0f;
    __syncthreads();
    if (!valid) return;

    int p = a.pos ? a.pos[b] : a.start + t;
    if (p >= a.t_max) p = a.t_max - 1;  // never read past the cache
    const int n_keys = p + 1;
    const int kvh = h / (a.H / a.Hkv);
    const T *K = (const T *)a.kc + ((int64_t)b * a.Hkv + kvh) * a.t_max * a.dh;
    const T *V = (const T *)a.vc + ((int64_t)b * a.Hkv + kvh) * a.t_max * a.dh;

    float m = -INFINITY, l = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = 0; j0 < n_keys; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        if (j < n_keys) {
            const T *kj = K + (int64_t)j * a.dh;
            float dot = 0.0f;
            for (int e = 0; e < a.dh; ++e) dot += qs[wave][e] * Elem<T>::load(kj, e);
            s = dot * a.scale;
        }
        const float m_new = fmaxf(m, wave_max(s));
        const float alpha = __expf(m - m_new);
        const float pj = (j < n_keys) ? __expf(s - m_new) : 0.0f;
        l = l * alpha + wave_sum(pj);
        m = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;
        const int cnt = min(64, n_keys - j0);
        for (int jj = 0; jj < cnt; ++jj) {
            const float pw = __shfl(pj, jj, 64);
            const T *vj = V + (int64_t)(j0 + jj) * a.dh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lane + 64 * i;
                if (e < a.dh) o[i] += pw * Elem<T>::load(vj, e);
            }
        }
    }
    T *out = (T *)a.o + ((int64_t)b * a.T + t) * ((int64_t)a.H * a.dh) + (int64_t)h * a.dh;
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < a.dh) Elem<T>::store(out, e, o[i] * inv);
    }
}

static hipError_t rowwise_launch(const AttnCall &a, hipStream_t s) {
    const int64_t waves = (int64_t)a.B * a.H * a.T;
    dim3 grid((unsigned)((waves + 3) / 4));
    if (a.dtype == TFB_BF16)
        hipLaunchKernelGGL(attn_rowwise_kernel<bf16_t>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(attn_rowwise_kernel<float>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t attention_prefill_launch(const AttnCall &a, hipStream_t s) { return rowwise_launch(a, s); }
hipError_t attention_decode_launch(const AttnCall &a, hipStream_t s) { return rowwise_launch(a, s); }
size_t attention_decode_scratch_bytes(int, int, int, int) { return 0; }

}  // namespace tfb
