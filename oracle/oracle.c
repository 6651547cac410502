/*
 * ORACLE — test infrastructure, not part of the product.
 *
 * A plain, slow, scalar fp32 CPU implementation of the pre-norm decoder block
 * (prefill and decode against a KV cache) and of the thin model around it.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no source with the GPU library and includes no HIP header.
 *
 * Precision: every value is fp32 and every sum runs in ascending index order,
 * as in the scalar block printed on tirogla "Transformer block" (section Code),
 * which computes in f32; that page's Implementation notes keep softmax and
 * norms in fp32 and run the GEMMs on bf16 operands with fp32 accumulation.
 * So with gemm_bf16 set (the bf16 storage configuration) each GEMM operand is
 * rounded to bf16 (nearest, ties to even) where it is produced: the normed
 * rows h and h2, q and k after RoPE, v, the attention output, the SwiGLU
 * product, the block output passed between layers and the final-norm rows.
 * Softmax probabilities and the residual inside a block stay fp32.
 * Build with -ffp-contract=off so no multiply-add is fused.
 * OpenMP only splits independent outputs (matmul rows, attention query rows),
 * never a sum, so results are bitwise independent of the thread count.
 *
 * Pages cited (title, address):
 *   [TIR] "Transformer block", tirogla.com/ml-training/transformer-architecture
 *   [PID] "The Transformer" (topic 09), infra.pidoku.co.in/inference-engineering
 *   [KIR] "The Transformer", kirito-excalibur.github.io/GenerativeAIDocs
 *   [GEN] "The Transformer Architecture", thegeniusblogs.com/modern-ai/transformers
 *   [MSA] "AI engineering: transformers", engineering.msaqlain.com
 *
 * Readings where the pages leave a choice open (each is also listed with its
 * reasons in the design notes): eps is a parameter (1e-5 on [TIR] Code, 1e-6 on
 * [PID] Tiny example); RoPE pairs are interleaved (2i, 2i+1) with frequency
 * base^(-2i/dh) over the head width; the cos/sin table is built from an fp64
 * angle and rounded to fp32 ([TIR] Implementation notes: precompute a
 * [T_max, dh/2] table); positions are 0-based absolute; weights are [in, out]
 * with y = x.W ([TIR] Code header comment).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t d, n_heads, n_kv_heads, head_dim, d_ff;
    float rope_base, rms_eps;
    int32_t gemm_bf16;  /* 1: GEMM operands rounded to bf16 (see Precision above) */
    int32_t window;     /* sliding window: keys per query, the query's own included; 0 = full causal */
} o_config;

/* fp32 -> nearest bf16 value (ties to even), returned widened to fp32.  A bf16
 * is the upper 16 bits of an fp32; NaN stays NaN. */
static float bf16_round(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return x;
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    memcpy(&x, &u, 4);
    return x;
}

/* Rounds n values in place when the configuration asks for bf16 operands. */
static void operand_round(const o_config *cfg, float *v, int64_t n) {
    if (!cfg->gemm_bf16) return;
    for (int64_t i = 0; i < n; ++i) v[i] = bf16_round(v[i]);
}

typedef struct {
    const float *g_attn, *g_mlp; /* [d] RMSNorm gains */
    const float *wq;             /* [d, H*dh] */
    const float *wk, *wv;        /* [d, Hkv*dh] */
    const float *wo;             /* [H*dh, d] */
    const float *w1, *w3;        /* gate, up: [d, f] */
    const float *w2;             /* down: [f, d] */
} o_weights;

/* Work actually done, counted where it is done. */
typedef struct {
    int64_t matmul_macs;   /* multiply-adds in weight matmuls */
    int64_t qk_macs;       /* multiply-adds in q.k scores */
    int64_t pv_macs;       /* multiply-adds in the weighted sum of v */
    int64_t cache_values;  /* K and V values appended to the cache */
} o_counters;

/* Optional intermediates for the selected rows (each nullable).  q, att and
 * act are the operands as handed on (bf16 values with gemm_bf16); the *_pre
 * arrays hold the same values as computed in fp32, before that rounding (equal
 * to the operands when gemm_bf16 is 0).  k_pre, v_pre cover every row. */
typedef struct {
    float *q;    /* [B, R, H*dh] after RoPE */
    float *att;  /* [B, R, H*dh] concatenated head outputs */
    float *r;    /* [B, R, d] first residual */
    float *act;  /* [B, R, f] SiLU(gate) * up */
    float *q_pre, *att_pre, *act_pre; /* as q, att, act */
    float *k_pre, *v_pre;             /* [B, T, Hkv*dh], k after RoPE */
} o_intermediates;

/* RMSNorm, one row: [TIR] Code (rms_norm) and How it works step 2;
 * [PID] Tiny example (rmsnorm).  ss = sum x_i^2; r = 1/sqrt(ss/d + eps);
 * y_i = x_i * r * g_i. */
static void rms_norm_row(const float *x, const float *g, int d, float eps, float *y) {
    float ss = 0.0f;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    float ms = ss / (float)d;
    float r = 1.0f / sqrtf(ms + eps);
    for (int i = 0; i < d; ++i) y[i] = x[i] * r * g[i];
}

void o_rms_norm(const float *x, const float *g, int64_t rows, int d, float eps, float *y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) rms_norm_row(x + i * d, g, d, eps, y + i * d);
}

/* y[t, n] = x[t, k] . w[k, n]: [TIR] Code (matmul, W is [in, out]).
 * Each y[i][j] is summed over p in ascending order starting from 0, exactly as
 * the i-p-j loop on that page; rows are processed in blocks so that a row of w
 * is read once per block, which does not change any sum. */
#define O_ROW_BLOCK 16
void o_matmul(const float *x, const float *w, int64_t t, int k, int n, float *y, o_counters *cnt) {
    int64_t nblk = (t + O_ROW_BLOCK - 1) / O_ROW_BLOCK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nblk; ++blk) {
        int64_t i0 = blk * O_ROW_BLOCK;
        int64_t i1 = i0 + O_ROW_BLOCK < t ? i0 + O_ROW_BLOCK : t;
        for (int64_t i = i0; i < i1; ++i) memset(y + i * (int64_t)n, 0, sizeof(float) * (size_t)n);
        for (int p = 0; p < k; ++p) {
            const float *wr = w + (int64_t)p * n;
            for (int64_t i = i0; i < i1; ++i) {
                float a = x[i * k + p];
                float *yr = y + i * (int64_t)n;
                for (int j = 0; j < n; ++j) yr[j] += a * wr[j];
            }
        }
    }
    if (cnt) cnt->matmul_macs += t * (int64_t)k * n;
}

/* RoPE cos/sin table [t_max][dh/2]: [TIR] Implementation notes (precompute a
 * [T_max, dh/2] table); [GEN] Positional encodings, RoPE (theta_i =
 * base^(-2i/d) over the rotated width).  Angle in fp64, stored as fp32. */
void o_rope_table(int t_max, int dh, double base, float *cos_tab, float *sin_tab) {
    int half = dh / 2;
    for (int t = 0; t < t_max; ++t)
        for (int i = 0; i < half; ++i) {
            double theta = pow(base, -2.0 * (double)i / (double)dh);
            double a = (double)t * theta;
            cos_tab[(int64_t)t * half + i] = (float)cos(a);
            sin_tab[(int64_t)t * half + i] = (float)sin(a);
        }
}

/* Rotate one head vector at one position: [TIR] Code (rope), pairs (2i, 2i+1):
 * v[2i] = a c - b s, v[2i+1] = a s + b c. */
static void rope_rotate(float *v, int dh, const float *c, const float *s) {
    for (int i = 0; i < dh / 2; ++i) {
        float a = v[2 * i], b = v[2 * i + 1];
        v[2 * i] = a * c[i] - b * s[i];
        v[2 * i + 1] = a * s[i] + b * c[i];
    }
}

void o_rope_apply(float *v, int64_t rows, int heads, int dh, const int32_t *pos, const float *cos_tab,
                  const float *sin_tab) {
    int half = dh / 2;
    for (int64_t r = 0; r < rows; ++r)
        for (int h = 0; h < heads; ++h)
            rope_rotate(v + (r * heads + h) * dh, dh, cos_tab + (int64_t)pos[r] * half,
                        sin_tab + (int64_t)pos[r] * half);
}

/* SiLU: [TIR] Code (silu), z / (1 + e^-z). */
static float silu(float z) { return z / (1.0f + expf(-z)); }

/* One query row of one head against keys j0..n_keys-1 of its KV head:
 * [TIR] How it works step 2 and Code (scores = q.k * scale, causal j <= i,
 * max-subtracted softmax in fp32, p = e/z, o += p v);
 * [MSA] 1.3 Scaled dot-product attention and 5.1 Causal masking.
 * kc, vc point at row 0 of the head's [t_max, dh] cache slab. */
static void attend_row(const float *q, const float *kc, const float *vc, int j0, int n_keys, int dh, float scale,
                       float *o, float *s) {
    float m = -INFINITY;
    for (int j = j0; j < n_keys; ++j) {
        const float *kj = kc + (int64_t)j * dh;
        float dot = 0.0f;
        for (int e = 0; e < dh; ++e) dot += q[e] * kj[e];
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
    }
    float z = 0.0f;
    for (int j = j0; j < n_keys; ++j) {
        s[j] = expf(s[j] - m);
        z += s[j];
    }
    for (int e = 0; e < dh; ++e) o[e] = 0.0f;
    for (int j = j0; j < n_keys; ++j) {
        const float *vj = vc + (int64_t)j * dh;
        float p = s[j] / z;
        for (int e = 0; e < dh; ++e) o[e] += p * vj[e];
    }
}

/* First key a query at position p sees under a sliding window of W keys:
 * [PID] Sliding-window attention (a query attends to the last W tokens, its
 * own included: with W = 4096 the query at 10000 sees 5905..10000).
 * W = 0 is full causal attention. */
int o_window_first_key(int p, int window) {
    if (window <= 0) return 0;
    int j0 = p - window + 1;
    return j0 > 0 ? j0 : 0;
}

/* Exported for the pins on attention alone (V = ones, T = 1, uniform scores,
 * windows). */
void o_attend_row_range(const float *q, const float *kc, const float *vc, int j0, int n_keys, int dh, float *o) {
    float *s = (float *)malloc(sizeof(float) * (size_t)(n_keys > 0 ? n_keys : 1));
    attend_row(q, kc, vc, j0, n_keys, dh, 1.0f / sqrtf((float)dh), o, s);
    free(s);
}

void o_attend_row(const float *q, const float *kc, const float *vc, int n_keys, int dh, float *o) {
    o_attend_row_range(q, kc, vc, 0, n_keys, dh, o);
}

/*
 * One block forward over x[B, T, d] whose row t of sequence b sits at absolute
 * position start[b] + t (start == NULL means 0: full-sequence prefill; T == 1
 * with start = current cache length is a decode step; [GEN] KV cache and
 * inference math, Two phases; [MSA] 5.2 The KV cache).
 *
 * Wiring: [TIR] How it works steps 2-3 and Code (Block::forward);
 * [KIR] 2. The block, in detail (pre-norm x <- x + Sub(Norm(x)), twice).
 *
 * kc, vc: [B, Hkv, t_max, dh] caches of post-RoPE k and v ([TIR] How it works,
 * KV cache).  Rows start[b] .. start[b]+T-1 are written, and attention for the
 * query at position p reads rows 0..p.  When kc is NULL a private cache of
 * t_max = T rows is used (start must then be NULL).
 *
 * rows: which of the T rows get an output (NULL = all T, in order); K and V
 * are always computed for every row because later rows attend to them.
 * out: [B, n_rows, d].
 */
int o_block_forward(const o_config *cfg, const o_weights *w, const float *cos_tab, const float *sin_tab,
                    int t_max_table, const float *x, int B, int T, const int32_t *start, float *kc, float *vc,
                    int t_max, const int32_t *rows, int n_rows, float *out, o_intermediates *inter,
                    o_counters *cnt) {
    const int d = cfg->d, H = cfg->n_heads, Hkv = cfg->n_kv_heads, dh = cfg->head_dim, f = cfg->d_ff;
    const int qd = H * dh, kvd = Hkv * dh;
    if (H % Hkv != 0 || dh % 2 != 0 || H * dh != d) return -2;
    int own_cache = 0;
    if (!kc) {
        if (start) return -2;
        t_max = T;
        kc = (float *)calloc((size_t)B * Hkv * t_max * dh, sizeof(float));
        vc = (float *)calloc((size_t)B * Hkv * t_max * dh, sizeof(float));
        own_cache = 1;
    }
    if (!rows) n_rows = T;
    for (int b = 0; b < B; ++b) {
        int s0 = start ? start[b] : 0;
        if (s0 < 0 || s0 + T > t_max || s0 + T > t_max_table) {
            if (own_cache) { free(kc); free(vc); }
            return -6;
        }
    }
    const int64_t M = (int64_t)B * T, R = (int64_t)B * n_rows;

    /* RMSNorm_1 of every row, then k and v of every row. */
    float *h = (float *)malloc(sizeof(float) * M * d);
    float *k = (float *)malloc(sizeof(float) * M * kvd);
    float *v = (float *)malloc(sizeof(float) * M * kvd);
    o_rms_norm(x, w->g_attn, M, d, cfg->rms_eps, h);
    operand_round(cfg, h, M * d);
    o_matmul(h, w->wk, M, d, kvd, k, cnt);
    o_matmul(h, w->wv, M, d, kvd, v, cnt);

    /* Selected rows: gather their normed input and residual input. */
    float *hs = (float *)malloc(sizeof(float) * R * d);
    float *xs = (float *)malloc(sizeof(float) * R * d);
    int32_t *pos_k = (int32_t *)malloc(sizeof(int32_t) * M);
    int32_t *pos_q = (int32_t *)malloc(sizeof(int32_t) * R);
    for (int b = 0; b < B; ++b) {
        int s0 = start ? start[b] : 0;
        for (int t = 0; t < T; ++t) pos_k[(int64_t)b * T + t] = s0 + t;
        for (int r = 0; r < n_rows; ++r) {
            int t = rows ? rows[r] : r;
            int64_t src = (int64_t)b * T + t, dst = (int64_t)b * n_rows + r;
            memcpy(hs + dst * d, h + src * d, sizeof(float) * d);
            memcpy(xs + dst * d, x + src * d, sizeof(float) * d);
            pos_q[dst] = s0 + t;
        }
    }
    free(h);
    float *q = (float *)malloc(sizeof(float) * R * qd);
    o_matmul(hs, w->wq, R, d, qd, q, cnt);
    free(hs);

    /* RoPE on q and k only, never on v ([TIR] Pitfalls). */
    o_rope_apply(q, R, H, dh, pos_q, cos_tab, sin_tab);
    o_rope_apply(k, M, Hkv, dh, pos_k, cos_tab, sin_tab);
    if (inter && inter->q_pre) memcpy(inter->q_pre, q, sizeof(float) * R * qd);
    if (inter && inter->k_pre) memcpy(inter->k_pre, k, sizeof(float) * M * kvd);
    if (inter && inter->v_pre) memcpy(inter->v_pre, v, sizeof(float) * M * kvd);
    operand_round(cfg, q, R * qd);
    operand_round(cfg, k, M * kvd);
    operand_round(cfg, v, M * kvd);

    /* Append post-RoPE k and v to the cache. */
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t) {
            int p = pos_k[(int64_t)b * T + t];
            for (int g = 0; g < Hkv; ++g) {
                int64_t dst = (((int64_t)b * Hkv + g) * t_max + p) * dh;
                int64_t src = ((int64_t)b * T + t) * kvd + (int64_t)g * dh;
                memcpy(kc + dst, k + src, sizeof(float) * dh);
                memcpy(vc + dst, v + src, sizeof(float) * dh);
            }
        }
    if (cnt) cnt->cache_values += M * 2 * kvd;
    free(k);
    free(v);

    /* Attention, one (row, head) at a time.  GQA: query head hd reads KV head
     * hd / (H / Hkv) ([TIR] Code; [PID] Tiny example).  With a sliding
     * window, the query at position p reads keys from o_window_first_key. */
    const float scale = 1.0f / sqrtf((float)dh);
    float *att = (float *)malloc(sizeof(float) * R * qd);
    const int group = H / Hkv;
    int64_t qk = 0;
#pragma omp parallel
    {
        float *s = (float *)malloc(sizeof(float) * (size_t)t_max);
#pragma omp for schedule(dynamic, 4) reduction(+ : qk)
        for (int64_t rh = 0; rh < R * H; ++rh) {
            int64_t rr = rh / H;
            int hd = (int)(rh % H);
            int b = (int)(rr / n_rows);
            int kvh = hd / group;
            int p = pos_q[rr];
            const float *kcs = kc + ((int64_t)b * Hkv + kvh) * t_max * dh;
            const float *vcs = vc + ((int64_t)b * Hkv + kvh) * t_max * dh;
            const int j0 = o_window_first_key(p, cfg->window);
            attend_row(q + rr * qd + (int64_t)hd * dh, kcs, vcs, j0, p + 1, dh, scale, att + rr * qd + (int64_t)hd * dh,
                       s);
            qk += (int64_t)(p + 1 - j0) * dh;
        }
        free(s);
    }
    if (cnt) { cnt->qk_macs += qk; cnt->pv_macs += qk; }
    if (inter && inter->q) memcpy(inter->q, q, sizeof(float) * R * qd);
    free(q);

    /* Wo and the first residual: r = x + att.Wo ([TIR] How it works step 2). */
    float *a = (float *)malloc(sizeof(float) * R * d);
    if (inter && inter->att_pre) memcpy(inter->att_pre, att, sizeof(float) * R * qd);
    operand_round(cfg, att, R * qd);
    o_matmul(att, w->wo, R, qd, d, a, cnt);
    if (inter && inter->att) memcpy(inter->att, att, sizeof(float) * R * qd);
    free(att);
    float *r = (float *)malloc(sizeof(float) * R * d);
    for (int64_t i = 0; i < R * d; ++i) r[i] = xs[i] + a[i];
    free(a);
    free(xs);
    if (inter && inter->r) memcpy(inter->r, r, sizeof(float) * R * d);

    /* SwiGLU MLP and the second residual: out = r + (SiLU(h2.W1) * h2.W3).W2
     * ([TIR] How it works step 3; [MSA] 2. Transformer Block Anatomy). */
    float *h2 = (float *)malloc(sizeof(float) * R * d);
    o_rms_norm(r, w->g_mlp, R, d, cfg->rms_eps, h2);
    operand_round(cfg, h2, R * d);
    float *gate = (float *)malloc(sizeof(float) * R * f);
    float *up = (float *)malloc(sizeof(float) * R * f);
    o_matmul(h2, w->w1, R, d, f, gate, cnt);
    o_matmul(h2, w->w3, R, d, f, up, cnt);
    free(h2);
    for (int64_t i = 0; i < R * f; ++i) gate[i] = silu(gate[i]) * up[i];
    free(up);
    if (inter && inter->act_pre) memcpy(inter->act_pre, gate, sizeof(float) * R * f);
    operand_round(cfg, gate, R * f);
    if (inter && inter->act) memcpy(inter->act, gate, sizeof(float) * R * f);
    float *m = (float *)malloc(sizeof(float) * R * d);
    o_matmul(gate, w->w2, R, f, d, m, cnt);
    free(gate);
    for (int64_t i = 0; i < R * d; ++i) out[i] = r[i] + m[i];
    free(m);
    free(r);
    free(pos_k);
    free(pos_q);
    if (own_cache) { free(kc); free(vc); }
    return 0;
}

/* Scatter k_new, v_new [B, n, Hkv, dh] into the caches at rows start[b]..:
 * [TIR] How it works, KV cache (store post-RoPE k and v of every past token). */
int o_kv_append(int B, int Hkv, int dh, int t_max, const float *k_new, const float *v_new, const int32_t *start,
                int n_new, float *kc, float *vc) {
    for (int b = 0; b < B; ++b)
        if (start[b] < 0 || start[b] + n_new > t_max) return -6;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < n_new; ++t)
            for (int g = 0; g < Hkv; ++g) {
                int64_t src = (((int64_t)b * n_new + t) * Hkv + g) * dh;
                int64_t dst = (((int64_t)b * Hkv + g) * t_max + start[b] + t) * dh;
                memcpy(kc + dst, k_new + src, sizeof(float) * dh);
                memcpy(vc + dst, v_new + src, sizeof(float) * dh);
            }
    return 0;
}

/* argmax over n logits, lowest index on ties (greedy next token). */
static int32_t argmax_row(const float *v, int n) {
    int32_t best = 0;
    for (int j = 1; j < n; ++j)
        if (v[j] > v[best]) best = j;
    return best;
}

/*
 * Model forward: [PID] 5. Technical explanation, The full model (embed, L
 * blocks, final norm, LM head) and Tiny example (forward); [TIR] How it works
 * steps 1 and 4 (untied W_U [d, V], final norm after the last block).
 * ids [B, T]; start[b] is the absolute position of ids[b, 0] (NULL = 0).
 * layers: host array [L]; kcs, vcs: host arrays [L] of [B, Hkv, t_max, dh].
 * logits: [B, n_rows, V] for the selected rows (rows NULL = all T rows).
 * next_ids (nullable): [B] argmax of the last selected row of each sequence.
 * k_pre, v_pre (nullable host arrays [L] of [B, T, Hkv*dh]): each layer's k
 * (after RoPE) and v as computed, before bf16 storage.
 */
int o_model_forward(const o_config *cfg, int n_layers, int vocab, const float *embed, const o_weights *layers,
                    const float *g_final, const float *w_unembed, const float *cos_tab, const float *sin_tab,
                    int t_max_table, const int32_t *ids, int B, int T, const int32_t *start, float **kcs,
                    float **vcs, int t_max, const int32_t *rows, int n_rows, float *logits, int32_t *next_ids,
                    float **k_pre, float **v_pre, o_counters *cnt) {
    const int d = cfg->d;
    const int64_t M = (int64_t)B * T;
    if (!rows) n_rows = T;
    float *x = (float *)malloc(sizeof(float) * M * d);
    float *y = (float *)malloc(sizeof(float) * M * d);
    for (int64_t i = 0; i < M; ++i) {
        if (ids[i] < 0 || ids[i] >= vocab) { free(x); free(y); return -2; }
        memcpy(x + i * d, embed + (int64_t)ids[i] * d, sizeof(float) * d);
    }
    int rc = 0;
    for (int l = 0; l < n_layers && rc == 0; ++l) {
        int last = (l == n_layers - 1);
        /* Only the last layer may restrict its rows: earlier layers feed the
         * keys and values of every row to the next. */
        o_intermediates kv = {0};
        if (k_pre) kv.k_pre = k_pre[l];
        if (v_pre) kv.v_pre = v_pre[l];
        rc = o_block_forward(cfg, &layers[l], cos_tab, sin_tab, t_max_table, x, B, T, start, kcs[l], vcs[l], t_max,
                             last ? rows : NULL, last ? n_rows : T, y, &kv, cnt);
        /* the block output is the next block's input activation */
        operand_round(cfg, y, (last ? (int64_t)B * n_rows : M) * d);
        float *tmp = x; x = y; y = tmp;
    }
    if (rc == 0) {
        const int64_t R = (int64_t)B * n_rows;
        float *hn = (float *)malloc(sizeof(float) * R * d);
        o_rms_norm(x, g_final, R, d, cfg->rms_eps, hn);
        operand_round(cfg, hn, R * d);
        o_matmul(hn, w_unembed, R, d, vocab, logits, cnt);
        free(hn);
        if (next_ids)
            for (int b = 0; b < B; ++b)
                next_ids[b] = argmax_row(logits + ((int64_t)b * n_rows + n_rows - 1) * vocab, vocab);
    }
    free(x);
    free(y);
    return rc;
}

/* Threads an OpenMP region uses here (reported with the CPU timing). */
int o_omp_threads(void) { return omp_get_max_threads(); }
