// C ABI of libtfb (include/tfb.h): argument validation, workspace layout and
// the launch sequence of each call.  Page short names: [TIR] tirogla
// "Transformer block", [PID] pidoku "The Transformer".
#include <math.h>
#include <stdint.h>
#include <cstdint>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kernels.h"

using namespace tfb;

namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t esize(int dtype) { return dtype == TFB_BF16 ? 2 : 4; }

// Decode attention splits each (sequence, KV head) key range into at most
// this many chunks; their partial results live in the workspace.
constexpr int kMaxSplits = 64;

struct WsLayout {
    size_t h, q, att, r, act, kv_k, kv_v, part, part_bytes, skinny, skinny_bytes, gsplit, gsplit_bytes, rss,
        rss_bytes, x0, x1, last, logits, total;
};

// A folded RMSNorm in flight between two large-M GEMMs: h holds bf16(x * g)
// and ss [M][parts] the partial sums of x^2 that the next GEMM adds up.
struct FoldedNorm {
    const float *ss;
    int parts;  // 0: nothing folded
};

// part_bytes: room for the decode-attention partials; the default holds
// kMaxSplits chunks per (sequence, head), whatever the call's positions.
WsLayout ws_layout(const tfb_block_config &c, int B, int T, int vocab, size_t part_bytes = SIZE_MAX) {
    WsLayout L{};
    const size_t es = esize(c.dtype), M = (size_t)B * T;
    const size_t qd = (size_t)c.n_heads * c.head_dim, kvd = (size_t)c.n_kv_heads * c.head_dim;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += up(bytes); return o; };
    L.h = take(M * c.d * es);
    L.q = take(M * qd * es);
    L.att = take(M * qd * es);
    L.r = take(M * c.d * sizeof(float));  // block-internal residual, fp32
    L.act = take(M * (size_t)c.d_ff * es);
    // keys and values when no cache is given; with a sliding window, also the
    // contiguous staging copy (chunk + the window's history) that a prefill
    // into a bounded window cache works in
    const size_t kv_rows = (c.window > 0 && T > 1) ? std::max(M, (size_t)B * ((size_t)T + c.window - 1)) : M;
    L.kv_k = take(kv_rows * kvd * es);
    L.kv_v = take(kv_rows * kvd * es);
    L.part_bytes =
        part_bytes == SIZE_MAX ? attention_decode_scratch_bytes(B, c.n_heads, c.head_dim, kMaxSplits) : part_bytes;
    L.part = take(L.part_bytes);
    if (c.dtype == TFB_BF16) {
        // split-K partials of the skinny GEMMs (rows <= kSkinnyMaxM): the
        // block's GEMMs in decode and the LM head over the last rows
        size_t sk = 0;
        if (M <= (size_t)kSkinnyMaxM)
            sk = std::max({skinny_part_bytes((int)M, c.d, (int)(qd + 2 * kvd)),
                           skinny_part_bytes((int)M, (int)qd, c.d), skinny_part_bytes((int)M, c.d, 2 * c.d_ff),
                           skinny_part_bytes((int)M, c.d_ff, c.d)});
        // the LM head runs on the last row of each sequence, or on every row
        // when all logits are wanted: both row counts may take this path
        if (vocab > 0 && B <= kSkinnyMaxM) sk = std::max(sk, skinny_part_bytes(B, c.d, vocab));
        if (vocab > 0 && M <= (size_t)kSkinnyMaxM) sk = std::max(sk, skinny_part_bytes((int)M, c.d, vocab));
        if (sk) {
            L.skinny_bytes = sk;
            L.skinny = take(sk);
        }
    }
    if (c.dtype == TFB_BF16) {
        // split-K tail partials of the large-M GEMMs (one GEMM at a time)
        const int Mi = (int)M;
        size_t gs = std::max({gemm_split_bytes(Mi, (int)(qd + 2 * kvd), c.d), gemm_split_bytes(Mi, c.d, (int)qd),
                              gemm_split_bytes(Mi, 2 * c.d_ff, c.d), gemm_split_bytes(Mi, c.d, c.d_ff)});
        if (vocab > 0) gs = std::max(gs, gemm_split_bytes(Mi, vocab, c.d));
        if (gs) {
            L.gsplit_bytes = gs;
            L.gsplit = take(gs);
        }
    }
    if (c.fold_norms && c.dtype == TFB_BF16 && M > (size_t)kSkinnyMaxM) {
        // partial sums of squares of a folded RMSNorm (large-M GEMMs)
        L.rss_bytes = M * kRowSsMaxParts * sizeof(float);
        L.rss = take(L.rss_bytes);
    }
    if (vocab > 0) {
        L.x0 = take(M * c.d * es);
        L.x1 = take(M * c.d * es);
        L.last = take((size_t)B * c.d * es);
        L.logits = take((size_t)B * vocab * sizeof(float));
    }
    L.total = off;
    return L;
}

tfb_status check_cfg(const tfb_block_config *c) {
    if (!c) return TFB_ERR_NULL;
    if (c->dtype != TFB_F32 && c->dtype != TFB_BF16) return TFB_ERR_DTYPE;
    if (c->d <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->d_ff <= 0) return TFB_ERR_SHAPE;
    if (c->n_heads % c->n_kv_heads != 0 || c->n_heads * c->head_dim != c->d || (c->head_dim & 1)) return TFB_ERR_SHAPE;
    if (!(c->rope_base > 0.0f) || !(c->rms_eps >= 0.0f) || !isfinite(c->rope_base) || !isfinite(c->rms_eps))
        return TFB_ERR_SHAPE;
    if (c->window < 0) return TFB_ERR_SHAPE;
    if (c->dtype == TFB_BF16) {
        if (c->d % 64 || c->d_ff % 64 || (c->head_dim != 64 && c->head_dim != 128)) return TFB_ERR_SHAPE;
    } else {
        if (c->head_dim > 256 || c->d % 4 || c->d_ff % 4) return TFB_ERR_SHAPE;
    }
    return TFB_OK;
}

tfb_status check_weights(const tfb_block_weights *w) {
    if (!w) return TFB_ERR_NULL;
    const void *p[] = {w->g_attn, w->g_mlp, w->wq, w->wk, w->wv, w->wo, w->w1, w->w3, w->w2};
    for (const void *x : p)
        if (!x) return TFB_ERR_NULL;
    for (const void *x : p)
        if (!aligned(x)) return TFB_ERR_ALIGN;
    return TFB_OK;
}

tfb_status check_cache(const tfb_kv_cache *kv, int B) {
    if (!kv->k || !kv->v) return TFB_ERR_NULL;
    if (!aligned(kv->k) || !aligned(kv->v)) return TFB_ERR_ALIGN;
    if (kv->batch != B || kv->t_max <= 0) return TFB_ERR_SHAPE;
    return TFB_OK;
}

#define TRY_HIP(expr)                                  \
    do {                                               \
        if ((expr) != hipSuccess) return TFB_ERR_HIP;  \
    } while (0)

// ---- optional per-stage event timing (tfb_profile_*) -----------------------
enum Stage {
    ST_RMSNORM_ATTN, ST_QKV, ST_ATTN, ST_ATTN_COMBINE, ST_WO, ST_RMSNORM_MLP, ST_GATEUP, ST_W2,
    ST_EMBED, ST_FINAL_NORM, ST_LM_HEAD, ST_ARGMAX, ST_KV_APPEND, ST_COUNT
};
const char *kStageNames[ST_COUNT] = {"rmsnorm_attn", "qkv_gemm", "attention", "attention_combine", "wo_gemm",
                                     "rmsnorm_mlp", "gateup_gemm", "w2_gemm", "embed", "final_norm", "lm_head",
                                     "argmax", "kv_append"};
struct ProfRec { int stage; hipEvent_t a, b; };
std::mutex g_prof_mu;
bool g_prof = false;
uint32_t g_prof_mask = 0xFFFFFFFFu;  // stages bracketed while profiling
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t prof_event() {
    if (!g_pool.empty()) { hipEvent_t e = g_pool.back(); g_pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDefault) != hipSuccess) return nullptr;
    return e;
}

// Runs one launch; when profiling, brackets it with an event pair.
template <typename F>
hipError_t staged(int stage, hipStream_t s, F &&launch) {
    if (!g_prof || !((g_prof_mask >> stage) & 1u)) return launch();
    std::lock_guard<std::mutex> lk(g_prof_mu);
    ProfRec r{stage, prof_event(), prof_event()};
    if (r.a) hipEventRecord(r.a, s);
    hipError_t e = launch();
    if (r.b) hipEventRecord(r.b, s);
    if (r.a && r.b) g_recs.push_back(r);
    return e;
}
#define STAGE(st, expr) staged((st), s, [&]() { return (expr); })

// The launches of one block for M = B*T rows ([TIR] How it works steps 2-3):
//   RMSNorm_1 -> fused QKV GEMM (+RoPE, q to workspace, k and v to the cache)
//   -> causal GQA attention -> Wo GEMM + residual -> RMSNorm_2
//   -> fused gate-up GEMM (+SiLU * up) -> W2 GEMM + residual.
// The RMSNorms that follow a residual GEMM run inside its reduce pass: on the
// skinny path (bf16, at most kSkinnyMaxM rows, with its partial buffer) and
// for widths the fused kernel holds in registers.
bool norms_fuse(const tfb_block_config &c, int M, const WsLayout &L) {
    return c.dtype == TFB_BF16 && M <= kSkinnyMaxM && L.skinny_bytes > 0 && c.d <= kSkinnyNormMaxN && c.d % 8 == 0;
}

tfb_status run_block(const tfb_block_config &c, const tfb_block_weights &w, const float *rope, int rope_rows,
                     int max_pos, const void *x, void *out, int B, int T, int start, const int32_t *pos, void *kc,
                     void *vc, const KvMap &kvm, uint8_t *ws, const WsLayout &L, hipStream_t s,
                     const int32_t *starts = nullptr, const int32_t *lens = nullptr, bool h_ready = false,
                     const void *next_g = nullptr, const FoldedNorm *h_fold = nullptr,
                     FoldedNorm *next_fold = nullptr) {
    // h_ready: h in the workspace already holds RMSNorm1(x) (written by the
    // previous layer's W2 step).  next_g: on the skinny path, the W2 step also
    // writes RMSNorm(out) with this gain into h for whoever reads h next.
    // h_fold (large-M path): h holds RMSNorm1's folded operand bf16(x * g_attn)
    // instead, with its row sums.  next_fold (large-M path, with next_g): the
    // W2 step folds the next norm into its epilogue and says so here.
    //
    // With fold_norms, on the large-M bf16 path RMSNorm2 is folded: the Wo
    // epilogue writes bf16(r * g_mlp) and per-tile sums of r^2, and the
    // gate-up GEMM scales each row's products by 1/rms(r) before SiLU.  The
    // norm's row scale distributes over the GEMM (row m of h W is
    // s_m (x_m * g) W), so only the place where the operand is rounded to
    // bf16 moves.  (The workspace holds the sums only with fold_norms.)
    // cache rows: contiguous [B, Hkv, t_max, dh], or a paged pool and block
    // table; a bounded window cache is only ever passed here for decode
    const int t_max = kvm.t_max;
    const int M = B * T, d = c.d, H = c.n_heads, Hkv = c.n_kv_heads, dh = c.head_dim, f = c.d_ff;
    const int qd = H * dh, kvd = Hkv * dh;
    void *h = ws + L.h, *q = ws + L.q, *att = ws + L.att, *r = ws + L.r, *act = ws + L.act;

    const bool folded_in = h_fold && h_fold->parts > 0;
    if (!h_ready && !folded_in)
        TRY_HIP(STAGE(ST_RMSNORM_ATTN, rmsnorm_launch(c.dtype, x, d, w.g_attn, h, d, M, d, c.rms_eps, s)));
    const bool fuse = norms_fuse(c, M, L);
    float *rss = L.rss_bytes ? (float *)(ws + L.rss) : nullptr;
    const int mlp_parts = rss ? gemm_fold_parts(M, d, qd) : 0;

    AttnCall a{};
    a.dtype = c.dtype;
    a.q = q; a.kc = kc; a.vc = vc; a.o = att; a.pos = pos;
    a.B = B; a.T = T; a.H = H; a.Hkv = Hkv; a.dh = dh; a.t_max = t_max; a.start = start;
    a.starts = starts;
    a.lens = lens;
    a.kvm = kvm;
    a.scale = 1.0f / sqrtf((float)dh);
    a.partials = ws + L.part;
    a.partial_bytes = L.part_bytes;
    a.max_keys = pos ? max_pos + 1 : start + T;
    a.max_splits = kMaxSplits;
    a.window = c.window;

    GemmCall g{};
    g.dtype = c.dtype;
    g.epi = EPI_QKV;
    g.A = h;
    g.lda = d;
    g.M = M;
    g.K = d;
    g.w[0] = w.wq; g.w[1] = w.wk; g.w[2] = w.wv;
    g.w_cols[0] = qd; g.w_cols[1] = kvd; g.w_cols[2] = kvd;
    g.ep.M = M;
    g.ep.N = qd + 2 * kvd;
    g.ep.q = q;
    g.ep.kc = kc;
    g.ep.vc = vc;
    g.ep.rope = rope;
    g.ep.rope_rows = rope_rows;
    g.ep.pos = pos;
    g.ep.T = T; g.ep.H = H; g.ep.Hkv = Hkv; g.ep.dh = dh; g.ep.t_max = t_max; g.ep.start = start;
    g.ep.starts = starts;
    g.ep.lens = lens;
    g.ep.kvm = kvm;
    g.scratch = L.skinny_bytes ? ws + L.skinny : nullptr;
    g.scratch_bytes = L.skinny_bytes;
    g.split_scratch = L.gsplit_bytes ? ws + L.gsplit : nullptr;
    g.split_bytes = L.gsplit_bytes;
    if (folded_in) {
        g.row_ss = h_fold->ss;
        g.row_ss_n = h_fold->parts;
        g.row_ss_eps = c.rms_eps;
    }
    // decode on the split attention kernel: the QKV GEMM leaves its split-K
    // partials, and the attention kernel reduces them (q, RoPE, the new cache
    // rows) instead of a separate reduce pass
    int qkv_splits = 0;
    if (pos && attention_decode_takes_qkv_partials(a)) g.qkv_deferred_splits = &qkv_splits;
    TRY_HIP(STAGE(ST_QKV, gemm_launch(g, s)));
    if (qkv_splits > 0) {
        a.qkv_part = (const float *)g.scratch;
        a.qkv_splits = qkv_splits;
        a.qkv_n = g.ep.N;
        a.rope = rope;
        a.rope_rows = rope_rows;
    }

    TRY_HIP(STAGE(ST_ATTN, pos ? attention_decode_launch(a, s) : attention_prefill_launch(a, s)));
    // with few (sequence, KV head) pairs the Wo GEMM merges the attention's
    // chunk partials itself, under its first weight loads, instead of a
    // separate merge pass
    AttnChunks chunks{};
    bool wo_merges = false;
    if (pos && attention_decode_takes_qkv_partials(a) && c.dtype == TFB_BF16 && M <= kSkinnyMaxM && L.skinny_bytes &&
        skinny_takes_attn_chunks(M, qd, d) && attention_decode_chunks(a, &chunks.chunk_keys, &chunks.max_chunks)) {
        chunks.part = (const float *)a.partials;
        chunks.pos = pos;
        chunks.H = H;
        chunks.dh = dh;
        chunks.window = c.window;
        chunks.kvm = kvm;
        chunks.att_out = att;
        wo_merges = true;
    }
    if (pos && !wo_merges) TRY_HIP(STAGE(ST_ATTN_COMBINE, attention_decode_merge_launch(a, s)));

    GemmCall o{};
    o.dtype = c.dtype;
    o.epi = EPI_RESID;
    o.A = att; o.lda = qd; o.M = M; o.K = qd;
    o.w[0] = w.wo; o.w_cols[0] = d;
    o.ep.M = M; o.ep.N = d; o.ep.out = r; o.ep.ldo = d; o.ep.res = x; o.ep.ldr = d; o.ep.out_f32 = 1;
    if (wo_merges) o.attn_chunks = &chunks;
    o.scratch = g.scratch;
    o.scratch_bytes = g.scratch_bytes;
    o.split_scratch = g.split_scratch;
    o.split_bytes = g.split_bytes;
    if (fuse) {  // RMSNorm2 of the stored residual rows, in the Wo reduce
        o.norm_g = w.g_mlp;
        o.norm_out = h;
        o.norm_eps = c.rms_eps;
    } else if (mlp_parts) {  // RMSNorm2 folded into the Wo epilogue and the gate-up
        o.norm_g = w.g_mlp;
        o.norm_out = h;
        o.norm_ss = rss;
    }
    TRY_HIP(STAGE(ST_WO, gemm_launch(o, s)));

    if (!fuse && !mlp_parts)
        TRY_HIP(STAGE(ST_RMSNORM_MLP, rmsnorm_launch(c.dtype, r, d, w.g_mlp, h, d, M, d, c.rms_eps, s, true)));

    GemmCall gu{};
    gu.dtype = c.dtype;
    gu.epi = EPI_SWIGLU;
    gu.A = h; gu.lda = d; gu.M = M; gu.K = d;
    gu.w[0] = w.w1; gu.w[1] = w.w3; gu.w_cols[0] = f; gu.w_cols[1] = f;
    gu.ep.M = M; gu.ep.N = f; gu.ep.out = act; gu.ep.ldo = f;
    gu.scratch = g.scratch;
    gu.scratch_bytes = g.scratch_bytes;
    gu.split_scratch = g.split_scratch;
    gu.split_bytes = g.split_bytes;
    if (mlp_parts) {
        gu.row_ss = rss;
        gu.row_ss_n = mlp_parts;
        gu.row_ss_eps = c.rms_eps;
    }
    TRY_HIP(STAGE(ST_GATEUP, gemm_launch(gu, s)));

    GemmCall dn{};
    dn.dtype = c.dtype;
    dn.epi = EPI_RESID;
    dn.A = act; dn.lda = f; dn.M = M; dn.K = f;
    dn.w[0] = w.w2; dn.w_cols[0] = d;
    dn.ep.M = M; dn.ep.N = d; dn.ep.out = out; dn.ep.ldo = d; dn.ep.res = r; dn.ep.ldr = d; dn.ep.res_f32 = 1;
    dn.scratch = g.scratch;
    dn.scratch_bytes = g.scratch_bytes;
    dn.split_scratch = g.split_scratch;
    dn.split_bytes = g.split_bytes;
    if (fuse && next_g) {
        dn.norm_g = next_g;
        dn.norm_out = h;
        dn.norm_eps = c.rms_eps;
    }
    const int next_parts = (rss && next_g && next_fold) ? gemm_fold_parts(M, d, f) : 0;
    if (next_parts) {  // the next RMSNorm folded into the W2 epilogue
        dn.norm_g = next_g;
        dn.norm_out = h;
        dn.norm_ss = rss;
    }
    if (next_fold) *next_fold = FoldedNorm{rss, next_parts};
    TRY_HIP(STAGE(ST_W2, gemm_launch(dn, s)));
    return TFB_OK;
}

// Prefill of rows start .. start+T-1.  A bounded sliding-window cache (ring)
// holds only the last `ring` positions.  When the chunk and the window's
// history before it (hist positions) fit in the ring, every position the
// call touches has its own slot and the block runs on the ring directly.
// Otherwise the chunk's own rows would overwrite history that its earlier
// rows still attend to, so the chunk works in a contiguous staging copy in
// the workspace: the history is copied in, the block runs on the copy
// exactly as on an uncapped cache, and the chunk's last rows go to their
// ring slots at the end.
tfb_status run_prefill(const tfb_block_config &c, const tfb_block_weights &w, const float *rope, int rope_rows,
                       const void *x, void *out, int B, int T, int start, void *kc, void *vc, const KvMap &kvm,
                       uint8_t *ws, const WsLayout &L, hipStream_t s, bool h_ready = false,
                       const void *next_g = nullptr, const FoldedNorm *h_fold = nullptr,
                       FoldedNorm *next_fold = nullptr) {
    const int hist = kvm.ring ? std::min(start, c.window - 1) : 0;
    if (!kvm.ring || (int64_t)T + hist <= kvm.ring)
        return run_block(c, w, rope, rope_rows, 0, x, out, B, T, start, nullptr, kc, vc, kvm, ws, L, s, nullptr,
                         nullptr, h_ready, next_g, h_fold, next_fold);
    const KvMap stg{nullptr, T + hist, 0, 0, 0, start - hist, 0};
    void *sk = ws + L.kv_k, *sv = ws + L.kv_v;
    TRY_HIP(kv_copy_launch(c.dtype, kc, vc, kvm, sk, sv, stg, B, c.n_kv_heads, c.head_dim, start - hist, hist, s));
    const tfb_status st = run_block(c, w, rope, rope_rows, 0, x, out, B, T, start, nullptr, sk, sv, stg, ws, L, s,
                                    nullptr, nullptr, h_ready, next_g, h_fold, next_fold);
    if (st != TFB_OK) return st;
    const int n = std::min(T, kvm.ring);
    TRY_HIP(kv_copy_launch(c.dtype, sk, sv, stg, kc, vc, kvm, B, c.n_kv_heads, c.head_dim, start + T - n, n, s));
    return TFB_OK;
}

// Row map of a contiguous cache; a ring cache holds the last t_max positions.
KvMap contig_map(const tfb_kv_cache &kv) { return KvMap{nullptr, kv.t_max, 0, 0, 0, 0, kv.ring ? kv.t_max : 0}; }

// A bounded window cache needs a window no longer than the cache and rows the
// staging copy moves in 16-byte pieces.
tfb_status check_ring(const tfb_block_config &c, int ring, int capacity) {
    if (!ring) return TFB_OK;
    if (c.window <= 0 || capacity < c.window) return TFB_ERR_SHAPE;
    if (c.dtype == TFB_F32 && c.head_dim % 4) return TFB_ERR_SHAPE;
    return TFB_OK;
}

}  // namespace

// ---- allocation-free decode (tfb_block_decode_noalloc) ----------------------
// The workspace of one decode step lives in this file-scope device array.  In
// host code `scratch` names a host-side stand-in; the device address of each
// GPU's own copy is looked up once per device and kept in g_scratch_dev.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_dev[kMaxDevices];  // nullptr: not looked up yet on that device

// Device address of the current device's `scratch` (hipGetSymbolAddress with
// that device current, once per device).
tfb_status scratch_on_current_device(uint8_t **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TFB_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TFB_ERR_HIP;
        g_scratch_dev[dev] = (uint8_t *)p;
    }
    *out = g_scratch_dev[dev];
    return TFB_OK;
}
}  // namespace

extern "C" {

int32_t tfb_version(void) { return 100; }

tfb_status tfb_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof = on != 0;
    return TFB_OK;
}

tfb_status tfb_profile_stages(uint32_t mask) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_mask = mask;
    return TFB_OK;
}

int32_t tfb_profile_read(float *ms, int32_t *calls, int32_t n) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    float acc[ST_COUNT] = {};
    int32_t cnt[ST_COUNT] = {};
    for (const ProfRec &r : g_recs) {
        float t = 0.0f;
        if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
            acc[r.stage] += t;
            cnt[r.stage] += 1;
        }
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    for (int i = 0; i < n && i < ST_COUNT; ++i) {
        if (ms) ms[i] = acc[i];
        if (calls) calls[i] = cnt[i];
    }
    return ST_COUNT;
}

const char *tfb_profile_stage_name(int32_t stage) {
    return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "";
}

const char *tfb_status_string(tfb_status st) {
    switch (st) {
        case TFB_OK: return "ok";
        case TFB_ERR_NULL: return "a required pointer is NULL";
        case TFB_ERR_SHAPE: return "invalid sizes";
        case TFB_ERR_DTYPE: return "unknown storage type";
        case TFB_ERR_ALIGN: return "pointer not 16-byte aligned";
        case TFB_ERR_WORKSPACE: return "workspace missing or too small";
        case TFB_ERR_CACHE_OVERFLOW: return "position bound not below cache or RoPE table length";
        case TFB_ERR_HIP: return "HIP launch failed";
        case TFB_ERR_UNSUPPORTED: return "unsupported request";
    }
    return "unknown status";
}

size_t tfb_workspace_bytes(const tfb_block_config *cfg, int32_t B, int32_t T, int32_t vocab) {
    if (check_cfg(cfg) != TFB_OK || B <= 0 || T <= 0 || vocab < 0) return 0;
    return ws_layout(*cfg, B, T, vocab).total;
}

tfb_status tfb_workspace_view(const tfb_block_config *cfg, int32_t B, int32_t T, int32_t vocab, int32_t which,
                              size_t *offset) {
    if (check_cfg(cfg) != TFB_OK || B <= 0 || T <= 0 || vocab < 0) return TFB_ERR_SHAPE;
    if (!offset) return TFB_ERR_NULL;
    const WsLayout L = ws_layout(*cfg, B, T, vocab);
    switch (which) {
        case TFB_VIEW_Q: *offset = L.q; return TFB_OK;
        case TFB_VIEW_ATT: *offset = L.att; return TFB_OK;
        case TFB_VIEW_R: *offset = L.r; return TFB_OK;
        case TFB_VIEW_ACT: *offset = L.act; return TFB_OK;
    }
    return TFB_ERR_SHAPE;
}

tfb_status tfb_rope_table_init(const tfb_block_config *cfg, int32_t t_max, float *table, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if (!table) return TFB_ERR_NULL;
    if (!aligned(table)) return TFB_ERR_ALIGN;
    if (t_max <= 0) return TFB_ERR_SHAPE;
    TRY_HIP(rope_table_launch(t_max, cfg->head_dim, (double)cfg->rope_base, table, (hipStream_t)stream));
    return TFB_OK;
}

tfb_status tfb_block_prefill(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                             int32_t t_max_table, const void *x, void *out, int32_t B, int32_t T, int32_t start_pos,
                             tfb_kv_cache *cache, void *ws, size_t ws_bytes, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if ((st = check_weights(w)) != TFB_OK) return st;
    if (!rope_table || !x || !out) return TFB_ERR_NULL;
    if (!aligned(rope_table) || !aligned(x) || !aligned(out)) return TFB_ERR_ALIGN;
    if (B <= 0 || T <= 0 || start_pos < 0) return TFB_ERR_SHAPE;
    if (cache) {
        if ((st = check_cache(cache, B)) != TFB_OK) return st;
        if ((st = check_ring(*cfg, cache->ring, cache->t_max)) != TFB_OK) return st;
        if (!cache->ring && (int64_t)start_pos + T > cache->t_max) return TFB_ERR_CACHE_OVERFLOW;
    } else if (start_pos != 0) {
        return TFB_ERR_SHAPE;
    }
    if ((int64_t)start_pos + T > t_max_table) return TFB_ERR_CACHE_OVERFLOW;
    const WsLayout L = ws_layout(*cfg, B, T, 0);
    if (!ws || ws_bytes < L.total) return TFB_ERR_WORKSPACE;
    if (!aligned(ws)) return TFB_ERR_ALIGN;
    uint8_t *wsb = (uint8_t *)ws;
    if (!cache)
        return run_block(*cfg, *w, rope_table, t_max_table, 0, x, out, B, T, 0, nullptr, wsb + L.kv_k, wsb + L.kv_v,
                         KvMap{nullptr, T, 0, 0, 0, 0, 0}, wsb, L, (hipStream_t)stream);
    return run_prefill(*cfg, *w, rope_table, t_max_table, x, out, B, T, start_pos, cache->k, cache->v,
                       contig_map(*cache), wsb, L, (hipStream_t)stream);
}

tfb_status tfb_block_prefill_varlen(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                    int32_t t_max_table, const void *x, void *out, int32_t B, int32_t T,
                                    const int32_t *start, const int32_t *len, int32_t h_max_end, tfb_kv_cache *cache,
                                    void *ws, size_t ws_bytes, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if ((st = check_weights(w)) != TFB_OK) return st;
    if (!rope_table || !x || !out || !cache || !start || !len) return TFB_ERR_NULL;
    if (!aligned(rope_table) || !aligned(x) || !aligned(out)) return TFB_ERR_ALIGN;
    if (B <= 0 || T <= 0 || h_max_end < 0) return TFB_ERR_SHAPE;
    if ((st = check_cache(cache, B)) != TFB_OK) return st;
    if (cache->ring) return TFB_ERR_UNSUPPORTED;  // per-sequence starts would need per-sequence staging
    if (h_max_end > cache->t_max || h_max_end > t_max_table) return TFB_ERR_CACHE_OVERFLOW;
    const WsLayout L = ws_layout(*cfg, B, T, 0);
    if (!ws || ws_bytes < L.total) return TFB_ERR_WORKSPACE;
    if (!aligned(ws)) return TFB_ERR_ALIGN;
    return run_block(*cfg, *w, rope_table, t_max_table, 0, x, out, B, T, 0, nullptr, cache->k, cache->v,
                     contig_map(*cache), (uint8_t *)ws, L, (hipStream_t)stream, start, len);
}

tfb_status tfb_block_decode(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                            int32_t t_max_table, const void *x, void *out, int32_t B, tfb_kv_cache *cache,
                            const int32_t *pos, int32_t h_max_pos, void *ws, size_t ws_bytes, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if ((st = check_weights(w)) != TFB_OK) return st;
    if (!rope_table || !x || !out || !cache || !pos) return TFB_ERR_NULL;
    if (!aligned(rope_table) || !aligned(x) || !aligned(out)) return TFB_ERR_ALIGN;
    if (B <= 0 || h_max_pos < 0) return TFB_ERR_SHAPE;
    if ((st = check_cache(cache, B)) != TFB_OK) return st;
    if ((st = check_ring(*cfg, cache->ring, cache->t_max)) != TFB_OK) return st;
    if ((!cache->ring && h_max_pos >= cache->t_max) || h_max_pos >= t_max_table) return TFB_ERR_CACHE_OVERFLOW;
    const WsLayout L = ws_layout(*cfg, B, 1, 0);
    if (!ws || ws_bytes < L.total) return TFB_ERR_WORKSPACE;
    if (!aligned(ws)) return TFB_ERR_ALIGN;
    return run_block(*cfg, *w, rope_table, t_max_table, h_max_pos, x, out, B, 1, 0, pos, cache->k, cache->v,
                     contig_map(*cache), (uint8_t *)ws, L, (hipStream_t)stream);
}

// ---- allocation-free decode: see scratch_on_current_device above ----
size_t tfb_noalloc_scratch_bytes(void) { return kScratchBytes; }

tfb_status tfb_block_decode_noalloc(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                    int32_t t_max_table, const void *x, void *out, int32_t B, tfb_kv_cache *cache,
                                    const int32_t *pos, int32_t h_max_pos, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if ((st = check_weights(w)) != TFB_OK) return st;
    if (!rope_table || !x || !out || !cache || !pos) return TFB_ERR_NULL;
    if (!aligned(rope_table) || !aligned(x) || !aligned(out)) return TFB_ERR_ALIGN;
    if (B <= 0 || h_max_pos < 0) return TFB_ERR_SHAPE;
    if ((st = check_cache(cache, B)) != TFB_OK) return st;
    if ((st = check_ring(*cfg, cache->ring, cache->t_max)) != TFB_OK) return st;
    if ((!cache->ring && h_max_pos >= cache->t_max) || h_max_pos >= t_max_table) return TFB_ERR_CACHE_OVERFLOW;
    // the decode-attention partials this call's chunk plan needs (the plan
    // is the one tfb_block_decode makes, so the launches are the same)
    AttnCall a{};
    a.dtype = cfg->dtype;
    a.B = B; a.T = 1; a.H = cfg->n_heads; a.Hkv = cfg->n_kv_heads; a.dh = cfg->head_dim;
    a.max_keys = h_max_pos + 1;
    a.max_splits = kMaxSplits;
    a.window = cfg->window;
    const WsLayout L = ws_layout(*cfg, B, 1, 0, attention_decode_call_bytes(a));
    if (L.total > kScratchBytes) return TFB_ERR_WORKSPACE;
    uint8_t *ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != TFB_OK) return st;
    return run_block(*cfg, *w, rope_table, t_max_table, h_max_pos, x, out, B, 1, 0, pos, cache->k, cache->v,
                     contig_map(*cache), ws, L, (hipStream_t)stream);
}

// Paged cache: validated host fields, and the row map the kernels use.
static tfb_status paged_map(const tfb_paged_kv_cache *pc, int B, KvMap &m) {
    if (!pc->k || !pc->v || !pc->block_table) return TFB_ERR_NULL;
    if (!aligned(pc->k) || !aligned(pc->v)) return TFB_ERR_ALIGN;
    if (pc->batch != B || pc->max_blocks <= 0 || pc->n_blocks <= 0) return TFB_ERR_SHAPE;
    const int bs = pc->block_size;
    if (bs < 8 || bs > (1 << 16) || (bs & (bs - 1))) return TFB_ERR_SHAPE;
    int shift = 0;
    while ((1 << shift) < bs) ++shift;
    if ((int64_t)pc->max_blocks * bs > INT32_MAX) return TFB_ERR_SHAPE;
    m = KvMap{pc->block_table, pc->max_blocks * bs, shift, pc->max_blocks, pc->n_blocks, 0,
              pc->ring ? pc->max_blocks * bs : 0};
    return TFB_OK;
}

tfb_status tfb_block_prefill_paged(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                   int32_t t_max_table, const void *x, void *out, int32_t B, int32_t T,
                                   int32_t start_pos, const tfb_paged_kv_cache *cache, void *ws, size_t ws_bytes,
                                   void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if ((st = check_weights(w)) != TFB_OK) return st;
    if (!rope_table || !x || !out || !cache) return TFB_ERR_NULL;
    if (!aligned(rope_table) || !aligned(x) || !aligned(out)) return TFB_ERR_ALIGN;
    if (B <= 0 || T <= 0 || start_pos < 0) return TFB_ERR_SHAPE;
    KvMap m;
    if ((st = paged_map(cache, B, m)) != TFB_OK) return st;
    if ((st = check_ring(*cfg, m.ring, m.t_max)) != TFB_OK) return st;
    if ((!m.ring && (int64_t)start_pos + T > m.t_max) || (int64_t)start_pos + T > t_max_table)
        return TFB_ERR_CACHE_OVERFLOW;
    const WsLayout L = ws_layout(*cfg, B, T, 0);
    if (!ws || ws_bytes < L.total) return TFB_ERR_WORKSPACE;
    if (!aligned(ws)) return TFB_ERR_ALIGN;
    return run_prefill(*cfg, *w, rope_table, t_max_table, x, out, B, T, start_pos, cache->k, cache->v, m,
                       (uint8_t *)ws, L, (hipStream_t)stream);
}

tfb_status tfb_block_decode_paged(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                  int32_t t_max_table, const void *x, void *out, int32_t B,
                                  const tfb_paged_kv_cache *cache, const int32_t *pos, int32_t h_max_pos, void *ws,
                                  size_t ws_bytes, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if ((st = check_weights(w)) != TFB_OK) return st;
    if (!rope_table || !x || !out || !cache || !pos) return TFB_ERR_NULL;
    if (!aligned(rope_table) || !aligned(x) || !aligned(out)) return TFB_ERR_ALIGN;
    if (B <= 0 || h_max_pos < 0) return TFB_ERR_SHAPE;
    KvMap m;
    if ((st = paged_map(cache, B, m)) != TFB_OK) return st;
    if ((st = check_ring(*cfg, m.ring, m.t_max)) != TFB_OK) return st;
    if ((!m.ring && h_max_pos >= m.t_max) || h_max_pos >= t_max_table) return TFB_ERR_CACHE_OVERFLOW;
    const WsLayout L = ws_layout(*cfg, B, 1, 0);
    if (!ws || ws_bytes < L.total) return TFB_ERR_WORKSPACE;
    if (!aligned(ws)) return TFB_ERR_ALIGN;
    return run_block(*cfg, *w, rope_table, t_max_table, h_max_pos, x, out, B, 1, 0, pos, cache->k, cache->v, m,
                     (uint8_t *)ws, L, (hipStream_t)stream);
}

tfb_status tfb_kv_append(const tfb_block_config *cfg, tfb_kv_cache *cache, const void *k_new, const void *v_new,
                         const int32_t *start, int32_t n_new, int32_t h_max_start, void *stream) {
    tfb_status st = check_cfg(cfg);
    if (st != TFB_OK) return st;
    if (!cache || !k_new || !v_new || !start) return TFB_ERR_NULL;
    if (!aligned(k_new) || !aligned(v_new)) return TFB_ERR_ALIGN;
    if (cache->batch <= 0) return TFB_ERR_SHAPE;
    if ((st = check_cache(cache, cache->batch)) != TFB_OK) return st;
    if (n_new <= 0 || h_max_start < 0) return TFB_ERR_SHAPE;
    if ((st = check_ring(*cfg, cache->ring, cache->t_max)) != TFB_OK) return st;
    // a ring takes at most t_max rows per call (more would share slots)
    if (cache->ring ? n_new > cache->t_max : (int64_t)h_max_start + n_new > cache->t_max) return TFB_ERR_CACHE_OVERFLOW;
    hipStream_t s = (hipStream_t)stream;
    const KvMap kvm = contig_map(*cache);
    TRY_HIP(STAGE(ST_KV_APPEND, kv_append_launch(cfg->dtype, cache->k, cache->v, k_new, v_new, start, cache->batch,
                                                 n_new, cfg->n_kv_heads, cfg->head_dim, kvm, s)));
    return TFB_OK;
}

tfb_status tfb_model_forward(const tfb_model *model, const float *rope_table, int32_t t_max_table, const int32_t *ids,
                             int32_t B, int32_t T, tfb_kv_cache *caches, int32_t *lens, int32_t h_max_len,
                             float *logits, int32_t last_only, int32_t *next_ids, void *ws, size_t ws_bytes,
                             void *stream) {
    if (!model) return TFB_ERR_NULL;
    const tfb_block_config &c = model->blk;
    tfb_status st = check_cfg(&c);
    if (st != TFB_OK) return st;
    if (!model->embed || !model->layers || !model->g_final || !model->w_unembed || !rope_table || !ids ||
        !caches || !lens)
        return TFB_ERR_NULL;
    if (!aligned(model->embed) || !aligned(model->g_final) || !aligned(model->w_unembed) || !aligned(rope_table) ||
        (logits && !aligned(logits)))
        return TFB_ERR_ALIGN;
    if (model->n_layers <= 0 || model->vocab <= 0 || B <= 0 || T <= 0 || h_max_len < 0) return TFB_ERR_SHAPE;
    if (c.dtype == TFB_BF16 && model->vocab % 64) return TFB_ERR_SHAPE;
    if (c.dtype == TFB_F32 && model->vocab % 4) return TFB_ERR_SHAPE;
    if (T > 1 && h_max_len != 0) return TFB_ERR_SHAPE;  // prefill starts every sequence at 0
    for (int l = 0; l < model->n_layers; ++l) {
        if ((st = check_weights(&model->layers[l])) != TFB_OK) return st;
        if ((st = check_cache(&caches[l], B)) != TFB_OK) return st;
        if ((st = check_ring(c, caches[l].ring, caches[l].t_max)) != TFB_OK) return st;
        if (!caches[l].ring && (int64_t)h_max_len + T > caches[l].t_max) return TFB_ERR_CACHE_OVERFLOW;
    }
    if ((int64_t)h_max_len + T > t_max_table) return TFB_ERR_CACHE_OVERFLOW;
    const WsLayout L = ws_layout(c, B, T, model->vocab);
    if (!ws || ws_bytes < L.total) return TFB_ERR_WORKSPACE;
    if (!aligned(ws)) return TFB_ERR_ALIGN;

    hipStream_t s = (hipStream_t)stream;
    uint8_t *wsb = (uint8_t *)ws;
    const int M = B * T, d = c.d, V = model->vocab;
    // Embed ([PID] Tiny example, forward), then the L blocks.
    TRY_HIP(STAGE(ST_EMBED, embed_launch(c.dtype, ids, model->embed, wsb + L.x0, M, d, V, s)));
    void *cur = wsb + L.x0, *nxt = wsb + L.x1;
    // On the skinny path each layer's W2 step also writes the next layer's
    // normed input, and the last one the final norm when the head reads
    // every row.
    const bool fuse = norms_fuse(c, M, L);
    const bool final_fused = fuse && (logits || next_ids) && !(last_only && T > 1);
    // On the large-M path each layer's W2 epilogue folds the next layer's
    // RMSNorm1 (the final norm stays a pass of its own).
    const bool fold = L.rss_bytes > 0;
    FoldedNorm fold_in{nullptr, 0}, fold_out{nullptr, 0};
    for (int l = 0; l < model->n_layers; ++l) {
        const bool last = l + 1 == model->n_layers;
        const void *next_g = last ? (final_fused ? model->g_final : nullptr)
                                  : ((fuse || fold) ? model->layers[l + 1].g_attn : nullptr);
        const bool h_ready = fuse && l > 0;
        const KvMap kvm = contig_map(caches[l]);
        fold_out = FoldedNorm{nullptr, 0};
        if (T > 1)
            st = run_prefill(c, model->layers[l], rope_table, t_max_table, cur, nxt, B, T, 0, caches[l].k, caches[l].v,
                             kvm, wsb, L, s, h_ready, next_g, &fold_in, fold && !last ? &fold_out : nullptr);
        else
            st = run_block(c, model->layers[l], rope_table, t_max_table, h_max_len, cur, nxt, B, 1, 0, lens,
                           caches[l].k, caches[l].v, kvm, wsb, L, s, nullptr, nullptr, h_ready, next_g, &fold_in,
                           fold && !last ? &fold_out : nullptr);
        if (st != TFB_OK) return st;
        fold_in = fold_out;
        void *tmp = cur; cur = nxt; nxt = tmp;
    }
    // Final norm and untied LM head ([TIR] How it works step 4), fp32 logits.
    const void *fin = cur;
    int rows = M;
    if (last_only && T > 1) {
        TRY_HIP(gather_last_launch(c.dtype, cur, wsb + L.last, B, T, d, s));
        fin = wsb + L.last;
        rows = B;
    }
    if (logits || next_ids) {
        void *hn = wsb + L.h;
        if (!final_fused)
            TRY_HIP(STAGE(ST_FINAL_NORM, rmsnorm_launch(c.dtype, fin, d, model->g_final, hn, d, rows, d, c.rms_eps, s)));
        float *lg = logits;
        if (!lg) {
            if (rows != B) {  // next ids only: the head runs on the last rows
                TRY_HIP(gather_last_launch(c.dtype, cur, wsb + L.last, B, T, d, s));
                TRY_HIP(rmsnorm_launch(c.dtype, wsb + L.last, d, model->g_final, hn, d, B, d, c.rms_eps, s));
                rows = B;
            }
            lg = (float *)(wsb + L.logits);
        }
        GemmCall hd{};
        hd.dtype = c.dtype;
        hd.epi = EPI_F32;
        hd.A = hn; hd.lda = d; hd.M = rows; hd.K = d;
        hd.w[0] = model->w_unembed; hd.w_cols[0] = V;
        hd.ep.M = rows; hd.ep.N = V; hd.ep.out = lg; hd.ep.ldo = V;
        hd.scratch = L.skinny_bytes ? wsb + L.skinny : nullptr;
        hd.scratch_bytes = L.skinny_bytes;
        hd.split_scratch = L.gsplit_bytes ? wsb + L.gsplit : nullptr;
        hd.split_bytes = L.gsplit_bytes;
        TRY_HIP(STAGE(ST_LM_HEAD, gemm_launch(hd, s)));
        if (next_ids) {
            // Greedy next token from each sequence's last row ([PID] Under the hood, step 6).
            if (rows == B) {
                TRY_HIP(STAGE(ST_ARGMAX, argmax_launch(lg, V, B, V, next_ids, s)));
            } else {
                TRY_HIP(STAGE(ST_ARGMAX, argmax_launch(lg + (int64_t)(T - 1) * V, (int64_t)T * V, B, V, next_ids, s)));
            }
        }
    }
    TRY_HIP(add_scalar_launch(lens, B, T, s));
    return TFB_OK;
}

}  // extern "C"
