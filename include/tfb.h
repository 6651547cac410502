/*
 * tfb.h — C ABI of libtfb.so: the forward pass of a pre-norm, Llama-style
 * transformer decoder block on AMD Instinct MI355X (gfx950), in full-sequence
 * prefill and in single-token decode against a KV cache, plus a thin model
 * (embedding, L blocks, final norm, untied LM head, greedy next token).
 *
 * The operation is the one described on the page "Transformer block"
 * (tirogla.com/ml-training/transformer-architecture), section "How it works":
 *   h = RMSNorm(x; g_attn); q = h Wq, k = h Wk, v = h Wv; RoPE on q and k;
 *   per head softmax(q k^T / sqrt(dh) + causal mask) v with fp32 softmax,
 *   heads concatenated, r = x + O Wo;
 *   out = r + W2-projection of (SiLU(RMSNorm(r; g_mlp) W1) * RMSNorm(r; g_mlp) W3).
 * Shapes and names follow that page's notation: B batch, T sequence, d width,
 * H query heads, Hkv KV heads (GQA shares each KV head among H/Hkv consecutive
 * query heads), dh = d/H head width, f MLP width, L layers, V vocabulary.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless their name starts with h_ or the
 *    comment says "host".  Arrays are row-major and densely packed.
 *  - Storage is fp32 (TFB_F32) or bf16 (TFB_BF16) as the config says, for
 *    x, out, weights, gains, embedding and the KV cache.  Accumulation, the
 *    softmax and the norms are fp32; logits are always fp32.
 *  - Weights are stored [in, out] and applied as y = x W, the layout of the
 *    scalar block in that page's Code section.
 *  - The caller owns all memory.  The library never allocates or frees device
 *    memory, never synchronises and never reads device memory back, so every
 *    call can be captured into a HIP graph.  Scratch space is the caller's
 *    workspace of at least tfb_workspace_bytes() bytes.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream).  Host-visible arguments are validated before anything is
 *    launched: on an error nothing is launched and no caller buffer changes.
 *    A launch failure returns TFB_ERR_HIP.  Faults that happen on the device
 *    surface at the caller's next synchronisation.
 *  - Pointers must be 16-byte aligned.  For TFB_BF16, d, f must be multiples
 *    of 64, dh must be 64 or 128 and the vocabulary a multiple of 64; for
 *    TFB_F32, dh must be even and at most 256.  Always H*dh == d, H % Hkv == 0.
 *  - No C++ exception crosses this interface.
 */
#ifndef TFB_H
#define TFB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TFB_OK = 0,
    TFB_ERR_NULL = -1,           /* a required pointer is NULL */
    TFB_ERR_SHAPE = -2,          /* sizes violate the constraints above */
    TFB_ERR_DTYPE = -3,          /* unknown storage type */
    TFB_ERR_ALIGN = -4,          /* a pointer is not 16-byte aligned */
    TFB_ERR_WORKSPACE = -5,      /* workspace NULL or smaller than required */
    TFB_ERR_CACHE_OVERFLOW = -6, /* a position bound is not below the cache (or RoPE table) length */
    TFB_ERR_HIP = -7,            /* a kernel launch failed */
    TFB_ERR_UNSUPPORTED = -8     /* valid request the library does not implement */
} tfb_status;

typedef enum { TFB_F32 = 0, TFB_BF16 = 1 } tfb_dtype;

/* Block hyper-parameters (the page's notation).  rope_base is the RoPE
 * frequency base (10000 or 500000 in the workloads); rms_eps is the RMSNorm
 * epsilon inside the square root.  window > 0 limits attention to a sliding
 * window: the query at position p attends to keys p - window + 1 .. p, its own
 * included (pidoku "The Transformer", Sliding-window attention); 0 is full
 * causal attention.  Rows below a query's window are never read.  With a
 * window, a cache may also be a bounded ring (the `ring` field of the cache
 * structs): that page notes that the window caps the KV cache. */
typedef struct {
    int32_t d, n_heads, n_kv_heads, head_dim, d_ff;
    float rope_base, rms_eps;
    int32_t dtype;  /* tfb_dtype */
    int32_t window; /* keys per query; 0 = full causal */
    /* fold_norms != 0 (bf16 calls over more than 64 rows, B * T > 64): an
     * RMSNorm whose input a GEMM of the block produces (RMSNorm2 after the Wo
     * GEMM; in tfb_model_forward also each later layer's RMSNorm1 after the
     * previous W2 GEMM) is folded into that GEMM and the next one instead of
     * running as a pass of its own.  The producing GEMM's epilogue stores
     * bf16(y * g) and per-row partial sums of y^2; the consuming GEMM scales
     * each row of its fp32 products by 1 / sqrt(mean(y^2) + eps).  This is
     * the same product (row m of (s_m y_m * g) W is s_m ((y_m * g) W)); only
     * the place where the GEMM operand is rounded to bf16 moves, from the
     * normalised row to y * g.  0: every RMSNorm's output is the GEMM operand
     * (the tirogla page, Implementation notes: norms in fp32, GEMM operands
     * in bf16).  Ignored for fp32 storage and for calls of at most 64 rows,
     * whose norms already run inside the GEMMs' reduce passes. */
    int32_t fold_norms;
} tfb_block_config;

/* One block's weights, all in the config's storage type, [in, out] layout:
 * g_attn, g_mlp [d]; wq [d, H*dh]; wk, wv [d, Hkv*dh]; wo [H*dh, d];
 * w1 (gate, the SiLU branch) and w3 (up) [d, f]; w2 (down) [f, d].
 * The block has no bias terms (that page's parameter count, How it works). */
typedef struct {
    const void *g_attn, *g_mlp;
    const void *wq, *wk, *wv, *wo;
    const void *w1, *w3, *w2;
} tfb_block_weights;

/* KV cache of one layer: k and v are each [batch, Hkv, t_max, dh] in the
 * config's storage type.  Keys are kept after RoPE, values as projected (the
 * KV cache paragraph of How it works).
 * ring == 0: row t of sequence b holds the token at absolute position t, and
 *   positions must stay below t_max.
 * ring != 0: a bounded sliding-window cache (pidoku "The Transformer",
 *   Sliding-window attention: the KV cache is capped at the window).  It
 *   holds the last t_max positions of each sequence: position p lives in row
 *   p mod t_max, positions are bounded only by the RoPE table, and rows older
 *   than t_max positions are overwritten.  Needs config window > 0 with
 *   window <= t_max (t_max == window is the smallest), and for fp32 storage
 *   dh % 4 == 0.  Every call gives the same results, bit for bit, as on an
 *   uncapped cache; a prefill chunk works in a contiguous copy of its window
 *   in the workspace.  Variable-length prefill does not take a ring cache
 *   (TFB_ERR_UNSUPPORTED). */
typedef struct {
    void *k, *v;
    int32_t batch, t_max;
    int32_t ring;
} tfb_kv_cache;

/* The thin model: embedding [V, d], L blocks, final RMSNorm gain [d] and an
 * untied LM head w_unembed [d, V].  `layers` is a HOST array of L weight sets
 * whose members are device pointers. */
typedef struct {
    tfb_block_config blk;
    int32_t n_layers, vocab;
    const void *embed;
    const tfb_block_weights *layers;
    const void *g_final;
    const void *w_unembed;
} tfb_model;

/* A paged KV cache (tirogla "Transformer block", Implementation notes: a
 * cache allocated in fixed-size blocks per sequence rather than one T_max
 * buffer per request).  k, v: pools [n_blocks, Hkv, block_size, dh] in the
 * config's storage type, device; post-RoPE keys and values as in
 * tfb_kv_cache.  block_table: [batch, max_blocks] int32, device, read-only:
 * row (position) p of sequence b is row p % block_size of pool block
 * block_table[b][p / block_size].  block_size is a power of two in
 * [8, 65536]; a sequence holds up to max_blocks * block_size positions.
 * Table entries must lie in [0, n_blocks) and the blocks of different live
 * sequences must not overlap (device data, not checked on the host: an
 * entry outside the range is clamped into it, so no access leaves the
 * pool).  The caller owns the pools and the table and may hand blocks out
 * and back in any order. */
typedef struct {
    void *k, *v;
    const int32_t *block_table;
    int32_t batch, block_size, max_blocks, n_blocks;
    int32_t ring; /* != 0: bounded window cache over max_blocks * block_size
                     slots, as in tfb_kv_cache: slot p mod that count */
} tfb_paged_kv_cache;

/* Bytes of workspace the calls below need for batch B, sequence T (T = 1 for
 * decode) and, for tfb_model_forward, vocabulary `vocab` (0 = block calls
 * only).  Returns 0 for an invalid config. */
size_t tfb_workspace_bytes(const tfb_block_config *cfg, int32_t B, int32_t T, int32_t vocab);

/* Where the block calls leave their intermediate tensors in the workspace,
 * for inspection after a call returns (tests and tools; the contents stay
 * valid until the next call that uses the workspace).  `which` selects one:
 *   TFB_VIEW_Q   q after RoPE, [B, H, T, dh], storage type;
 *   TFB_VIEW_ATT the concatenated head outputs, [B, T, H*dh], storage type;
 *   TFB_VIEW_R   the first residual r = x + att Wo, [B, T, d], fp32;
 *   TFB_VIEW_ACT the SwiGLU product SiLU(h2 W1) * (h2 W3), [B, T, f],
 *                storage type
 * (the names of the tirogla page, How it works steps 2-3).  Sizes as for
 * tfb_workspace_bytes.  *offset receives the byte offset from the start of
 * the workspace.  Returns TFB_ERR_SHAPE for an invalid config or `which`. */
enum { TFB_VIEW_Q = 0, TFB_VIEW_ATT = 1, TFB_VIEW_R = 2, TFB_VIEW_ACT = 3 };
tfb_status tfb_workspace_view(const tfb_block_config *cfg, int32_t B, int32_t T, int32_t vocab, int32_t which,
                              size_t *offset);

/* Fill the RoPE table: table[t][i] = (cos, sin) of t * base^(-2i/dh) for
 * t < t_max, i < dh/2, angle computed in fp64 and stored as fp32
 * ([t_max, dh/2, 2] fp32, device).  The tirogla page's Implementation notes
 * recommend such a precomputed [T_max, dh/2] table; rotation pairs are the
 * interleaved (2i, 2i+1) components. */
tfb_status tfb_rope_table_init(const tfb_block_config *cfg, int32_t t_max, float *table, void *stream);

/* Full-sequence (or chunked) prefill of one block, the page's How it works
 * steps 2-3.  x, out: [B, T, d]; out may alias x.  Token t of sequence b is
 * at absolute position start_pos + t (0 for a fresh prompt; a positive value
 * continues a sequence whose rows 0..start_pos-1 are already in the cache:
 * chunked prefill).  When cache is non-NULL, rows start_pos..start_pos+T-1 of
 * every sequence are written and attention reads rows 0..start_pos+t; cache
 * batch must equal B and start_pos+T <= t_max.  With cache NULL, start_pos
 * must be 0 and the keys and values stay in the workspace.
 * rope_table: from tfb_rope_table_init with t_max_table >= start_pos + T. */
tfb_status tfb_block_prefill(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                             int32_t t_max_table, const void *x, void *out, int32_t B, int32_t T, int32_t start_pos,
                             tfb_kv_cache *cache, void *ws, size_t ws_bytes, void *stream);

/* Batched prefill of sequences of different lengths and start positions
 * (variable-length, right-padded): row t of sequence b holds a real token
 * when t < len[b], at absolute position start[b] + t, and is padding
 * otherwise.  A real token attends to rows 0..start[b]+t of its own
 * sequence's cache, so it never attends to a pad key (the tirogla page's
 * Pitfalls: pad tokens must be masked in batched prefill); padding rows write
 * nothing to the cache, and their rows of out hold unspecified values.
 * x, out: [B, T, d]; start, len: [B] int32, device, read-only, with
 * 0 <= len[b] <= T; rows 0..start[b]-1 of the cache must already hold the
 * sequence's earlier keys and values.  h_max_end: host upper bound of
 * max_b (start[b] + len[b]), at most cache t_max and t_max_table (checked;
 * the device values are trusted to respect it).  Other arguments as
 * tfb_block_prefill; the workspace is tfb_workspace_bytes(cfg, B, T, 0). */
tfb_status tfb_block_prefill_varlen(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                    int32_t t_max_table, const void *x, void *out, int32_t B, int32_t T,
                                    const int32_t *start, const int32_t *len, int32_t h_max_end, tfb_kv_cache *cache,
                                    void *ws, size_t ws_bytes, void *stream);

/* One decode step of one block for B sequences: each new token's q
 * [B, H, 1, dh] attends over its sequence's cache (KV cache paragraph of
 * How it works).  x, out: [B, 1, d], out may alias x.  pos: [B] int32 (device,
 * read-only): the position of each new token, which is also the number of
 * valid cache rows before the step.  Row pos[b] of the cache is written with
 * the new post-RoPE k and v and attention reads rows 0..pos[b].  h_max_pos is
 * a host upper bound of max(pos) and must be < t_max and < t_max_table;
 * device code additionally never touches rows >= t_max.  Positions are not
 * advanced (the caller, or tfb_model_forward, does that). */
tfb_status tfb_block_decode(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                            int32_t t_max_table, const void *x, void *out, int32_t B, tfb_kv_cache *cache,
                            const int32_t *pos, int32_t h_max_pos, void *ws, size_t ws_bytes, void *stream);

/* tfb_block_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and the same kernels, with the workspace taken from a
 * static device array of the library instead of a caller buffer.  The array
 * holds tfb_noalloc_scratch_bytes() bytes (32 MiB) on every GPU the library
 * runs on, until the process ends; its device address is looked up once per
 * device, on the first call with that device current (the calling thread's
 * current device must be the device of `stream`).  A call whose workspace
 * would exceed it returns TFB_ERR_WORKSPACE before launching anything (the
 * GQA decode step with B = 64, d = 4096, f = 14336 and 4096 cached rows needs
 * ~23 MiB).  Nothing in the array needs to start at zero: every partial
 * result is written before it is read.  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (different streams, or
 * threads) race; serialise them.  No device memory is allocated or freed. */
tfb_status tfb_block_decode_noalloc(const tfb_block_config *cfg, const tfb_block_weights *w,
                                    const float *rope_table, int32_t t_max_table, const void *x, void *out, int32_t B,
                                    tfb_kv_cache *cache, const int32_t *pos, int32_t h_max_pos, void *stream);
/* Size of the static array tfb_block_decode_noalloc works in, per GPU. */
size_t tfb_noalloc_scratch_bytes(void);

/* tfb_block_prefill and tfb_block_decode on a paged cache: the same
 * computation, with cache rows found through the block table (positions and
 * bounds as in the contiguous calls, with t_max = max_blocks * block_size).
 * Prefill writes rows start_pos..start_pos+T-1 of every sequence; decode
 * writes row pos[b] and attends over rows 0..pos[b] (or the window). */
tfb_status tfb_block_prefill_paged(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                   int32_t t_max_table, const void *x, void *out, int32_t B, int32_t T,
                                   int32_t start_pos, const tfb_paged_kv_cache *cache, void *ws, size_t ws_bytes,
                                   void *stream);
tfb_status tfb_block_decode_paged(const tfb_block_config *cfg, const tfb_block_weights *w, const float *rope_table,
                                  int32_t t_max_table, const void *x, void *out, int32_t B,
                                  const tfb_paged_kv_cache *cache, const int32_t *pos, int32_t h_max_pos, void *ws,
                                  size_t ws_bytes, void *stream);

/* Append n_new rows per sequence to the cache: the tirogla page, How it
 * works, KV cache paragraph (the keys, after RoPE, and the values of every
 * past token are stored so that a decode step computes only the new token's).
 * k_new, v_new: [B, n_new, Hkv, dh] device, storage type, already rotated;
 * row t of sequence b, KV head g goes to cache row start[b] + t of that
 * sequence and head.  start: [B] int32 device, read-only; h_max_start is a
 * host upper bound of max(start) with h_max_start + n_new <= t_max (checked;
 * device code also skips any row outside [0, t_max)).  Rows outside the
 * written range are never touched.  Any even dh is accepted for fp32 storage.
 * A ring cache takes rows at their slots p mod t_max, n_new <= t_max. */
tfb_status tfb_kv_append(const tfb_block_config *cfg, tfb_kv_cache *cache, const void *k_new, const void *v_new,
                         const int32_t *start, int32_t n_new, int32_t h_max_start, void *stream);

/* Model forward (the pidoku page "The Transformer", section 5 "The full
 * model": embed, L blocks, final norm, LM head; the tirogla page, How it
 * works steps 1 and 4).  ids: [B, T] int32 device, each in [0, V).
 * caches: HOST array of n_layers caches.  lens: [B] int32 device, in/out:
 *   T > 1  prefill of a fresh prompt: lens must be 0 on entry (every
 *          sequence starts at position 0) and becomes T;
 *   T == 1 decode: the new token sits at position lens[b]; lens[b] += 1.
 * h_max_len: host upper bound of max(lens) on entry (0 for prefill); must
 * satisfy h_max_len + T <= t_max (ring caches: h_max_len + T <= t_max_table).
 * logits (nullable): fp32 [B, T, V], or [B, 1, V] when last_only != 0 (the
 * last row of each sequence only).
 * next_ids (nullable): [B] int32, argmax of each sequence's last row, lowest
 * index on ties (greedy decoding). */
tfb_status tfb_model_forward(const tfb_model *model, const float *rope_table, int32_t t_max_table, const int32_t *ids,
                             int32_t B, int32_t T, tfb_kv_cache *caches, int32_t *lens, int32_t h_max_len,
                             float *logits, int32_t last_only, int32_t *next_ids, void *ws, size_t ws_bytes,
                             void *stream);

/* Benchmark instrumentation (host side, off by default).  While enabled,
 * every launch of a selected stage made by the calls above is bracketed by a
 * pair of HIP events recorded on the call's stream.  tfb_profile_stages
 * selects the stages: bit i of mask selects stage i (default: all; an event
 * pair costs the stream a short gap, so timing one kernel inside a timed
 * region selects just that one).  tfb_profile_read waits for the recorded
 * events, writes the summed milliseconds and launch counts per stage into
 * ms[i] and calls[i] for i < n (either may be NULL), forgets the records and
 * returns the number of stages.  Stage i is named by tfb_profile_stage_name.
 * Not for use under graph capture; the event pool is created lazily on the
 * host and holds no device memory. */
tfb_status tfb_profile_enable(int32_t on);
tfb_status tfb_profile_stages(uint32_t mask);
int32_t tfb_profile_read(float *ms, int32_t *calls, int32_t n);
const char *tfb_profile_stage_name(int32_t stage);

/* Static description of a status code. */
const char *tfb_status_string(tfb_status s);

/* Library version (major*10000 + minor*100 + patch). */
int32_t tfb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TFB_H */
