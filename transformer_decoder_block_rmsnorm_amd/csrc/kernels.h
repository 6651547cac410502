// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tfb.h"
#include "epilogue.h"

namespace tfb {

// Decode attention's chunk partials as the activations of the Wo GEMM: the
// skinny kernel merges them itself (what the chunk merge pass computes) and
// writes the merged rows to att_out for later readers of the workspace.
struct AttnChunks {
    const float *part;     // [B][H][max_chunks][dh + 4]: (m, l, -, -, o[dh])
    const int32_t *pos;    // [B] decode positions
    int H, dh, chunk_keys, max_chunks, window;
    KvMap kvm;             // for the key count of each sequence
    void *att_out;         // [B, H*dh] bf16
};

struct GemmCall {
    int dtype;             // TFB_F32 / TFB_BF16
    int epi;               // EpiKind
    const void *A;         // [M, K] activations
    int64_t lda;
    int M, K;
    const void *w[3];      // QKV: wq, wk, wv; SWIGLU: w1, w3; else w[0]
    int w_cols[3];
    EpiParams ep;
    void *scratch;         // split-K partials for skinny (decode) shapes, may be NULL
    size_t scratch_bytes;
    void *split_scratch;   // large-M split-K tail partials (gemm_split_bytes), may be NULL
    size_t split_bytes;
    // EPI_RESID on the skinny path only (see kSkinnyNormMaxN): after storing
    // each output row, RMSNorm the stored row with gain norm_g and write the
    // bf16 result to norm_out [M, N] (the next GEMM's normed input)
    const void *norm_g;
    void *norm_out;
    float norm_eps;
    // EPI_QKV on the skinny path: when set, the split-K partials are left for
    // the decode attention kernel to reduce (no reduce pass is launched) and
    // the split count goes here; other paths leave it untouched (the caller
    // starts it at 0).
    int *qkv_deferred_splits;
    // EPI_RESID on the skinny path only: the activations A are the decode
    // attention's chunk partials (see skinny_takes_attn_chunks); A is unused
    const AttnChunks *attn_chunks;
    // EPI_RESID on the large-M bf16 path (M > kSkinnyMaxM): fold the next
    // RMSNorm (gain norm_g).  The epilogue writes bf16(y * norm_g) to
    // norm_out [M, N] and gemm_fold_parts(M, N, K) partial sums of y^2 per
    // row to norm_ss [M][parts]; the GEMM that reads norm_out passes them
    // as row_ss.
    float *norm_ss;
    // Large-M bf16 path: A holds bf16(x * gain) of a folded RMSNorm, row_ss
    // [M][row_ss_n] the partial sums of x^2 over the K columns; the products
    // of each row are scaled by 1 / sqrt(sum / K + row_ss_eps).
    const float *row_ss;
    int row_ss_n;
    float row_ss_eps;
};
constexpr int kSkinnyNormMaxN = 8192;
// Compute units of the current device (queried once per device; 256 if the
// query fails).
int device_cus();
hipError_t gemm_launch(const GemmCall &c, hipStream_t s);
// Scratch the large-M bf16 GEMM uses for its split-K tail (0: none); with
// less, it runs without splitting.  N_virtual: B columns (gate-up: 2 f).
size_t gemm_split_bytes(int M, int N_virtual, int K);
// Most partial sums of squares per row a folded norm may bring (two threads
// of a GEMM workgroup load a row's partials, kRowSsMaxParts / 2 each).
constexpr int kRowSsMaxParts = 32;
// Partial sums of squares per row that a RESID GEMM of this shape writes when
// it folds the next RMSNorm (0: it cannot fold one).
int gemm_fold_parts(int M, int N, int K);
// Skinny (M <= 64) weight-streaming GEMM with split-K partials in `part`.
constexpr int kSkinnyMaxM = 64;
hipError_t skinny_gemm_launch(const GemmCall &c, void *part, size_t part_bytes, hipStream_t s);
size_t skinny_part_bytes(int M, int K, int N);
// Whether the skinny GEMM of this shape can take its activations as decode
// attention chunk partials (one 16-row tile, a k range of at most 512 per
// workgroup).
bool skinny_takes_attn_chunks(int M, int K, int N);

// y[m] = x[m] * rsqrt(mean(x[m]^2) + eps) * g, rows of width d.
// x_f32: the input rows are fp32 (the block-internal residual) whatever the storage type.
hipError_t rmsnorm_launch(int dtype, const void *x, int64_t ldx, const void *g, void *y, int64_t ldy, int rows, int d,
                          float eps, hipStream_t s, bool x_f32 = false);

// RoPE table [t_max][dh/2] of (cos, sin) from an fp64 angle.
hipError_t rope_table_launch(int t_max, int dh, double base, float *table, hipStream_t s);

// Attention over the KV cache: query row t of sequence b sits at position
// pos[b] (decode, T == 1) or start + t (prefill) and reads cache rows 0..pos.
struct AttnCall {
    int dtype;
    const void *q;        // [B, H, T, dh]
    const void *kc, *vc;  // [B, Hkv, t_max, dh]
    void *o;              // [B, T, H*dh]
    const int32_t *pos;   // decode positions or NULL
    const int32_t *starts, *lens;  // varlen prefill: [B] first position, valid rows (NULL: start, T)
    int B, T, H, Hkv, dh, t_max, start;
    float scale;
    void *partials;       // split-KV scratch (decode), may be NULL
    size_t partial_bytes;
    int max_keys;         // host bound on keys per query (for work sizing)
    int max_splits;       // chunks per (b, h) the partial buffer holds
    int window;           // sliding window: keys per query (0: full causal)
    KvMap kvm;            // cache row addressing (contiguous or paged)
    // decode only: the QKV projection's split-K partials [splits][B][qkv_n]
    // (NULL: q and the new cache rows are already in place).  The attention
    // kernel then sums them in split order, applies RoPE from `rope`
    // ([rope_rows][dh/2] (cos, sin)), writes q to `q` and the new key and
    // value rows to the cache, as the QKV reduce pass would.
    const float *qkv_part;
    int qkv_splits, qkv_n;
    const float *rope;
    int rope_rows;
};
hipError_t attention_prefill_launch(const AttnCall &a, hipStream_t s);
hipError_t attention_decode_launch(const AttnCall &a, hipStream_t s);
// Merge of the split-KV chunk partials into o (after attention_decode_launch).
hipError_t attention_decode_merge_launch(const AttnCall &a, hipStream_t s);
size_t attention_decode_scratch_bytes(int B, int H, int dh, int max_splits);
// Partial-buffer bytes the decode kernels use for this call (its chunk count),
// never more than attention_decode_scratch_bytes(B, H, dh, a.max_splits).
size_t attention_decode_call_bytes(const AttnCall &a);
// Whether attention_decode_launch runs the split MFMA kernel for this call
// (the one that can take the QKV partials in place of the reduce pass).
bool attention_decode_takes_qkv_partials(const AttnCall &a);
// The split decode kernel's chunking of this call (what the chunk merge and
// AttnChunks readers index by); false when the split kernel does not run.
bool attention_decode_chunks(const AttnCall &a, int *chunk_keys, int *max_chunks);

hipError_t kv_append_launch(int dtype, void *kc, void *vc, const void *k_new, const void *v_new, const int32_t *start,
                            int B, int n_new, int Hkv, int dh, const KvMap &kvm, hipStream_t s);
// Keys and values of positions p_lo .. p_lo+n-1 from one cache map to another
// (row width dh in the storage type must be a multiple of 16 bytes).
hipError_t kv_copy_launch(int dtype, const void *sk, const void *sv, const KvMap &sm, void *dk, void *dv,
                          const KvMap &dm, int B, int Hkv, int dh, int p_lo, int n, hipStream_t s);
hipError_t embed_launch(int dtype, const int32_t *ids, const void *table, void *x, int64_t rows, int d, int vocab,
                        hipStream_t s);
// Copy row (T-1) of each sequence of x [B, T, d] into y [B, d].
hipError_t gather_last_launch(int dtype, const void *x, void *y, int B, int T, int d, hipStream_t s);
hipError_t argmax_launch(const float *logits, int64_t ld, int rows, int n, int32_t *out, hipStream_t s);
hipError_t add_scalar_launch(int32_t *v, int n, int32_t add, hipStream_t s);
hipError_t fill_i32_launch(int32_t *v, int n, int32_t value, hipStream_t s);

}  // namespace tfb
