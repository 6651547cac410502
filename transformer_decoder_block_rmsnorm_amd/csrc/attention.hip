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
#include <algorithm>

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

    if (a.lens && t >= a.lens[b]) return;  // padding row (after the only barrier)
    int p = a.pos ? a.pos[b] : (a.starts ? a.starts[b] : a.start) + t;
    // never read past the cache (a ring holds every position asked of it)
    if (!a.kvm.ring && p - a.kvm.pos0 >= a.kvm.t_max) p = a.kvm.pos0 + a.kvm.t_max - 1;
    const int n_keys = p + 1;
    const int kvh = h / (a.H / a.Hkv);
    const T *K = (const T *)a.kc;
    const T *V = (const T *)a.vc;

    // sliding window: keys from p - window + 1 ([PID] Sliding-window attention)
    const int k_first = a.window > 0 ? max(0, p - a.window + 1) : 0;
    float m = -INFINITY, l = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j0 = k_first; j0 < n_keys; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        if (j < n_keys) {
            const T *kj = K + kv_row(a.kvm, b, a.Hkv, kvh, j) * a.dh;
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
            const T *vj = V + kv_row(a.kvm, b, a.Hkv, kvh, j0 + jj) * a.dh;
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

// ---------------------------------------------------------------------------
// bf16 prefill: flash-style attention on MFMA 32x32x16 ([GEN] FlashAttention
// entry and [MSA] 6: exact attention computed tile by tile with a running
// softmax, never materialising the T x T score matrix).
//
// Workgroup = NGRP groups of 4 waves over the same 128 query rows of one KV
// head's group (HG heads of the group side by side times 128/HG positions),
// so every K/V tile loaded into LDS serves all query heads that share it
// (GQA).  Each wave owns 32 queries.  With NGRP = 2 the two groups take the
// lower and the upper half of the workgroup's key tiles, each with its own
// LDS ring and running softmax, and are merged through LDS at the end: used
// when the whole grid is resident at once, where the longest causal key
// range is the critical path.  Larger grids run NGRP = 1 at two workgroups
// per CU, where one workgroup's start and end overlap the other's work.
//   S^T[keys, queries] = K . Q^T : lane l holds query l%32, so the softmax of
//                                  a query lives in one lane (plus lane l^32).
//   O^T[e, queries]   += V^T . P^T : P^T comes straight from the S^T
//                                  accumulators, as a hi + lo pair of bf16
//                                  fragments (two products per V^T
//                                  fragment), so the fp32 softmax weights
//                                  keep ~16 significant bits.  Rounded to
//                                  one bf16 operand instead, they made the
//                                  block output's error sigma against the
//                                  fp32 reference 15% larger at the 7B
//                                  shape (the attention delta's 84%).
// K and V tiles of 64 keys go from global memory straight into LDS
// (global_load_lds_dwordx4) in their cache layout, rows of dh values: two K
// slots and two V slots, K loaded two steps ahead of its softmax and V one
// (the loop is a two-step pipeline, described below).
// K rows are read as 16-byte fragments (chunks XOR-swizzled by key); the V^T
// fragments come from the transpose read ds_read_b64_tr_b16 on rows of V
// (32-byte granules swizzled by key), taking keys in the order in which the
// S^T accumulator holds them, so nothing is transposed in registers.
// Tiles entirely above the causal diagonal are skipped per wave; the
// workgroups with the longest key ranges are scheduled first.  Rows a tile
// holds beyond start + T, or (sliding window) below the earliest window of the
// workgroup, are fetched from a clamped valid row and masked out of the
// softmax, so cache rows no query may read (even NaN) never reach the result.
// ---------------------------------------------------------------------------
struct FlashArgs {
    const bf16_t *q, *kc, *vc;
    bf16_t *o;
    int B, T, H, Hkv, t_max, start;
    const int32_t *starts, *lens;  // varlen: [B] first position and valid rows (NULL: start, T)
    int window;  // keys per query (0: full causal)
    KvMap kvm;   // cache row addressing
    int HG, PB, n_qblocks, n_hsub;
    float scale_log2e;
};

// 32-byte granule swizzle of V rows: the four rows one 16-lane group of a
// transpose read touches fall in four different bank groups.
template <int DH>
__device__ __forceinline__ int v_granule_swz(int key) {
    if constexpr (DH >= 128) return swz_tr(key);
    else return key & 3;
}

// Cache row map of the flash kernel: a contiguous slab per (sequence, KV
// head), a paged pool, or a ring (bounded window cache, contiguous or paged).
enum FlashMap { FM_CONTIG = 0, FM_PAGED = 1, FM_RING = 2 };

template <int DH, int MAP, int NGRP>
__global__ __launch_bounds__(NGRP * 256, 3 - NGRP) void flash_prefill_kernel(FlashArgs a) {
    constexpr bool PAGED = MAP != FM_CONTIG;  // rows through the map, one by one
    constexpr int BKV = 64;                    // keys per tile
    constexpr int NS = DH / 16;                // 16-wide dh slices of q.k
    constexpr int NE = DH / 32;                // 32-row e tiles of O^T
    constexpr int KCH = DH / 8;                // 16-byte chunks per row
    constexpr int TILE = BKV * DH;             // elements of one K (or V) tile
    constexpr int NSTG = 2;                    // two stages, each a K slot and a V slot
    constexpr int BLK = 2 * TILE * 2 / 1024;   // 1 KB blocks per stage (K then V)
    constexpr int PER = BLK / 4;               // DMA instructions per wave per tile
    constexpr int RPB = 1024 / (DH * 2);       // keys per 1 KB block
    static_assert(PER * 4 == BLK && RPB * DH * 2 == 1024, "tile splits into 1 KB blocks per wave");
    __shared__ __attribute__((aligned(1024))) bf16_t lds[NGRP * NSTG * 2 * TILE];  // a ring per wave group
    static_assert(NGRP == 1 || 2 * NSTG * 2 * TILE * 2 >= 4 * (NE * 16 + 2) * 64 * 4, "merge staging fits");
    // wave group: lower / upper half of the key tiles
    const int grp = NGRP == 2 ? (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 8) : 0;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_t *)lds + grp * (NSTG * 2 * TILE * 2);
    bf16_t *const ring = lds + grp * (NSTG * 2 * TILE);

    const int tid = threadIdx.x & 255, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    const int nbh = a.B * a.Hkv * a.n_hsub;
    const int qb = a.n_qblocks - 1 - (int)(blockIdx.x / nbh);  // longest key ranges first
    int rem = blockIdx.x % nbh;
    const int hsub = rem % a.n_hsub;
    rem /= a.n_hsub;
    const int kvh = rem % a.Hkv, b = rem / a.Hkv;
    const int G = a.H / a.Hkv;
    const int hl = wave % a.HG, pw = wave / a.HG;
    const int h = kvh * G + hsub * a.HG + hl;
    const int t0 = qb * a.PB + pw * 32;
    // this sequence: rows 0..Tb-1 at positions start+0.. (varlen: its own start and length)
    const int start = a.starts ? a.starts[b] : a.start;
    const int Tb = a.lens ? min(a.lens[b], a.T) : a.T;
    if (qb * a.PB >= Tb) return;  // only padding rows here: the whole block leaves before any barrier
    const int kv_len = start + Tb;
    const int t_last_wg = min(qb * a.PB + a.PB - 1, Tb - 1);
    const int n_tiles = (start + t_last_wg) / BKV + 1;
    const bool wave_active = t0 < Tb;
    const int wave_tiles = wave_active ? (start + min(t0 + 31, Tb - 1)) / BKV + 1 : 0;
    // sliding window: query position p sees keys from p - window + 1, so
    // tiles below the earliest query's window are never loaded, and a wave
    // skips tiles below its own earliest query's window
    const int W = a.window;
    const int key_floor = W > 0 ? max(0, start + qb * a.PB - W + 1) : 0;  // no query here reads below it
    const int first_tile = key_floor / BKV;
    const int wave_first_tile = W > 0 ? max(0, start + t0 - W + 1) / BKV : 0;

    // q fragments (B operand of S^T): row t0 + lr, dh [16s + 8lh, +8)
    bf16x8 qf[NS];
    {
        const int t = t0 + lr;
        const bf16_t *qrow = a.q + (((int64_t)b * a.H + h) * a.T + min(t, Tb - 1)) * DH;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 v = *(const u32x4 *)(qrow + 16 * s + 8 * lh);
            if (t >= Tb) v = u32x4{0, 0, 0, 0};
            qf[s] = as_bf16x8(v);
        }
    }
    const int qpos = start + t0 + lr;
    // cache row j of this sequence and KV head (a contiguous slab unless paged)
    const int64_t slab = ((int64_t)b * a.Hkv + kvh) * a.t_max - a.kvm.pos0;
    auto row = [&](int j) -> int64_t {
        if constexpr (MAP == FM_CONTIG) return slab + j;
        else if constexpr (MAP == FM_PAGED) return kv_row_of_slot(a.kvm, b, a.Hkv, kvh, j - a.kvm.pos0);
        else return kv_row(a.kvm, b, a.Hkv, kvh, j);
    };

    // Per-lane part of this wave's DMA blocks: block bi (K for bi < BLK/2,
    // then V) holds keys RPB*(bi % (BLK/2)) .. +RPB-1; lane slot -> key and
    // the element offset inside the row that belongs in that LDS slot.
    // Computed where needed rather than kept for the whole loop.
    auto blk_key = [&](int i) { return ((wave * PER + i) % (BLK / 2)) * RPB + lane / KCH; };
    auto blk_off = [&](int i) {
        const int key = blk_key(i), pch = lane % KCH;
        return wave * PER + i >= BLK / 2 ? 16 * ((pch >> 1) ^ v_granule_swz<DH>(key)) + 8 * (pch & 1)  // V: granules
                                         : 8 * (pch ^ (key & (KCH - 1)));                              // K: chunks
    };
    // a wave's blocks are all K or all V; byte offset of each lane's chunk
    // from the tile's first cache row (contiguous cache).  Four blocks on,
    // the keys are 4 RPB further and the swizzles (key mod KCH, key mod 4)
    // repeat, so the offsets of blocks 4.. are those of blocks 0..3 plus
    // 4 RPB rows, moved into the scalar base.
    static_assert((BLK / 2) % PER == 0, "a wave fills K blocks or V blocks only");
    constexpr int NVO = PER > 4 ? 4 : PER;
    static_assert(PER == NVO || ((4 * RPB) % KCH == 0 && (4 * RPB) % 4 == 0), "lane offsets repeat every 4 blocks");
    const bf16_t *const kv_src = wave * PER < BLK / 2 ? a.kc : a.vc;
    uint32_t voff[NVO];
#pragma unroll
    for (int i = 0; i < NVO; ++i) voff[i] = (uint32_t)(blk_key(i) * DH + blk_off(i)) * 2u;
    auto issue = [&](int it, int stg) {
        const int j0 = it * BKV;
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base + stg * (2 * TILE * 2) + wave * PER * 1024);
        // every row of the tile is a valid row, and (paged cache) the tile
        // lies in one pool block of at least BKV rows, whose rows for this KV
        // head are consecutive: scalar base + fixed lane offsets.  (A paged
        // ring has a multiple of the block size in slots, so an aligned tile
        // never wraps; a contiguous ring has bs_shift 0 and takes the
        // general path.)
        if ((!PAGED || (1 << a.kvm.bs_shift) >= BKV) && j0 >= key_floor && j0 + BKV <= kv_len) {
            const bf16_t *src = kv_src + row(j0) * DH;
#pragma unroll
            for (int i = 0; i < PER; ++i) dma16_sbase(src + (i / NVO) * (NVO * RPB * DH), voff[i % NVO], base + i * 1024);
            return;
        }
        int64_t rows[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) rows[i] = row(min(max(j0 + blk_key(i), key_floor), kv_len - 1));
#pragma unroll
        for (int i = 0; i < PER; ++i) dma16(kv_src + rows[i] * DH + blk_off(i), base + i * 1024);
    };

    f32x16 oacc[NE];
#pragma unroll
    for (int te = 0; te < NE; ++te)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[te][v] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // transpose-read geometry: 16-lane group q reads e columns 16(q&1)+..,
    // keys 4(q>>1)+.. of each 8-key half of a 16-key slice
    const int q4 = lane >> 4, sl = lane & 15;
    const int v_row = 4 * (q4 >> 1) + (sl >> 2), v_in = (sl & 3) * 4;

    // key tiles of this wave group; both groups run n_lo steps so that their
    // barriers pair up
    const int n_lo = NGRP == 2 ? (n_tiles - first_tile + 1) / 2 : n_tiles - first_tile;
    const int g_first = grp ? first_tile + n_lo : first_tile, g_end = grp ? n_tiles : first_tile + n_lo;
    // tiles this wave computes: its group's, inside its own causal and window range
    const int w_lo = max(g_first, wave_first_tile), w_hi = min(g_end, wave_tiles);

    // S^T of a tile from K slot ks
    auto scores = [&](int ks, f32x16 (&S)[2]) {
        const bf16_t *Ks = ring + ks * 2 * TILE;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) S[kt][v] = 0.0f;
            const int key = kt * 32 + lr;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 kf = as_bf16x8(*(const u32x4 *)(Ks + key * DH + (((2 * s + lh) ^ (key & (KCH - 1))) * 8)));
                S[kt] = mfma32(kf, qf[s], S[kt]);
            }
        }
    };
    // Softmax and P.V of tile it (scores S, V slot vs), online in the log2
    // domain.  The reference max of a query moves only when a tile raises it
    // by more than 2^8 (in exponent units): until then the weights 2^(x - m)
    // stay below 256 and the running sums stay exact up to rounding, so the
    // output accumulators are rescaled only on those rare tiles.
    // The first part: mask, max and the rare rescale; returns the max the
    // weights of this tile are taken against.
    auto softmax_head = [&](int it, f32x16 (&S)[2]) -> float {
        const int j0 = it * BKV;
        // The diagonal crosses this tile, or (window) its lower edge does;
        // rows past start + T sit above every real query's diagonal.  One
        // wave-uniform branch around the masking selects (a test per element
        // would put a branch in front of every score; the empty asm keeps the
        // compiler from executing the selects on every tile instead of
        // branching).
        const bool need_mask = (j0 + BKV - 1 > start + t0) || (W > 0 && j0 < start + t0 + 31 - W + 1);
        const int key_lo = W > 0 ? qpos - W + 1 : 0;
        if (need_mask) {
            asm volatile("");
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = j0 + kt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    S[kt][v] = (key > qpos || key < key_lo) ? -INFINITY : S[kt][v];
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, S[kt][v]);
        mx = max_halves(mx) * a.scale_log2e;  // lane l holds keys 4lh.. of its query, l ^ 32 the rest
        const bool grow = mx > m_run + 8.0f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
            if (grow) m_run = mx;
            l_run *= alpha;
#pragma unroll
            for (int te = 0; te < NE; ++te)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[te][v] *= alpha;
        }
        return m_run == -INFINITY ? 0.0f : m_run;
    };
    // The rest: the weights and their products with V (slot vs).
    auto softmax_tail = [&](int vs, f32x16 (&S)[2], float msub) {
        const bf16_t *Vs = ring + vs * 2 * TILE + TILE;
        float sum = -0.0f;  // the additive identity: the first add folds away
        // One 16-key slice at a time, so that the products of a slice run
        // while the next slice's weights are formed.  P^T fragment of slice
        // s2: lane (query lr, half lh) holds keys 16 s2 + {4lh .. 4lh+3,
        // 8+4lh .. 8+4lh+3}.  The weights are fp32 softmax values; they enter
        // the bf16 product as a hi + lo pair of bf16 fragments, both against
        // the same V^T fragment.
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            f32x16 &src = S[s2 >> 1];
            const int o = 8 * (s2 & 1);
#pragma unroll
            for (int v = o; v < o + 8; ++v) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(src[v], a.scale_log2e, -msub));
                src[v] = p;
                sum += p;
            }
            u32x4 w, wl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 hl = split_bf16x2(src[o + 2 * i], src[o + 2 * i + 1]);
                w[i] = hl[0];
                wl[i] = hl[1];
            }
            const bf16x8 pf = as_bf16x8(w), pl = as_bf16x8(wl);
#pragma unroll
            for (int te = 0; te < NE; ++te) {
                const int gran = 2 * te + (q4 & 1);
                const int r0 = 16 * s2 + v_row, r1 = r0 + 8;
                const u32x2 lo = lds_read_tr16(Vs + r0 * DH + ((gran ^ v_granule_swz<DH>(r0)) * 16) + v_in);
                const u32x2 hi = lds_read_tr16(Vs + r1 * DH + ((gran ^ v_granule_swz<DH>(r1)) * 16) + v_in);
                const bf16x8 vf = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                oacc[te] = mfma32(vf, pf, oacc[te]);
                oacc[te] = mfma32(vf, pl, oacc[te]);
            }
        }
        l_run += sum_halves(sum);
    };

    // Software pipeline over the key tiles: step s issues the score products
    // of tile s+1, then the softmax and P.V of tile s, so the matrix cores
    // still work on the next scores while this tile's vector work starts.
    // K tile j sits in K slot (j - g_first) % 2 and is loaded two steps
    // before its softmax, V tile j in V slot (j - g_first) % 2, one step
    // before.  Each wave loads K blocks or V blocks only.
    const bool kwave = wave * PER < BLK / 2;
    if (kwave) {
        if (g_first < g_end) issue(g_first, 0);
        if (g_first + 1 < g_end) issue(g_first + 1, 1);
    } else if (g_first < g_end) {
        issue(g_first, 0);
    }
    f32x16 S0[2], S1[2];
    wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    if (g_first >= w_lo && g_first < w_hi) scores(0, S0);
    auto step = [&](int s, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
        const int it = g_first + s;
        wait_vmcnt<0>();                         // this wave's loads of the previous step landed
        asm volatile("s_barrier" ::: "memory");  // every wave's did; every wave is done with the previous step
        if (kwave) {
            if (it + 2 < g_end) issue(it + 2, s & 1);
        } else if (it + 1 < g_end) {
            issue(it + 1, (s + 1) & 1);
        }
        const bool cur = it >= w_lo && it < w_hi, nxt = it + 1 >= w_lo && it + 1 < w_hi;
        if (nxt) scores((s + 1) & 1, Sn);
        // With two workgroups per CU, a wave in its softmax competes with
        // waves issuing the next tile's products; a raised wave priority over
        // the softmax (and the P.V products interleaved with it) took 1.7%
        // off the long-context attention.  Around the score products instead
        // it cost 4%; the single-workgroup layout (NGRP = 2) gained nothing.
        if constexpr (NGRP == 1) __builtin_amdgcn_s_setprio(1);
        if (cur) softmax_tail(s & 1, Sc, softmax_head(it, Sc));
        if constexpr (NGRP == 1) __builtin_amdgcn_s_setprio(0);
    };
    for (int s = 0; s < n_lo; s += 2) {
        step(s, S0, S1);
        if (s + 1 < n_lo) step(s + 1, S1, S0);
    }
    wait_vmcnt<0>();
    if constexpr (NGRP == 2) {
        __syncthreads();  // both rings are free: they hold the merge staging now

        // Merge the two groups' partial softmax states: (m, l, O) of the
        // upper group go through LDS to the wave of the lower group that owns
        // the same queries; both are relative to 2^m of their own group.
        float *xs = (float *)lds + wave * ((NE * 16 + 2) * 64);
        if (grp == 1) {
#pragma unroll
            for (int te = 0; te < NE; ++te)
#pragma unroll
                for (int v = 0; v < 16; ++v) xs[(te * 16 + v) * 64 + lane] = oacc[te][v];
            xs[NE * 16 * 64 + lane] = m_run;
            xs[(NE * 16 + 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (grp == 1) return;
        {
            const float m1 = xs[NE * 16 * 64 + lane], l1 = xs[(NE * 16 + 1) * 64 + lane];
            const float m = fmaxf(m_run, m1);
            const float c0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
            const float c1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
            l_run = l_run * c0 + l1 * c1;
#pragma unroll
            for (int te = 0; te < NE; ++te)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[te][v] = oacc[te][v] * c0 + xs[(te * 16 + v) * 64 + lane] * c1;
        }
    }

    const int t = t0 + lr;
    if (wave_active && t < Tb) {
        const float inv = 1.0f / l_run;
        bf16_t *orow = a.o + ((int64_t)b * a.T + t) * ((int64_t)a.H * DH) + (int64_t)h * DH;
#pragma unroll
        for (int te = 0; te < NE; ++te)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int e = te * 32 + 8 * g + 4 * lh;
                u32x2 w;
                w[0] = pack_bf16x2(oacc[te][4 * g] * inv, oacc[te][4 * g + 1] * inv);
                w[1] = pack_bf16x2(oacc[te][4 * g + 2] * inv, oacc[te][4 * g + 3] * inv);
                *(u32x2 *)(orow + e) = w;
            }
    }
}

static hipError_t flash_launch(const AttnCall &c, hipStream_t s) {
    FlashArgs a;
    a.q = (const bf16_t *)c.q;
    a.kc = (const bf16_t *)c.kc;
    a.vc = (const bf16_t *)c.vc;
    a.o = (bf16_t *)c.o;
    a.B = c.B; a.T = c.T; a.H = c.H; a.Hkv = c.Hkv; a.t_max = c.t_max; a.start = c.start;
    a.starts = c.starts;
    a.lens = c.lens;
    a.window = c.window;
    a.kvm = c.kvm;
    const int G = c.H / c.Hkv;
    a.HG = G >= 4 ? 4 : (G >= 2 ? 2 : 1);
    if (G % a.HG) a.HG = 1;
    a.PB = 128 / a.HG;
    a.n_hsub = G / a.HG;
    a.n_qblocks = (c.T + a.PB - 1) / a.PB;
    a.scale_log2e = c.scale * 1.4426950408889634f;
    const int blocks = a.n_qblocks * c.B * c.Hkv * a.n_hsub;
    // the whole grid resident at once (two single-group workgroups per CU):
    // split each workgroup's key range over two wave groups
    const bool two = blocks <= 2 * device_cus();
    // a ring (bounded window cache) maps every row through kv_row, as a
    // paged cache does; the caller guarantees the call's rows do not share slots
    const dim3 g(blocks), b1(256), b2(512);
    const int map = a.kvm.ring ? FM_RING : (a.kvm.table ? FM_PAGED : FM_CONTIG);
#define TFB_FLASH(DH, MAP)                                                                          \
    do {                                                                                           \
        if (two) hipLaunchKernelGGL((flash_prefill_kernel<DH, MAP, 2>), g, b2, 0, s, a);           \
        else hipLaunchKernelGGL((flash_prefill_kernel<DH, MAP, 1>), g, b1, 0, s, a);               \
    } while (0)
    if (c.dh == 128) {
        if (map == FM_RING) TFB_FLASH(128, FM_RING);
        else if (map == FM_PAGED) TFB_FLASH(128, FM_PAGED);
        else TFB_FLASH(128, FM_CONTIG);
    } else {
        if (map == FM_RING) TFB_FLASH(64, FM_RING);
        else if (map == FM_PAGED) TFB_FLASH(64, FM_PAGED);
        else TFB_FLASH(64, FM_CONTIG);
    }
#undef TFB_FLASH
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 decode: split-KV streaming over the cache ([GEN] KV cache and inference
// math: a decode step reads the whole cache and is bandwidth bound).
// One workgroup per (sequence b, KV head, chunk of keys); all G = H/Hkv query
// heads of the KV head are served by one read of each K and V row, and both
// products run on MFMA 16x16x32 with the heads as matrix columns.
// Each workgroup writes (max, sum, unnormalised o) per head; a second kernel
// merges the chunks of a (b, h) with log-sum-exp weights.  Keys at or beyond
// pos[b] + 1 are never loaded.
// ---------------------------------------------------------------------------
constexpr int kDecChunk = 768;       // keys per workgroup (multiple of 256)
constexpr int kDecChunkFew = 256;    // ... when (sequence, KV head) pairs are few

struct DecArgs {
    const bf16_t *q, *kc, *vc;
    bf16_t *o;
    const int32_t *pos;
    float *part;      // [B][H][max_chunks][DH + 4]
    int B, H, Hkv, t_max, max_chunks, chunk_keys;
    int window;       // keys per query (0: full causal)
    KvMap kvm;        // cache row addressing
    float scale_log2e;
    // QKV split-K partials [splits][B][qkv_n] (NULL: q and the new rows are
    // in place); see AttnCall
    const float *qkv_part;
    int qkv_splits, qkv_n;
    const float *rope;
    int rope_rows;
};

// Sum of the QKV partials of columns c, c+1 of sequence b, in split order
// (as the reduce pass adds them).  Every split is loaded before any is
// added: with the count known only at run time, a plain loop would wait for
// each load in turn.
constexpr int kQkvMaxSplits = 16;
__device__ __forceinline__ float2 qkv_pair_sum(const DecArgs &a, int b, int c) {
    const float *p = a.qkv_part + (int64_t)b * a.qkv_n + c;
    const int64_t stride = (int64_t)a.B * a.qkv_n;
    float2 t[kQkvMaxSplits];
#pragma unroll
    for (int s = 0; s < kQkvMaxSplits; ++s)
        if (s < a.qkv_splits) t[s] = *(const float2 *)(p + s * stride);
    float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
    for (int s = 0; s < kQkvMaxSplits; ++s)
        if (s < a.qkv_splits) {
            v0 += t[s].x;
            v1 += t[s].y;
        }
    return make_float2(v0, v1);
}
// RoPE of the pair (e, e+1) of a head at position ps ([TIR] Code, rope).
__device__ __forceinline__ float2 rope_pair(const DecArgs &a, int dh, int ps, int e, float2 v) {
    const int pr = min(max(ps, 0), a.rope_rows - 1);
    const float2 cs = ((const float2 *)a.rope)[(int64_t)pr * (dh >> 1) + (e >> 1)];
    return make_float2(v.x * cs.x - v.y * cs.y, v.x * cs.y + v.y * cs.x);
}

template <int DH, int G, bool RING, bool QKV>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecArgs a) {
    // Per wave, 64 keys at a time on MFMA 16x16x32 (lane l: column l%16,
    // k group g = l/16):
    //   S^T[keys, heads] = K . Q^T   K loaded as whole rows (each load
    //                                 instruction covers 1 KB of consecutive
    //                                 rows, the fastest streaming pattern),
    //                                 written to a wave-private LDS slot
    //                                 (16-byte chunks swizzled by row) and
    //                                 read back as MFMA fragments;
    //   O[heads, e]     += P . V     V loaded 8 rows x 16 bytes per lane
    //                                 (whole rows per instruction) and
    //                                 transposed 8x8 in registers; output
    //                                 column n of tile c is e = 8n + c.
    // Heads are MFMA columns: G <= 16 (unused columns are zero).
    // QKV: a.qkv_part holds the QKV projection's split-K partials; this
    // kernel builds q and the new key and value rows from them.
    static_assert(G <= 16, "at most 16 query heads per KV head");
    constexpr int NS = DH / 32;        // 32-wide dh slices
    constexpr int NCH = DH / 8;        // 16-byte chunks per row
    __shared__ __attribute__((aligned(16))) float red_o[4][G][DH];
    __shared__ float red_ml[4][G][2];
    __shared__ __attribute__((aligned(16))) bf16_t kst[4][64 * DH];  // per wave: 64 K rows
    // QKV: the new key and value row, and q, built from the partials
    __shared__ __attribute__((aligned(16))) bf16_t newkv[QKV ? 2 : 1][QKV ? DH : 8];
    __shared__ __attribute__((aligned(16))) bf16_t qsh[QKV ? G : 1][QKV ? DH : 8];
    constexpr int RPI = 64 / NCH;  // K rows per whole-row load instruction

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, g4 = lane >> 4;
    // grid (Hkv, B, chunks): consecutive workgroups, which the hardware deals
    // to the 8 XCDs in turn, are different (sequence, KV head) pairs of one
    // chunk index, so every XCD gets the same mix of long and empty chunks
    const int kvh = blockIdx.x, b = blockIdx.y, ch = blockIdx.z;
    const int n_keys = a.kvm.ring ? a.pos[b] + 1 : min(a.pos[b] + 1, a.kvm.pos0 + a.kvm.t_max);
    // keys [k_first, n_keys): all of them, or the last `window` ones
    const int k_first = a.window > 0 ? max(0, n_keys - a.window) : 0;
    const int k_begin = k_first + ch * a.chunk_keys;
    if (k_begin >= n_keys) return;  // whole block leaves before any barrier
    const int k_end = min(n_keys, k_begin + a.chunk_keys);
    const int h0 = kvh * G;
    const int pos_b = a.pos[b];
    // with the QKV partials: this workgroup holds the new key (position
    // pos[b]) when its chunk ends there and the cache has a row for it
    const bool has_new = QKV && k_end == pos_b + 1 && kv_has(a.kvm, pos_b);

    if constexpr (QKV) {
        // q of the G heads and (the workgroup holding position pos[b]) the
        // new key and value row, one pair of columns per item: summed over
        // the splits, rotated, rounded to bf16 as the reduce pass does.  All
        // items' partials are loaded before anything is stored.
        constexpr int NQ = G * (DH / 2), NIT = (NQ + DH + 255) / 256;
        float2 sum[NIT];
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
            const int i = tid + 256 * k, j = i - NQ;
            const bool item = i < NQ || (has_new && j < DH);
            const int col = i < NQ ? (h0 + i / (DH / 2)) * DH + 2 * (i % (DH / 2))
                                   : a.H * DH + (j / (DH / 2)) * a.Hkv * DH + kvh * DH + 2 * (j % (DH / 2));
            sum[k] = item ? qkv_pair_sum(a, b, col) : make_float2(0.0f, 0.0f);
        }
#pragma unroll
        for (int k = 0; k < NIT; ++k) {
            const int i = tid + 256 * k, j = i - NQ;
            if (i < NQ) {
                const int hh = i / (DH / 2), e = 2 * (i % (DH / 2));
                const float2 r = rope_pair(a, DH, pos_b, e, sum[k]);
                const uint32_t w = pack_bf16x2(r.x, r.y);
                *(uint32_t *)&qsh[hh][e] = w;
                if (ch == 0) *(uint32_t *)((bf16_t *)a.q + ((int64_t)b * a.H + h0 + hh) * DH + e) = w;  // q in the workspace
            } else if (has_new && j < DH) {
                const int kv = j / (DH / 2), e = 2 * (j % (DH / 2));
                const float2 r = kv == 0 ? rope_pair(a, DH, pos_b, e, sum[k]) : sum[k];
                const uint32_t w = pack_bf16x2(r.x, r.y);
                *(uint32_t *)&newkv[kv][e] = w;
                bf16_t *dst = (bf16_t *)(kv == 0 ? a.kc : a.vc);
                *(uint32_t *)(dst + kv_row(a.kvm, b, a.Hkv, kvh, pos_b) * DH + e) = w;
            }
        }
        __syncthreads();  // q and the new row are in LDS for every wave
    }
    // Q^T operand: column = head ln, k slots = dh chunk 4s + g4
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4 v = {0, 0, 0, 0};
        if (ln < G)
            v = QKV ? *(const u32x4 *)&qsh[ln][(4 * s + g4) * 8]
                    : *(const u32x4 *)(a.q + ((int64_t)b * a.H + h0 + ln) * DH + (4 * s + g4) * 8);
        qf[s] = as_bf16x8(v);
    }
    const bool v_lane = ln < NCH;  // dh = 64 uses half the output columns

    float m_run = -INFINITY, l_run = 0.0f;  // for head ln
    f32x4 oacc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) oacc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int base = k_begin + wave * 64; base < k_end; base += 256) {
        // cache row of key base + o, o < 64.  A ring (bounded window cache):
        // the slot of `base` once, then a wrap by a compare
        int sbase = base;
        if constexpr (RING) sbase = kv_slot(a.kvm, base);
        auto row_at = [&](int o) -> int64_t {
            if constexpr (RING) {
                int sl = sbase + o;
                if (sl >= a.kvm.ring) sl = sl - a.kvm.ring < a.kvm.ring ? sl - a.kvm.ring : sl % a.kvm.ring;
                return kv_row_of_slot(a.kvm, b, a.Hkv, kvh, sl);
            } else {
                return kv_row_of_slot(a.kvm, b, a.Hkv, kvh, base + o - a.kvm.pos0);
            }
        };
        u32x4 kw[NCH], vr[2][8];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int r = RPI * i + lane / NCH, j = base + r;
            kw[i] = (j < k_end) ? ld_stream(a.kc + row_at(r) * DH + (lane % NCH) * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                // slots 0-3: keys 32u + 4g + v; slots 4-7: keys 32u + 16 + 4g + v
                const int o = 32 * u + 16 * (r >> 2) + 4 * g4 + (r & 3), j = base + o;
                vr[u][r] = (v_lane && j < k_end) ? ld_stream(a.vc + row_at(o) * DH + ln * 8) : u32x4{0, 0, 0, 0};
            }
        bf16_t *ks = kst[wave];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int r = RPI * i + lane / NCH, c = lane % NCH;
            *(u32x4 *)(ks + r * DH + ((c ^ (r & (NCH - 1))) * 8)) = kw[i];
        }
        // the new key and value (their cache rows are being written by this
        // workgroup): key row pos[b] - base of this tile, if it is here
        const int rn = pos_b - base;
        if (QKV && has_new && rn >= 0 && rn < 64) {
            asm volatile("");
            if (lane < NCH) *(u32x4 *)(ks + rn * DH + ((lane ^ (rn & (NCH - 1))) * 8)) = *(const u32x4 *)&newkv[0][lane * 8];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int o = 32 * u + 16 * (r >> 2) + 4 * g4 + (r & 3);
                    if (v_lane && o == rn) vr[u][r] = *(const u32x4 *)&newkv[1][ln * 8];
                }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 sacc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const int r = 16 * t + ln;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 kf = *(const u32x4 *)(ks + r * DH + (((4 * s + g4) ^ (r & (NCH - 1))) * 8));
                sacc[t] = mfma16(as_bf16x8(kf), qf[s], sacc[t]);
            }
        }
        // the slot is rewritten by the next iteration: its reads come first
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // online softmax for head ln over keys 16t + 4g + v
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int j = base + 16 * t + 4 * g4 + v;
                const float x = (j < k_end) ? sacc[t][v] * a.scale_log2e : -INFINITY;
                sacc[t][v] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);  // key `base` is valid: finite
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float p = __builtin_amdgcn_exp2f(sacc[t][v] - m_new);
                sacc[t][v] = p;
                sum += p;
            }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        l_run = l_run * alpha + sum;
        m_run = m_new;
        // O rows are heads 4*g4 + v: fetch their rescale factors
        float al[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) al[v] = __shfl(alpha, 4 * g4 + v, 64);
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) oacc[c][v] *= al[v];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            // fp32 softmax weights as a hi + lo pair of bf16 operands
            u32x4 pw, pwl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 hl = split_bf16x2(sacc[2 * u + (i >> 1)][2 * (i & 1)], sacc[2 * u + (i >> 1)][2 * (i & 1) + 1]);
                pw[i] = hl[0];
                pwl[i] = hl[1];
            }
            const bf16x8 pf = as_bf16x8(pw), pl = as_bf16x8(pwl);
            u32x4 vt[8];
            transpose8x8_bf16(vr[u], vt);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                oacc[c] = mfma16(pf, as_bf16x8(vt[c]), oacc[c]);
                oacc[c] = mfma16(pl, as_bf16x8(vt[c]), oacc[c]);
            }
        }
    }
    // per-wave results to LDS: head 4*g4 + v, e = 8*ln + c
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int h = 4 * g4 + v;
        if (h < G && v_lane) {
#pragma unroll
            for (int c = 0; c < 8; ++c) red_o[wave][h][8 * ln + c] = oacc[c][v];
        }
    }
    if (g4 == 0 && ln < G) {
        red_ml[wave][ln][0] = m_run;
        red_ml[wave][ln][1] = l_run;
    }
    __syncthreads();
    // merge the four waves and write this chunk's partial result
    for (int i = tid; i < G * DH; i += 256) {
        const int h = i / DH, e = i % DH;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[w][h][0]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sc = (red_ml[w][h][0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(red_ml[w][h][0] - M);
            L += sc * red_ml[w][h][1];
            O += sc * red_o[w][h][e];
        }
        float *dst = a.part + (((int64_t)b * a.H + h0 + h) * a.max_chunks + ch) * (DH + 4);
        dst[4 + e] = O;
        if (e == 0) { dst[0] = M; dst[1] = L; }
    }
}

// Merge the chunk partials of each (b, h): one wave per pair.
// Chunk count up to which the merge loads every chunk's partial at once.
constexpr int kCombineBatch = 16;

template <int DH>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + wave;
    if (bh >= a.B * a.H) return;
    const int b = bh / a.H;
    const int n_keys = a.kvm.ring ? a.pos[b] + 1 : min(a.pos[b] + 1, a.kvm.pos0 + a.kvm.t_max);
    const int n_range = a.window > 0 ? min(n_keys, a.window) : n_keys;
    const int n_ch = min((n_range + a.chunk_keys - 1) / a.chunk_keys, a.max_chunks);
    const float *base = a.part + (int64_t)bh * a.max_chunks * (DH + 4);
    constexpr int EPL = DH / 64;
    float M = -INFINITY, L = 0.0f, O[EPL] = {};
    if (n_ch <= kCombineBatch) {
        // every chunk's (m, l, o) loaded at once, then combined in chunk
        // order: a loop over a run-time count would wait for each load in turn
        float pm[kCombineBatch], pl[kCombineBatch], po[kCombineBatch][EPL];
#pragma unroll
        for (int c = 0; c < kCombineBatch; ++c) {
            const float *p = base + c * (DH + 4);
            const bool in = c < n_ch;
            pm[c] = in ? p[0] : -INFINITY;
            pl[c] = in ? p[1] : 0.0f;
#pragma unroll
            for (int i = 0; i < EPL; ++i) po[c][i] = in ? p[4 + lane * EPL + i] : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < kCombineBatch; ++c) M = fmaxf(M, pm[c]);
#pragma unroll
        for (int c = 0; c < kCombineBatch; ++c) {
            if (c < n_ch) {
                const float sc = __builtin_amdgcn_exp2f(pm[c] - M);
                L += sc * pl[c];
#pragma unroll
                for (int i = 0; i < EPL; ++i) O[i] += sc * po[c][i];
            }
        }
    } else {
        for (int c = 0; c < n_ch; ++c) M = fmaxf(M, base[c * (DH + 4)]);
        for (int c = 0; c < n_ch; ++c) {
            const float *p = base + c * (DH + 4);
            const float sc = __builtin_amdgcn_exp2f(p[0] - M);
            L += sc * p[1];
#pragma unroll
            for (int i = 0; i < EPL; ++i) O[i] += sc * p[4 + lane * EPL + i];
        }
    }
    const float inv = 1.0f / L;
    bf16_t *out = a.o + (int64_t)bh * DH + lane * EPL;
    if constexpr (EPL == 2) {
        *(uint32_t *)out = pack_bf16x2(O[0] * inv, O[1] * inv);
    } else {
        out[0] = f32_to_bf16(O[0] * inv);
    }
}

size_t decode_part_bytes(int B, int H, int dh, int max_chunks) {
    return (size_t)B * H * max_chunks * (dh + 4) * sizeof(float);
}

template <int DH, bool RING, bool QKV>
static hipError_t decode_launch_g(const AttnCall &c, DecArgs &a, hipStream_t s) {
    const int G = c.H / c.Hkv;
    dim3 grid(c.Hkv, c.B, a.max_chunks);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_attn_kernel<DH, 1, RING, QKV>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((decode_attn_kernel<DH, 2, RING, QKV>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_attn_kernel<DH, 4, RING, QKV>), grid, dim3(256), 0, s, a); break;
        case 8: hipLaunchKernelGGL((decode_attn_kernel<DH, 8, RING, QKV>), grid, dim3(256), 0, s, a); break;
        case 16: hipLaunchKernelGGL((decode_attn_kernel<DH, 16, RING, QKV>), grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
template <int DH>
static hipError_t decode_launch_dh(const AttnCall &c, DecArgs &a, hipStream_t s) {
    if (c.qkv_part)
        return c.kvm.ring ? decode_launch_g<DH, true, true>(c, a, s) : decode_launch_g<DH, false, true>(c, a, s);
    return c.kvm.ring ? decode_launch_g<DH, true, false>(c, a, s) : decode_launch_g<DH, false, false>(c, a, s);
}

// Arguments of the split decode kernels for one call.
static bool split_decode_args(const AttnCall &c, DecArgs &a) {
    a.q = (const bf16_t *)c.q;
    a.kc = (const bf16_t *)c.kc;
    a.vc = (const bf16_t *)c.vc;
    a.o = (bf16_t *)c.o;
    a.pos = c.pos;
    a.part = (float *)c.partials;
    a.B = c.B; a.H = c.H; a.Hkv = c.Hkv; a.t_max = c.t_max;
    // chunk size: kDecChunk keys (768 streamed 5% faster than 512 and 1024
    // at B=64); kDecChunkFew when (sequence, KV head) pairs are few, so that
    // a small batch still spreads over the CUs; grown in steps of kDecChunk
    // when the longest sequence would need more chunks than the partial
    // buffer holds
    const int max_keys = c.window > 0 ? std::min(c.max_keys, c.window) : c.max_keys;
    a.window = c.window;
    int chunks = (max_keys + kDecChunk - 1) / kDecChunk;
    int chunk_keys = kDecChunk;
    if ((int64_t)c.B * c.Hkv * chunks < 2 * (int64_t)device_cus()) {
        chunk_keys = kDecChunkFew;
        chunks = (max_keys + chunk_keys - 1) / chunk_keys;
    }
    if (chunks > c.max_splits) {
        chunk_keys = kDecChunk * ((chunks + c.max_splits - 1) / c.max_splits);
        chunks = (max_keys + chunk_keys - 1) / chunk_keys;
    }
    a.chunk_keys = chunk_keys;
    a.max_chunks = chunks;
    a.kvm = c.kvm;
    a.scale_log2e = c.scale * 1.4426950408889634f;
    a.qkv_part = c.qkv_part;
    a.qkv_splits = c.qkv_splits;
    a.qkv_n = c.qkv_n;
    a.rope = c.rope;
    a.rope_rows = c.rope_rows;
    return decode_part_bytes(c.B, c.H, c.dh, chunks) <= c.partial_bytes;
}

static bool split_decode_applies(const AttnCall &a) {
    const int G = a.H / a.Hkv;
    return a.dtype == TFB_BF16 && (a.dh == 128 || a.dh == 64) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
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

hipError_t attention_prefill_launch(const AttnCall &a, hipStream_t s) {
    if (a.dtype == TFB_BF16 && (a.dh == 128 || a.dh == 64)) return flash_launch(a, s);
    return rowwise_launch(a, s);
}
hipError_t attention_decode_launch(const AttnCall &a, hipStream_t s) {
    if (!split_decode_applies(a)) return rowwise_launch(a, s);
    DecArgs d;
    if (!split_decode_args(a, d)) return hipErrorInvalidValue;
    return a.dh == 128 ? decode_launch_dh<128>(a, d, s) : decode_launch_dh<64>(a, d, s);
}

hipError_t attention_decode_merge_launch(const AttnCall &a, hipStream_t s) {
    if (!split_decode_applies(a)) return hipSuccess;  // the row-wise kernel needs no merge
    DecArgs d;
    if (!split_decode_args(a, d)) return hipErrorInvalidValue;
    const dim3 grid((a.B * a.H + 3) / 4);
    if (a.dh == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(256), 0, s, d);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(256), 0, s, d);
    return hipGetLastError();
}
size_t attention_decode_scratch_bytes(int B, int H, int dh, int max_splits) {
    return decode_part_bytes(B, H, dh, max_splits);
}
// Only for few (sequence, KV head) pairs: there the reduce pass is a launch
// of its own for little work, while with many pairs every workgroup of the
// attention grid would rebuild q from the partials at its start.
bool attention_decode_takes_qkv_partials(const AttnCall &a) {
    return split_decode_applies(a) && 2 * (int64_t)a.B * a.Hkv <= device_cus();
}
bool attention_decode_chunks(const AttnCall &a, int *chunk_keys, int *max_chunks) {
    if (!split_decode_applies(a)) return false;
    DecArgs d;
    if (!split_decode_args(a, d)) return false;
    *chunk_keys = d.chunk_keys;
    *max_chunks = d.max_chunks;
    return true;
}
size_t attention_decode_call_bytes(const AttnCall &a) {
    if (!split_decode_applies(a)) return 0;
    DecArgs d;
    split_decode_args(a, d);
    return decode_part_bytes(a.B, a.H, a.dh, d.max_chunks);
}

}  // namespace tfb
