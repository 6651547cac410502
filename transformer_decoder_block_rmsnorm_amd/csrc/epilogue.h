// Fused GEMM epilogues of the decoder block (shared by the bf16 MFMA GEMM and
// the fp32 GEMM).  Page short names: [TIR] tirogla "Transformer block".
#pragma once
#include "common.h"

namespace tfb {

enum EpiKind {
    EPI_QKV = 0,    // RoPE on q and k, q -> [B,H,T,dh] workspace, k and v -> KV cache rows
    EPI_RESID = 1,  // out = residual + acc            ([TIR] How it works steps 2 and 3)
    EPI_SWIGLU = 2, // act = SiLU(gate) * up           ([TIR] How it works step 3)
    EPI_F32 = 3,    // fp32 store (logits)
};

struct EpiParams {
    int M, N;                // logical output rows / columns
    void *out;               // RESID, SWIGLU: storage type T; F32: float
    int64_t ldo;
    const void *res;         // RESID residual input (may alias out)
    int64_t ldr;
    int res_f32, out_f32;    // RESID: residual / output held in fp32 instead of the storage type
    // QKV
    void *q, *kc, *vc;       // q [B,H,T,dh]; caches [B,Hkv,t_max,dh]
    const float *rope;       // [t_max_table][dh/2][2] (cos, sin)
    const int32_t *pos;      // decode: [B] positions (T == 1); NULL: start + t
    const int32_t *starts;   // varlen prefill: [B] position of row 0 (NULL: start)
    const int32_t *lens;     // varlen prefill: [B] valid rows; later rows are padding (NULL: all T)
    int T, H, Hkv, dh, t_max, start;
    KvMap kvm;               // cache row addressing (contiguous or paged)
    int rope_rows;           // rows of the RoPE table (device positions are clamped to it)
    int vec8;                // set by the GEMM launcher: 8-column groups may use 16-byte accesses
    // RESID on the large-M bf16 GEMM, with the next RMSNorm folded in (nu
    // non-null): besides y, write nu[m, c] = bf16(y[m, c] * ng[c]) and, per
    // row and column tile of the launch, the sum of y^2 over the tile's
    // columns to nss[m * nss_n + tile] (y as stored: rounded to bf16 unless
    // out_f32).  The GEMM that takes nu as its A operand applies the row
    // scale 1 / sqrt(sum / N + eps) to its products.
    const bf16_t *ng;
    bf16_t *nu;
    int64_t ldu;
    float *nss;
    int nss_n;
};

// Eight consecutive bf16 values -> one 16-byte store.
// Output stores of the epilogues take the nontemporal policy: a round of
// GEMM tiles writes about an L2's worth of output per XCD, which would
// otherwise push out the operand panels the next tiles read (the long-context
// step ran ~0.35% faster this way; decode unchanged).
__device__ __forceinline__ void store_bf16x8(bf16_t *dst, const float (&v)[8]) {
    u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    __builtin_nontemporal_store(w, (u32x4 *)dst);
}
// y as the RESID epilogue stored it: fp32, or rounded to the storage type.
__device__ __forceinline__ float as_stored(const EpiParams &p, float y) {
    return p.out_f32 ? y : bf16_lo(pack_bf16x2(y, 0.0f));
}

// The folded norm's part of one 8-column group of row m: nu = bf16(y * g)
// (gains g of the group's columns, already widened) and the group's sum of
// y^2, returned.  A group lies wholly inside the row or wholly past its end
// (N is a multiple of 8, checked by the launcher); rows past M and groups
// past N contribute nothing and write nothing.
__device__ __forceinline__ float epi_norm8(const EpiParams &p, int m, int c, const float (&y)[8],
                                           const float (&g)[8]) {
    if (m >= p.M || c >= p.N) return 0.0f;
    float u[8], ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        u[k] = y[k] * g[k];
        ss += y[k] * y[k];
    }
    // plain stores: the next GEMM reads these rows right away, many times
    // over, and they should stay in the caches for it
    *(u32x4 *)(p.nu + (int64_t)m * p.ldu + c) =
        u32x4{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(u[4], u[5]), pack_bf16x2(u[6], u[7])};
    return ss;
}

// Position of output row m (token t of sequence b).
__device__ __forceinline__ void qkv_row(const EpiParams &p, int m, int &b, int &t, int &ps) {
    b = m / p.T;
    t = m - b * p.T;
    ps = p.pos ? p.pos[b] : (p.starts ? p.starts[b] : p.start) + t;
}

// Store the pair of output columns (c, c+1), c even, of row m.
template <int KIND, typename T>
__device__ __forceinline__ void epi_store_pair(const EpiParams &p, int m, int c, float v0, float v1) {
    if (m >= p.M || c >= p.N) return;
    if constexpr (KIND == EPI_RESID) {
        // The block-internal residual r stays fp32 so that only the block
        // output is rounded to the storage type.
        int64_t ir = (int64_t)m * p.ldr + c, io = (int64_t)m * p.ldo + c;
        float r0, r1;
        if (p.res_f32) {
            float2 rr = *(const float2 *)((const float *)p.res + ir);
            r0 = rr.x; r1 = rr.y;
        } else {
            r0 = Elem<T>::load((const T *)p.res, ir);
            r1 = Elem<T>::load((const T *)p.res, ir + 1);
        }
        if (p.out_f32) {
            *(float2 *)((float *)p.out + io) = make_float2(r0 + v0, r1 + v1);
        } else {
            Elem<T>::store((T *)p.out, io, r0 + v0);
            Elem<T>::store((T *)p.out, io + 1, r1 + v1);
        }
    } else if constexpr (KIND == EPI_F32) {
        float *out = (float *)p.out;
        int64_t io = (int64_t)m * p.ldo + c;
        out[io] = v0;
        out[io + 1] = v1;
    } else if constexpr (KIND == EPI_QKV) {
        int b, t, ps;
        qkv_row(p, m, b, t, ps);
        const int qd = p.H * p.dh, kvd = p.Hkv * p.dh;
        // RoPE on q and k only, pairs (2i, 2i+1) rotated by ps * theta_i
        // ([TIR] Code, rope; never on v: [TIR] Pitfalls).
        if (c < qd + kvd) {
            int e = c % p.dh;
            const int pr = min(max(ps, 0), p.rope_rows - 1);
            float2 cs = ((const float2 *)p.rope)[(int64_t)pr * (p.dh >> 1) + (e >> 1)];
            float a = v0, bb = v1;
            v0 = a * cs.x - bb * cs.y;
            v1 = a * cs.y + bb * cs.x;
        }
        if (c < qd) {
            int h = c / p.dh, e = c - h * p.dh;
            T *q = (T *)p.q;
            int64_t iq = (((int64_t)b * p.H + h) * p.T + t) * p.dh + e;
            Elem<T>::store(q, iq, v0);
            Elem<T>::store(q, iq + 1, v1);
        } else {
            if (!kv_has(p.kvm, ps)) return;  // never write outside the cache
            if (p.lens && t >= p.lens[b]) return;  // padding rows leave the cache alone
            int cc = c - qd;
            T *dst = (T *)p.kc;
            if (cc >= kvd) { cc -= kvd; dst = (T *)p.vc; }
            int g = cc / p.dh, e = cc - g * p.dh;
            int64_t ic = kv_row(p.kvm, b, p.Hkv, g, ps) * p.dh + e;
            Elem<T>::store(dst, ic, v0);
            Elem<T>::store(dst, ic + 1, v1);
        }
    }
}

__device__ __forceinline__ void load_bf16x8(const bf16_t *src, float (&v)[8]) {
    const u32x4 w = *(const u32x4 *)src;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
    }
}

// Store output columns c .. c+7 (c a multiple of 8) of row m with 16-byte
// accesses.  The launcher sets p.vec8 when every such group starts 16-byte
// aligned in every tensor it touches (leading dimensions, head width); a
// group that is not whole inside the output, or a launch without vec8, goes
// through the pairwise path, which checks each column.  KIND == EPI_SWIGLU
// takes the finished SiLU(gate) * up values.
// y (RESID with a folded norm, p.nu): receives the values as stored; only the
// 16-byte path fills it (the launcher folds a norm only where every group
// takes that path).
template <int KIND>
__device__ __forceinline__ void epi_store8(const EpiParams &p, int m, int c, const float (&v)[8], float (&y)[8]) {
    if (!p.vec8 || c + 8 > p.N) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            if constexpr (KIND == EPI_SWIGLU) {
                if (m < p.M && c + k < p.N) Elem<bf16_t>::store((bf16_t *)p.out, (int64_t)m * p.ldo + c + k, v[k]);
                if (m < p.M && c + k + 1 < p.N)
                    Elem<bf16_t>::store((bf16_t *)p.out, (int64_t)m * p.ldo + c + k + 1, v[k + 1]);
            } else {
                epi_store_pair<KIND, bf16_t>(p, m, c + k, v[k], v[k + 1]);
            }
        }
        return;
    }
    if (m >= p.M) return;
    if constexpr (KIND == EPI_SWIGLU) {
        store_bf16x8((bf16_t *)p.out + (int64_t)m * p.ldo + c, v);
    } else if constexpr (KIND == EPI_RESID) {
        const int64_t ir = (int64_t)m * p.ldr + c, io = (int64_t)m * p.ldo + c;
        float r[8];
        if (p.res_f32) {
            const f32x4 a = *(const f32x4 *)((const float *)p.res + ir), b = *(const f32x4 *)((const float *)p.res + ir + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) { r[k] = a[k]; r[k + 4] = b[k]; }
        } else {
            load_bf16x8((const bf16_t *)p.res + ir, r);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] += v[k];
        if (p.nu)
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = as_stored(p, r[k]);
        if (p.out_f32) {
            float *o = (float *)p.out + io;
            __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, (f32x4 *)o);
            __builtin_nontemporal_store(f32x4{r[4], r[5], r[6], r[7]}, (f32x4 *)(o + 4));
        } else {
            store_bf16x8((bf16_t *)p.out + io, r);
        }
    } else if constexpr (KIND == EPI_F32) {
        float *o = (float *)p.out + (int64_t)m * p.ldo + c;
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4 *)o);
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, (f32x4 *)(o + 4));
    } else if constexpr (KIND == EPI_QKV) {
        int b, t, ps;
        qkv_row(p, m, b, t, ps);
        const int qd = p.H * p.dh, kvd = p.Hkv * p.dh;
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = v[k];
        if (c < qd + kvd) {
            // RoPE on the four pairs (e, e+1) .. (e+6, e+7) of one head
            const int e = c % p.dh;
            const int pr = min(max(ps, 0), p.rope_rows - 1);
            const f32x4 *cs = (const f32x4 *)(p.rope + ((int64_t)pr * (p.dh >> 1) + (e >> 1)) * 2);
            const f32x4 t0 = cs[0], t1 = cs[1];
            const float co[4] = {t0[0], t0[2], t1[0], t1[2]}, si[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = v[2 * k], bb = v[2 * k + 1];
                w[2 * k] = a * co[k] - bb * si[k];
                w[2 * k + 1] = a * si[k] + bb * co[k];
            }
        }
        if (c < qd) {
            const int h = c / p.dh, e = c - h * p.dh;
            store_bf16x8((bf16_t *)p.q + (((int64_t)b * p.H + h) * p.T + t) * p.dh + e, w);
        } else {
            if (!kv_has(p.kvm, ps)) return;  // never write outside the cache
            if (p.lens && t >= p.lens[b]) return;  // padding rows leave the cache alone
            int cc = c - qd;
            bf16_t *dst = (bf16_t *)p.kc;
            if (cc >= kvd) { cc -= kvd; dst = (bf16_t *)p.vc; }
            const int g = cc / p.dh, e = cc - g * p.dh;
            store_bf16x8(dst + kv_row(p.kvm, b, p.Hkv, g, ps) * p.dh + e, w);
        }
    }
}

template <int KIND>
__device__ __forceinline__ void epi_store8(const EpiParams &p, int m, int c, const float (&v)[8]) {
    float y[8];
    epi_store8<KIND>(p, m, c, v, y);
}

// What the epilogue of one 8-column group reads from memory besides the
// accumulators: the residual (EPI_RESID) or the RoPE (cos, sin) pairs and the
// row's position (EPI_QKV).  Loading it apart from the store lets a caller
// issue the loads of its next rows before it stores the current ones.
struct EpiPre {
    f32x4 a, b;  // RESID: fp32 residual columns 0..3 and 4..7, or the 16 bytes of the bf16 residual in a;
                 // QKV: table entries of pairs 0..1 (a) and 2..3 (b), each (cos, sin)
    int ps;      // QKV: position of the row
};

// Whole-tile fast path.  In a tile that lies wholly inside the output with
// 16-byte groups (p.vec8), a lane keeps the same 8-column group over all of
// its rows, so what depends on the column is computed once (EpiLane), and
// its rows only move forward, so the row's sequence and token are carried
// along instead of divided out for every group.
struct EpiLane {
    int c;          // first column of the group
    int part, head, e;  // QKV: 0 q, 1 k, 2 v; head within that part; offset in the head
    int b, t;       // QKV: sequence and token of the lane's current row
    int m;          // that row
};

template <int KIND>
__device__ __forceinline__ void epi_lane_init(const EpiParams &p, int c, int m, EpiLane &L) {
    L.c = c;
    L.m = m;
    if constexpr (KIND == EPI_QKV) {
        const int qd = p.H * p.dh, kvd = p.Hkv * p.dh;
        int cc = c;
        L.part = cc < qd ? 0 : (cc < qd + kvd ? 1 : 2);
        cc -= L.part == 0 ? 0 : (L.part == 1 ? qd : qd + kvd);
        L.head = cc / p.dh;
        L.e = cc - L.head * p.dh;
        L.b = m / p.T;
        L.t = m - L.b * p.T;
    }
}

// Move the lane to row m (m >= the current row).
template <int KIND>
__device__ __forceinline__ void epi_lane_seek(const EpiParams &p, int m, EpiLane &L) {
    if constexpr (KIND == EPI_QKV) {
        L.t += m - L.m;
        while (L.t >= p.T) { L.t -= p.T; ++L.b; }
    }
    L.m = m;
}

template <int KIND>
__device__ __forceinline__ void epi_load8_lane(const EpiParams &p, const EpiLane &L, EpiPre &pre) {
    if constexpr (KIND == EPI_RESID) {
        const int64_t ir = (int64_t)L.m * p.ldr + L.c;
        if (p.res_f32) {
            pre.a = *(const f32x4 *)((const float *)p.res + ir);
            pre.b = *(const f32x4 *)((const float *)p.res + ir + 4);
        } else {
            pre.a = __builtin_bit_cast(f32x4, *(const u32x4 *)((const bf16_t *)p.res + ir));
        }
    } else if constexpr (KIND == EPI_QKV) {
        pre.ps = p.pos ? p.pos[L.b] : (p.starts ? p.starts[L.b] : p.start) + L.t;
        if (L.part < 2) {
            const int pr = min(max(pre.ps, 0), p.rope_rows - 1);
            const f32x4 *cs = (const f32x4 *)(p.rope + ((int64_t)pr * (p.dh >> 1) + (L.e >> 1)) * 2);
            pre.a = cs[0];
            pre.b = cs[1];
        }
    }
}

template <int KIND>
__device__ __forceinline__ void epi_store8_lane(const EpiParams &p, const EpiLane &L, const float (&v)[8],
                                                const EpiPre &pre, float (&y)[8]) {
    if constexpr (KIND == EPI_SWIGLU) {
        store_bf16x8((bf16_t *)p.out + (int64_t)L.m * p.ldo + L.c, v);
    } else if constexpr (KIND == EPI_RESID) {
        const int64_t io = (int64_t)L.m * p.ldo + L.c;
        float r[8];
        if (p.res_f32) {
#pragma unroll
            for (int k = 0; k < 4; ++k) { r[k] = pre.a[k]; r[k + 4] = pre.b[k]; }
        } else {
            const u32x4 w = __builtin_bit_cast(u32x4, pre.a);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r[2 * k] = bf16_lo(w[k]);
                r[2 * k + 1] = bf16_hi(w[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) r[k] += v[k];
        if (p.nu)
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = as_stored(p, r[k]);
        if (p.out_f32) {
            float *o = (float *)p.out + io;
            __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, (f32x4 *)o);
            __builtin_nontemporal_store(f32x4{r[4], r[5], r[6], r[7]}, (f32x4 *)(o + 4));
        } else {
            store_bf16x8((bf16_t *)p.out + io, r);
        }
    } else if constexpr (KIND == EPI_F32) {
        float *o = (float *)p.out + (int64_t)L.m * p.ldo + L.c;
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4 *)o);
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, (f32x4 *)(o + 4));
    } else if constexpr (KIND == EPI_QKV) {
        float w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = v[k];
        if (L.part < 2) {
            // RoPE on the four pairs of the group ([TIR] Code, rope; never on v)
            const float co[4] = {pre.a[0], pre.a[2], pre.b[0], pre.b[2]}, si[4] = {pre.a[1], pre.a[3], pre.b[1], pre.b[3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = v[2 * k], bb = v[2 * k + 1];
                w[2 * k] = a * co[k] - bb * si[k];
                w[2 * k + 1] = a * si[k] + bb * co[k];
            }
        }
        if (L.part == 0) {
            store_bf16x8((bf16_t *)p.q + (((int64_t)L.b * p.H + L.head) * p.T + L.t) * p.dh + L.e, w);
        } else {
            if (!kv_has(p.kvm, pre.ps)) return;  // never write outside the cache
            if (p.lens && L.t >= p.lens[L.b]) return;  // padding rows leave the cache alone
            bf16_t *dst = (bf16_t *)(L.part == 1 ? p.kc : p.vc);
            store_bf16x8(dst + kv_row(p.kvm, L.b, p.Hkv, L.head, pre.ps) * p.dh + L.e, w);
        }
    }
}

// SwiGLU epilogue: one logical column c of act.
template <typename T>
__device__ __forceinline__ void epi_store_swiglu(const EpiParams &p, int m, int c, float gate, float up) {
    if (m >= p.M || c >= p.N) return;
    Elem<T>::store((T *)p.out, (int64_t)m * p.ldo + c, silu_f(gate) * up);
}

template <int KIND>
__device__ __forceinline__ void epi_store8_lane(const EpiParams &p, const EpiLane &L, const float (&v)[8],
                                                const EpiPre &pre) {
    float y[8];
    epi_store8_lane<KIND>(p, L, v, pre, y);
}

}  // namespace tfb
