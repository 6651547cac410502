// Device-side helpers shared by the gfx950 kernels of libtfb.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfb {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu); }

// Two fp32 values as a sum of two bf16 pairs: hi = nearest bf16, lo = nearest
// bf16 of what that rounding left (a - hi is exact in fp32).  hi + lo carries
// ~16 significant bits, so a bf16 product fed with both halves and fp32
// accumulation matches an fp32 operand to ~2^-17 relative.  Used for the
// softmax weights of P.V, which the method keeps in fp32.
// Returns {hi, lo}.
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
    const uint32_t hi = pack_bf16x2(a, b);
    return u32x2{hi, pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u))};
}

// Storage-type traits: load/store one element as fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(bf16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// MFMA 32x32x16 bf16 -> fp32 (gfx950).  Lane l supplies row/column l%32 of A/B
// and eight consecutive k values in half (l/32) of the 16-wide k slice.  The
// accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + v%4,
// column l%32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// MFMA 16x16x32 bf16 -> fp32 (gfx950).  Lane l supplies row/column l%16 and
// eight k values in quarter (l/16); accumulator register v holds row
// 4*(l/16) + v, column l%16.
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte load of data read once (KV cache in decode, weights in skinny
// GEMMs): the nontemporal hint keeps it from displacing reused lines and
// measured ~7.0 TB/s on MI355X against ~5 TB/s for plain loads.
__device__ __forceinline__ u32x4 ld_stream(const void *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// 8x8 transpose of bf16 held as eight 16-byte rows: in[r] holds row r
// (8 values along the fast axis); out[c] receives column c (8 values, one per
// input row).  32 byte permutes.
__device__ __forceinline__ void transpose8x8_bf16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t lo = in[2 * w][c >> 1], hi = in[2 * w + 1][c >> 1];
            // even column: low halves of the two rows; odd column: high halves
            out[c][w] = __builtin_amdgcn_perm(hi, lo, (c & 1) ? 0x07060302u : 0x05040100u);
        }
    }
}

// LDS swizzles (XOR on 16-byte chunks / 32-byte granules), chosen so that
// the fragment reads below hit distinct banks whether the LDS interleaves 32
// or 64 four-byte banks:
//  - rows of 128 bytes read as 16-byte chunks, one chunk column, 16
//    consecutive rows at a time: chunk ^ swz_row(row);
//  - rows read by ds_read_b64_tr_b16 (four consecutive rows of 32 bytes per
//    16-lane group, two groups on adjacent granules): granule ^ swz_tr(row).
__device__ __forceinline__ int swz_row(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz_tr(int k) { return (0x6530 >> (4 * (k & 3))) & 0xF; }  // 0, 3, 5, 6

// The values of lanes l % 32 and l % 32 + 32, in that order on both halves
// of the wave: v_permlane32_swap (gfx950) exchanges the halves of two
// registers in one instruction, where a shuffle goes through LDS
// (ds_bpermute, with a wait that also drains the wave's other LDS reads).
__device__ __forceinline__ void halves_of(float x, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
// max / sum of a value over lanes l and l ^ 32 (same result on both lanes;
// max of values that are never NaN)
__device__ __forceinline__ float max_halves(float x) {
    float lo, hi;
    halves_of(x, lo, hi);
    return lo > hi ? lo : hi;
}
__device__ __forceinline__ float sum_halves(float x) {
    float lo, hi;
    halves_of(x, lo, hi);
    return lo + hi;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Where the key and value of absolute position j of sequence b, KV head g
// live in a KV cache.  A position first maps to a slot of the sequence:
//  - slot = j - pos0 (pos0 = 0 except for a prefill's staging copy, whose
//    row 0 holds position pos0);
//  - bounded sliding-window cache (ring > 0): slot = (j - pos0) mod ring, so
//    the cache holds the last `ring` positions ([PID] "The Transformer",
//    Sliding-window attention: with a window the KV cache is capped);
// and a slot to a row (the element offset is row * dh):
//  - contiguous cache [B, Hkv, t_max, dh] (table == NULL);
//  - paged cache: a pool [n_blocks, Hkv, 2^bs_shift, dh] of fixed-size
//    blocks, and a block table [B, max_blocks] giving the pool block of each
//    logical block slot >> bs_shift of a sequence (tirogla "Transformer
//    block", Implementation notes: a KV cache allocated in fixed blocks per
//    sequence).  A table entry outside [0, n_blocks) is clamped into it, so a
//    bad table can give wrong values but never an access outside the pool.
struct KvMap {
    const int32_t *table;
    int t_max;        // slots per sequence (paged: max_blocks << bs_shift)
    int bs_shift, max_blocks, n_blocks;
    int pos0;         // position held by slot 0 (no ring)
    int ring;         // > 0: position j lives in slot (j - pos0) mod ring (ring == t_max)
};
__device__ __forceinline__ int kv_slot(const KvMap &m, int j) {
    const int s = j - m.pos0;  // callers pass j >= pos0
    return m.ring ? s % m.ring : s;
}
// Whether position j has a slot (writes outside the cache are skipped).
__device__ __forceinline__ bool kv_has(const KvMap &m, int j) {
    const int s = j - m.pos0;
    return s >= 0 && (m.ring || s < m.t_max);
}
__device__ __forceinline__ int64_t kv_row_of_slot(const KvMap &m, int b, int Hkv, int g, int s) {
    if (!m.table) return ((int64_t)b * Hkv + g) * m.t_max + s;
    int blk = m.table[(int64_t)b * m.max_blocks + (s >> m.bs_shift)];
    blk = min(max(blk, 0), m.n_blocks - 1);
    return (((int64_t)blk * Hkv + g) << m.bs_shift) + (s & ((1 << m.bs_shift) - 1));
}
__device__ __forceinline__ int64_t kv_row(const KvMap &m, int b, int Hkv, int g, int j) {
    return kv_row_of_slot(m, b, Hkv, g, kv_slot(m, j));
}

// ---- LDS staging helpers (gfx950) ----------------------------------------
// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
// (j % 4) of the 8-byte rows addressed by lanes j/4 + 4i, i = 0..3.  So when
// lane s of a group points at B[kb + s/4][n0 + 4 (s % 4)], lane j receives
// B[kb + 0..3][n0 + j]: four consecutive k values of column n0 + j, the
// layout of an MFMA B fragment.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ u32x2 lds_read_tr16(const bf16_t *p) {
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(__attribute__((address_space(3))) void *)p);
    return __builtin_bit_cast(u32x2, v);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// A wave-uniform value as a scalar register (read from the first lane).
__device__ __forceinline__ int uniform_i32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    return (const void *)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b));
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Issued as inline assembly so that the compiler neither tracks the LDS write
// nor inserts its own vmcnt waits; callers order it with wait_vmcnt and a
// barrier.  An LDS DMA that reads m0 right after a scalar write of m0 needs
// one wait state on this chip family (the compiler adds it for its own
// instructions, not inside inline assembly): without the s_nop, the first
// 16 lanes of the load could still take the previous m0 and land in the
// previous block.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_byte_addr), "v"(gptr)
                 : "memory", "m0");
}

// The same with the address split into a wave-uniform base (SGPR pair) and
// a 32-bit per-lane byte offset: a loop that walks a fixed per-lane pattern
// over consecutive tiles then moves only the scalar base.
// (The base must be the same on every lane; it is read from the first one.)
__device__ __forceinline__ void dma16_sbase(const void *sbase, uint32_t voff, uint32_t lds_byte_addr) {
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_byte_addr), "v"(voff),
                 "s"((const void *)(uintptr_t)ub)
                 : "memory", "m0");
}

// The same for data streamed once (weights in decode GEMMs): the nontemporal
// policy keeps it from displacing reused lines in the caches; measured on
// MI355X it roughly doubles the rate of a weight stream over the plain form.
__device__ __forceinline__ void dma16_stream(const void *gptr, uint32_t lds_byte_addr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_byte_addr), "v"(gptr)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

}  // namespace tfb
