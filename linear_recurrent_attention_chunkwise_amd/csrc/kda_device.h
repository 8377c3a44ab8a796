// kda_device.h -- device-side helpers shared by the KDA kernels (gfx950).
//
// Conventions used by every kernel:
//  * A "K16 fragment" is the per-lane slice of a 16 x 16 MFMA operand over a
//    16-deep slab of the contraction index: lane l holds the 4 consecutive
//    contraction indices k = 4*(l/16) + e (e = 0..3) of row/column l % 16.
//    The same slice feeds v_mfma_f32_16x16x16_bf16 (one instruction) and
//    v_mfma_f32_16x16x4_f32 (four instructions, one per e), so one tile
//    routine serves the bf16 and the fp32 paths.
//  * A 16 x 16 fp32 accumulator tile D[M][N] holds D[4*(l/16) + e][l % 16] in
//    element e of lane l.  Read along M, that is exactly a K16 fragment, so an
//    accumulator tile can be fed back as the B operand of a product that
//    contracts over its rows (B[k][n] = D[k][n]) without any data movement.
//  * Two K16 fragments over contraction indices [k0, k0+16) and
//    [k0+16, k0+32) form one v_mfma_f32_16x16x32_bf16 operand: the
//    instruction sums over its 32 indices in any order, so putting the two
//    4-element slices side by side (elements 0..3 and 4..7) is a consistent
//    relabelling of k for A and B alike.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// Lower bound of the log-decay (the K3 gate bound g_min = -5).
constexpr float kGMin = -5.0f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Per-key-channel decay alpha = exp(g), g = g_min * sigma(e^A z), evaluated as
// alpha = 2^(K s), s = 1 / (1 + 2^(c2 z)), c2 = -e^A log2(e), K = g_min log2(e),
// with the scale folded into the reciprocal: K s = 1 / (c + c 2^(c2 z)),
// c = 1 / K (one fused multiply-add instead of an add and a multiply).
// For c2*z -> +inf: 2^inf = inf, c + c inf = -inf, 1/-inf = -0, alpha = 1
// exactly; for c2*z -> -inf: 1/c = K, alpha = e^(g_min).  No NaN for any
// finite z.
__device__ __forceinline__ float kda_alpha(float c2, float z) {
    constexpr float c = 1.0f / (kGMin * kLog2e);
    const float e = __builtin_amdgcn_exp2f(c2 * z);
    return __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(__builtin_fmaf(e, c, c)));
}

// Two floats -> a packed pair of bf16 (round to nearest even), low half first:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// Four floats -> four bf16 as two packed conversions.
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
    return __builtin_bit_cast(bf16x4, (uint64_t)pack_bf16x2(a, b) |
                                          ((uint64_t)pack_bf16x2(c, d) << 32));
}

// ---------------------------------------------------------------- MFMA ----

template <typename TO> struct Frag;
template <> struct Frag<bf16> { bf16x4 v; };
template <> struct Frag<float> { f32x4 v; };

__device__ __forceinline__ void mma16(f32x4 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], acc, 0, 0, 0);
}
// Contraction over two adjacent 16-slabs: (a0,b0) over [k0,k0+16), (a1,b1)
// over [k0+16,k0+32).
__device__ __forceinline__ void mma32(f32x4 &acc, const Frag<bf16> &a0, const Frag<bf16> &a1,
                                      const Frag<bf16> &b0, const Frag<bf16> &b1) {
    const bf16x8 a = {a0.v[0], a0.v[1], a0.v[2], a0.v[3], a1.v[0], a1.v[1], a1.v[2], a1.v[3]};
    const bf16x8 b = {b0.v[0], b0.v[1], b0.v[2], b0.v[3], b1.v[0], b1.v[1], b1.v[2], b1.v[3]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x4 &acc, const Frag<float> &a0, const Frag<float> &a1,
                                      const Frag<float> &b0, const Frag<float> &b1) {
    mma16(acc, a0, b0);
    mma16(acc, a1, b1);
}

// K16 fragment from a K-contiguous LDS tile: row (lane % 16) of `tile`
// (row stride `ld` elements), contraction indices k0 + 4*(lane/16) + 0..3.
template <typename TO>
__device__ __forceinline__ Frag<TO> lds_frag(const TO *tile, int ld, int k0, int lane) {
    Frag<TO> f;
    const TO *p = tile + (lane & 15) * ld + k0 + 4 * (lane >> 4);
    if constexpr (sizeof(TO) == 2) {
        f.v = *reinterpret_cast<const bf16x4 *>(p);
    } else {
        f.v = *reinterpret_cast<const f32x4 *>(p);
    }
    return f;
}

// Accumulator tile reused as a K16 fragment (rounded to the operand type).
template <typename TO>
__device__ __forceinline__ Frag<TO> acc_frag(const f32x4 &d) {
    Frag<TO> f;
    if constexpr (sizeof(TO) == 2) {
        f.v = to_bf16x4(d[0], d[1], d[2], d[3]);
    } else {
        f.v = d;
    }
    return f;
}

// Same, with element e scaled by s[e] before rounding.
template <typename TO>
__device__ __forceinline__ Frag<TO> acc_frag_scaled(const f32x4 &d, const f32x4 &s) {
    return acc_frag<TO>(d * s);
}

// Scale a fragment elementwise by fp32 factors (used for per-channel decay
// factors along the contraction index).
template <typename TO>
__device__ __forceinline__ Frag<TO> frag_scaled(const Frag<TO> &f, const f32x4 &s) {
    Frag<TO> r;
    if constexpr (sizeof(TO) == 2) {
        r.v = to_bf16x4((float)f.v[0] * s[0], (float)f.v[1] * s[1], (float)f.v[2] * s[2],
                        (float)f.v[3] * s[3]);
    } else {
        r.v = f.v * s;
    }
    return r;
}

// Raw buffer resource over [p, p + bytes): loads past the end return 0 and
// stores past the end are dropped, which masks a partial last chunk.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// ------------------------------------------------------- sequences ----

// Token range of sequence b: dense layout (cu == NULL: b*T .. b*T+T) or the
// packed layout [cu[b], cu[b+1]), clamped into [0, T] so that malformed
// offsets can never move an access outside the tensors.
struct SeqRange {
    int64_t start, len;
};
__device__ __forceinline__ SeqRange seq_range(const int64_t *cu, int64_t b, int64_t T) {
    if (!cu) return SeqRange{b * T, T};
    int64_t lo = cu[b], hi = cu[b + 1];
    lo = lo < 0 ? 0 : (lo > T ? T : lo);
    hi = hi < lo ? lo : (hi > T ? T : hi);
    return SeqRange{lo, hi - lo};
}

// Workgroup -> (head unit, value-column slice).  A head unit is r*H + h for
// the sequence of rank r (rank order: `order[r]` when given, else r itself).
// Workgroups are dealt to the 8 XCDs round-robin in dispatch order; within each
// run of 8*nsplit consecutive workgroups, workgroup 8*nsplit*a + 8*s + i takes
// slice s of unit 8a + i.  So the slices of one head land on one XCD (and
// share its L2 for the head's q, k, z), and units are dispatched in order,
// which lets a longest-first ranking of packed sequences balance the load.
struct BlockMap {
    int64_t b;      // sequence (batch entry)
    int h;          // head
    int split;      // value-column slice
};
__device__ __forceinline__ BlockMap block_map(int64_t x, int64_t nblk, int nsplit, int64_t H,
                                              const int32_t *order) {
    const int64_t grp = 8 * (int64_t)nsplit;
    int64_t unit;
    int split;
    if (nblk % grp == 0) {
        const int64_t a = x / grp, rem = x % grp;
        split = (int)(rem / 8);
        unit = 8 * a + rem % 8;
    } else {
        unit = x / nsplit;
        split = (int)(x % nsplit);
    }
    const int64_t r = unit / H;
    return BlockMap{order ? (int64_t)order[r] : r, (int)(unit % H), split};
}

// First checkpoint row of sequence b: the rows of earlier sequences come
// first, floor(len / every) per sequence.
__device__ __forceinline__ int64_t ckpt_row0(const int64_t *cu, int64_t b, int64_t T, int every) {
    int64_t r = 0;
    for (int64_t j = 0; j < b; ++j) r += seq_range(cu, j, T).len / every;
    return r;
}

// Workgroup barrier that waits for LDS traffic only: outstanding global loads
// (prefetches of the next chunk) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace kda
