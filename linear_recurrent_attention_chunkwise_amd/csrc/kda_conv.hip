// kda_conv.hip -- the prologue of a KDA layer (gfx950): short causal depthwise
// convolutions of q, k and v over tokens, an optional SiLU, and L2
// normalization of q and k per token and head.
//
// "Kimi K3 Open Weights: What Is Actually New", section 1, puts short
// convolutions and Q/K normalization ahead of the decay products and chunk
// interactions of a KDA prefill.  The page fixes neither the width nor an
// activation nor the normalization's guard; this library reads them as: per
// channel c,  y_t[c] = sum_{j<W} w[c][j] x_{t-(W-1)+j}[c]  (tap W-1 on the
// current token, earlier tokens of the sequence from a convolution state of
// the last W-1 raw inputs, zeros for a fresh sequence), then optionally
// y * logistic(y), then q, k <- y / sqrt(sum_c y^2 + eps).
//
// The pass is bound by HBM: each input element is read once and each output
// written once, ~2 * sizeof(dtype) bytes per element and tensor.  Layout of
// the work:
//  * A lane owns one octet of 8 consecutive channels of a token row (16 bytes
//    in bf16: one buffer_load_dwordx4), so 64 lanes cover 512 channels of a
//    row, four heads of 128.  A head's 128 channels are 16 lanes, one DPP row,
//    and the per-token sum of squares reduces inside it with four DPP adds.
//  * A wave owns TT consecutive tokens of its 512 channels and keeps the TT
//    rows plus the three rows before them in registers; the convolution is a
//    sliding window over those rows (W <= 4 taps, zero-padded to 4).  All
//    TT + 3 loads are issued before any arithmetic.
//  * The four waves of a workgroup take four consecutive tiles of the same
//    channels, so a tile's three leading rows are its neighbour's last rows
//    (a cache hit, not a second HBM read).  The workgroup stages its 512
//    channels' taps through LDS once (coalesced), transposed so that each
//    lane's reads are conflict-free.
//  * Consecutive workgroups take the 512-channel slabs of the same tokens, so
//    the workgroups in flight stream whole token rows.
//  * Outputs are written with nontemporal stores: the next kernel reads them
//    from HBM anyway, and streaming them past the caches keeps the read
//    stream at full rate (measured on MI355X: 105 us instead of 117 us for
//    the K3 prefill shape).
//  * The wave holding a sequence's last tile writes the new convolution state
//    (the last W-1 raw rows, exact copies) from its registers.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

__device__ __forceinline__ float lo16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(bf16)a, (bf16)b});
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of a buffer store: the nt (nontemporal) bit.
constexpr int kNontemporal = 2;

// Eight consecutive channels of one token row, as loaded.
template <typename TI> struct Oct;
template <> struct Oct<bf16> {
    uint32_t u[4];
    __device__ __forceinline__ float at(int e) const { return e & 1 ? hi16(u[e >> 1]) : lo16(u[e >> 1]); }
    __device__ __forceinline__ void zero() { u[0] = u[1] = u[2] = u[3] = 0u; }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
        const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
        u[0] = r[0]; u[1] = r[1]; u[2] = r[2]; u[3] = r[3];
    }
    __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, int voff, int soff) const {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{u[0], u[1], u[2], u[3]}, rs, voff, soff, 0);
    }
    __device__ __forceinline__ static void store_f32(const float *y, __amdgpu_buffer_rsrc_t rs,
                                                     int voff, int soff) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])}, rs,
            voff, soff, kNontemporal);
    }
};
template <> struct Oct<float> {
    uint32_t u[8];
    __device__ __forceinline__ float at(int e) const { return __uint_as_float(u[e]); }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = 0u;
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, 0);
        u[0] = a[0]; u[1] = a[1]; u[2] = a[2]; u[3] = a[3];
        u[4] = b[0]; u[5] = b[1]; u[6] = b[2]; u[7] = b[3];
    }
    __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, int voff, int soff) const {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{u[0], u[1], u[2], u[3]}, rs, voff, soff, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{u[4], u[5], u[6], u[7]}, rs, voff + 16, soff, 0);
    }
    __device__ __forceinline__ static void store_f32(const float *y, __amdgpu_buffer_rsrc_t rs,
                                                     int voff, int soff) {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                  __float_as_uint(y[3])}, rs, voff, soff, kNontemporal);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                  __float_as_uint(y[7])}, rs, voff + 16, soff, kNontemporal);
    }
};

// DPP lane exchange inside a row of 16 lanes.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i within each half row
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i within the row

// Sum over the LPR consecutive lanes that hold one head's channels (LPR in
// {2, 16}; groups are aligned to LPR).
template <int LPR> __device__ __forceinline__ float head_sum(float x) {
    static_assert(LPR == 2 || LPR == 16, "one head = 2 or 16 lanes");
    x += dpp<kQuadXor1>(x);
    if constexpr (LPR == 16) {
        x += dpp<kQuadXor2>(x);
        x += dpp<kRowHalfMirror>(x);
        x += dpp<kRowMirror>(x);
    }
    return x;
}

__device__ __forceinline__ float silu(float y) {
    // y * logistic(y); e = 2^(-y log2 e) -> inf for y -> -inf gives y * 0
    const float e = __builtin_amdgcn_exp2f(-y * kLog2e);
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace


// Sequence of packed token t: the largest b < N with cu[b] <= t (offsets
// clamped into [0, T] as in seq_range).
__device__ __forceinline__ int64_t seq_of(const int64_t *cu, int64_t N, int64_t T, int64_t t) {
    int64_t lo = 0, hi = N - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        int64_t c = cu[mid];
        c = c < 0 ? 0 : (c > T ? T : c);
        if (c <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The tile of one wave: TT tokens x 512 channels (lane = channel octet).
// VL: the token axis packs N sequences (cu offsets); a row's taps that reach
// before its sequence's first token read that sequence's convolution state.
template <typename TI, int D, int TT, int W, bool ACT, bool NORM, bool VL>
__device__ __forceinline__ void conv_body(const ConvTensor &ct, const ConvNormArgs &p, int64_t b,
                                          int64_t slab, int64_t tile, int lane,
                                          const float *sw) {
    constexpr int ESZ = sizeof(TI);
    constexpr int LPR = D / 8;
    const int64_t H = p.H, T = p.T;
    const int64_t rowoct = H * (D / 8);
    const int64_t c8 = slab * 64 + lane;
    const bool active = c8 < rowoct;
    const int rowbytes = (int)(H * D * ESZ);
    const int voff = (int)(c8 * 8 * ESZ);
    const int64_t t0 = tile * TT;
    float wt[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) wt[e][j] = j >= 4 - W ? sw[(e * W + j - (4 - W)) * 64 + lane] : 0.0f;
    Oct<TI> xr[TT + 3];
    const int64_t nrows = T - t0 < TT ? (T - t0 > 0 ? T - t0 : 0) : TT;
    const int64_t rowel = H * D;
    const char *xb = static_cast<const char *>(ct.x) + ((b * T + t0) * rowel) * ESZ;
    {
        const auto rs = make_rsrc(xb, nrows * rowbytes);
#pragma unroll
        for (int s = 0; s < TT; ++s) xr[3 + s].load(rs, voff, s * rowbytes);
    }
    if (tile > 0) {
        const auto rs = make_rsrc(xb - 3 * (int64_t)rowbytes, 3 * (int64_t)rowbytes);
#pragma unroll
        for (int r = 0; r < 3; ++r) xr[r].load(rs, voff, r * rowbytes);
    } else if (VL) {
#pragma unroll
        for (int r = 0; r < 3; ++r) xr[r].zero();   // replaced per row below
    } else if (ct.sin && W > 1) {
        const char *sb = static_cast<const char *>(ct.sin) + (b * (W - 1) * rowel) * ESZ;
        const auto rs = make_rsrc(sb, (int64_t)(W - 1) * rowbytes);
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int sr = r - (4 - W);
            if (sr >= 0) xr[r].load(rs, voff, sr * rowbytes);
            else xr[r].zero();
        }
    } else {
#pragma unroll
        for (int r = 0; r < 3; ++r) xr[r].zero();
    }
    char *yb = static_cast<char *>(ct.y) + ((b * T + t0) * rowel) * ESZ;
    const auto ys = make_rsrc(yb, nrows * rowbytes);
    const float eps = p.eps;
    // packed sequences: the sequence of the current row and its first token
    int64_t sq = 0, sq_start = 0, sq_next = 0;
    if constexpr (VL) {
        sq = seq_of(p.cu, p.N, T, t0);
        auto clampT = [&](int64_t c) { return c < 0 ? 0 : (c > T ? T : c); };
        sq_start = clampT(p.cu[sq]);
        sq_next = sq + 1 < p.N ? clampT(p.cu[sq + 1]) : T;
    }
#pragma unroll
    for (int s = 0; s < TT; ++s) {
        Oct<TI> src[4] = {xr[s], xr[s + 1], xr[s + 2], xr[s + 3]};
        if constexpr (VL) {
            const int64_t t = t0 + s;
            // next sequence(s) starting at or before this row (empty ones skipped)
            while (sq + 1 < p.N && sq_next <= t) {
                ++sq;
                sq_start = sq_next;
                int64_t c = sq + 1 < p.N ? p.cu[sq + 1] : T;
                sq_next = c < sq_start ? sq_start : (c > T ? T : c);
            }
            if (t - 3 < sq_start) {
                // taps before the sequence start: its state rows, or zeros
                const char *sb = ct.sin ? static_cast<const char *>(ct.sin) +
                                              (sq * (W - 1) * rowel) * ESZ
                                        : nullptr;
                const auto rs = make_rsrc(sb, sb ? (int64_t)(W - 1) * rowbytes : 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t tok = t - 3 + j;
                    if (tok < sq_start) {
                        const int64_t sr = (W - 1) + (tok - sq_start);
                        if (sb && sr >= 0) src[j].load(rs, voff, (int)sr * rowbytes);
                        else src[j].zero();
                    }
                }
            }
        }
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[e] = wt[e][0] * src[0].at(e);
            y[e] = fmaf(wt[e][1], src[1].at(e), y[e]);
            y[e] = fmaf(wt[e][2], src[2].at(e), y[e]);
            y[e] = fmaf(wt[e][3], src[3].at(e), y[e]);
        }
        if constexpr (ACT) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = silu(y[e]);
        }
        if constexpr (NORM) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
            ss = head_sum<LPR>(ss);
            const float r = __builtin_amdgcn_rsqf(ss + eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= r;
        }
        if (active) Oct<TI>::store_f32(y, ys, voff, s * rowbytes);
    }
    if (!VL && tile == p.ntile - 1 && ct.sout && W > 1 && active) {
        char *sb = static_cast<char *>(ct.sout) + (b * (W - 1) * rowel) * ESZ;
        const auto rs = make_rsrc(sb, (int64_t)(W - 1) * rowbytes);
        const int64_t first = T - (W - 1);
#pragma unroll
        for (int r = 0; r < TT + 3; ++r) {
            const int64_t i = t0 - 3 + r - first;
            if (i >= 0 && i < W - 1) xr[r].store(rs, voff, (int)i * rowbytes);
        }
    }
}

// One workgroup = 4 waves = 4 consecutive token tiles of one 512-channel slab
// of one tensor (blockIdx.y: q, k, v) of one sequence.
template <typename TI, int D, int TT, int W, bool ACT, bool VL>
__global__ __launch_bounds__(256) void kda_conv_norm_kernel(ConvNormArgs p) {
    __shared__ float sw[8 * 4 * 64];   // taps of the slab's 512 channels, [e*W + j][lane]
    const ConvTensor ct = blockIdx.y == 0 ? p.t[0] : (blockIdx.y == 1 ? p.t[1] : p.t[2]);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t H = p.H;
    const int64_t rowoct = H * (D / 8);
    const int64_t nslab = (rowoct + 63) / 64;
    int64_t x = blockIdx.x;
    const int64_t slab = x % nslab;
    x /= nslab;
    const int64_t grp = x % p.ngroup;
    const int64_t b = x / p.ngroup;
    {
        // the slab's taps are contiguous: channels slab*512 .. +512, W each
        const int64_t base = slab * 64 * 8 * W;
        const int64_t lim = H * D * W;
        for (int i = threadIdx.x; i < 64 * 8 * W; i += 256) {
            const int l = i / (8 * W), r = i % (8 * W);
            sw[r * 64 + l] = base + i < lim ? ct.w[base + i] : 0.0f;
        }
    }
    __syncthreads();
    const int64_t tile = grp * 4 + wave;
    if (tile >= p.ntile) return;
    if (ct.norm) conv_body<TI, D, TT, W, ACT, true, VL>(ct, p, b, slab, tile, lane, sw);
    else conv_body<TI, D, TT, W, ACT, false, VL>(ct, p, b, slab, tile, lane, sw);
}

bool conv_supported(int dtype, int64_t D) {
    return (dtype == 0 || dtype == 1) && (D == 16 || D == 128);
}

// Tokens per wave tile, as launch_conv_norm instantiates the kernel.
int conv_tile_tokens(int dtype, int64_t D) { return dtype == 1 && D != 128 ? 16 : 8; }

// New convolution states of packed sequences: row i of sequence b's state is
// raw token end_b - (W-1) + i, or, for a sequence shorter than W-1, a row of
// its old state (zeros without one).  One thread per (sequence, channel
// octet, tensor).
template <typename TI>
__global__ __launch_bounds__(256) void kda_conv_state_varlen_kernel(ConvNormArgs p) {
    constexpr int ESZ = sizeof(TI);
    const ConvTensor ct = blockIdx.y == 0 ? p.t[0] : (blockIdx.y == 1 ? p.t[1] : p.t[2]);
    const int64_t rowoct = p.H * (p.D / 8);
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (!ct.sout || i >= p.N * rowoct) return;
    const int64_t b = i / rowoct, c8 = i % rowoct;
    const SeqRange sr = seq_range(p.cu, b, p.T);
    const int64_t rowel = p.H * p.D;
    const int W = p.W;
    for (int r = 0; r < W - 1; ++r) {
        const int64_t tok = sr.start + sr.len - (W - 1) + r;
        Oct<TI> val;
        if (tok >= sr.start) {
            const auto rs = make_rsrc(static_cast<const char *>(ct.x) + tok * rowel * ESZ,
                                      rowel * ESZ);
            val.load(rs, (int)(c8 * 8 * ESZ), 0);
        } else if (ct.sin) {
            const int64_t srow = (W - 1) + (tok - sr.start);   // >= 0: tok >= start - (W-1)
            const auto rs = make_rsrc(static_cast<const char *>(ct.sin) +
                                          ((b * (W - 1) + srow) * rowel) * ESZ,
                                      rowel * ESZ);
            val.load(rs, (int)(c8 * 8 * ESZ), 0);
        } else {
            val.zero();
        }
        const auto ws = make_rsrc(static_cast<char *>(ct.sout) + ((b * (W - 1) + r) * rowel) * ESZ,
                                  rowel * ESZ);
        val.store(ws, (int)(c8 * 8 * ESZ), 0);
    }
}

template <typename TI, int D, int TT, int W, bool ACT>
static hipError_t launch_conv_t(const ConvNormArgs &a0) {
    ConvNormArgs a = a0;
    const int64_t ntile = a.T > 0 ? (a.T + TT - 1) / TT : 1;
    const int64_t rowoct = a.H * (D / 8);
    const int64_t nslab = (rowoct + 63) / 64;
    a.ntile = ntile;
    a.ngroup = (ntile + 3) / 4;
    if (a.cu) {
        // packed sequences: tiles over the whole token axis, then the states
        if (a.T > 0)
            hipLaunchKernelGGL((kda_conv_norm_kernel<TI, D, TT, W, ACT, true>),
                               dim3((unsigned)(nslab * a.ngroup), 3), dim3(256), 0, a.stream, a);
        const int64_t nst = a.N * rowoct;
        if (W > 1 && nst > 0)
            hipLaunchKernelGGL((kda_conv_state_varlen_kernel<TI>),
                               dim3((unsigned)((nst + 255) / 256), 3), dim3(256), 0, a.stream, a);
        return hipGetLastError();
    }
    const int64_t nblk = a.B * nslab * a.ngroup;
    hipLaunchKernelGGL((kda_conv_norm_kernel<TI, D, TT, W, ACT, false>), dim3((unsigned)nblk, 3),
                       dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

template <typename TI, int D, int TT>
static hipError_t launch_conv_w(const ConvNormArgs &a) {
    switch (a.W * 2 + (a.act ? 1 : 0)) {
        case 2: return launch_conv_t<TI, D, TT, 1, false>(a);
        case 3: return launch_conv_t<TI, D, TT, 1, true>(a);
        case 4: return launch_conv_t<TI, D, TT, 2, false>(a);
        case 5: return launch_conv_t<TI, D, TT, 2, true>(a);
        case 6: return launch_conv_t<TI, D, TT, 3, false>(a);
        case 7: return launch_conv_t<TI, D, TT, 3, true>(a);
        case 8: return launch_conv_t<TI, D, TT, 4, false>(a);
        default: return launch_conv_t<TI, D, TT, 4, true>(a);
    }
}

hipError_t launch_conv_norm(const ConvNormArgs &a) {
    // tile sizes as conv_tile_tokens states them; bf16 at d = 128 takes 8-token
    // tiles, ~2% faster than 16 (more workgroups in flight; 32 costs 7.5%)
    if (a.dtype == 1) {
        if (a.D == 128) return launch_conv_w<bf16, 128, 8>(a);
        return launch_conv_w<bf16, 16, 16>(a);
    }
    if (a.D == 128) return launch_conv_w<float, 128, 8>(a);
    return launch_conv_w<float, 16, 8>(a);
}

}  // namespace kda
