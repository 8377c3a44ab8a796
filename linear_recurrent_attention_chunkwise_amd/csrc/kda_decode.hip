// kda_decode.hip -- fused one-token KDA decode step (gfx950).
//
// The step is the KDA recurrence of "Kimi K3 Open Weights: What Is Actually
// New", section 1 (its prefill/decode split), for a single token: decode
// updates the recurrent state once per token and layer, and the state stays
// in HBM from one call to the next.  Writing a = alpha*k, b = alpha*q:
//
//     w = S^T a,  y = S^T b           (one pass over S, reductions over dk)
//     u = beta (v - w)
//     o = y + (q . k) u               (= S_t^T q)
//     S <- Diag(alpha) S + k u^T      (= (I - beta k k^T) Diag(alpha) S + beta k v^T)
//
// Memory-bound: every state entry is read once and written once.  One
// workgroup owns one (b, h); the dk x dv fp32 state is held in registers
// between the read and the write-back, as float4 column quads, so each wave
// load/store instruction touches whole contiguous state rows.  The new state
// is written with nontemporal stores: it is not read again within the step,
// and streaming it past the caches keeps the read stream of the other heads'
// states at full rate (measured on MI355X: 6.9 TB/s instead of 5.3 TB/s).
//
// The CONV instantiation fuses the layer's prologue into the step (the same
// section has decode keep a convolution state alongside the recurrent one):
// each of q, k, v is convolved with its W-1 previous raw inputs, held in a
// per-sequence convolution state that the step shifts in place, and q, k are
// L2-normalized.  The normalization is a scalar per vector, so it is applied
// after the pass over S:  S^T(alpha k^) = S^T(alpha k) / |k|,  and likewise
// for q and for q^.k^.  The prologue adds about 4% to the step's HBM bytes.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// One channel of the fused prologue.  load(): the current raw input x, the
// W-1 raw inputs before it (convolution state rows, oldest first) and the W
// taps.  conv(): the short causal convolution (tap W-1 weighs x), optionally
// followed by SiLU.  shift(): the state rows move down by one and x becomes
// the newest row, in place; the stored values are the raw inputs, so the
// state stays exact.  Every load of the three tensors is issued before any
// state store, so the loads do not wait on stores they might alias.
template <typename TI> struct ConvChannel {
    TI x, raw[3];
    float w[4];
    __device__ __forceinline__ void load(const TI *xp, const float *wp, const TI *st,
                                         int64_t stride, int W) {
        x = *xp;
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < W - 1) raw[j] = st[j * stride];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < W) w[j] = wp[j];
    }
    __device__ __forceinline__ float conv(int W, int act) const {
        float y = 0.0f;
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < W - 1) y = fmaf(w[j], to_f32(raw[j]), y);
#pragma unroll
        for (int j = 1; j <= 4; ++j)
            if (j == W) y = fmaf(w[j - 1], to_f32(x), y);
        if (act) {
            const float e = __builtin_amdgcn_exp2f(-y * kLog2e);
            y *= __builtin_amdgcn_rcpf(1.0f + e);
        }
        return y;
    }
    __device__ __forceinline__ void shift(TI *st, int64_t stride, int W) const {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (j < W - 2) st[j * stride] = raw[j + 1];
#pragma unroll
        for (int j = 1; j <= 3; ++j)
            if (j == W - 1) st[(j - 1) * stride] = x;
    }
};

template <typename TI, int D, int NT, bool CONV>
__global__ __launch_bounds__(NT) void kda_decode_kernel(DecodeArgs p) {
    constexpr int NCG = D / 4;          // float4 column quads per state row
    constexpr int RG = NT / NCG;        // row groups
    constexpr int RPT = D / RG;         // state rows per thread
    constexpr int NWAVE = NT / 64;
    constexpr int NRED = CONV ? 3 : 1;  // q.k, and with the prologue |q|^2, |k|^2
    static_assert(RG * RPT == D && NCG <= 64 && NT % 64 == 0, "bad decode tiling");

    __shared__ float s_alpha[D], s_k[D], s_ak[D], s_aq[D];
    __shared__ __attribute__((aligned(16))) float s_v[CONV ? D : 1];
    __shared__ __attribute__((aligned(16))) float s_red[NWAVE][2][D];
    __shared__ float s_qk[NWAVE][NRED];

    const TI *__restrict__ q = static_cast<const TI *>(p.q);
    const TI *__restrict__ k = static_cast<const TI *>(p.k);
    const TI *__restrict__ v = static_cast<const TI *>(p.v);
    const TI *__restrict__ z = static_cast<const TI *>(p.z);
    const TI *__restrict__ beta = static_cast<const TI *>(p.beta);
    const int64_t H = p.H;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % NCG, rg = tid / NCG;
    float *Sp = p.S + bh * (int64_t)(D * D);

    // The token's own inputs are loaded first and the whole state read right
    // after: loads return in order, so the gate and prologue arithmetic runs
    // while the state streams in.
    const int64_t off = bh * D + tid;
    TI zr{}, kr{}, qr{};
    ConvChannel<TI> cnq, cnk, cnv;
    TI *cq = nullptr, *ck = nullptr, *cv = nullptr;
    int64_t hd = 0;
    if (tid < D) {
        zr = z[off];
        if constexpr (CONV) {
            const int W = p.W;
            const int64_t b = bh / H;
            hd = H * D;
            const int64_t sb = b * (W - 1) * hd + (int64_t)h * D + tid;
            const int64_t wb = ((int64_t)h * D + tid) * W;
            cq = static_cast<TI *>(p.cq) + sb;
            ck = static_cast<TI *>(p.ck) + sb;
            cv = static_cast<TI *>(p.cv) + sb;
            cnk.load(k + off, p.wk + wb, ck, hd, W);
            cnq.load(q + off, p.wq + wb, cq, hd, W);
            cnv.load(v + off, p.wv + wb, cv, hd, W);
        } else {
            kr = k[off];
            qr = q[off];
        }
    }
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = *reinterpret_cast<const f32x4 *>(Sp + (rg + RG * m) * D + 4 * cg);

    float red[NRED];
#pragma unroll
    for (int r = 0; r < NRED; ++r) red[r] = 0.0f;
    if (tid < D) {
        const float zi = to_f32(zr);
        float ki, qi;
        if constexpr (CONV) {
            // prologue: convolve q, k, v (states updated in place); q and k are
            // normalized below through their squared norms
            const int W = p.W;
            ki = cnk.conv(W, p.act);
            qi = cnq.conv(W, p.act);
            s_v[tid] = cnv.conv(W, p.act);
            cnk.shift(ck, hd, W);
            cnq.shift(cq, hd, W);
            cnv.shift(cv, hd, W);
            red[1] = qi * qi;
            red[2] = ki * ki;
        } else {
            ki = to_f32(kr);
            qi = to_f32(qr);
        }
        const float c2 = -__builtin_amdgcn_exp2f(p.A[h] * kLog2e) * kLog2e;
        const float al = kda_alpha(c2, zi);
        s_alpha[tid] = al;
        s_k[tid] = ki;
        s_ak[tid] = al * ki;
        s_aq[tid] = al * qi;
        red[0] = qi * ki;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
        for (int r = 0; r < NRED; ++r) red[r] += __shfl_xor(red[r], off);
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < NRED; ++r) s_qk[wave][r] = red[r];
    }
    __syncthreads();

    f32x4 w = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        w += s[m] * s_ak[i];
        y += s[m] * s_aq[i];
    }
    // Lanes holding the same column quad differ by multiples of NCG.
#pragma unroll
    for (int off = NCG; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] += __shfl_xor(w[e], off);
            y[e] += __shfl_xor(y[e], off);
        }
    }
    if (lane < NCG) {
        *reinterpret_cast<f32x4 *>(&s_red[wave][0][4 * cg]) = w;
        *reinterpret_cast<f32x4 *>(&s_red[wave][1][4 * cg]) = y;
    }
    __syncthreads();

    f32x4 wt = {0.f, 0.f, 0.f, 0.f}, yt = {0.f, 0.f, 0.f, 0.f};
    float tot[NRED];
#pragma unroll
    for (int r = 0; r < NRED; ++r) tot[r] = 0.0f;
#pragma unroll
    for (int wv = 0; wv < NWAVE; ++wv) {
        wt += *reinterpret_cast<const f32x4 *>(&s_red[wv][0][4 * cg]);
        yt += *reinterpret_cast<const f32x4 *>(&s_red[wv][1][4 * cg]);
#pragma unroll
        for (int r = 0; r < NRED; ++r) tot[r] += s_qk[wv][r];
    }
    float qkt = tot[0], kscale = 1.0f;
    f32x4 vv;
    if constexpr (CONV) {
        // q^ = q / sqrt(|q|^2 + eps), k^ likewise: S^T(alpha k^) = rk S^T(alpha k), ...
        const float rq = __builtin_amdgcn_rsqf(tot[1] + p.eps);
        const float rk = __builtin_amdgcn_rsqf(tot[2] + p.eps);
        wt *= rk;
        yt *= rq;
        qkt *= rq * rk;
        kscale = rk;
        vv = *reinterpret_cast<const f32x4 *>(&s_v[4 * cg]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = to_f32(v[bh * D + 4 * cg + e]);
    }
    const float bt = to_f32(beta[bh]);
    const f32x4 u = bt * (vv - wt);
    if (rg == 0) {
        const f32x4 ov = yt + qkt * u;
        TI *op = static_cast<TI *>(p.o) + bh * D + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e) op[e] = from_f32<TI>(ov[e]);
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        const f32x4 ns = s_alpha[i] * s[m] + (kscale * s_k[i]) * u;
        __builtin_nontemporal_store(ns, reinterpret_cast<f32x4 *>(Sp + i * D + 4 * cg));
    }
}

bool decode_supported(int dtype, int64_t D) {
    return (dtype == 0 || dtype == 1) && (D == 16 || D == 128);
}

template <typename TI, int D, int NT>
static hipError_t launch_decode_t(const DecodeArgs &a) {
    const int64_t nblk = a.B * a.H;
    if (a.conv)
        hipLaunchKernelGGL((kda_decode_kernel<TI, D, NT, true>), dim3((unsigned)nblk), dim3(NT), 0,
                           a.stream, a);
    else
        hipLaunchKernelGGL((kda_decode_kernel<TI, D, NT, false>), dim3((unsigned)nblk), dim3(NT),
                           0, a.stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a) {
    if (a.dtype == 1) {
        if (a.D == 128) return launch_decode_t<bf16, 128, 512>(a);
        return launch_decode_t<bf16, 16, 64>(a);
    }
    if (a.D == 128) return launch_decode_t<float, 128, 512>(a);
    return launch_decode_t<float, 16, 64>(a);
}

}  // namespace kda
