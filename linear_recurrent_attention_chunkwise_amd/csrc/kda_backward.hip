// kda_backward.hip -- chunk-parallel reverse mode of the KDA prefill (gfx950).
//
// The training form the K3 coverage page lists as the next KDA primitive
// (nishifamily.com K3 page, innovation table, row "Kimi Delta Attention
// (linear)"): gradients of a loss through the recurrence of "Kimi K3 Open
// Weights: What Is Actually New", section 1, computed chunk by chunk.  Per
// 16-token chunk with entering state S, in-chunk cumulative log-decay G
// (chunk-start reference), Q^ = Q e^G, K^ = K e^G, Ki = K e^-G,
// Kb = K e^{G_n - G}, A = strict_tril(K^ Ki^T), P = tril(Q^ Ki^T),
// T = (I + diag(beta) A)^-1, W = T diag(beta) K^, U = T diag(beta) V - W S:
//
//   dU = P^T dO + Kb dS'                  dS = Q^^T dO + e^{G_n} dS' - W^T dU
//   dP = tril(dO U^T)                     dW = -dU S^T
//   dT = dW (beta K^)^T + dU (beta V)^T   dL = -T^T dT T^T  (strictly lower)
//
// and the decayed products pass the rest to q, k, beta and G; the reverse
// cumulative sum of dG is dg, and the gate gives dz and dA.  Every decayed
// product factors as (X e^G)(Y e^-G)^T: over 16 tokens e^-G <= e^80 stays in
// fp32 range, so all of them are plain 16 x 16 x d products.
//
// Kernels:
//   prep   -- one workgroup per (sequence, head, chunk): the chunk's W, Q^,
//             Kb, P, T, e^{G_n} and A (S-independent, fp32; A, P, T and W on
//             fp32 matrix-core tiles), into the workspace.
//   dstate -- (bf16, d = 128) one workgroup per (sequence, head, 64 value
//             columns): walks the chunks backwards carrying dS in fp32
//             accumulator tiles (bf16 matrix-core products) and stores every
//             chunk's incoming dS'; the final dS is dS0.
//   part   -- (bf16, d = 128) one workgroup per (sequence, head, chunk), all
//             chunks at once: from the forward rerun's checkpoint S and the
//             stored dS' it forms dV and the sums over all value columns
//             (dQ^, dKb, dW, dP, the V parts of dT and dbeta, sum_j dS' S).
//   chain  -- (fp32 inputs, d = 16) dstate and part in one fp32 kernel per
//             (sequence, head, value-column slice), carrying dS through LDS.
//   grad   -- one workgroup per (sequence, head, chunk): adds the slices'
//             partials in slice order and, with A and T from prep's record,
//             forms dq, dk, dbeta, dz and the chunk's share of dA (fp32; its
//             chunk products on fp32 matrix-core tiles).
//   dA     -- one workgroup per head: sums its (sequence, chunk) shares in a
//             fixed order (strided per thread, then a fixed tree).
// No atomics: results are bitwise reproducible.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int C = 16;   // chunk length of the backward

__device__ __forceinline__ float sigmoidf_(float x) {
    return 1.0f / (1.0f + __expf(-x));
}

// Per-chunk prep record in the workspace (floats):
//   W [C][D], Qh [C][D], Kb [C][D], P [C][C], T [C][C], Gn [D] (= e^{G_n}), A [C][C]
template <int D> struct PrepLayout {
    static constexpr int W = 0, QH = C * D, KB = 2 * C * D, P = 3 * C * D, T = 3 * C * D + C * C,
                         GN = 3 * C * D + 2 * C * C, A = 3 * C * D + 2 * C * C + D,
                         SIZE = 3 * C * D + 3 * C * C + D;
};

// Per-(chunk, slice) partial record (floats):
//   dQh [C][D], dKb [C][D], dW [C][D], dP [C][C], dTV [C][C], dbV [C], dGn [D]
template <int D> struct PartLayout {
    static constexpr int DQH = 0, DKB = C * D, DW = 2 * C * D, DP = 3 * C * D,
                         DTV = 3 * C * D + C * C, DBV = 3 * C * D + 2 * C * C,
                         DGN = 3 * C * D + 2 * C * C + C, SIZE = 3 * C * D + 2 * C * C + C + D;
};

// The S-independent quantities of one chunk, in LDS.  Rows r >= n are absent
// tokens: zero inputs, beta 0 and g 0 (alpha 1), so they contribute nothing.
// With G the in-chunk cumulative log-decay, the decayed operands are kept:
// Qh = q e^{G}, Kh = k e^{G}, Ki = k e^{-G} (over 16 tokens e^{-G} <= e^80
// stays in fp32 range), and E = e^{G}; so k_r k_s e^{G_r - G_s} = Kh_r Ki_s.
// [C][D] rows are padded by one float: threads that read one column d of
// several rows then hit distinct LDS banks.
template <int D> constexpr int rowpad() { return D + 1; }
template <typename TI, int D> struct ChunkOps {
    float Qh[C][rowpad<D>()], Kh[C][rowpad<D>()], Ki[C][rowpad<D>()], E[C][rowpad<D>()];
    float A[C][C + 1], P[C][C + 1], T[C][C + 1];
    float beta[C];
};

// fp32 K16 fragments of an LDS matrix M with row stride ld (see kda_device.h):
// rowfrag -- lane (m, g) holds M[r0 + m][k0 + 4g + e]  (A operand M, or B = M^T)
// colfrag -- lane (n, g) holds M[k0 + 4g + e][c0 + n]  (B operand M, or A = M^T)
__device__ __forceinline__ Frag<float> rowfrag(const float *M, int ld, int r0, int k0, int lane) {
    Frag<float> f;
    const float *p = M + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = p[e];
    return f;
}
__device__ __forceinline__ Frag<float> colfrag(const float *M, int ld, int k0, int c0, int lane) {
    Frag<float> f;
    const float *p = M + (k0 + 4 * (lane >> 4)) * ld + c0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) f.v[e] = p[e * ld];
    return f;
}

// Eight consecutive inputs (16-byte aligned) as fp32.
__device__ __forceinline__ void load8(const bf16 *p, float *out) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float *out) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[i] = a[i];
        out[4 + i] = b[i];
    }
}

template <typename TI, int D>
__device__ void chunk_ops(ChunkOps<TI, D> &s, const BwdArgs &p, int64_t b, int64_t h, int64_t c,
                          int n) {
    const TI *q = static_cast<const TI *>(p.q), *k = static_cast<const TI *>(p.k),
             *z = static_cast<const TI *>(p.z), *beta = static_cast<const TI *>(p.beta);
    const int64_t H = p.H;
    const int64_t row0 = (b * p.T + c * C) * H + h;   // token row of the chunk's first token
    const float cA = __expf(p.A[h]);
    // q, k, z: a thread takes 8 consecutive channels of one token row (16- or
    // 32-byte loads, all three issued before any use)
    constexpr int VEC = 8, NVEC = C * D / VEC;   // 256 for D = 128 (blockDim.x == 256)
    for (int t = threadIdx.x; t < NVEC; t += blockDim.x) {
        const int r = t / (D / VEC), d0 = VEC * (t % (D / VEC));
        float qv[VEC], kv[VEC], zv[VEC];
        if (r < n) {
            const int64_t off = (row0 + (int64_t)r * H) * D + d0;
            load8(q + off, qv);
            load8(k + off, kv);
            load8(z + off, zv);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) qv[e] = kv[e] = zv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            s.Qh[r][d0 + e] = qv[e];
            s.Kh[r][d0 + e] = kv[e];
            s.E[r][d0 + e] = r < n ? kGMin * sigmoidf_(cA * zv[e]) : 0.f;
        }
    }
    for (int r = threadIdx.x; r < C; r += blockDim.x)
        s.beta[r] = r < n ? to_f32(beta[row0 + (int64_t)r * H]) : 0.f;
    __syncthreads();
    // cumulative log-decay over the chunk, applied to q and k
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            acc += s.E[r][d];
            const float e = __expf(acc), ei = __expf(-acc), kv = s.Kh[r][d];
            s.E[r][d] = e;
            s.Qh[r][d] *= e;
            s.Kh[r][d] = kv * e;
            s.Ki[r][d] = kv * ei;
        }
    }
    __syncthreads();
    // A[r][s] = sum_d k_r k_s e^{G_r - G_s} (s < r),  P[r][s] = sum_d q_r k_s e^{G_r - G_s} (s <= r):
    // Kh Ki^T and Qh Ki^T on fp32 matrix-core tiles, wave 0 and wave 1 (two
    // accumulators each, to halve the dependent chain)
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        const int g = lane >> 4, nn = lane & 15;
        constexpr int LDD = rowpad<D>();
        if (wave < 2) {
            const float *X = wave == 0 ? &s.Kh[0][0] : &s.Qh[0][0];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += 16) {
                if ((k0 / 16) % 2 == 0)
                    mma16(acc, rowfrag(X, LDD, 0, k0, lane), rowfrag(&s.Ki[0][0], LDD, 0, k0, lane));
                else
                    mma16(acc2, rowfrag(X, LDD, 0, k0, lane), rowfrag(&s.Ki[0][0], LDD, 0, k0, lane));
            }
            acc += acc2;
            if (wave == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    s.P[r][nn] = nn <= r ? acc[e] : 0.f;
                }
            } else {
                // T = (I + N)^-1 with N = diag(beta) A strictly lower, so N^16 = 0:
                // T = (I - N)(I + N^2)(I + N^4)(I + N^8), on fp32 tiles in
                // registers.  A tile in accumulator layout (lane (g, nn) holds
                // X[4g+e][nn]) is the B operand of X and the A operand of X^T, so
                // mm(a, b) below, with a holding X^T and b holding Y, gives X Y.
                f32x4 N, I;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    const float a = nn < r ? acc[e] : 0.f;
                    s.A[r][nn] = a;
                    N[e] = s.beta[r] * a;
                    I[e] = r == nn ? 1.f : 0.f;
                }
                auto mm = [](const f32x4 &a, const f32x4 &b) {
                    Frag<float> fa, fb;
                    fa.v = a;
                    fb.v = b;
                    f32x4 d = {0.f, 0.f, 0.f, 0.f};
                    mma16(d, fa, fb);
                    return d;
                };
                const f32x4 NT = mm(N, I);            // N^T I
                const f32x4 N2 = mm(NT, N), N2T = mm(N, NT);
                const f32x4 N4 = mm(N2T, N2), N4T = mm(N2, N2T);
                const f32x4 N8 = mm(N4T, N4);
                const f32x4 Y = mm(I + N4T, I + N8);  // (I + N^4)(I + N^8)
                const f32x4 XT = mm(I + N2, I - NT);  // ((I - N)(I + N^2))^T
                const f32x4 Tm = mm(XT, Y);           // T
#pragma unroll
                for (int e = 0; e < 4; ++e) s.T[4 * g + e][nn] = Tm[e];
            }
        }
    }
    __syncthreads();
}

}  // namespace

// ------------------------------------------------------------------ prep ----

template <typename TI, int D>
__global__ __launch_bounds__(256) void kda_bwd_prep_kernel(BwdArgs p) {
    __shared__ ChunkOps<TI, D> s;
    static_assert(sizeof(ChunkOps<TI, D>) <= 150 * 1024, "LDS budget");
    using Lay = PrepLayout<D>;
    const int64_t x = blockIdx.x;
    const int64_t c = x % p.nchunk, bh = x / p.nchunk;
    const int64_t b = bh / p.H, h = bh % p.H;
    const int n = (int)(p.T - c * C < C ? p.T - c * C : C);
    chunk_ops<TI, D>(s, p, b, h, c, n);
    float *rec = p.prep + x * (int64_t)Lay::SIZE;
    // W = T diag(beta) Kh on fp32 matrix-core tiles: wave w takes the 16-column
    // tiles w, w+4, ...; lane (g, nn) gets W[4g+e][16t+nn]  (blockDim.x == 256)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, nn = lane & 15;
        constexpr int LDD = rowpad<D>();
        Frag<float> tb;   // A operand: T[nn][4g+e] beta[4g+e]
#pragma unroll
        for (int e = 0; e < 4; ++e) tb.v[e] = s.T[nn][4 * g + e] * s.beta[4 * g + e];
        for (int t = wave; t < D / 16; t += 4) {
            f32x4 w = {0.f, 0.f, 0.f, 0.f};
            mma16(w, tb, colfrag(&s.Kh[0][0], LDD, 0, 16 * t, lane));
#pragma unroll
            for (int e = 0; e < 4; ++e) rec[Lay::W + (4 * g + e) * D + 16 * t + nn] = w[e];
        }
    }
    for (int i = threadIdx.x; i < C * D; i += blockDim.x) {
        const int r = i / D, d = i % D;
        rec[Lay::QH + i] = s.Qh[r][d];
        rec[Lay::KB + i] = s.Ki[r][d] * s.E[C - 1][d];
    }
    for (int i = threadIdx.x; i < C * C; i += blockDim.x) {
        rec[Lay::P + i] = s.P[i / C][i % C];
        rec[Lay::T + i] = s.T[i / C][i % C];
        rec[Lay::A + i] = s.A[i / C][i % C];
    }
    for (int d = threadIdx.x; d < D; d += blockDim.x) rec[Lay::GN + d] = s.E[C - 1][d];
}

// ----------------------------------------------------------------- chain ----

template <int D, int NC> struct ChainLds {
    float S[D][NC], dS[D][NC];
    float W[C][D], Qh[C][D], Kb[C][D];
    float P[C][C], T[C][C];
    float Gn[D];
    float dO[C][NC], V[C][NC], U[C][NC], dU[C][NC], BV[C][NC];
    float beta[C];
};

template <typename TI, int D, int NC, int NT>
__global__ __launch_bounds__(NT) void kda_bwd_chain_kernel(BwdArgs p) {
    __shared__ ChainLds<D, NC> s;
    static_assert(sizeof(ChainLds<D, NC>) <= 150 * 1024, "LDS budget");
    using Lay = PrepLayout<D>;
    using PL = PartLayout<D>;
    const TI *v = static_cast<const TI *>(p.v), *beta = static_cast<const TI *>(p.beta),
             *dO = static_cast<const TI *>(p.dO);
    constexpr int NS = D / NC;   // column slices per head
    const int64_t x = blockIdx.x;
    const int sl = (int)(x % NS);
    const int64_t bh = x / NS;
    const int64_t b = bh / p.H, h = bh % p.H, H = p.H;
    const int j0 = sl * NC;
    const int tid = threadIdx.x;
    const int64_t nfull = p.T / C;   // checkpoints per sequence

    // dS' of the last chunk: dL/dS_T (or 0)
    for (int i = tid; i < D * NC; i += NT) {
        const int d = i / NC, j = i % NC;
        s.dS[d][j] = p.dST ? p.dST[(bh * D + d) * D + j0 + j] : 0.f;
    }
    for (int64_t c = p.nchunk - 1; c >= 0; --c) {
        const int n = (int)(p.T - c * C < C ? p.T - c * C : C);
        const int64_t row0 = (b * p.T + c * C) * H + h;
        const float *Sin = c == 0 ? (p.S0 ? p.S0 + bh * (int64_t)(D * D) : nullptr)
                                  : p.ckpt + ((b * nfull + c - 1) * H + h) * (int64_t)(D * D);
        const float *rec = p.prep + (bh * p.nchunk + c) * (int64_t)Lay::SIZE;
        for (int i = tid; i < D * NC; i += NT) {
            const int d = i / NC, j = i % NC;
            s.S[d][j] = Sin ? Sin[(int64_t)d * D + j0 + j] : 0.f;
        }
        for (int i = tid; i < C * D; i += NT) {
            const int r = i / D, d = i % D;
            s.W[r][d] = rec[Lay::W + i];
            s.Qh[r][d] = rec[Lay::QH + i];
            s.Kb[r][d] = rec[Lay::KB + i];
        }
        for (int i = tid; i < C * C; i += NT) {
            (&s.P[0][0])[i] = rec[Lay::P + i];
            (&s.T[0][0])[i] = rec[Lay::T + i];
        }
        for (int d = tid; d < D; d += NT) s.Gn[d] = rec[Lay::GN + d];
        for (int i = tid; i < C * NC; i += NT) {
            const int r = i / NC, j = i % NC;
            float ov = 0.f, vv = 0.f;
            if (r < n) {
                const int64_t off = (row0 + (int64_t)r * H) * D + j0 + j;
                ov = to_f32(dO[off]);
                vv = to_f32(v[off]);
            }
            s.dO[r][j] = ov;
            s.V[r][j] = vv;
        }
        for (int r = tid; r < C; r += NT) s.beta[r] = r < n ? to_f32(beta[row0 + (int64_t)r * H]) : 0.f;
        __syncthreads();

        // U = T diag(beta) V - W S;  dU = P^T dO + Kb dS'
        for (int i = tid; i < C * NC; i += NT) {
            const int r = i / NC, j = i % NC;
            float u = 0.f, du = 0.f;
            for (int sc = 0; sc < C; ++sc) {
                u += s.T[r][sc] * s.beta[sc] * s.V[sc][j];
                du += s.P[sc][r] * s.dO[sc][j];
            }
            for (int d = 0; d < D; ++d) {
                u -= s.W[r][d] * s.S[d][j];
                du += s.Kb[r][d] * s.dS[d][j];
            }
            s.U[r][j] = u;
            s.dU[r][j] = du;
        }
        __syncthreads();

        // partial sums over this slice's value columns, and dV
        float *part = p.part + ((bh * p.nchunk + c) * NS + sl) * (int64_t)PL::SIZE;
        for (int i = tid; i < C * D; i += NT) {
            const int r = i / D, d = i % D;
            float a = 0.f, bb = 0.f, w = 0.f;
            for (int j = 0; j < NC; ++j) {
                a += s.dO[r][j] * s.S[d][j];
                bb += s.U[r][j] * s.dS[d][j];
                w -= s.dU[r][j] * s.S[d][j];
            }
            part[PL::DQH + i] = a;
            part[PL::DKB + i] = bb;
            part[PL::DW + i] = w;
        }
        for (int i = tid; i < C * C; i += NT) {
            const int r = i / C, sc = i % C;
            float dp = 0.f, dtv = 0.f;
            for (int j = 0; j < NC; ++j) {
                dp += s.dO[r][j] * s.U[sc][j];
                dtv += s.dU[r][j] * s.beta[sc] * s.V[sc][j];
            }
            part[PL::DP + i] = dp;
            part[PL::DTV + i] = dtv;
        }
        for (int d = tid; d < D; d += NT) {
            float a = 0.f;
            for (int j = 0; j < NC; ++j) a += s.dS[d][j] * s.S[d][j];
            part[PL::DGN + d] = a;
        }
        // dBV = T^T dU;  dV = beta dBV
        for (int i = tid; i < C * NC; i += NT) {
            const int r = i / NC, j = i % NC;
            float a = 0.f;
            for (int sc = 0; sc < C; ++sc) a += s.T[sc][r] * s.dU[sc][j];
            s.BV[r][j] = a;
            if (r < n) p.dv[(row0 + (int64_t)r * H) * D + j0 + j] = s.beta[r] * a;
        }
        __syncthreads();
        for (int r = tid; r < C; r += NT) {
            float a = 0.f;
            for (int j = 0; j < NC; ++j) a += s.BV[r][j] * s.V[r][j];
            part[PL::DBV + r] = a;
        }
        // dS <- Q^^T dO + e^{G_n} dS' - W^T dU   (each thread its own entries)
        for (int i = tid; i < D * NC; i += NT) {
            const int d = i / NC, j = i % NC;
            float a = s.Gn[d] * s.dS[d][j];
            for (int r = 0; r < C; ++r) a += s.Qh[r][d] * s.dO[r][j] - s.W[r][d] * s.dU[r][j];
            s.dS[d][j] = a;
        }
        __syncthreads();
    }
    for (int i = tid; i < D * NC; i += NT) {
        const int d = i / NC, j = i % NC;
        p.dS0[(bh * D + d) * D + j0 + j] = s.dS[d][j];
    }
}

// ------------------------------------------- bf16, d = 128: MFMA kernels ----
//
// For bf16 inputs at d = 128 the chain is split in two, both on bf16 MFMA
// tiles with fp32 accumulation (the forward's operand precision):
//   dstate -- sequential over chunks, one workgroup per (b, h, 64 value
//             columns), a wave per 16 columns with its 128 x 16 slice of dS in
//             accumulator tiles.  Per chunk (reverse order) it stores the
//             incoming dS' and applies
//                dU = P^T dO + Kb dS',   dS = e^{G_n} dS' + Q^^T dO - W^T dU.
//             The chunk's prep record is staged through LDS (double buffer,
//             one barrier per chunk).
//   part   -- one workgroup per (b, h, chunk), all chunks in parallel: from the
//             chunk-entry state S (forward checkpoints) and the stored dS' it
//             recomputes U and dU and forms, over all 128 value columns at once,
//             the sums the grad kernel consumes (dQ^, dKb, dW, dP, the V part of
//             dT and of dbeta, sum_j dS' S), plus dV.  The record has a single
//             column slice.

namespace {

constexpr int BD = 128;          // head size of the MFMA backward
constexpr int BLD = BD + 8;      // bf16 row stride of [.][d] / [.][j] LDS tiles
constexpr int BLT = C + 8;       // bf16 row stride of [.][token] LDS tiles
constexpr int BLQ = BD + 16;     // bf16 row stride of tiles read only by transposing reads
                                 // (8 banks between rows: the 16 rows of a read do not collide)

// K16 fragment over k = r0 + 4*(lane/16) + e of column col0 + lane%16 of a
// row-major LDS tile, tile[k][col0 + lane%16], from one transposing 8-byte
// LDS read per lane (gfx950's ds_read_b64_tr_b16, in place of four 2-byte
// reads): within each 16-lane group the hardware hands lane i,
// element e, element i % 4 of the 8 bytes that lane 4e + i/4 addressed.  So
// lane (g, j) addresses row r0 + 4g + j/4, columns col0 + 4(j%4) .. +3, and
// lane (g, n) receives tile[r0 + 4g + e][col0 + n].  `tile` must be in LDS,
// col0 a multiple of 4 and the row stride a multiple of 4 elements.
__device__ __forceinline__ Frag<bf16> frag_rows_tr(const bf16 *tile, int ld, int r0, int col0,
                                                   int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int g = lane >> 4, j = lane & 15;
    const bf16 *a = tile + (r0 + 4 * g + (j >> 2)) * ld + col0 + 4 * (j & 3);
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(a));
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x4, r);
    return f;
}

__device__ __forceinline__ void store_bf16x4(bf16 *p, float a, float b, float c, float d) {
    *reinterpret_cast<bf16x4 *>(p) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}

// Sum over the 16 lanes n of each row group (lanes 16g .. 16g+15), fixed order.
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 8, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 1, 16);
    return x;
}

struct DstateBuf {
    bf16 Kb[C][BLD];      // Kb [r][d]
    bf16 Qh[C][BLQ];      // Q^ [r][d]  (read transposed by ds_read_b64_tr_b16)
    bf16 Wn[C][BLQ];      // -W [r][d]
    bf16 PT[C][BLT];      // P transposed [r][s] = P[s][r]
    float Gn[BD];         // e^{G_n}
};

}  // namespace

template <int NW>
__global__ __launch_bounds__(64 * NW) void kda_bwd_dstate_kernel(BwdArgs p, bf16 *dsp) {
    using Lay = PrepLayout<BD>;
    constexpr int NDT = BD / 16, NT = 64 * NW, NSL = BD / (16 * NW);
    __shared__ __attribute__((aligned(16))) DstateBuf buf[2];
    static_assert(2 * sizeof(DstateBuf) <= 150 * 1024, "LDS budget");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t x = blockIdx.x;
    const int64_t bh = x / NSL;
    const int jw = (int)(x % NSL) * 16 * NW + 16 * wave;   // this wave's first value column
    const int64_t b = bh / p.H, h = bh % p.H, H = p.H;
    const int64_t nchunk = p.nchunk;
    const bf16 *dO = static_cast<const bf16 *>(p.dO);

    f32x4 dS[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[i][e] = p.dST ? p.dST[(bh * BD + 16 * i + 4 * g + e) * BD + jw + n] : 0.f;

    // Staging registers: this thread's float4s of the record of one chunk and
    // the wave's dO fragment.  Two sets alternate, so every chunk's loads are
    // issued two chunk steps before the step that writes them to LDS.
    struct Regs {
        f32x4 rw[2048 / 4 / NT], rq[2048 / 4 / NT], rk[2048 / 4 / NT], rp, rg;
        short dr[4];
    };
    const int64_t tok_stride = H * BD, row_bytes = tok_stride * 2;
    const int64_t base = (b * p.T * H + h) * BD;
    auto load = [&](int64_t c, Regs &R) {
        const f32x4 *rec =
            reinterpret_cast<const f32x4 *>(p.prep + (bh * nchunk + c) * (int64_t)Lay::SIZE);
#pragma unroll
        for (int u = 0; u < 2048 / 4 / NT; ++u) {
            // W and Q^ in (token, 4-column group) order, Kb row-major
            const int f = tid + NT * u, r = f % C, q4 = f / C;
            R.rw[u] = rec[Lay::W / 4 + r * (BD / 4) + q4];
            R.rq[u] = rec[Lay::QH / 4 + r * (BD / 4) + q4];
            R.rk[u] = rec[Lay::KB / 4 + f];
        }
        if (tid < C * C / 4) R.rp = rec[Lay::P / 4 + tid];
        if (tid < BD / 4) R.rg = rec[Lay::GN / 4 + tid];
        // dO fragment: dO[t0 + 4g + e][jw + n] (zero past T)
        const int64_t t0 = c * C, rows = p.T - t0 < C ? p.T - t0 : (int64_t)C;
        const auto rs = make_rsrc(dO + base + t0 * tok_stride + jw, rows * row_bytes);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            R.dr[e] = __builtin_amdgcn_raw_buffer_load_b16(rs, (4 * g + e) * (int)row_bytes + 2 * n, 0, 0);
    };
    auto store = [&](const Regs &R, DstateBuf &B) {
#pragma unroll
        for (int u = 0; u < 2048 / 4 / NT; ++u) {
            const int f = tid + NT * u, r = f / (BD / 4), d = 4 * (f % (BD / 4));
            store_bf16x4(&B.Kb[r][d], R.rk[u][0], R.rk[u][1], R.rk[u][2], R.rk[u][3]);
        }
        // Q^ and -W row-major (the products read them transposed)
#pragma unroll
        for (int u = 0; u < 2048 / 4 / NT; ++u) {
            const int f = tid + NT * u, r = f % C, d = 4 * (f / C);
            store_bf16x4(&B.Qh[r][d], R.rq[u][0], R.rq[u][1], R.rq[u][2], R.rq[u][3]);
            store_bf16x4(&B.Wn[r][d], -R.rw[u][0], -R.rw[u][1], -R.rw[u][2], -R.rw[u][3]);
        }
        if (tid < C * C / 4) {
            const int sidx = tid / 4, r0 = 4 * (tid % 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) B.PT[r0 + e][sidx] = (bf16)R.rp[e];
        }
        if (tid < BD / 4) *reinterpret_cast<f32x4 *>(&B.Gn[4 * tid]) = R.rg;
    };
    auto dO_frag = [](const Regs &R) {
        Frag<bf16> f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f.v[e] = __builtin_bit_cast(bf16, R.dr[e]);
        return f;
    };
    // one chunk step (reverse order), from the chunk's record in buf[c & 1]
    auto step = [&](int64_t c, const Frag<bf16> &dOf) {
        const DstateBuf &B = buf[c & 1];
        // dU = P^T dO + Kb dS'; the incoming dS' of chunk c is stored as the
        // same bf16 values the products use
        Frag<bf16> dSf[NDT];
#pragma unroll
        for (int i = 0; i < NDT; ++i) dSf[i] = acc_frag<bf16>(dS[i]);
        // stored in 4-row blocks, element (d, j) at ((d/4)*D + j)*4 + d%4: a
        // lane's four rows of a tile are one 8-byte group, and the 16 lanes of
        // a row group write 128 contiguous bytes
        bf16 *out = dsp + (bh * nchunk + c) * (int64_t)(BD * BD) + (g * BD + jw + n) * 4;
#pragma unroll
        for (int i = 0; i < NDT; ++i)
            *reinterpret_cast<bf16x4 *>(out + i * 4 * 4 * BD) = dSf[i].v;
        f32x4 ua = {0.f, 0.f, 0.f, 0.f}, ub = {0.f, 0.f, 0.f, 0.f};
        mma16(ua, lds_frag(&B.PT[0][0], BLT, 0, lane), dOf);
#pragma unroll
        for (int i = 0; i < NDT; i += 2) {
            f32x4 &acc = (i / 2) % 2 ? ua : ub;
            mma32(acc, lds_frag(&B.Kb[0][0], BLD, 16 * i, lane),
                  lds_frag(&B.Kb[0][0], BLD, 16 * i + 16, lane), dSf[i], dSf[i + 1]);
        }
        const Frag<bf16> dUf = acc_frag<bf16>(ua + ub);
        // dS = e^{G_n} dS' + Q^^T dO - W^T dU
#pragma unroll
        for (int i = 0; i < NDT; ++i) {
            const f32x4 gn = *reinterpret_cast<const f32x4 *>(&B.Gn[16 * i + 4 * g]);
            dS[i] *= gn;
            mma32(dS[i], frag_rows_tr(&B.Qh[0][0], BLQ, 0, 16 * i, lane),
                  frag_rows_tr(&B.Wn[0][0], BLQ, 0, 16 * i, lane), dOf, dUf);
        }
    };

    Regs RA, RB;
    if (nchunk > 0) {
        load(nchunk - 1, RA);
        store(RA, buf[(nchunk - 1) & 1]);
    }
    if (nchunk > 1) load(nchunk - 2, RB);
    __syncthreads();
    for (int64_t c = nchunk - 1; c >= 0; c -= 2) {
        // chunk c: RA holds its dO; RB (chunk c-1) is in flight
        const Frag<bf16> dOa = dO_frag(RA);
        if (c >= 2) load(c - 2, RA);
        step(c, dOa);
        if (c >= 1) store(RB, buf[(c - 1) & 1]);
        __syncthreads();
        if (c < 1) break;
        // chunk c-1: RB holds its dO; RA (chunk c-2) is in flight
        const Frag<bf16> dOb = dO_frag(RB);
        if (c >= 3) load(c - 3, RB);
        step(c - 1, dOb);
        if (c >= 2) store(RA, buf[c & 1]);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.dS0[(bh * BD + 16 * i + 4 * g + e) * BD + jw + n] = dS[i][e];
}

namespace {
struct PartLds {
    bf16 S[BD][BLD], dS[BD][BLD];          // chunk-entry state, incoming dS' [d][j]
    bf16 W[C][BLD], Kb[C][BLD];            // [r][d]
    bf16 V[C][BLD], dO[C][BLD], U[C][BLD], dU[C][BLD];   // [r][j]
    bf16 Ulo[C][BLD], dUlo[C][BLD];        // U - bf16(U), dU - bf16(dU): U, dU to ~16 bits
    bf16 Tb[C][BLT], PT[C][BLT], TT[C][BLT];            // T, P^T, T^T
    float beta[C];
    float dbV[8][C];
};
}  // namespace

// 16 waves per chunk (the LDS of one chunk allows one workgroup per CU, so
// its waves are what hides latency): value-column phase split into U (waves
// 0-7) and dU (waves 8-15), key-row phase into dQ^, dW (0-7) and dKb, dP,
// dT's V part (8-15).
__global__ __launch_bounds__(1024) void kda_bwd_part_kernel(BwdArgs p, const bf16 *dsp) {
    using Lay = PrepLayout<BD>;
    using PL = PartLayout<BD>;
    __shared__ __attribute__((aligned(16))) PartLds s;
    static_assert(sizeof(PartLds) <= 150 * 1024, "LDS budget");   // blockDim.x == 1024
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t x = blockIdx.x;
    const int64_t c = x % p.nchunk, bh = x / p.nchunk;
    const int64_t b = bh / p.H, h = bh % p.H, H = p.H;
    const int nv = (int)(p.T - c * C < C ? p.T - c * C : C);   // tokens in the chunk
    const int64_t nfull = p.T / C;
    const int64_t row0 = (b * p.T + c * C) * H + h;            // token row of the chunk's first token
    const bf16 *v = static_cast<const bf16 *>(p.v), *dOg = static_cast<const bf16 *>(p.dO),
               *betag = static_cast<const bf16 *>(p.beta);
    float *part = p.part + x * (int64_t)PL::SIZE;

    // ---- stage: every global load first, then the LDS tiles ----
    // S (fp32 S0 for the first chunk, else the bf16 checkpoint) and dS' come as
    // 4 x 4 blocks, rows d0..d0+3 by columns j0..j0+3, so that a thread holds
    // both operands of its 16 products of sum_j dS' S; 32 consecutive threads
    // cover one block row and reduce it in a fixed order.
    {
        const float *Sin = c == 0 && p.S0 ? p.S0 + bh * (int64_t)(BD * BD) : nullptr;
        const bf16 *Ck = c >= 1 ? reinterpret_cast<const bf16 *>(p.ckpt) +
                                      ((b * nfull + c - 1) * H + h) * (int64_t)(BD * BD)
                                : nullptr;
        const bf16 *Dt = dsp + x * (int64_t)(BD * BD);   // 4-row blocks, as dstate stores them
        const float *rec = p.prep + x * (int64_t)Lay::SIZE;
        const int d0 = 4 * (tid / 32), j0 = 4 * (tid % 32);
        f32x4 sv[4];    // sv[r] = S[d0 + r][j0 .. j0+3]
        bf16x4 tv[4];   // tv[e] = dS'[d0 .. d0+3][j0 + e]
        if (c == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sv[e] = Sin ? *reinterpret_cast<const f32x4 *>(Sin + (d0 + e) * BD + j0)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
            bf16x4 cv[4];   // cv[e] = S[d0 .. d0+3][j0 + e]
#pragma unroll
            for (int e = 0; e < 4; ++e)
                cv[e] = *reinterpret_cast<const bf16x4 *>(Ck + ((d0 / 4) * BD + j0 + e) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sv[r] = f32x4{(float)cv[0][r], (float)cv[1][r], (float)cv[2][r], (float)cv[3][r]};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            tv[e] = *reinterpret_cast<const bf16x4 *>(Dt + ((d0 / 4) * BD + j0 + e) * 4);
        // one float4 of W (threads 0-511) or Kb (512-1023), T or P rows, beta,
        // and one 16-byte piece of a V (0-255) or dO (256-511) row
        const int t5 = tid & 511, rW = t5 / 32, dW = 4 * (t5 % 32);
        const f32x4 wk4 = reinterpret_cast<const f32x4 *>(rec + (tid < 512 ? Lay::W : Lay::KB))[t5];
        f32x4 tp4 = {0.f, 0.f, 0.f, 0.f};
        if (tid < C * C / 4)
            tp4 = reinterpret_cast<const f32x4 *>(rec + Lay::T)[tid];
        else if (tid < 2 * C * C / 4)
            tp4 = reinterpret_cast<const f32x4 *>(rec + Lay::P)[tid - C * C / 4];
        const int rb = tid - 2 * C * C / 4;
        float bv = 0.f;
        if (rb >= 0 && rb < nv) bv = (float)betag[row0 + (int64_t)rb * H];
        const int t2 = tid & 255, rv = t2 / 16, pc = t2 % 16;
        uint4 val = {0u, 0u, 0u, 0u};
        if (tid < 512 && rv < nv)
            val = *reinterpret_cast<const uint4 *>((tid < 256 ? v : dOg) +
                                                   (row0 + (int64_t)rv * H) * BD + 8 * pc);

#pragma unroll
        for (int e = 0; e < 4; ++e) {
            store_bf16x4(&s.S[d0 + e][j0], sv[e][0], sv[e][1], sv[e][2], sv[e][3]);
            *reinterpret_cast<bf16x4 *>(&s.dS[d0 + e][j0]) =
                bf16x4{tv[0][e], tv[1][e], tv[2][e], tv[3][e]};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // row d0 + r: S[d0+r][j0+e] * dS'[d0+r][j0+e]
            float a = sv[r][0] * (float)tv[0][r] + sv[r][1] * (float)tv[1][r] +
                      sv[r][2] * (float)tv[2][r] + sv[r][3] * (float)tv[3][r];
            a += __shfl_xor(a, 16, 32);
            a += __shfl_xor(a, 8, 32);
            a += __shfl_xor(a, 4, 32);
            a += __shfl_xor(a, 2, 32);
            a += __shfl_xor(a, 1, 32);
            if ((tid & 31) == 0) part[PL::DGN + d0 + r] = a;
        }
        store_bf16x4(tid < 512 ? &s.W[rW][dW] : &s.Kb[rW][dW], wk4[0], wk4[1], wk4[2], wk4[3]);
        if (tid < C * C / 4) {
            // T row rr, columns s0 .. s0+3 (beta is applied to V below)
            const int rr = tid / 4, s0 = 4 * (tid % 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s.Tb[rr][s0 + e] = (bf16)tp4[e];
                s.TT[s0 + e][rr] = (bf16)tp4[e];
            }
        } else if (tid < 2 * C * C / 4) {
            // P row sidx, columns r0 .. r0+3  ->  P^T[r][sidx]
            const int f2 = tid - C * C / 4, sidx = f2 / 4, r0 = 4 * (f2 % 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) s.PT[r0 + e][sidx] = (bf16)tp4[e];
        }
        if (rb >= 0 && rb < C) s.beta[rb] = bv;
        if (tid < 512)
            *reinterpret_cast<uint4 *>(tid < 256 ? &s.V[rv][8 * pc] : &s.dO[rv][8 * pc]) = val;
    }
    __syncthreads();

    // ---- value columns jw .. jw+15: U = T diag(b) V - W S (waves 0-7);
    //      dU = P^T dO + Kb dS', T^T dU, dV, dbeta's V part (waves 8-15) ----
    {
        const int jw = 16 * (wave & 7);
        static_assert(BLD % 4 == 0, "transposing reads need 8-byte rows");
        const Frag<bf16> Vf = frag_rows_tr(&s.V[0][0], BLD, 0, jw, lane);
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
        if (wave < 8) {
            Frag<bf16> bVf;   // diag(beta) V, rows 4g + e
#pragma unroll
            for (int e = 0; e < 4; ++e) bVf.v[e] = (bf16)(s.beta[4 * g + e] * (float)Vf.v[e]);
            mma16(a0, lds_frag(&s.Tb[0][0], BLT, 0, lane), bVf);
#pragma unroll
            for (int i = 0; i < BD / 16; i += 2) {
                f32x4 &acc = (i / 2) % 2 == 0 ? a1 : a2;
                mma32(acc, lds_frag(&s.W[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.W[0][0], BLD, 16 * i + 16, lane),
                      frag_rows_tr(&s.S[0][0], BLD, 16 * i, jw, lane),
                      frag_rows_tr(&s.S[0][0], BLD, 16 * i + 16, jw, lane));
            }
            const f32x4 U = a0 - (a1 + a2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                const bf16 uh = (bf16)U[e];
                s.U[r][jw + n] = uh;
                s.Ulo[r][jw + n] = (bf16)(U[e] - (float)uh);
            }
        } else {
            const Frag<bf16> dOf = frag_rows_tr(&s.dO[0][0], BLD, 0, jw, lane);
            mma16(a0, lds_frag(&s.PT[0][0], BLT, 0, lane), dOf);
#pragma unroll
            for (int i = 0; i < BD / 16; i += 2) {
                f32x4 &acc = (i / 2) % 2 == 0 ? a1 : a2;
                mma32(acc, lds_frag(&s.Kb[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.Kb[0][0], BLD, 16 * i + 16, lane),
                      frag_rows_tr(&s.dS[0][0], BLD, 16 * i, jw, lane),
                      frag_rows_tr(&s.dS[0][0], BLD, 16 * i + 16, jw, lane));
            }
            const f32x4 dU = a0 + (a1 + a2);
            // dU enters the products below as a bf16 pair hi + lo
            const Frag<bf16> dUh = acc_frag<bf16>(dU);
            f32x4 dUl4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dUl4[e] = dU[e] - (float)dUh.v[e];
            f32x4 BV = {0.f, 0.f, 0.f, 0.f};
            const Frag<bf16> TTf = lds_frag(&s.TT[0][0], BLT, 0, lane);
            mma16(BV, TTf, dUh);
            mma16(BV, TTf, acc_frag<bf16>(dUl4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                s.dU[r][jw + n] = dUh.v[e];
                s.dUlo[r][jw + n] = (bf16)dUl4[e];
                if (r < nv) p.dv[(row0 + (int64_t)r * H) * BD + jw + n] = s.beta[r] * BV[e];
                const float part_bv = sum16(BV[e] * (float)Vf.v[e]);
                if (n == 0) s.dbV[wave - 8][r] = part_bv;
            }
        }
    }
    __syncthreads();

    // ---- key rows dw .. dw+15 (sums over all columns): dQ^ and dW (waves
    //      0-7), dKb (8-15); dP (wave 8) and dT's V part (wave 9) ----
    {
        const int dw = 16 * (wave & 7);
        if (wave < 8) {
            f32x4 aq = {0.f, 0.f, 0.f, 0.f}, aw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < BD / 16; i += 2) {
                const Frag<bf16> s0 = lds_frag(&s.S[dw][0], BLD, 16 * i, lane),
                                 s1 = lds_frag(&s.S[dw][0], BLD, 16 * i + 16, lane);
                mma32(aq, lds_frag(&s.dO[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.dO[0][0], BLD, 16 * i + 16, lane), s0, s1);
                mma32(aw, lds_frag(&s.dU[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.dU[0][0], BLD, 16 * i + 16, lane), s0, s1);
                mma32(aw, lds_frag(&s.dUlo[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.dUlo[0][0], BLD, 16 * i + 16, lane), s0, s1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                part[PL::DQH + r * BD + dw + n] = aq[e];
                part[PL::DW + r * BD + dw + n] = -aw[e];
            }
        } else {
            f32x4 ak = {0.f, 0.f, 0.f, 0.f}, ak2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < BD / 16; i += 2) {
                const Frag<bf16> t0 = lds_frag(&s.dS[dw][0], BLD, 16 * i, lane),
                                 t1 = lds_frag(&s.dS[dw][0], BLD, 16 * i + 16, lane);
                mma32(ak, lds_frag(&s.U[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.U[0][0], BLD, 16 * i + 16, lane), t0, t1);
                mma32(ak2, lds_frag(&s.Ulo[0][0], BLD, 16 * i, lane),
                      lds_frag(&s.Ulo[0][0], BLD, 16 * i + 16, lane), t0, t1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                part[PL::DKB + (4 * g + e) * BD + dw + n] = ak[e] + ak2[e];
            if (wave == 8 || wave == 9) {
                // dP = dO U^T (wave 8);  dT's V part = dU (beta V)^T (wave 9)
                // (U, dU as hi + lo pairs)
                const bool w8 = wave == 8;
                const bf16 *A = w8 ? &s.dO[0][0] : &s.dU[0][0];
                const bf16 *Bm = w8 ? &s.U[0][0] : &s.V[0][0];
                const bf16 *A2 = w8 ? &s.dO[0][0] : &s.dUlo[0][0];
                const bf16 *B2 = w8 ? &s.Ulo[0][0] : &s.V[0][0];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < BD / 16; i += 2) {
                    mma32(acc, lds_frag(A, BLD, 16 * i, lane), lds_frag(A, BLD, 16 * i + 16, lane),
                          lds_frag(Bm, BLD, 16 * i, lane), lds_frag(Bm, BLD, 16 * i + 16, lane));
                    mma32(acc2, lds_frag(A2, BLD, 16 * i, lane), lds_frag(A2, BLD, 16 * i + 16, lane),
                          lds_frag(B2, BLD, 16 * i, lane), lds_frag(B2, BLD, 16 * i + 16, lane));
                }
                const float sc = w8 ? 1.f : s.beta[n];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    part[(w8 ? PL::DP : PL::DTV) + (4 * g + e) * C + n] = (acc[e] + acc2[e]) * sc;
            } else if (wave == 10 && lane < C) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < 8; ++w) a += s.dbV[w][lane];
                part[PL::DBV + lane] = a;
            }
        }
    }
}

// ------------------------------------------------------------------ grad ----

// Only what several waves read goes through LDS: Kh (dT's row fragments), A,
// T, beta and the partial sums.  q e^{G}, k e^{-G} and e^{G} are read only
// at each thread's own tile elements and stay in its registers (so that four
// workgroups fit per CU).
template <int D> struct GradLds {
    float Kh[C][rowpad<D>()];          // k e^{G}
    float A[C][C + 1], T[C][C + 1];    // from the chunk's prep record
    float beta[C];
    float dW[C][rowpad<D>()];
    float dP[C][C + 1], dTV[C][C + 1], dL[C][C + 1];
    float dbV[C], dGn[D];   // dGn: sum_j dS' S (times e^{G_n} where used)
    float dbk[4][C];   // per-wave sums over d of (T^T dW)[r][d] Kh[r][d]
    float dbL[C];      // sum_s dL[r][s] A[r][s]
};

template <typename TI, int D, int NS>
__global__ __launch_bounds__(256, 4) void kda_bwd_grad_kernel(BwdArgs p) {
    __shared__ GradLds<D> s;
    static_assert(sizeof(GradLds<D>) <= 150 * 1024, "LDS budget");
    using PL = PartLayout<D>;
    using Lay = PrepLayout<D>;
    const int64_t x = blockIdx.x;
    const int64_t c = x % p.nchunk, bh = x / p.nchunk;
    const int64_t b = bh / p.H, h = bh % p.H, H = p.H;
    const int n = (int)(p.T - c * C < C ? p.T - c * C : C);
    const int tid = threadIdx.x;
    // the slices' partial sums, added in slice order (4-float loads, all issued
    // before any use; blockDim.x == 256)
    const float *part = p.part + x * NS * (int64_t)PL::SIZE;
    const float *rec = p.prep + x * (int64_t)Lay::SIZE;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, nn = lane & 15;
    constexpr int LDD = rowpad<D>(), LDC = C + 1, NDT = D / 16, TPW = (NDT + 3) / 4;
    const TI *qg = static_cast<const TI *>(p.q), *kg = static_cast<const TI *>(p.k),
             *zg = static_cast<const TI *>(p.z), *bg = static_cast<const TI *>(p.beta);
    const int64_t row0 = (b * p.T + c * C) * H + h;   // token row of the chunk's first token
    const float cA = __expf(p.A[h]);
    // per thread, rows 4g..4g+3 of column 16t + nn of each of its tiles t:
    // dQ^ and dKb partial sums, q, k, z; then e^{G}, q e^{G}, k e^{G}, k e^{-G}
    float tq[TPW][4], tkb[TPW][4], tz[TPW][4];
    float ev[TPW][4], qh[TPW][4], kh[TPW][4], ki[TPW][4];
    {
        float qv[TPW][4], kv[TPW][4];
        f32x4 at4 = {0.f, 0.f, 0.f, 0.f};   // A (threads < 64), T (64 .. 127)
        if (tid < C * C / 4)
            at4 = reinterpret_cast<const f32x4 *>(rec + Lay::A)[tid];
        else if (tid < C * C / 2)
            at4 = reinterpret_cast<const f32x4 *>(rec + Lay::T)[tid - C * C / 4];
        const float bt = tid < n ? to_f32(bg[row0 + (int64_t)tid * H]) : 0.f;   // tid < C
        constexpr int NV4 = C * D / 4, PER = (NV4 + 255) / 256;
        f32x4 w[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int v = tid + 256 * j;
            w[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (v < NV4) {
#pragma unroll
                for (int q = 0; q < NS; ++q)
                    w[j] += reinterpret_cast<const f32x4 *>(part + q * PL::SIZE)[PL::DW / 4 + v];
            }
        }
        // dQ^, dKb and z at this thread's elements of its column tiles (rows
        // 4g..4g+3 of column 16t + nn), used directly by the dq/dk pass
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wave + 4 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e, d = 16 * t + nn;
                float a = 0.f, bq = 0.f;
                if (t < NDT) {
#pragma unroll
                    for (int q = 0; q < NS; ++q) {
                        a += part[q * PL::SIZE + PL::DQH + r * D + d];
                        bq += part[q * PL::SIZE + PL::DKB + r * D + d];
                    }
                }
                tq[j][e] = a;
                tkb[j][e] = bq;
                const bool in = t < NDT && r < n;
                const int64_t off = (row0 + (int64_t)r * H) * D + d;
                qv[j][e] = in ? to_f32(qg[off]) : 0.f;
                kv[j][e] = in ? to_f32(kg[off]) : 0.f;
                tz[j][e] = in ? to_f32(zg[off]) : 0.f;
            }
        }
        // dP, dT's V part (64 float4 each), dbeta's V part (4), sum_j dS' S (D/4)
        f32x4 e4 = {0.f, 0.f, 0.f, 0.f}, f4 = {0.f, 0.f, 0.f, 0.f};
        const int u = tid - C * C / 4;       // dbV / dGn lanes
        if (tid < C * C / 4) {
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const f32x4 *pq = reinterpret_cast<const f32x4 *>(part + q * PL::SIZE);
                e4 += pq[PL::DP / 4 + tid];
                f4 += pq[PL::DTV / 4 + tid];
            }
        } else if (u < C / 4 + D / 4) {
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const f32x4 *pq = reinterpret_cast<const f32x4 *>(part + q * PL::SIZE);
                e4 += u < C / 4 ? pq[PL::DBV / 4 + u] : pq[PL::DGN / 4 + (u - C / 4)];
            }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int v = tid + 256 * j;
            if (v < NV4) {
                const int r = (4 * v) / D, d = (4 * v) % D;
#pragma unroll
                for (int e = 0; e < 4; ++e) s.dW[r][d + e] = w[j][e];
            }
        }
        if (tid < C * C / 4) {
            const int r = (4 * tid) / C, s0 = (4 * tid) % C;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s.dP[r][s0 + e] = s0 + e <= r ? e4[e] : 0.f;   // P is lower triangular
                s.dTV[r][s0 + e] = f4[e];
            }
        } else if (u < C / 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s.dbV[4 * u + e] = e4[e];
        } else if (u < C / 4 + D / 4) {
            const int d = 4 * (u - C / 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) s.dGn[d + e] = e4[e];
        }
        if (tid < C * C / 2) {
            const int f = 4 * (tid % (C * C / 4)), r = f / C, s0 = f % C;
            float(*M)[C + 1] = tid < C * C / 4 ? s.A : s.T;
#pragma unroll
            for (int e = 0; e < 4; ++e) M[r][s0 + e] = at4[e];
        }
        if (tid < C) s.beta[tid] = bt;
        // G = cumulative sum over the rows of g_min sigma(c z) (0 past the
        // chunk's tokens): within the lane's four rows, then the totals of the
        // lower lane groups, added in group order
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wave + 4 * j;
            float cs[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gz = 4 * g + e < n ? kGMin * sigmoidf_(cA * tz[j][e]) : 0.f;
                cs[e] = e == 0 ? gz : cs[e - 1] + gz;
            }
            const float t0 = __shfl(cs[3], nn), t1 = __shfl(cs[3], 16 + nn),
                        t2 = __shfl(cs[3], 32 + nn);
            const float pre = g == 0 ? 0.f : g == 1 ? t0 : g == 2 ? t0 + t1 : (t0 + t1) + t2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float G = pre + cs[e], E = __expf(G), Ei = __expf(-G);
                ev[j][e] = E;
                qh[j][e] = qv[j][e] * E;
                kh[j][e] = kv[j][e] * E;
                ki[j][e] = kv[j][e] * Ei;
                if (t < NDT) s.Kh[4 * g + e][16 * t + nn] = kh[j][e];
            }
        }
    }
    __syncthreads();
    // wave 0: dT = dW (beta K^)^T + dU (beta V)^T (a 16 x 16 tile over d), then
    // dL = -(T^T dT) T^T (strictly lower), its share of dbeta and dA = diag(beta) dL,
    // all on fp32 matrix-core tiles in registers.  A tile in accumulator layout
    // (lane (g, n) holds X[4g+e][n]) is the B operand of X and the A operand of X^T.
    if (wave == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += 16) {
            if ((k0 / 16) % 2 == 0)
                mma16(acc, rowfrag(&s.dW[0][0], LDD, 0, k0, lane), rowfrag(&s.Kh[0][0], LDD, 0, k0, lane));
            else
                mma16(acc2, rowfrag(&s.dW[0][0], LDD, 0, k0, lane), rowfrag(&s.Kh[0][0], LDD, 0, k0, lane));
        }
        Frag<float> dTf;   // dT[4g+e][nn]
#pragma unroll
        for (int e = 0; e < 4; ++e) dTf.v[e] = s.dTV[4 * g + e][nn] + s.beta[nn] * (acc[e] + acc2[e]);
        f32x4 m1t = {0.f, 0.f, 0.f, 0.f};   // M1^T = dT^T T:  M1^T[4g+e][nn]
        mma16(m1t, dTf, colfrag(&s.T[0][0], LDC, 0, 0, lane));
        Frag<float> m1f;
        m1f.v = m1t;
        f32x4 tm = {0.f, 0.f, 0.f, 0.f};    // T M1^T = -dL^T:  -dL[nn][4g+e]
        mma16(tm, rowfrag(&s.T[0][0], LDC, 0, 0, lane), m1f);
        float lb = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int sc = 4 * g + e;
            const float dl = sc < nn ? -tm[e] : 0.f;   // dL[nn][sc]
            lb += dl * s.A[nn][sc];
            s.dL[nn][sc] = dl * s.beta[nn];            // now dA
        }
        lb += __shfl_xor(lb, 16);
        lb += __shfl_xor(lb, 32);
        if (g == 0) s.dbL[nn] = lb;
    }
    // T^T dW: wave w takes the 16-column tiles w, w+4, ..., keeps them in
    // registers for dk below, and sums its share of (T^T dW) . K^ per row
    f32x4 tdw[TPW];
    {
        float part_b[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wave + 4 * j;
            tdw[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (t < NDT) {
                mma16(tdw[j], colfrag(&s.T[0][0], LDC, 0, 0, lane),
                      colfrag(&s.dW[0][0], LDD, 0, 16 * t, lane));
#pragma unroll
                for (int e = 0; e < 4; ++e) part_b[e] += tdw[j][e] * kh[j][e];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = sum16(part_b[e]);
            if (nn == 0) s.dbk[wave][4 * g + e] = v;
        }
    }
    __syncthreads();
    // dbeta: V part, K^ part (through W), L part
    if (tid < C) {
        const int r = tid;
        const float a = s.dbV[r] + ((s.dbk[0][r] + s.dbk[1][r]) + (s.dbk[2][r] + s.dbk[3][r])) +
                        s.dbL[r];
        if (r < n) p.dbeta[(b * p.T + c * C + r) * H + h] = a;
    }
    // dq, dk, dG and dz on the same column tiles:
    //   dQ^ += dP Ki,  dK^ = dA Ki + beta (T^T dW),  dKi = dA^T K^ + dP^T Q^
    // (products over the 16 tokens s on fp32 matrix-core tiles).  A tile's
    // rows 4g..4g+3 of column d sit in lane group g, so the column's dG_n terms
    // and the reverse cumulative sum of dG over the 16 rows are formed across
    // the four lane groups, and the gate's derivative gives dz in place.
    float dA_acc = 0.f;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int t = wave + 4 * j;
        if (t < NDT) {
            const int d = 16 * t + nn;
            f32x4 dqh, dkh = {0.f, 0.f, 0.f, 0.f}, dki = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) dqh[e] = tq[j][e];
            // B operands straight from the registers (lane (g, nn) holds rows
            // 4g..4g+3 of column d)
            Frag<float> kiB, khB, qhB;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kiB.v[e] = ki[j][e];
                khB.v[e] = kh[j][e];
                qhB.v[e] = qh[j][e];
            }
            mma16(dqh, rowfrag(&s.dP[0][0], LDC, 0, 0, lane), kiB);
            mma16(dkh, rowfrag(&s.dL[0][0], LDC, 0, 0, lane), kiB);
            mma16(dki, colfrag(&s.dL[0][0], LDC, 0, 0, lane), khB);
            mma16(dki, colfrag(&s.dP[0][0], LDC, 0, 0, lane), qhB);
            const float En = __shfl(ev[j][3], 48 + nn);   // e^{G} of the last row
            float dGv[4], colp = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                const float dk_h = dkh[e] + s.beta[r] * tdw[j][e];   // through W = T diag(beta) K^
                const float Em = ev[j][e], Ei = 1.0f / Em;   // e^{G}, e^{-G}
                const float dKb = tkb[j][e], kb = ki[j][e] * En;   // Kb = k e^{G_n - G}
                const float dq = dqh[e] * Em;
                const float dk = dk_h * Em + dki[e] * Ei + dKb * En * Ei;
                dGv[e] = dqh[e] * qh[j][e] + dk_h * kh[j][e] - dki[e] * ki[j][e] - dKb * kb;
                colp += dKb * kb;   // d/dG_n of Kb = k e^{G_n - G}
                if (r < n) {
                    const int64_t off = ((b * p.T + c * C + r) * H + h) * D + d;
                    p.dq[off] = dq;
                    p.dk[off] = dk;
                }
            }
            // G_n is G of the last row: it collects the column's Kb terms and
            // e^{G_n} (sum_j dS' S)
            colp += __shfl_xor(colp, 16);
            colp += __shfl_xor(colp, 32);
            if (g == 3) dGv[3] += s.dGn[d] * En + colp;   // d/dG_n of e^{G_n} (sum_j dS' S)
            // dg = reverse cumulative sum of dG over the rows: within the lane,
            // then the totals of the higher lane groups
            float suf[4];
            suf[3] = dGv[3];
            suf[2] = dGv[2] + suf[3];
            suf[1] = dGv[1] + suf[2];
            suf[0] = dGv[0] + suf[1];
            const float t1 = __shfl_xor(suf[0], 16), t2 = __shfl_xor(suf[0], 32),
                        t3 = __shfl_xor(suf[0], 48);
            const float higher = ((g ^ 1) > g ? t1 : 0.f) + ((g ^ 2) > g ? t2 : 0.f) +
                                 ((g ^ 3) > g ? t3 : 0.f);
            // gate: g = g_min sigma(c z)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                if (r < n) {
                    const int64_t off = ((b * p.T + c * C + r) * H + h) * D + d;
                    const float xz = cA * tz[j][e];
                    const float sg = sigmoidf_(xz);
                    const float dx = (suf[e] + higher) * kGMin * sg * (1.0f - sg);
                    p.dz[off] = cA * dx;
                    dA_acc += dx * xz;
                }
            }
        }
    }
    // the chunk's share of dA: block sum in a fixed order (16 partial sums of
    // 16 consecutive threads each, then their sum)
    __shared__ float red[256 + 16];
    red[tid] = dA_acc;
    __syncthreads();
    if (tid < 16) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a += red[16 * tid + i];
        red[256 + tid] = a;
    }
    __syncthreads();
    if (tid == 0) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a += red[256 + i];
        p.dA_part[x] = a;
    }
}

// dA[h] = sum over (sequence, chunk) of the shares: one workgroup per head,
// thread t sums shares t, t + 256, ... (in order), then a fixed-order tree.
__global__ __launch_bounds__(256) void kda_bwd_dA_kernel(const float *dA_part, float *dA,
                                                          int64_t B, int64_t H, int64_t nchunk) {
    __shared__ float red[256];
    const int64_t h = blockIdx.x;
    const int t = threadIdx.x;
    float a = 0.f;
    for (int64_t i = t; i < B * nchunk; i += 256) {
        const int64_t b = i / nchunk, c = i % nchunk;
        a += dA_part[(b * H + h) * nchunk + c];
    }
    red[t] = a;
    __syncthreads();
#pragma unroll
    for (int w = 128; w > 0; w /= 2) {
        if (t < w) red[t] += red[t + w];
        __syncthreads();
    }
    if (t == 0) dA[h] = red[0];
}

size_t bwd_prep_floats(int64_t D) {
    return D == 128 ? PrepLayout<128>::SIZE : PrepLayout<16>::SIZE;
}
size_t bwd_part_floats(int64_t D) {
    return D == 128 ? 2 * PartLayout<128>::SIZE : PartLayout<16>::SIZE;
}

template <typename TI, int D, int NC, int NT>
static hipError_t launch_bwd_t(const BwdArgs &a) {
    const int64_t bh = a.B * a.H, units = bh * a.nchunk;
    if (units > 0)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<TI, D>), dim3((unsigned)units), dim3(256), 0,
                           a.stream, a);
    // with no tokens the chain only writes dS0 = dS_T
    if (bh > 0)
        hipLaunchKernelGGL((kda_bwd_chain_kernel<TI, D, NC, NT>), dim3((unsigned)(bh * (D / NC))),
                           dim3(NT), 0, a.stream, a);
    if (units > 0)
        hipLaunchKernelGGL((kda_bwd_grad_kernel<TI, D, D / NC>), dim3((unsigned)units), dim3(256),
                           0, a.stream, a);
    if (a.H > 0)
        hipLaunchKernelGGL(kda_bwd_dA_kernel, dim3((unsigned)a.H), dim3(256), 0, a.stream,
                           a.dA_part, a.dA, a.B, a.H, a.nchunk);
    return hipGetLastError();
}

// bf16, d = 128: prep, the dS recurrence (dstate) and the chunk-parallel sums
// (part) on MFMA tiles, then grad with a single column slice.  prep reads no
// checkpoint (the front); the rest follows the forward rerun (the back).
hipError_t launch_bwd_front(const BwdArgs &a) {
    if (!(a.dtype == 1 && a.D == BD)) return hipErrorInvalidValue;
    const int64_t units = a.B * a.H * a.nchunk;
    if (units > 0)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<bf16, BD>), dim3((unsigned)units), dim3(256), 0,
                           a.stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_back(const BwdArgs &a) {
    if (!(a.dtype == 1 && a.D == BD)) return hipErrorInvalidValue;
    const int64_t bh = a.B * a.H, units = bh * a.nchunk;
    if (bh > 0)
        hipLaunchKernelGGL(kda_bwd_dstate_kernel<4>, dim3((unsigned)(bh * 2)), dim3(256), 0,
                           a.stream, a, static_cast<bf16 *>(a.dsp));
    if (units > 0) {
        hipLaunchKernelGGL(kda_bwd_part_kernel, dim3((unsigned)units), dim3(1024), 0, a.stream, a,
                           static_cast<const bf16 *>(a.dsp));
        hipLaunchKernelGGL((kda_bwd_grad_kernel<bf16, BD, 1>), dim3((unsigned)units), dim3(256), 0,
                           a.stream, a);
    }
    if (a.H > 0)
        hipLaunchKernelGGL(kda_bwd_dA_kernel, dim3((unsigned)a.H), dim3(256), 0, a.stream,
                           a.dA_part, a.dA, a.B, a.H, a.nchunk);
    return hipGetLastError();
}

static hipError_t launch_bwd_mfma(const BwdArgs &a) {
    const hipError_t e = launch_bwd_front(a);
    return e != hipSuccess ? e : launch_bwd_back(a);
}

size_t bwd_dsp_bytes(int dtype, int64_t D) { return dtype == 1 && D == 128 ? D * D * 2 : 0; }

hipError_t launch_bwd(const BwdArgs &a) {
    if (a.dtype == 1) {
        if (a.D == 128) return launch_bwd_mfma(a);
        return launch_bwd_t<bf16, 16, 16, 256>(a);
    }
    if (a.D == 128) return launch_bwd_t<float, 128, 64, 512>(a);
    return launch_bwd_t<float, 16, 16, 256>(a);
}

}  // namespace kda
