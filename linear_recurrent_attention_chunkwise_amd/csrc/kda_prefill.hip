// kda_prefill.hip -- chunkwise KDA prefill (gfx950).
//
// Method: the KDA recurrence and bounded decay gate of "Kimi K3 Open Weights:
// What Is Actually New", section 1, with the state carried sequentially from
// chunk to chunk and each chunk's tokens handled in parallel (kimi-k3-course
// capstone, one-page map, SEQUENCE block).
// The in-chunk algebra is the WY / UT form of the delta rule, derived from the
// recurrence.  For a chunk of C tokens with entering state S, per key channel
// cumulative log-decay G_r = sum_{s<=r} g_s (r = 0..C-1, chunk-relative):
//
//   L[r,s] = beta_r sum_d k_r[d] k_s[d] e^{G_r[d]-G_s[d]}      (s <  r)
//   P[r,s] =        sum_d q_r[d] k_s[d] e^{G_r[d]-G_s[d]}      (s <= r)
//   U  = (I+L)^-1 diag(beta) (V - (K * e^G) S)
//   O  = (Q * e^G) S + P U
//   S <- e^{G_C} * S + (K * e^{G_C - G})^T U
//
// Range (the reason for the K3 gate bound): g >= -5, so the decay over any
// 16 tokens is >= e^-80 and its reciprocal <= e^80 < bf16 max.  The chunk is
// therefore cut into 16-token sub-tiles p; every pairwise decay factor is
// split at the END of a sub-tile into a factor >= 1 on the row side (at most
// e^75) and a factor <= 1 on the column side, so all MFMA operands stay
// finite and normal-range, and both diagonal and off-diagonal sub-tile blocks
// are plain dense products:
//   row side    Qd_r = q_r e^{G_r - E_p}      (E_p = G at the end of r's sub-tile p)
//   column side Kt_s = k_s e^{E_p' - G_s}     (s in sub-tile p')
//   block (p,p') = Qd_p (Kt_p' * F_{p,p'})^T,  F_{p,p'} = e^{E_p - E_p'} <= 1.
// T = (I+L)^-1 is formed as 16 x 16 blocks: the diagonal ones by nilpotent
// doubling on MFMA, the others from them by block forward substitution, and
// the chain applies T to its rounded V - K e^G S (one product per block).
//
// Work split (one workgroup per (b, h, slice of value columns)):
//   * value columns of the state evolve independently, so a workgroup owns
//     DVB = 16 * NW of them (bf16, dk = 128, 64-token chunks: all 128, eight
//     waves, so a chunk's key-side work is done once per head); each wave
//     owns 16 columns and the full dk x 16 fp32 state slice in registers, and
//     runs the S-dependent chain (U, O, state update) with no cross-wave
//     traffic;
//   * the S-independent per-chunk work (gate, decay factors, P, L and the
//     blocks of T) is done cooperatively by the waves into LDS;
//   * the next chunk's q, k, z, beta, v are prefetched into registers while
//     the current chunk is processed.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

struct PrefillParams {
    const void *q, *k, *v, *z, *beta;
    const float *A, *S0;
    void *o;
    float *S_T;
    int64_t T, H;   // T: tokens per sequence (dense) or in the packing (cu != NULL)
    int nsplit;
    const int64_t *cu;   // packed sequence offsets, or NULL
    const int32_t *order;   // longest-first sequence order, or NULL
    float *ckpt;         // state checkpoints [n_ckpt, H, D, D], or NULL
    int64_t n_ckpt;
    int ckpt_every;      // tokens between checkpoints (0: none)
    int mode;            // 0: prefill; 1: final states only; 3: the state map M
};

template <typename T, int D, int C, int NW>
struct PrefillCfg {
    static constexpr int NT = 64 * NW;
    static constexpr int DVB = 16 * NW;
    static constexpr int NP = C / 16;
    static constexpr int NDT = D / 16;
    // Row strides.  LDS serves each group of 16 lanes from 32 four-byte banks;
    // a fragment read (16 rows, one 8-byte piece each) is conflict-free when
    // the stride is 2 mod 32 words.  [token][d] tiles take D + 4 elements
    // (66 words for bf16, 132 for fp32, whose 16-byte pieces need 4 mod 32),
    // and so do [d][token] / [token][token] tiles (C + 4: 34 words for bf16
    // at C = 64, 10 at C = 16, 68 for fp32 at C = 64), whose rows are then
    // only 8-byte aligned.  The output staging tile is read 16 bytes per row.
    static constexpr int PADE = sizeof(T) == 2 ? 8 : 4;
    static constexpr int DP = D + 4;         // row stride of [token][d] tiles
    static constexpr int CP = C + 4;         // row stride of [d][token] / [token][token] tiles
    static constexpr int LP = C + 4;         // row stride of the fp32 L tile
    static constexpr int OP = DVB + PADE;    // row stride of the output staging tile
    static constexpr int NPAIR = D / 2;
    static constexpr int NSEG_RAW = NT / (NPAIR * NP);
    static constexpr int NSEG = NSEG_RAW < 1 ? 1 : (NSEG_RAW > 16 ? 16 : NSEG_RAW);
    static constexpr int SEGLEN = 16 / NSEG;
    static constexpr int NITEM = NPAIR * NP * NSEG;
    static constexpr int IPT = NITEM / NT;   // gate items per thread
    static constexpr int NOFF = NP * (NP - 1) / 2;
    static constexpr int NB = NP * (NP + 1) / 2;  // lower sub-tile blocks
    static constexpr int BPW = (NB + NW - 1) / NW;
    static constexpr int VQ = C * DVB / (4 * NT);  // v quads per thread
    static_assert(NITEM % NT == 0 && IPT >= 1, "gate items must tile the workgroup");
    static_assert(16 % NSEG == 0, "segments must tile a sub-tile");
    static_assert(VQ >= 1 && (C * DVB) % (4 * NT) == 0, "v quads must tile the workgroup");

    // LDS map (bytes).  Small fp32 tables first, then region X, which holds
    // Qd, Kd, Kt while P and L are formed, then P, T, L and the output
    // staging tile (after the chain only); then the chain operands.
    static constexpr int SZ_TOKD = C * DP * (int)sizeof(T);
    static constexpr int SZ_DTOK = D * CP * (int)sizeof(T);
    static constexpr int SZ_P = C * CP * (int)sizeof(T);
    static constexpr int SZ_L = C * LP * 4;
    static constexpr int SZ_O = C * OP * (int)sizeof(T);
    static constexpr int OFF_GC = 0;
    static constexpr int OFF_F = OFF_GC + D * 4;
    static constexpr int OFF_E = OFF_F + (NOFF > 0 ? NOFF : 1) * D * 4;
    static constexpr int OFF_BETA = OFF_E + NP * NSEG * D * 4;
    static constexpr int OFF_X = (OFF_BETA + C * 4 + 15) / 16 * 16;
    static constexpr int SZ_X1 = 3 * SZ_TOKD;
    static constexpr int SZ_X2 = 2 * SZ_P + SZ_L + SZ_O;
    static constexpr int SZ_X = SZ_X1 > SZ_X2 ? SZ_X1 : SZ_X2;
    static constexpr int OFF_QD = OFF_X;
    static constexpr int OFF_KD = OFF_QD + SZ_TOKD;
    static constexpr int OFF_KT = OFF_KD + SZ_TOKD;
    static constexpr int OFF_P = OFF_X;
    static constexpr int OFF_T = OFF_P + SZ_P;
    static constexpr int OFF_L = OFF_T + SZ_P;
    static constexpr int OFF_O = OFF_L + SZ_L;
    static constexpr int OFF_QG = OFF_X + SZ_X;             // Q e^G        [token][d]
    static constexpr int OFF_KG = OFF_QG + SZ_TOKD;         // beta K e^G   [token][d]
    static constexpr int OFF_KHT = OFF_KG + SZ_TOKD;        // (K e^{G_C-G})^T [d][token]
    static constexpr int OFF_VBT = OFF_KHT + SZ_DTOK;       // (beta V)^T   [column][token]
    static constexpr int LDS_BYTES = OFF_VBT + DVB * CP * (int)sizeof(T);
    static_assert(LDS_BYTES <= 150 * 1024, "LDS budget exceeded");
    static_assert(OFF_O + SZ_O <= OFF_X + SZ_X, "region X overflow");
};

// Index of the off-diagonal sub-tile block (p, p'), p' < p, in the F table.
__host__ __device__ constexpr int off_index(int p, int pq) { return p * (p - 1) / 2 + pq; }

template <typename T> struct PairOf;
template <> struct PairOf<bf16> { typedef uint32_t type; };
template <> struct PairOf<float> { typedef uint2 type; };

__device__ __forceinline__ void unpack2(uint32_t u, float &a, float &b) {
    a = __uint_as_float(u << 16);
    b = __uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ void unpack2(uint2 u, float &a, float &b) {
    a = __uint_as_float(u.x);
    b = __uint_as_float(u.y);
}
__device__ __forceinline__ void store_pair(bf16 *p, float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<bf16x2 *>(p) = bf16x2{(bf16)a, (bf16)b};
}
__device__ __forceinline__ void store_pair(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}
// two values as one bf16 pair (a at the lower address)
__device__ __forceinline__ uint32_t pack_pair_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(bf16)a, (bf16)b});
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_from_f32(const f32x4 &x) {
    return acc_frag<T>(x);
}

// acc += A[16 x K] * B[K x 16], A rows from a K-contiguous LDS tile, B given
// as K16 fragments.
template <typename T, int K>
__device__ __forceinline__ void contract_lds_frag(f32x4 &acc, const T *A, int lda,
                                                  const Frag<T> *Bf, int lane) {
    if constexpr (K >= 32) {
#pragma unroll
        for (int kk = 0; kk + 32 <= K; kk += 32)
            mma32(acc, lds_frag(A, lda, kk, lane), lds_frag(A, lda, kk + 16, lane),
                  Bf[kk / 16], Bf[kk / 16 + 1]);
        if constexpr (K % 32 != 0)
            mma16(acc, lds_frag(A, lda, K - 16, lane), Bf[K / 16 - 1]);
    } else {
#pragma unroll
        for (int kk = 0; kk < K; kk += 16) mma16(acc, lds_frag(A, lda, kk, lane), Bf[kk / 16]);
    }
}

// Item vi of a thread's share of a chunk's v tile (C tokens x DVB/4 column
// quads): each group of 64 items is 16 consecutive tokens x 4 quads, so the
// transposed LDS stores of a wave (rows 4 quads apart, C + 4 elements each)
// fall into disjoint bank ranges.
template <int C, int DVB, int NT>
__device__ __forceinline__ void v_item(int tid, int vi, int &r, int &cq) {
    const int Q = tid + NT * vi;
    const int l = Q & 63, grp = Q >> 6;
    r = 16 * (grp % (C / 16)) + (l & 15);
    cq = 4 * (grp / (C / 16)) + (l >> 4);
}

// One workgroup's share: sequence, head and value-column slice from block
// `blk` of `nblk`.  prm.mode: 0 the prefill; 1 final states only (o is not
// written); 3 the linear part M of the segment's affine state map
// S_end = M S_start + N (the state starts at the identity and v is read as
// zero; M goes to S_T; o is not written).
template <typename T, int D, int C, int NW, bool CKPT>
__device__ __forceinline__ void prefill_block(const PrefillParams &prm, char *smem, int64_t blk,
                                              int64_t nblk) {
    using Cfg = PrefillCfg<T, D, C, NW>;
    using Pair = typename PairOf<T>::type;
    constexpr int NT = Cfg::NT, DVB = Cfg::DVB, NP = Cfg::NP, NDT = Cfg::NDT;
    constexpr int DP = Cfg::DP, CP = Cfg::CP, LP = Cfg::LP, OP = Cfg::OP;
    constexpr int NSEG = Cfg::NSEG, SEGLEN = Cfg::SEGLEN, IPT = Cfg::IPT, NPAIR = Cfg::NPAIR;
    constexpr int VQ = Cfg::VQ;

    T *sQd = reinterpret_cast<T *>(smem + Cfg::OFF_QD);
    T *sKd = reinterpret_cast<T *>(smem + Cfg::OFF_KD);
    T *sKt = reinterpret_cast<T *>(smem + Cfg::OFF_KT);
    T *sP = reinterpret_cast<T *>(smem + Cfg::OFF_P);
    T *sT = reinterpret_cast<T *>(smem + Cfg::OFF_T);
    float *sL = reinterpret_cast<float *>(smem + Cfg::OFF_L);
    T *sO = reinterpret_cast<T *>(smem + Cfg::OFF_O);
    T *sQG = reinterpret_cast<T *>(smem + Cfg::OFF_QG);
    T *sKG = reinterpret_cast<T *>(smem + Cfg::OFF_KG);
    T *sKhT = reinterpret_cast<T *>(smem + Cfg::OFF_KHT);
    T *sVbT = reinterpret_cast<T *>(smem + Cfg::OFF_VBT);
    float *sGC = reinterpret_cast<float *>(smem + Cfg::OFF_GC);
    float *sF = reinterpret_cast<float *>(smem + Cfg::OFF_F);
    float *sE = reinterpret_cast<float *>(smem + Cfg::OFF_E);
    float *sBeta = reinterpret_cast<float *>(smem + Cfg::OFF_BETA);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int g = lane >> 4, n = lane & 15;

    // Workgroup -> (b, h, value-column slice); the slices of one head share
    // an XCD (and its L2), which dedupes their reads of q, k, z.
    const int64_t H = prm.H;
    const BlockMap bm = block_map(blk, nblk, prm.nsplit, H, prm.order);
    const int64_t b = bm.b;
    const int split = bm.split;
    const int64_t bh = b * H + bm.h;
    const SeqRange sr = seq_range(prm.cu, b, prm.T);
    const int64_t Tn = sr.len;
    const int h = (int)(bh % H);
    const int j0 = split * DVB;         // first value column of the workgroup
    const int jw = j0 + 16 * wave;      // first value column of this wave

    const T *gq = static_cast<const T *>(prm.q);
    const T *gk = static_cast<const T *>(prm.k);
    const T *gz = static_cast<const T *>(prm.z);
    const T *gv = static_cast<const T *>(prm.v);
    const T *gbeta = static_cast<const T *>(prm.beta);
    T *go = static_cast<T *>(prm.o);
    const int64_t tok_stride = H * D;               // elements between tokens
    const int64_t base = (sr.start * H + h) * D;     // token 0 of (b, h)
    const int64_t bbase = sr.start * H + h;          // beta of token 0
    const float c2 = -__builtin_amdgcn_exp2f(prm.A[h] * kLog2e) * kLog2e;

    // ---- state slice: S[16 i + 4 g + e][jw + n] -------------------------
    // Modes 1 and 3 write final states only.  They still form the output
    // tiles and skip only the global stores: branching around the output
    // products, or fixing the mode at compile time, costs the plain prefill
    // 2-40% through a worse register allocation at 8 waves.
    const bool want_o = prm.mode == 0;
    const bool vzero = prm.mode == 3;    // the map M: v read as zero
    f32x4 S[NDT];
    if (prm.mode == 3) {   // the identity
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][e] = 16 * i + 4 * g + e == jw + n ? 1.0f : 0.0f;
    } else if (prm.S0) {
        const float *s0 = prm.S0 + bh * (int64_t)(D * D);
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][e] = s0[(16 * i + 4 * g + e) * D + jw + n];
    } else {
#pragma unroll
        for (int i = 0; i < NDT; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- prefetch registers --------------------------------------------
    // gate item it = tid + NT*ii: channel pair cp, segment sg of sub-tile sp
    Pair rq[IPT][SEGLEN], rk[IPT][SEGLEN], rz[IPT][SEGLEN];
    T rb[IPT][SEGLEN];   // raw beta bits; converted where used
    typedef typename std::conditional<sizeof(T) == 2, uint2, uint4>::type Quad;
    Quad rv[VQ];

    // Loads are branch-free: tokens past the end read the last token (Tn >= 1
    // whenever a chunk is loaded) and are masked where they are used, so the
    // compiler keeps every prefetch in flight instead of waiting on each one.
    auto load_chunk = [&](int64_t t0) {
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int it = tid + NT * ii;
            const int cp = it % NPAIR, rest = it / NPAIR;
            const int sg = rest % NSEG, sp = rest / NSEG;
#pragma unroll
            for (int s = 0; s < SEGLEN; ++s) {
                const int r = 16 * sp + sg * SEGLEN + s;
                const int64_t t = t0 + r < Tn ? t0 + r : Tn - 1;
                const int64_t off = base + t * tok_stride + 2 * cp;
                rq[ii][s] = *reinterpret_cast<const Pair *>(gq + off);
                rk[ii][s] = *reinterpret_cast<const Pair *>(gk + off);
                rz[ii][s] = *reinterpret_cast<const Pair *>(gz + off);
                rb[ii][s] = gbeta[bbase + t * H];
            }
        }
#pragma unroll
        for (int vi = 0; vi < VQ; ++vi) {
            int r, cq;
            v_item<C, DVB, NT>(tid, vi, r, cq);
            const int64_t t = t0 + r < Tn ? t0 + r : Tn - 1;
            rv[vi] = *reinterpret_cast<const Quad *>(gv + base + t * tok_stride + j0 + 4 * cq);
        }
    };

    const int64_t nchunks = (Tn + C - 1) / C;
    // Wide workgroups prefetch the next chunk into registers during the
    // current one.  With one or two waves each thread owns so many gate items
    // that the prefetch would not fit the register file; those variants load
    // each chunk at the top of its step instead.
    constexpr bool kPrefetch = NW >= 4;
    if (kPrefetch && nchunks > 0) load_chunk(0);

    // state checkpoints: the state after every ckpt_every tokens
    const int every = CKPT ? prm.ckpt_every : 0;   // CKPT: prm.ckpt set, every > 0
    int64_t ck_row = every > 0 ? ckpt_row0(prm.cu, b, prm.T, every) : 0;
    int64_t ck_next = every;   // token count of the next checkpoint
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = ch * C;
        if (!kPrefetch) load_chunk(t0);

        // ================= phase A: gate, decay factors, operands ==========
        float fl0[IPT][SEGLEN], fl1[IPT][SEGLEN], al0[IPT][SEGLEN], al1[IPT][SEGLEN];
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int it = tid + NT * ii;
            const int cp = it % NPAIR, rest = it / NPAIR;
            const int sg = rest % NSEG, sp = rest / NSEG;
            float run0 = 1.0f, run1 = 1.0f;
#pragma unroll
            for (int s = 0; s < SEGLEN; ++s) {
                const int r = 16 * sp + sg * SEGLEN + s;
                float z0, z1;
                unpack2(rz[ii][s], z0, z1);
                const bool valid = t0 + r < Tn;
                const float a0 = valid ? kda_alpha(c2, z0) : 1.0f;
                const float a1 = valid ? kda_alpha(c2, z1) : 1.0f;
                run0 *= a0;
                run1 *= a1;
                fl0[ii][s] = run0;
                fl1[ii][s] = run1;
                al0[ii][s] = a0;
                al1[ii][s] = a1;
            }
            sE[(sp * NSEG + sg) * D + 2 * cp] = run0;
            sE[(sp * NSEG + sg) * D + 2 * cp + 1] = run1;
            if (cp == 0) {
#pragma unroll
                for (int s = 0; s < SEGLEN; ++s) {
                    const int r = 16 * sp + sg * SEGLEN + s;
                    sBeta[r] = t0 + r < Tn ? to_f32(rb[ii][s]) : 0.0f;
                }
            }
        }
        lds_barrier();

#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int it = tid + NT * ii;
            const int cp = it % NPAIR, rest = it / NPAIR;
            const int sg = rest % NSEG, sp = rest / NSEG;
            const int d0 = 2 * cp;
            // products of the segment decays: within this sub-tile before /
            // after this segment, and whole sub-tiles before / after it
            float bef0 = 1.f, bef1 = 1.f, aft0 = 1.f, aft1 = 1.f;
            float pre0 = 1.f, pre1 = 1.f, post0 = 1.f, post1 = 1.f;
            float tot[NP][2];
#pragma unroll
            for (int p2 = 0; p2 < NP; ++p2) {
                float t0v = 1.f, t1v = 1.f;
#pragma unroll
                for (int s2 = 0; s2 < NSEG; ++s2) {
                    const float e0 = sE[(p2 * NSEG + s2) * D + d0];
                    const float e1 = sE[(p2 * NSEG + s2) * D + d0 + 1];
                    t0v *= e0;
                    t1v *= e1;
                    if (p2 == sp && s2 < sg) { bef0 *= e0; bef1 *= e1; }
                    if (p2 == sp && s2 > sg) { aft0 *= e0; aft1 *= e1; }
                }
                tot[p2][0] = t0v;
                tot[p2][1] = t1v;
                if (p2 < sp) { pre0 *= t0v; pre1 *= t1v; }
                if (p2 > sp) { post0 *= t0v; post1 *= t1v; }
            }
            const float itot0 = __builtin_amdgcn_rcpf(tot[sp][0]);
            const float itot1 = __builtin_amdgcn_rcpf(tot[sp][1]);
            float rl0 = aft0, rl1 = aft1;   // decay over (r, end of sub-tile]
            // bf16 with whole 8-token groups: the transposed rows d0, d0+1 of
            // Kh are packed in registers and written 8 tokens at a time (two
            // 8-byte stores per row instead of eight 2-byte ones, whose rows
            // 2*cp fell into the same few LDS banks)
            constexpr bool kPackT = sizeof(T) == 2 && SEGLEN % 8 == 0;
            uint32_t ph0[4], ph1[4];
            float nh0 = 0.f, nh1 = 0.f;   // token s+1's values
#pragma unroll
            for (int s = SEGLEN - 1; s >= 0; --s) {
                const int r = 16 * sp + sg * SEGLEN + s;
                float q0, q1, k0, k1;
                unpack2(rq[ii][s], q0, q1);
                unpack2(rk[ii][s], k0, k1);
                const bool valid = t0 + r < Tn;   // padded tokens: q = k = beta = 0
                q0 = valid ? q0 : 0.0f;
                q1 = valid ? q1 : 0.0f;
                k0 = valid ? k0 : 0.0f;
                k1 = valid ? k1 : 0.0f;
                const float F0 = bef0 * fl0[ii][s], F1 = bef1 * fl1[ii][s];  // e^{G_r - start}
                const float bt = valid ? to_f32(rb[ii][s]) : 0.0f;
                store_pair(sQd + r * DP + d0, q0 * F0 * itot0, q1 * F1 * itot1);
                store_pair(sKd + r * DP + d0, k0 * F0 * itot0, k1 * F1 * itot1);
                store_pair(sKt + r * DP + d0, k0 * rl0, k1 * rl1);
                store_pair(sQG + r * DP + d0, q0 * F0 * pre0, q1 * F1 * pre1);
                store_pair(sKG + r * DP + d0, bt * k0 * F0 * pre0, bt * k1 * F1 * pre1);
                const float h0 = k0 * rl0 * post0, h1 = k1 * rl1 * post1;
                if constexpr (kPackT) {
                    if (s % 2 == 0) {
                        ph0[(s / 2) % 4] = pack_pair_bf16(h0, nh0);
                        ph1[(s / 2) % 4] = pack_pair_bf16(h1, nh1);
                    }
                    if (s % 8 == 0) {   // tokens r .. r+7 complete
                        *reinterpret_cast<uint2 *>(sKhT + d0 * CP + r) = uint2{ph0[0], ph0[1]};
                        *reinterpret_cast<uint2 *>(sKhT + d0 * CP + r + 4) = uint2{ph0[2], ph0[3]};
                        *reinterpret_cast<uint2 *>(sKhT + (d0 + 1) * CP + r) = uint2{ph1[0], ph1[1]};
                        *reinterpret_cast<uint2 *>(sKhT + (d0 + 1) * CP + r + 4) = uint2{ph1[2], ph1[3]};
                    }
                    nh0 = h0;
                    nh1 = h1;
                } else {
                    sKhT[d0 * CP + r] = from_f32<T>(h0);
                    sKhT[(d0 + 1) * CP + r] = from_f32<T>(h1);
                }
                rl0 *= al0[ii][s];
                rl1 *= al1[ii][s];
            }
            if (sp == 0 && sg == 0) {
                float gc0 = 1.f, gc1 = 1.f;
#pragma unroll
                for (int p2 = 0; p2 < NP; ++p2) { gc0 *= tot[p2][0]; gc1 *= tot[p2][1]; }
                sGC[d0] = gc0;
                sGC[d0 + 1] = gc1;
#pragma unroll
                for (int p2 = 1; p2 < NP; ++p2) {
#pragma unroll
                    for (int pq = 0; pq < p2; ++pq) {
                        float f0 = 1.f, f1 = 1.f;
#pragma unroll
                        for (int x2 = pq + 1; x2 <= p2; ++x2) { f0 *= tot[x2][0]; f1 *= tot[x2][1]; }
                        sF[off_index(p2, pq) * D + d0] = f0;
                        sF[off_index(p2, pq) * D + d0 + 1] = f1;
                    }
                }
            }
        }
        // beta * v, transposed to [column][token]
#pragma unroll
        for (int vi = 0; vi < VQ; ++vi) {
            int r, cq;
            v_item<C, DVB, NT>(tid, vi, r, cq);
            const float bt = sBeta[r];
            float vv[4];
            if constexpr (sizeof(T) == 2) {
                unpack2(rv[vi].x, vv[0], vv[1]);
                unpack2(rv[vi].y, vv[2], vv[3]);
            } else {
                vv[0] = __uint_as_float(rv[vi].x);
                vv[1] = __uint_as_float(rv[vi].y);
                vv[2] = __uint_as_float(rv[vi].z);
                vv[3] = __uint_as_float(rv[vi].w);
            }
            const bool valid = t0 + r < Tn;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sVbT[(4 * cq + e) * CP + r] = from_f32<T>(valid && !vzero ? bt * vv[e] : 0.0f);
        }
        lds_barrier();

        // prefetch the next chunk while this one is processed
        if (kPrefetch && ch + 1 < nchunks) load_chunk(t0 + C);

        // ================= phase B: P and L sub-tile blocks ================
        // Block (p, pq) of P and of L on one wave: they share the column-side
        // fragments (scaled by F_{p,pq} off the diagonal); the contraction
        // over the D channels runs on 16x16x32 MFMAs.
        f32x4 accP[Cfg::BPW], accL[Cfg::BPW];
#pragma unroll
        for (int bi = 0; bi < Cfg::BPW; ++bi) {
            const int blk = wave + NW * bi;
            accP[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
            accL[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (blk < Cfg::NB) {
                // blk -> (p, pq), pq <= p, row-major over the lower triangle
                int p = 0;
                while ((p + 1) * (p + 2) / 2 <= blk) ++p;
                const int pq = blk - p * (p + 1) / 2;
                const T *Aq = sQd + 16 * p * DP;
                const T *Ak = sKd + 16 * p * DP;
                const T *Bk = sKt + 16 * pq * DP;
                const float *Fs = pq < p ? sF + off_index(p, pq) * D : nullptr;
                auto bfrag = [&](int kk) {
                    Frag<T> bf = lds_frag(Bk, DP, kk, lane);
                    if (Fs) bf = frag_scaled(bf, *reinterpret_cast<const f32x4 *>(Fs + kk + 4 * g));
                    return bf;
                };
                if constexpr (D % 32 == 0) {
#pragma unroll
                    for (int kk = 0; kk < D; kk += 32) {
                        const Frag<T> b0 = bfrag(kk), b1 = bfrag(kk + 16);
                        mma32(accP[bi], lds_frag(Aq, DP, kk, lane), lds_frag(Aq, DP, kk + 16, lane), b0, b1);
                        mma32(accL[bi], lds_frag(Ak, DP, kk, lane), lds_frag(Ak, DP, kk + 16, lane), b0, b1);
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < D; kk += 16) {
                        const Frag<T> bf = bfrag(kk);
                        mma16(accP[bi], lds_frag(Aq, DP, kk, lane), bf);
                        mma16(accL[bi], lds_frag(Ak, DP, kk, lane), bf);
                    }
                }
            }
        }
        lds_barrier();   // region X switches from Qd/Kd/Kt to P/T/L
#pragma unroll
        for (int bi = 0; bi < Cfg::BPW; ++bi) {
            const int blk = wave + NW * bi;
            if (blk < Cfg::NB) {
                int p = 0;
                while ((p + 1) * (p + 2) / 2 <= blk) ++p;
                const int pq = blk - p * (p + 1) / 2;
                // beta of rows 4g..4g+3, read once and unconditionally: a read
                // under the strict-lower mask made every store wait on it
                const f32x4 bt4 = *reinterpret_cast<const f32x4 *>(sBeta + 16 * p + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * p + 4 * g + e, s = 16 * pq + n;
                    const bool lower = pq < p || s <= r;
                    const bool strict = pq < p || s < r;
                    sP[r * CP + s] = from_f32<T>(lower ? accP[bi][e] : 0.0f);
                    sL[r * LP + s] = strict ? bt4[e] * accL[bi][e] : 0.0f;
                }
            }
        }
        lds_barrier();

        // ================= phase C: 16 x 16 diagonal inverses ==============
        // T_pp = (I + L_pp)^-1 by L's nilpotency (L_pp^16 = 0):
        //    T = (I - L)(I + L^2)(I + L^4)(I + L^8),
        // nine 16 x 16 MFMA products; wave p % NW takes block p.  An
        // accumulator tile (lane (g, n) holding X[4g+e][n]) is the B operand
        // of X and the A operand of X^T, so each product is formed together
        // with the transpose the next one needs.
        for (int p = wave; p < NP; p += NW) {
            const float *Lp = sL + 16 * p * LP + 16 * p;
            f32x4 Lb, LTb, ImLT;   // L (B layout), L^T (B layout), I - L^T
            LTb = *reinterpret_cast<const f32x4 *>(Lp + n * LP + 4 * g);   // L[n][4g+e]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Lb[e] = Lp[(4 * g + e) * LP + n];                             // L[4g+e][n]
                ImLT[e] = (4 * g + e == n ? 1.0f : 0.0f) - LTb[e];
            }
            auto mm = [](const Frag<T> &a, const Frag<T> &b) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
                mma16(d, a, b);
                return d;
            };
            auto plus_i = [&](f32x4 x) {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] += (4 * g + e == n) ? 1.0f : 0.0f;
                return x;
            };
            auto fr = [](const f32x4 &x) { return acc_frag<T>(x); };
            const Frag<T> fL = fr(Lb), fLT = fr(LTb);
            const f32x4 L2 = mm(fLT, fL), L2T = mm(fL, fLT);           // L^2, (L^2)^T
            const Frag<T> fL2 = fr(L2), fL2T = fr(L2T);
            const f32x4 L4 = mm(fL2T, fL2), L4T = mm(fL2, fL2T);       // L^4, (L^4)^T
            const Frag<T> fL4 = fr(L4), fL4T = fr(L4T);
            const f32x4 L8 = mm(fL4T, fL4);                            // L^8
            const f32x4 Y = mm(fr(plus_i(L4T)), fr(plus_i(L8)));       // (I+L^4)(I+L^8)
            const f32x4 XT = mm(fr(plus_i(L2)), fr(ImLT));             // (I+L^2)^T (I-L)^T
            const f32x4 TT = mm(fr(Y), fr(XT));                        // T^T = Y^T X^T
            // lane (g, n) holds T[n][4g+e]: row n, four consecutive columns
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sT[(16 * p + n) * CP + 16 * p + 4 * g + e] = from_f32<T>(TT[e]);
        }
        lds_barrier();

        // ================= phase D: off-diagonal blocks of T ================
        // T = (I + L)^-1 is block lower triangular; with its diagonal blocks
        // from phase C, block row p follows from the rows above:
        //    T_pj = -T_pp sum_{j <= m < p} L_pm T_mj     (j < p).
        // One wave forms the NP(NP-1)/2 blocks in order, keeping them in
        // accumulator layout (the B operand of the next products), and writes
        // them into sT for the chain.
        if constexpr (NP > 1) {
            if (wave == 0) {
                f32x4 Tblk[NP][NP];   // T_mj, m > j, accumulator layout
#pragma unroll
                for (int p = 1; p < NP; ++p) {
                    const Frag<T> Tpp = lds_frag(sT + 16 * p * CP, CP, 16 * p, lane);
#pragma unroll
                    for (int j = 0; j < p; ++j) {
                        f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int m = j; m < p; ++m) {
                            // L_pm in A layout: L[16p + n][16m + 4g + e]
                            const f32x4 lf = *reinterpret_cast<const f32x4 *>(
                                sL + (16 * p + n) * LP + 16 * m + 4 * g);
                            Frag<T> tb;   // T_mj in B layout: T[16m + 4g + e][16j + n]
                            if (m == j) {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    tb.v[e] = sT[(16 * m + 4 * g + e) * CP + 16 * j + n];
                            } else {
                                tb = acc_frag<T>(Tblk[m][j]);
                            }
                            mma16(X, frag_from_f32<T>(lf), tb);
                        }
                        f32x4 R = {0.f, 0.f, 0.f, 0.f};
                        mma16(R, Tpp, acc_frag<T>(X));
                        Tblk[p][j] = -R;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sT[(16 * p + 4 * g + e) * CP + 16 * j + n] = from_f32<T>(-R[e]);
                    }
                }
            }
            lds_barrier();
        }

        // ================= phase E: the state chain (per wave) =============
        {
            Frag<T> Sf[NDT];
#pragma unroll
            for (int i = 0; i < NDT; ++i) Sf[i] = acc_frag<T>(S[i]);
            // A product of one MFMA shape never accumulates directly onto the
            // result of the other shape: a 16x16x16 product issued shortly
            // after a 16x16x32 product writing its accumulator returned wrong
            // values on MI355X (the compiler inserts no wait states between
            // the two shapes), so mixed-shape sums go through separate
            // accumulators and a VALU add.
            // U = T (beta V - beta K e^G S): Y rounded once, then the block
            // lower-triangular product with T
            f32x4 U[NP], O[NP];
            Frag<T> Yf[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                f32x4 X = {0.f, 0.f, 0.f, 0.f};
                contract_lds_frag<T, D>(X, sKG + 16 * p * DP, DP, Sf, lane);
                // beta V[16p + 4g + e][jw + n]
                const Frag<T> vb = lds_frag(sVbT + 16 * wave * CP, CP, 16 * p, lane);
                f32x4 Y;
#pragma unroll
                for (int e = 0; e < 4; ++e) Y[e] = to_f32(vb.v[e]) - X[e];
                Yf[p] = acc_frag<T>(Y);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                U[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j <= p; ++j)
                    mma16(U[p], lds_frag(sT + 16 * p * CP, CP, 16 * j, lane), Yf[j]);
            }
            Frag<T> Uf[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) Uf[p] = acc_frag<T>(U[p]);
            // O = (Q e^G) S + P U, from the entering state's bf16 image Sf
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                O[p] = f32x4{0.f, 0.f, 0.f, 0.f};
                contract_lds_frag<T, D>(O[p], sQG + 16 * p * DP, DP, Sf, lane);
                f32x4 Opu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j <= p; ++j)
                    mma16(Opu, lds_frag(sP + 16 * p * CP, CP, 16 * j, lane), Uf[j]);
                O[p] += Opu;
            }
            // S <- e^{G_C} * S + Kh^T U
#pragma unroll
            for (int i = 0; i < NDT; ++i) {
                const f32x4 gc = *reinterpret_cast<const f32x4 *>(sGC + 16 * i + 4 * g);
                S[i] *= gc;
#pragma unroll
                for (int j = 0; j < NP; ++j)
                    mma16(S[i], lds_frag(sKhT + 16 * i * CP, CP, 16 * j, lane), Uf[j]);
            }
            // stage O for coalesced stores
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sO[(16 * p + 4 * g + e) * OP + 16 * wave + n] = from_f32<T>(O[p][e]);
        }
        lds_barrier();
        if (want_o) {
            constexpr int E16 = 16 / (int)sizeof(T);
            constexpr int CPR = DVB / E16;          // 16-byte pieces per row
            const int64_t nvalid = Tn - t0 < C ? Tn - t0 : C;
            for (int idx = tid; idx < C * CPR; idx += NT) {
                const int r = idx / CPR, c = idx % CPR;
                if (r < nvalid) {
                    const uint4 val = *reinterpret_cast<const uint4 *>(sO + r * OP + c * E16);
                    *reinterpret_cast<uint4 *>(go + base + (t0 + r) * tok_stride + j0 + c * E16) = val;
                }
            }
        }
        lds_barrier();
        // state checkpoint after this chunk (S is final for the chunk here)
        if (CKPT && t0 + C == ck_next) {
            if (t0 + C <= Tn && ck_row < prm.n_ckpt) {
                // one lane offset, row offsets as scalars: no per-store addresses
                const auto crs = make_rsrc(prm.ckpt + (ck_row * H + h) * (int64_t)(D * D),
                                           (int64_t)(D * D) * 4);
                const int voff = (4 * g * D + jw + n) * 4;
#pragma unroll
                for (int i = 0; i < NDT; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[i][e]), crs, voff,
                                                              (16 * i + e) * D * 4, 0);
            }
            ++ck_row;
            ck_next += every;
        }
    }

    // ---- final state ------------------------------------------------------
    float *sT_out = prm.S_T + bh * (int64_t)(D * D);
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sT_out[(16 * i + 4 * g + e) * D + jw + n] = S[i][e];
}

template <typename T, int D, int C, int NW, bool CKPT>
__global__ __launch_bounds__(64 * NW) void kda_prefill_kernel(PrefillParams prm) {
    __shared__ __attribute__((aligned(16))) char smem[PrefillCfg<T, D, C, NW>::LDS_BYTES];
    prefill_block<T, D, C, NW, CKPT>(prm, smem, blockIdx.x, gridDim.x);
}

// Three independent runs in one launch (the first pass of a sequence split):
// blocks [0, n0) run p0, [n0, n0 + n1) p1 and the rest p2, so that together
// they fill the chip.
template <typename T, int D, int C, int NW>
__global__ __launch_bounds__(64 * NW) void kda_prefill_multi_kernel(PrefillParams p0,
                                                                    PrefillParams p1,
                                                                    PrefillParams p2, int n0,
                                                                    int n1) {
    __shared__ __attribute__((aligned(16))) char smem[PrefillCfg<T, D, C, NW>::LDS_BYTES];
    const int x = blockIdx.x;
    if (x < n0)
        prefill_block<T, D, C, NW, false>(p0, smem, x, n0);
    else if (x < n0 + n1)
        prefill_block<T, D, C, NW, false>(p1, smem, x - n0, n1);
    else
        prefill_block<T, D, C, NW, false>(p2, smem, x - n0 - n1, (int)gridDim.x - n0 - n1);
}

// Longest-first ranking of packed sequences: sequence j gets the rank
// #{i : L_i > L_j, or L_i == L_j and i < j}, and order[rank] = j.  One thread
// per sequence, O(N) each; lengths are the clamped ranges the prefill uses.
__global__ __launch_bounds__(256) void kda_seq_order_kernel(const int64_t *cu, int64_t N,
                                                            int64_t T, int32_t *order) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= N) return;
    const int64_t Lj = seq_range(cu, j, T).len;
    int64_t rank = 0;
    for (int64_t i = 0; i < N; ++i) {
        const int64_t Li = seq_range(cu, i, T).len;
        rank += (Li > Lj || (Li == Lj && i < j)) ? 1 : 0;
    }
    order[rank] = (int32_t)j;
}

// ---------------------------------------------------------------- host ----

bool prefill_ckpt_supported(int dtype, int64_t D, int chunk, int dv_per_block) {
    (void)dtype; (void)D; (void)chunk; (void)dv_per_block;
    return true;
}

template <int D, int NW>
static PrefillParams prefill_params(const PrefillArgs &a) {
    PrefillParams prm;
    prm.q = a.q; prm.k = a.k; prm.v = a.v; prm.z = a.z; prm.beta = a.beta;
    prm.A = a.A; prm.S0 = a.S0; prm.o = a.o; prm.S_T = a.S_T;
    prm.T = a.T; prm.H = a.H;
    prm.cu = a.cu_seqlens; prm.order = a.order; prm.ckpt = a.ckpt; prm.n_ckpt = a.n_ckpt;
    prm.ckpt_every = a.ckpt_every;
    prm.nsplit = (int)(D / (16 * NW));
    prm.mode = a.mode;
    return prm;
}

template <typename T, int D, int C, int NW>
static hipError_t launch_prefill_t(const PrefillArgs &a) {
    const PrefillParams prm = prefill_params<D, NW>(a);
    const int64_t nblk = a.B * a.H * prm.nsplit;
    if (a.ckpt != nullptr && a.ckpt_every > 0)
        hipLaunchKernelGGL((kda_prefill_kernel<T, D, C, NW, true>), dim3((unsigned)nblk),
                           dim3(64 * NW), 0, a.stream, prm);
    else
        hipLaunchKernelGGL((kda_prefill_kernel<T, D, C, NW, false>), dim3((unsigned)nblk),
                           dim3(64 * NW), 0, a.stream, prm);
    return hipGetLastError();
}

#define KDA_PREFILL_CASES(X)                                                             \
    X(bf16, 128, 16, 1) X(bf16, 128, 16, 2) X(bf16, 128, 16, 4) X(bf16, 128, 16, 8)        \
    X(bf16, 128, 64, 2) X(bf16, 128, 64, 4) X(bf16, 128, 64, 8)                            \
    X(bf16, 16, 16, 1) X(bf16, 16, 64, 1)                                                  \
    X(float, 128, 16, 1) X(float, 128, 16, 2) X(float, 128, 16, 4)                         \
    X(float, 16, 16, 1) X(float, 16, 64, 1)

template <typename T> constexpr int dtype_code();
template <> constexpr int dtype_code<bf16>() { return 1; }
template <> constexpr int dtype_code<float>() { return 0; }

bool prefill_supported(int dtype, int64_t D, int chunk, int dv_per_block) {
#define X(T_, D_, C_, NW_)                                                               \
    if (dtype == dtype_code<T_>() && D == D_ && chunk == C_ && dv_per_block == 16 * NW_)  \
        return true;
    KDA_PREFILL_CASES(X)
#undef X
    return false;
}

int prefill_default_dv_per_block(int dtype, int64_t B, int64_t H, int64_t D, int chunk) {
    (void)B; (void)H;
    if (D == 16) return 16;
    // bf16 at 64-token chunks: one 8-wave workgroup per head (two waves per
    // SIMD, and the key-side work of a chunk is done once per head)
    if (dtype == dtype_code<bf16>() && D == 128 && chunk == 64) return 128;
    return 64;
}

hipError_t launch_seq_order(const int64_t *cu, int64_t N, int64_t T, int32_t *order,
                            hipStream_t stream) {
    const unsigned nb = (unsigned)((N + 255) / 256);
    hipLaunchKernelGGL(kda_seq_order_kernel, dim3(nb), dim3(256), 0, stream, cu, N, T, order);
    return hipGetLastError();
}

// bf16, d = 128, 64-token chunks, 128 columns per workgroup: runs a[0..3)
// (modes 0, 1 or 3, no checkpoints) in one launch.
hipError_t launch_prefill_multi(const PrefillArgs *a) {
    for (int i = 0; i < 3; ++i)
        if (a[i].dtype != dtype_code<bf16>() || a[i].D != 128 || a[i].chunk != 64 ||
            a[i].dv_per_block != 128 || a[i].ckpt != nullptr || a[i].H != a[0].H ||
            (a[i].mode != 0 && a[i].mode != 1 && a[i].mode != 3))
            return hipErrorInvalidValue;
    const int64_t n0 = a[0].B * a[0].H, n1 = a[1].B * a[1].H, n2 = a[2].B * a[2].H;
    if (n0 + n1 + n2 == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_prefill_multi_kernel<bf16, 128, 64, 8>), dim3((unsigned)(n0 + n1 + n2)),
                       dim3(512), 0, a[0].stream, prefill_params<128, 8>(a[0]),
                       prefill_params<128, 8>(a[1]), prefill_params<128, 8>(a[2]), (int)n0, (int)n1);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a) {
#define X(T_, D_, C_, NW_)                                                               \
    if (a.dtype == dtype_code<T_>() && a.D == D_ && a.chunk == C_ &&                       \
        a.dv_per_block == 16 * NW_)                                                        \
        return launch_prefill_t<T_, D_, C_, NW_>(a);
    KDA_PREFILL_CASES(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace kda
