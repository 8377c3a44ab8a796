// kda_prefill16.hip -- chunkwise KDA prefill, 16-token chunks, bf16, d = 128,
// with role-split waves (gfx950).
//
// Same method and chunk algebra as kda_prefill.hip (the KDA recurrence and
// bounded gate of "Kimi K3 Open Weights: What Is Actually New", section 1,
// with the state carried sequentially from chunk to chunk and the tokens
// inside a 16-token chunk handled in parallel, as the kimi-k3-course
// capstone's one-page map describes), organised for overlap instead of
// lock-step phases:
//
//  * PREP waves (NPW per workgroup).  Prep wave w owns chunks w, w+NPW, ...
//    and does the S-independent work of a chunk by itself, with no workgroup
//    barrier: gate, decay factors, the P and L tiles and the 16 x 16
//    inverse T.  It writes the chain operands into an LDS slot (chunk m uses
//    slot m mod NSLOT).
//  * CHAIN waves (NCW per workgroup, 16 value columns each, fp32 state slice
//    in registers).  They consume the slots in chunk order and run the
//    S-dependent chain: S' = e^{G_C} S, U = T diag(beta) (V - K~ S'),
//    O = Q~ S' + P U, S <- S' + Kh^T U.  Each chain wave reads its own 16
//    columns of V (staged by the prep) as an MFMA fragment.
//  Slot hand-off uses LDS counters: `ready[slot]` (stored by the prep wave
//  as u+1 once the slot holds its u-th chunk) and `done[slot][chain wave]`
//  (stored by each chain wave as u+1 once it has issued every read of the
//  slot's u-th use; a wave's LDS operations execute in order, so a later
//  write by a prep wave cannot overtake them).  A prep wave waits until every
//  chain wave's count for the slot is >= u before writing its u-th use; chain
//  waves wait for ready >= u+1.  Production of chunk m only depends on
//  consumption of chunk m - NSLOT, so the hand-off cannot deadlock; every
//  wait is additionally bounded.  Each SIMD hosts one chain wave and two prep
//  waves, whose work overlaps.
//
// With one chunk per 16-token sub-tile, every decay factor can be referred to
// the chunk end: with G_r = sum_{s<=r} g_s and G_C the chunk total,
//    Q~ = Q * e^{G - G_C}   (row operand of P; the read O = Q~ (e^{G_C} S))
//    K~ = K * e^{G - G_C}   (row operand of L, and of the chain's K~ S')
//    Kh = K * e^{G_C - G}   (column operand of P and L; the state update)
// so P = tril(Q~ Kh^T), L = diag(beta) strict_tril(K~ Kh^T).  Over at most 15
// later tokens of a chunk, 1 <= e^{G - G_C} <= e^75 and e^{-75} <= e^{G_C - G}
// <= 1, inside bf16 range: the range argument of the pages.  Referring to
// the end (not the start) makes the factors of a chunk's last token 1 up to
// fp32 rounding, so after rounding to bf16 the diagonal entry q.k of P, which
// can cancel, is formed from the unscaled inputs for that token.
//
// The 16 x 16 inverse T = (I + L)^-1 uses L's nilpotency (L^16 = 0):
//    T = (I - L)(I + L^2)(I + L^4)(I + L^8),
// nine bf16 MFMAs kept in registers.  An MFMA result tile sits in B-operand
// layout (lane (g,n) holds rows 4g..4g+3 of column n), and the A-operand
// layout of M is the B-operand layout of M^T, so every product is formed
// together with the transposes the next one needs.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

struct Prefill16Params {
    const bf16 *q, *k, *v, *z, *beta;
    const float *A, *S0;
    bf16 *o;
    float *S_T;
    float *S_T2;         // MODE 2: final states of the value-carrying columns (N)
    int64_t T, H;   // T: tokens per sequence (dense) or in the packing (cu != NULL)
    int nsplit;
    const int64_t *cu;   // packed sequence offsets, or NULL
    const int32_t *order;   // longest-first sequence order, or NULL
    float *ckpt;         // state checkpoints [n_ckpt, H, D, D], or NULL
    int64_t n_ckpt;
    int ckpt_every;      // tokens between checkpoints (0: none)
    int ckpt_blocked;    // 1: bf16 checkpoints in 4-row blocks ((d/4)*D + j)*4 + d%4
    int spin_limit;      // sleeps before a slot wait gives up
};

template <int NCW, int NPW, int NSLOT>
struct P16Cfg {
    static constexpr int D = 128, C = 16;
    static constexpr int DVB = 16 * NCW;           // value columns per workgroup
    // Row strides, for LDS served as 32 four-byte banks to each group of 16
    // lanes.  A fragment read (16 rows, one 8-byte piece each) is
    // conflict-free when the stride is 2 mod 32 words (rows 2 banks apart).
    // Tiles that are also read by transposing reads (4 rows x 4 pieces) use a
    // stride of 8 mod 32 words and store 8-byte piece p of row r at piece
    // p ^ ((r >> 2) & 3) (swz_piece): the transposing read's 4 rows then fall
    // 8 banks apart with its 4 pieces in distinct banks, and the 16 rows of a
    // fragment read spread over 4 row strides x 4 piece positions.
    static constexpr int DP = D + 4;               // Q~ [token][d] row stride (66 words)
    static constexpr int CP = C + 4;               // [token][token] row stride (10 words)
    static constexpr int KP = D + 16;              // K~ and Kh row stride (72 words, swizzled)
    // slot: the chain operands of one chunk
    static constexpr int S_QG = 0;                         // Q~         [C][DP]
    static constexpr int S_KT = S_QG + C * DP * 2;         // K~         [C][KP], swizzled
    static constexpr int S_KH = S_KT + C * KP * 2;         // Kh         [C][KP], swizzled
    static constexpr int S_P = S_KH + C * KP * 2;          // P          [C][CP]
    static constexpr int S_TB = S_P + C * CP * 2;          // T diag(b)  [C][CP]
    static constexpr int S_GC = S_TB + C * CP * 2;         // e^{G_C}    [D] fp32, permuted
                                                           // (gc_word)
    static constexpr int VP = DVB + 16;                    // V row stride (transposing reads:
                                                           // the rows they touch in distinct banks)
    static constexpr int S_V = S_GC + D * 4;               // V, this workgroup's columns [C][VP]
    static constexpr int SLOT = S_V + C * VP * 2;
    // prep-wave scratch
    static constexpr int W_BETA = 0;                        // beta  [C] fp32
    static constexpr int SCR = (W_BETA + C * 4 + 15) / 16 * 16;
    static constexpr int OFF_FLAGS = 0;                     // ready[8], done[NSLOT][NCW], poison
    static constexpr int OFF_DONE = 32;
    static constexpr int OFF_POISON = OFF_DONE + NSLOT * NCW * 4;
    static constexpr int OFF_SLOTS = (OFF_POISON + 4 + 15) / 16 * 16;
    static constexpr int OFF_SCR = OFF_SLOTS + NSLOT * SLOT;
    static constexpr int LDS_BYTES = OFF_SCR + NPW * SCR;
    static_assert(NSLOT <= 8, "ready[] holds 8 slots");
    static_assert(NCW + NPW <= 16, "workgroup size");
    static_assert(SLOT % 16 == 0 && SCR % 16 == 0, "alignment");
    static_assert(LDS_BYTES <= 150 * 1024, "LDS budget");
};

// Swizzled 8-byte piece of row r of a [token][d] tile with a row stride of 8
// mod 32 words (see the row strides): piece p is stored at p ^ ((r >> 2) & 3).
__device__ __forceinline__ int swz_piece(int r, int p) { return p ^ ((r >> 2) & 3); }

// K16 fragment of a swizzled tile (row stride `ld` elements): rows lane % 16,
// contraction indices k0 + 4 (lane / 16) + 0..3, k0 a multiple of 32.
__device__ __forceinline__ Frag<bf16> frag_swz(const bf16 *tile, int ld, int k0, int lane) {
    const int r = lane & 15;
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x4 *>(tile + r * ld + k0 + 4 * swz_piece(r, lane >> 4));
    return f;
}

// Transposing read of a swizzled tile: the K16 fragment tile[4g + e][col0 + n]
// of frag_rows_tr, col0 a multiple of 16.  The 4 rows 4g .. 4g + 3 a lane
// group touches share (r >> 2) & 3 = g, so piece j % 4 of the group sits at
// (j % 4) ^ g.
__device__ __forceinline__ Frag<bf16> frag_rows_tr_swz(const bf16 *tile, int ld, int col0,
                                                       int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int g = lane >> 4, j = lane & 15;
    const bf16 *a = tile + (4 * g + (j >> 2)) * ld + col0 + 4 * ((j & 3) ^ g);
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(a));
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x4, r);
    return f;
}

// Word of the slot's e^{G_C} vector that holds key channel d.  A chain wave's
// lane (g, n) needs e^{G_C} of rows 16 i + 4 g + e of its state tiles; lane
// (g, n) reads the two words 32 g + 2 n, +1 (the 16 lanes of a group read 128
// contiguous bytes), and row i, element e of the group is then in lane
// 2 i + e / 2 of the group, word e % 2: broadcast within the 16-lane row.
__device__ __forceinline__ int gc_word(int d) { return 32 * ((d >> 2) & 3) + 4 * (d >> 4) + (d & 3); }

// Value of lane I of this lane's 16-lane row (DPP row broadcast).
template <int I>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x150 + I, 0xF, 0xF, true));
}

// Bounded LDS wait: true once *flag >= target (workgroup-scope acquire);
// false after `limit` sleeps without it.  A wave that gives up raises the
// workgroup's poison flag, and every state column it may have corrupted is
// then written as NaN (see the chain's final store), so a give-up can never
// pass for a valid result.
__device__ __forceinline__ bool wait_at_least(int *flag, int target, int limit, int *poison) {
    for (int it = 0;; ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target)
            return true;
        if (it >= limit) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(poison, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return false;
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return pack_bf16x2(a, b); }

// 16 values -> one [.][token] row of 16 bf16 (two 16-byte stores).
__device__ __forceinline__ void store_row16(bf16 *row, const float *x) {
    uint4 *r = reinterpret_cast<uint4 *>(row);
    r[0] = uint4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                 pack_bf16(x[6], x[7])};
    r[1] = uint4{pack_bf16(x[8], x[9]), pack_bf16(x[10], x[11]), pack_bf16(x[12], x[13]),
                 pack_bf16(x[14], x[15])};
}

// K16 fragment over rows 4*(lane/16) + e of column col0 + lane%16 of a
// row-major LDS tile, tile[4g + e][col0 + n], from one transposing 8-byte LDS
// read per lane (gfx950's ds_read_b64_tr_b16): within each 16-lane group the
// hardware hands lane i, element e, element i % 4 of the 8 bytes that lane
// 4e + i/4 addressed, so lane (g, j) addresses row 4g + j/4, columns
// col0 + 4(j%4) .. +3.  col0 and the row stride are multiples of 4.
__device__ __forceinline__ Frag<bf16> frag_rows_tr(const bf16 *tile, int ld, int col0, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const int g = lane >> 4, j = lane & 15;
    const bf16 *a = tile + (4 * g + (j >> 2)) * ld + col0 + 4 * (j & 3);
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(a));
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x4, r);
    return f;
}

// MODE 0: the prefill.  MODE 1: the final states only (no o).  MODE 2: a
// sequence's affine state map S_end = M S_start + N, for splitting one long
// sequence into segments that run in parallel: no o, and each chain wave
// carries two 16-column state slices on the same prep, columns jw.. of M
// (started from the identity with V taken as zero; written to S_T) and of N
// (the final state from S0, or from zero, with V; written to S_T2).
//
// The work of one workgroup (block `blk` of `nblk`), on the LDS block `smem`
// of P16Cfg::LDS_BYTES; the kernels below are its entry points.
template <int NCW, int NPW, int NSLOT, bool CKPT, int MODE>
__device__ __forceinline__ void prefill16_block(const Prefill16Params &prm, char *smem,
                                                int64_t blk, int64_t nblk) {
    using Cfg = P16Cfg<NCW, NPW, NSLOT>;
    constexpr int D = Cfg::D, C = Cfg::C, DVB = Cfg::DVB, DP = Cfg::DP, CP = Cfg::CP,
                  NDT = D / 16;
    int *ready = reinterpret_cast<int *>(smem + Cfg::OFF_FLAGS);
    int *done = reinterpret_cast<int *>(smem + Cfg::OFF_DONE);   // [slot][chain wave]
    int *poison = reinterpret_cast<int *>(smem + Cfg::OFF_POISON);
    const int spin = prm.spin_limit;

    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep it
    // (and every address derived from it) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;

    const int64_t H = prm.H;
    const BlockMap bm = block_map(blk, nblk, prm.nsplit, H, prm.order);
    const int64_t b = bm.b;
    const int h = bm.h;
    const int split = bm.split;
    const int64_t bh = b * H + h;
    const SeqRange sr = seq_range(prm.cu, b, prm.T);
    const int64_t Tn = sr.len;
    const int j0 = split * DVB;
    const int64_t tok_stride = H * D;
    const int64_t base = (sr.start * H + h) * D;   // token 0 of (b, h)
    const int64_t bbase = sr.start * H + h;
    const int64_t nchunks = (Tn + C - 1) / C;

    if (tid < Cfg::OFF_SLOTS / 4) ready[tid] = 0;   // every flag
    __syncthreads();

    if (wave < NCW) {
        // ============================ chain wave ============================
        const int jw = j0 + 16 * wave;
        // S: the state slice (MODE 2: of M, from the identity); S2: MODE 2's
        // value-carrying slice (of N)
        f32x4 S[NDT], S2[NDT];
        // state element (16 i + 4 g + e, jw + n) of a [D][D] matrix: one lane
        // offset, the row offsets as constants (no per-element addresses)
        const int svoff = (4 * g * D + jw + n) * 4;
        auto load_s0 = [&](f32x4 (&X)[NDT]) {
            if (prm.S0) {
                const auto srs = make_rsrc(prm.S0 + bh * (int64_t)(D * D), (int64_t)(D * D) * 4);
#pragma unroll
                for (int i = 0; i < NDT; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        X[i][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                            srs, svoff, (16 * i + e) * D * 4, 0));
            } else {
#pragma unroll
                for (int i = 0; i < NDT; ++i) X[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        if constexpr (MODE == 2) {
#pragma unroll
            for (int i = 0; i < NDT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i][e] = 16 * i + 4 * g + e == jw + n ? 1.f : 0.f;
            load_s0(S2);
        } else {
            load_s0(S);
        }
        const int64_t row_bytes = tok_stride * 2;
        auto chunk_rows = [&](int64_t t0) { return (Tn - t0 < C ? Tn - t0 : (int64_t)C); };
        // per-lane byte offsets of the fragment reads, fixed over chunks; a
        // chunk adds its slot's (uniform) byte offset once per tile layout
        const int offDP = ((lane & 15) * DP + 4 * (lane >> 4)) * 2;   // Q~ tile
        const int offKP = ((lane & 15) * Cfg::KP + 4 * swz_piece(lane & 15, lane >> 4)) * 2;
        const int offCP = ((lane & 15) * CP + 4 * (lane >> 4)) * 2;   // [.][CP] tiles
        const int offG = 4 * (32 * g + 2 * n);                         // e^{G_C} pair (gc_word)
        auto frag_at = [](const char *p) {
            Frag<bf16> f;
            f.v = *reinterpret_cast<const bf16x4 *>(p);
            return f;
        };
        // K~, T diag(beta), Kh^T and V fragments and the decay e^{G_C} of a chunk
        // (read one chunk ahead; Kh^T and V by transposing reads of token-major
        // tiles: V as V[t0 + 4g + e][jw + n], staged by the prep wave, zero past T)
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        Frag<bf16> Ktf[NDT], Kf[NDT], Tf, Vn;
        f32x2 gvn;
        bool waited_ok = true;   // every slot wait of this wave succeeded
        auto read_wtk = [&](int sl, int use) {
            waited_ok &= wait_at_least(&ready[sl], use + 1, spin, poison);
            const int off = Cfg::OFF_SLOTS + sl * Cfg::SLOT;
            const char *pk = smem + off + offKP;
            const char *pc = smem + off + offCP;
            gvn = *reinterpret_cast<const f32x2 *>(smem + off + Cfg::S_GC + offG);
#pragma unroll
            for (int i = 0; i < NDT; ++i) Ktf[i] = frag_at(pk + Cfg::S_KT + 32 * i);
            Tf = frag_at(pc + Cfg::S_TB);
            const bf16 *kh = reinterpret_cast<const bf16 *>(smem + off + Cfg::S_KH);
#pragma unroll
            for (int i = 0; i < NDT; ++i) Kf[i] = frag_rows_tr_swz(kh, Cfg::KP, 16 * i, lane);
            Vn = frag_rows_tr(reinterpret_cast<const bf16 *>(smem + off + Cfg::S_V), Cfg::VP,
                              16 * wave, lane);
        };
        // The output of chunk m, O = Q~ (e^{G_C} S) + P U, does not feed the
        // state, so it is software-pipelined: its products are issued at the
        // top of step m + 1, where they run on the matrix cores while that
        // step's decay is applied to S, and it is stored after the state update
        // of step m + 1.  Carried over: chunk m's S', U (bf16), Q~, P fragments.
        const int64_t row_stride_el = tok_stride;           // elements between token rows
        const bf16 *obase = prm.o + base + jw;              // token 0, this wave's columns
        const int ovoff = 4 * g * (int)row_bytes + 2 * n;   // lane offset of element e = 0
        Frag<bf16> Sp[NDT], Qp[NDT], Pp, Up;
        f32x4 Oa, Ob;
        auto out_issue = [&]() {
            Oa = f32x4{0.f, 0.f, 0.f, 0.f};
            Ob = f32x4{0.f, 0.f, 0.f, 0.f};
            mma32(Oa, Qp[0], Qp[1], Sp[0], Sp[1]);
            mma32(Ob, Qp[2], Qp[3], Sp[2], Sp[3]);
            mma32(Oa, Qp[4], Qp[5], Sp[4], Sp[5]);
            mma32(Ob, Qp[6], Qp[7], Sp[6], Sp[7]);
            mma16(Oa, Pp, Up);
        };
        auto out_store = [&](int64_t t0) {
            const f32x4 O = Oa + Ob;
            const auto ors = make_rsrc(obase + t0 * row_stride_el, chunk_rows(t0) * row_bytes);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (bf16)O[e]), ors,
                                                      ovoff, e * (int)row_bytes, 0);
        };
        // Loop bounds and the output pointer are wave-uniform: keep them in
        // scalar registers (readfirstlane) so the per-chunk bookkeeping is SALU
        // on constants, and run the chunks NSLOT at a time so that every slot
        // offset is a compile-time constant.
        const int nch = __builtin_amdgcn_readfirstlane((int)nchunks);
        if (nch > 0) read_wtk(0, 0);
        // state checkpoints: the state after every ckpt_every tokens
        const int every = CKPT ? prm.ckpt_every : 0;   // CKPT: prm.ckpt set, every > 0
        int64_t ck_row = every > 0 ? ckpt_row0(prm.cu, b, prm.T, every) : 0;
        int64_t ck_next = every;   // token count of the next checkpoint
        for (int m0 = 0, use = 0; m0 < nch; m0 += NSLOT, ++use) {
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) {
            const int m = m0 + sl;
            if (m >= nch) break;
            const int64_t t0 = (int64_t)m * C;
            const int off = Cfg::OFF_SLOTS + sl * Cfg::SLOT;
            const int sl1 = sl + 1 == NSLOT ? 0 : sl + 1;
            const int use1 = sl + 1 == NSLOT ? use + 1 : use;
            const char *pd = smem + off + offDP;
            const char *pc = smem + off + offCP;
            const f32x2 gv = gvn;
            const Frag<bf16> Vf = Vn;
            // (1) the previous chunk's output products (matrix cores), then
            // S <- e^{G_C} S and the products K~ S' of U = T diag(beta) (V - K~ S')
            // (two accumulators halve the dependent chain; the product with
            // T diag(beta), of the other MFMA shape, starts from zero: no MFMA
            // takes the fresh result of an MFMA of another shape as its
            // accumulator, which MI355X does not order)
            if constexpr (MODE == 0)
                if (m > 0) out_issue();
            __builtin_amdgcn_sched_barrier(0);
            f32x4 Ua = {0.f, 0.f, 0.f, 0.f}, Ub = {0.f, 0.f, 0.f, 0.f};
            Frag<bf16> Sf[NDT], Sf2[NDT];
            // X <- e^{G_C} X: row 16 i + 4 g + e scaled by lane 2 i + e/2's word e%2
#define KDA_DECAY_TILE(X, Xf, i)                                            \
            X[i][0] *= row_bcast<2 * (i)>(gv[0]);                           \
            X[i][1] *= row_bcast<2 * (i)>(gv[1]);                           \
            X[i][2] *= row_bcast<2 * (i) + 1>(gv[0]);                       \
            X[i][3] *= row_bcast<2 * (i) + 1>(gv[1]);                       \
            Xf[i] = acc_frag<bf16>(X[i]);
#define KDA_DECAY(X, Xf)                                                    \
            KDA_DECAY_TILE(X, Xf, 0) KDA_DECAY_TILE(X, Xf, 1)               \
            KDA_DECAY_TILE(X, Xf, 2) KDA_DECAY_TILE(X, Xf, 3)               \
            KDA_DECAY_TILE(X, Xf, 4) KDA_DECAY_TILE(X, Xf, 5)               \
            KDA_DECAY_TILE(X, Xf, 6) KDA_DECAY_TILE(X, Xf, 7)
            static_assert(NDT == 8, "decay broadcast covers 8 row tiles");
            KDA_DECAY(S, Sf)
            mma32(Ub, Ktf[0], Ktf[1], Sf[0], Sf[1]);
            mma32(Ua, Ktf[2], Ktf[3], Sf[2], Sf[3]);
            mma32(Ub, Ktf[4], Ktf[5], Sf[4], Sf[5]);
            mma32(Ua, Ktf[6], Ktf[7], Sf[6], Sf[7]);
            // MODE 2: the value-carrying slice, K~ S2' (its U2 takes V)
            f32x4 U2a = {0.f, 0.f, 0.f, 0.f}, U2b = {0.f, 0.f, 0.f, 0.f};
            if constexpr (MODE == 2) {
                KDA_DECAY(S2, Sf2)
                mma32(U2b, Ktf[0], Ktf[1], Sf2[0], Sf2[1]);
                mma32(U2a, Ktf[2], Ktf[3], Sf2[2], Sf2[3]);
                mma32(U2b, Ktf[4], Ktf[5], Sf2[4], Sf2[5]);
                mma32(U2a, Ktf[6], Ktf[7], Sf2[6], Sf2[7]);
            }
#undef KDA_DECAY
#undef KDA_DECAY_TILE
            // (2) this chunk's Q~ and P for its output (next step)
            compiler_fence();
            Frag<bf16> Qf[NDT], Pf;
            if constexpr (MODE == 0) {
#pragma unroll
                for (int i = 0; i < NDT; ++i) Qf[i] = frag_at(pd + Cfg::S_QG + 32 * i);
                Pf = frag_at(pc + Cfg::S_P);
            }
            // Every read of slot m has now been issued.  A wave's LDS operations
            // execute in order, so a prep wave that sees this count and then
            // writes the slot writes after these reads have executed: no wait
            // for the data to arrive is needed before releasing the slot.
            compiler_fence();
            __hip_atomic_store(&done[sl * NCW + wave], use + 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
            compiler_fence();
            // U = T diag(beta) (V - K~ S'): Y = V - K~ S' rounded once, then one
            // product with T diag(beta)
            Frag<bf16> Uf, Uf2;
            auto apply_t = [&](const f32x4 &X, bool with_v) {
                f32x4 Y;
#pragma unroll
                for (int e = 0; e < 4; ++e) Y[e] = (with_v ? (float)Vf.v[e] : 0.0f) - X[e];
                Frag<bf16> Yf;
                Yf.v = to_bf16x4(Y[0], Y[1], Y[2], Y[3]);
                f32x4 U = {0.f, 0.f, 0.f, 0.f};
                mma16(U, Tf, Yf);
                Frag<bf16> r;
                r.v = to_bf16x4(U[0], U[1], U[2], U[3]);
                return r;
            };
            if constexpr (MODE == 2) {
                Uf = apply_t(Ua + Ub, false);
                Uf2 = apply_t(U2a + U2b, true);
            } else {
                Uf = apply_t(Ua + Ub, true);
            }
            // (3) S <- S + Kh^T U
#pragma unroll
            for (int i = 0; i < NDT; ++i) mma16(S[i], Kf[i], Uf);
            if constexpr (MODE == 2)
#pragma unroll
                for (int i = 0; i < NDT; ++i) mma16(S2[i], Kf[i], Uf2);
            if (CKPT && t0 + C == ck_next) {
                if (t0 + C <= Tn && ck_row < prm.n_ckpt) {
                    // one lane offset, row offsets as scalars: no per-store addresses
                    const auto crs = make_rsrc(prm.ckpt + (ck_row * H + h) * (int64_t)(D * D),
                                               (int64_t)(D * D) * 4);
                    if (prm.ckpt_blocked) {
                        // bf16, rows 16i+4g .. 16i+4g+3 of column jw+n: one 8-byte group
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        const auto brs = make_rsrc(reinterpret_cast<bf16 *>(prm.ckpt) +
                                                       (ck_row * H + h) * (int64_t)(D * D),
                                                   (int64_t)(D * D) * 2);
                        const int voff = ((g * D + jw + n) * 4) * 2;
#pragma unroll
                        for (int i = 0; i < NDT; ++i)
                            __builtin_amdgcn_raw_buffer_store_b64(
                                u32x2{pack_bf16(S[i][0], S[i][1]), pack_bf16(S[i][2], S[i][3])},
                                brs, voff, i * 4 * D * 4 * 2, 0);
                    } else {
                        const int voff = (4 * g * D + jw + n) * 4;
#pragma unroll
                        for (int i = 0; i < NDT; ++i)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[i][e]), crs,
                                                                      voff, (16 * i + e) * D * 4, 0);
                    }
                }
                ++ck_row;
                ck_next += every;
            }
            __builtin_amdgcn_sched_barrier(0);
            // (4) the previous chunk's output, then chunk m+1's operands
            if constexpr (MODE == 0)
                if (m > 0) out_store(t0 - C);
            if (m + 1 < nch) read_wtk(sl1, use1);
            if constexpr (MODE == 0) {
#pragma unroll
                for (int i = 0; i < NDT; ++i) {
                    Sp[i] = Sf[i];
                    Qp[i] = Qf[i];
                }
                Pp = Pf;
                Up = Uf;
            }
        }
        }
        // the last chunk's output
        if constexpr (MODE == 0)
            if (nch > 0) {
                out_issue();
                out_store((int64_t)(nch - 1) * C);
            }
        // A prep wave that gave up a wait may have overwritten a slot this
        // wave was still reading: its poison store precedes a release of
        // `ready` that this wave has acquired since.  Another chain wave's
        // give-up corrupts only that wave's own columns.
        if (!waited_ok ||
            __hip_atomic_load(poison, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) {
            const float nan = __builtin_nanf("");
#pragma unroll
            for (int i = 0; i < NDT; ++i) S[i] = S2[i] = f32x4{nan, nan, nan, nan};
        }
        auto store_state = [&](float *dst, const f32x4 (&X)[NDT]) {
            const auto srs = make_rsrc(dst + bh * (int64_t)(D * D), (int64_t)(D * D) * 4);
#pragma unroll
            for (int i = 0; i < NDT; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(X[i][e]), srs, svoff,
                                                          (16 * i + e) * D * 4, 0);
        };
        store_state(prm.S_T, S);
        if constexpr (MODE == 2) store_state(prm.S_T2, S2);
        return;
    }

    // ============================== prep wave ===============================
    const int pw = wave - NCW;
    char *scr = smem + Cfg::OFF_SCR + pw * Cfg::SCR;
    float *sBeta = reinterpret_cast<float *>(scr + Cfg::W_BETA);

    const float c2 = -__builtin_amdgcn_exp2f(prm.A[h] * kLog2e) * kLog2e;
    const int d0 = 2 * lane;                           // this lane's channel pair

    uint32_t rq[C], rk[C], rz[C];
    short rb;   // lane s < 16: beta of token s
    // V of this workgroup's DVB columns: lane -> row lane / 4, columns
    // (lane % 4) * DVB/4 + 8u, u < DVB/32 (16-byte loads, zero past T)
    constexpr int VU = DVB / 32;
    const int vrow = lane >> 2, vcol = (lane & 3) * (DVB / 4);
    uint4 rvv[VU];
    const int64_t row_bytes = tok_stride * 2;
    auto load_chunk = [&](int64_t t0) {
        // one uniform buffer resource per tensor and chunk; rows past T read 0
        const int64_t rows = Tn - t0 < C ? Tn - t0 : (int64_t)C;
        const auto rq_ = make_rsrc(prm.q + base + t0 * tok_stride, rows * row_bytes);
        const auto rk_ = make_rsrc(prm.k + base + t0 * tok_stride, rows * row_bytes);
        const auto rz_ = make_rsrc(prm.z + base + t0 * tok_stride, rows * row_bytes);
        const auto rb_ = make_rsrc(prm.beta + bbase + t0 * H, rows * H * 2);
        rb = __builtin_amdgcn_raw_buffer_load_b16(rb_, (lane & 15) * (int)H * 2, 0, 0);
        {
            const auto rv_ = make_rsrc(prm.v + base + t0 * tok_stride, rows * row_bytes);
#pragma unroll
            for (int u = 0; u < VU; ++u) {
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(
                    rv_, vrow * (int)row_bytes + (j0 + vcol + 8 * u) * 2, 0, 0);
                rvv[u] = uint4{w[0], w[1], w[2], w[3]};
            }
        }
#pragma unroll
        for (int s = 0; s < C; ++s) {
            const int so = s * (int)row_bytes;
            rq[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rq_, 4 * lane, so, 0);
            rk[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rk_, 4 * lane, so, 0);
            rz[s] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rz_, 4 * lane, so, 0);
        }
    };
    if (pw < nchunks) load_chunk((int64_t)pw * C);

    for (int kk = 0;; ++kk) {
        const int64_t m = pw + (int64_t)NPW * kk;
        if (m >= nchunks) break;
        const int64_t t0 = m * C;
        const int s_ = (int)(m % NSLOT);
        const int use = (int)(m / NSLOT);
        char *slot = smem + Cfg::OFF_SLOTS + s_ * Cfg::SLOT;
        bf16 *sQG = reinterpret_cast<bf16 *>(slot + Cfg::S_QG);
        bf16 *sKt = reinterpret_cast<bf16 *>(slot + Cfg::S_KT);   // K~ token-major
        bf16 *sKh = reinterpret_cast<bf16 *>(slot + Cfg::S_KH);   // Kh token-major
        bf16 *sP = reinterpret_cast<bf16 *>(slot + Cfg::S_P);
        bf16 *sTb = reinterpret_cast<bf16 *>(slot + Cfg::S_TB);
        float *sGC = reinterpret_cast<float *>(slot + Cfg::S_GC);
        const bool full = t0 + C <= Tn;

        // decays, all 32 evaluations independent (no per-token branch, so
        // their transcendental latencies overlap); tokens past the end load
        // as 0 and are then given alpha = 1
        float a0[C], a1[C];
#pragma unroll
        for (int s = 0; s < C; ++s) {
            a0[s] = kda_alpha(c2, bf_lo(rz[s]));
            a1[s] = kda_alpha(c2, bf_hi(rz[s]));
        }
        if (!full) {
            const int nvalid = (int)(Tn - t0);
#pragma unroll
            for (int s = 0; s < C; ++s) {
                a0[s] = s < nvalid ? a0[s] : 1.0f;
                a1[s] = s < nvalid ? a1[s] : 1.0f;
            }
        }
        const float beta_l = __uint_as_float((uint32_t)(unsigned short)rb << 16);  // lane < 16

        // every chain wave has read the previous use of the slot
#pragma unroll
        for (int w = 0; w < NCW; ++w) wait_at_least(&done[s_ * NCW + w], use, spin, poison);

        {
            bf16 *sV = reinterpret_cast<bf16 *>(slot + Cfg::S_V);
#pragma unroll
            for (int u = 0; u < VU; ++u)
                *reinterpret_cast<uint4 *>(sV + vrow * Cfg::VP + vcol + 8 * u) = rvv[u];
        }
        // ---- decay factors and operands (lane = channel pair d0, d0+1) ------
        // Backward over the chunk: R = decay over (s, end of chunk], so that
        // Kh = K e^{G_C - G} (<= 1), written token-major into the slot (for P
        // and L here, and read transposed by the state update).  At the end R
        // is the decay over the whole chunk, e^{G_C}.
        float R0 = 1.f, R1 = 1.f;
#pragma unroll
        for (int s = C - 1; s >= 0; --s) {
            const float h0 = bf_lo(rk[s]) * R0, h1 = bf_hi(rk[s]) * R1;
            *reinterpret_cast<uint32_t *>(sKh + s * Cfg::KP + 4 * swz_piece(s, lane >> 1) +
                                          2 * (lane & 1)) = pack_bf16(h0, h1);
            R0 *= a0[s];
            R1 *= a1[s];
        }
        *reinterpret_cast<float2 *>(sGC + gc_word(d0)) = float2{R0, R1};   // d0 even: adjacent words
        // Forward: e^{G - G_C} = e^{G} / e^{G_C} (in [1, e^75]): Q~ = Q e^{G-G_C},
        // K~ = K e^{G-G_C}, as a running product started at 1 / e^{G_C}.  For
        // the chunk's last token both factors are 1 up to a few fp32 ulps, so
        // that token's bf16 operands are its unscaled inputs.
        {
            float f0 = __builtin_amdgcn_rcpf(R0), f1 = __builtin_amdgcn_rcpf(R1);
#pragma unroll
            for (int s = 0; s < C; ++s) {
                f0 *= a0[s];
                f1 *= a1[s];
                if constexpr (MODE == 0)   // Q~ feeds the output only
                    *reinterpret_cast<uint32_t *>(sQG + s * DP + d0) =
                        pack_bf16(bf_lo(rq[s]) * f0, bf_hi(rq[s]) * f1);
                *reinterpret_cast<uint32_t *>(sKt + s * Cfg::KP + 4 * swz_piece(s, lane >> 1) +
                                              2 * (lane & 1)) =
                    pack_bf16(bf_lo(rk[s]) * f0, bf_hi(rk[s]) * f1);
            }
        }
        // this wave's next chunk streams in while the rest of this one runs
        if (m + NPW < nchunks) load_chunk(t0 + (int64_t)NPW * C);
        if (lane < C) sBeta[lane] = beta_l;
        compiler_fence();

        // ---- P^T, L, L^T from Q~, K~, Kh (B-layout results) --------------------
        // accP[e]  = sum_d Kh[4g+e][d] Q~[n][d]   = P'[n][4g+e]   (P = tril P')
        // accL[e]  = sum_d K~[4g+e][d] Kh[n][d]   = L'[4g+e][n]
        // accLT[e] = sum_d Kh[4g+e][d] K~[n][d]   = L'[n][4g+e]   (L = beta strict_tril L')
        f32x4 accP = {0.f, 0.f, 0.f, 0.f}, accL = {0.f, 0.f, 0.f, 0.f},
              accLT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k32 = 0; k32 < D; k32 += 32) {
            const Frag<bf16> c0 = frag_swz(sKh, Cfg::KP, k32, lane),
                             c1 = frag_swz(sKh, Cfg::KP, k32 + 16, lane);
            const Frag<bf16> h0f = frag_swz(sKt, Cfg::KP, k32, lane),
                             h1f = frag_swz(sKt, Cfg::KP, k32 + 16, lane);
            if constexpr (MODE == 0) {
                const Frag<bf16> q0f = lds_frag(sQG, DP, k32, lane),
                                 q1f = lds_frag(sQG, DP, k32 + 16, lane);
                mma32(accP, c0, c1, q0f, q1f);
            }
            mma32(accL, h0f, h1f, c0, c1);
            mma32(accLT, c0, c1, h0f, h1f);
        }
        const f32x4 brow = *reinterpret_cast<const f32x4 *>(sBeta + 4 * g);   // beta_{4g+e}
        const float bcol = sBeta[n];                                            // beta_n
        f32x4 Lb, LTb, ImLT;   // L, L^T (B layout); I - L^T
        {
            f32x4 pm;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                pm[e] = r <= n ? accP[e] : 0.0f;                    // P[n][4g+e]
                Lb[e] = n < r ? brow[e] * accL[e] : 0.0f;           // L[4g+e][n]
                LTb[e] = r < n ? bcol * accLT[e] : 0.0f;            // L[n][4g+e]
                ImLT[e] = (r == n ? 1.0f : 0.0f) - LTb[e];
            }
            if constexpr (MODE == 0)
                *reinterpret_cast<bf16x4 *>(sP + n * CP + 4 * g) = to_bf16x4(pm[0], pm[1], pm[2], pm[3]);
        }
        // ---- T^T = Y^T X^T with X = (I-L)(I+L^2), Y = (I+L^4)(I+L^8) ----------
        // B-layout inputs: M (B) and M^T (= A-layout of M).
        auto bf = [](const f32x4 &x) { return acc_frag<bf16>(x); };
        auto mm = [](const Frag<bf16> &a, const Frag<bf16> &b) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            mma16(d, a, b);
            return d;
        };
        auto plus_i = [&](f32x4 x) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] += (4 * g + e == n) ? 1.0f : 0.0f;
            return x;
        };
        const Frag<bf16> fL = bf(Lb), fLT = bf(LTb);
        const f32x4 L2 = mm(fLT, fL), L2T = mm(fL, fLT);                 // L^2, (L^2)^T
        const Frag<bf16> fL2 = bf(L2), fL2T = bf(L2T);
        const f32x4 L4 = mm(fL2T, fL2), L4T = mm(fL2, fL2T);             // L^4, (L^4)^T
        const Frag<bf16> fL4 = bf(L4), fL4T = bf(L4T);
        const f32x4 L8 = mm(fL4T, fL4);                                  // L^8
        const f32x4 Y = mm(bf(plus_i(L4T)), bf(plus_i(L8)));            // (I+L^4)(I+L^8)
        const f32x4 XT = mm(bf(plus_i(L2)), bf(ImLT));                   // (I+L^2)^T (I-L)^T
        const f32x4 TT = mm(bf(Y), bf(XT));                              // T^T = Y^T X^T
        // T^T in B layout = T in A layout: lane (g,n) holds T[n][4g+e]
        Frag<bf16> Tf;   // A-layout of Tb = T diag(beta): T[n][4g+e] beta_{4g+e}
        Tf.v = to_bf16x4(TT[0] * brow[0], TT[1] * brow[1], TT[2] * brow[2], TT[3] * brow[3]);
        *reinterpret_cast<bf16x4 *>(sTb + n * CP + 4 * g) = Tf.v;

        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __hip_atomic_store(&ready[s_], use + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

template <int NCW, int NPW, int NSLOT, bool CKPT, int MODE>
__global__ __launch_bounds__(64 * (NCW + NPW)) void kda_prefill16_kernel(Prefill16Params prm) {
    __shared__ __attribute__((aligned(16))) char smem[P16Cfg<NCW, NPW, NSLOT>::LDS_BYTES];
    prefill16_block<NCW, NPW, NSLOT, CKPT, MODE>(prm, smem, blockIdx.x, gridDim.x);
}

// First pass of a sequence split, one launch: blocks [0, nblk0) run the
// prefill (MODE 0) of every sequence's first segment from its start state,
// the others the state maps (MODE 2) of the segments between the first and
// the last.  Both halves fill the chip together.
template <int NCW, int NPW, int NSLOT>
__global__ __launch_bounds__(64 * (NCW + NPW)) void kda_prefill16_split_head_kernel(
    Prefill16Params p0, Prefill16Params p2, int nblk0) {
    __shared__ __attribute__((aligned(16))) char smem[P16Cfg<NCW, NPW, NSLOT>::LDS_BYTES];
    if ((int)blockIdx.x < nblk0)
        prefill16_block<NCW, NPW, NSLOT, false, 0>(p0, smem, blockIdx.x, nblk0);
    else
        prefill16_block<NCW, NPW, NSLOT, false, 2>(p2, smem, blockIdx.x - nblk0,
                                                   gridDim.x - nblk0);
}

template <int NCW, int NPW, int NSLOT>
static Prefill16Params p16_params(const PrefillArgs &a) {
    Prefill16Params prm;
    prm.q = static_cast<const bf16 *>(a.q);
    prm.k = static_cast<const bf16 *>(a.k);
    prm.v = static_cast<const bf16 *>(a.v);
    prm.z = static_cast<const bf16 *>(a.z);
    prm.beta = static_cast<const bf16 *>(a.beta);
    prm.A = a.A;
    prm.S0 = a.S0;
    prm.o = static_cast<bf16 *>(a.o);
    prm.S_T = a.S_T;
    prm.S_T2 = a.S_T2;
    prm.T = a.T;
    prm.H = a.H;
    prm.nsplit = 128 / (16 * NCW);
    prm.cu = a.cu_seqlens;
    prm.order = a.order;
    prm.ckpt = a.ckpt;
    prm.n_ckpt = a.n_ckpt;
    prm.ckpt_every = a.ckpt_every;
    prm.ckpt_blocked = a.ckpt_blocked ? 1 : 0;
    prm.spin_limit = wait_spin_limit();
    return prm;
}

template <int NCW, int NPW, int NSLOT, bool CKPT, int MODE = 0>
static hipError_t launch_p16(const PrefillArgs &a) {
    const Prefill16Params prm = p16_params<NCW, NPW, NSLOT>(a);
    const int64_t nblk = a.B * a.H * prm.nsplit;
    hipLaunchKernelGGL((kda_prefill16_kernel<NCW, NPW, NSLOT, CKPT, MODE>), dim3((unsigned)nblk),
                       dim3(64 * (NCW + NPW)), 0, a.stream, prm);
    return hipGetLastError();
}

bool prefill16_supported(int dtype, int64_t D, int chunk, int dv_per_block) {
    return dtype == 1 && D == 128 && chunk == 16 && (dv_per_block == 32 || dv_per_block == 64);
}

hipError_t launch_prefill16_split_head(const PrefillArgs &a0, const PrefillArgs &a2) {
    if (a0.dv_per_block != 64 || a2.dv_per_block != 64 || a0.mode != 0 || a2.mode != 2 ||
        !a2.S_T2 || a0.H != a2.H)
        return hipErrorInvalidValue;
    const Prefill16Params p0 = p16_params<4, 8, 8>(a0), p2 = p16_params<4, 8, 8>(a2);
    const int64_t nblk0 = a0.B * a0.H * p0.nsplit, nblk2 = a2.B * a2.H * p2.nsplit;
    if (nblk0 + nblk2 == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_prefill16_split_head_kernel<4, 8, 8>), dim3((unsigned)(nblk0 + nblk2)),
                       dim3(64 * 12), 0, a0.stream, p0, p2, (int)nblk0);
    return hipGetLastError();
}

hipError_t launch_prefill16(const PrefillArgs &a) {
    const bool ck = a.ckpt != nullptr && a.ckpt_every > 0;
    if (a.mode != 0) {   // final states only: 64 columns
        if (a.dv_per_block != 64 || a.mode != 1) return hipErrorInvalidValue;
        if (a.mode == 1) return ck ? launch_p16<4, 8, 8, true, 1>(a) : launch_p16<4, 8, 8, false, 1>(a);
        return hipErrorInvalidValue;   // mode 2 runs inside launch_prefill16_split_head
    }
    if (a.dv_per_block == 64)
        return ck ? launch_p16<4, 8, 8, true>(a) : launch_p16<4, 8, 8, false>(a);
    if (a.dv_per_block == 32)
        return ck ? launch_p16<2, 6, 6, true>(a) : launch_p16<2, 6, 6, false>(a);
    return hipErrorInvalidValue;
}

}  // namespace kda
