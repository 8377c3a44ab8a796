// kda_api.hip -- the extern "C" entry points of libkda.so (see include/kda.h).
//
// Every check runs before anything is enqueued; on an error status no kernel
// is launched and no output is touched.  No device memory is allocated here.
// The one piece of state kept across calls is the per-device address of the
// static scratch of kda_prefill_varlen_noalloc (looked up once per device);
// the backward's optional second stream belongs to the caller.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdlib.h>

#include "kda_launch.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 62;

// The kernels read a tile of up to 64 consecutive tokens (rows of H*D
// elements) through one buffer resource with 32-bit offsets: such a tile
// must stay below 2^31 bytes (bf16, d = 128: H <= 131071).
bool tile_rows_fit(int64_t H, int64_t D, int64_t esz) {
    return H <= ((int64_t)0x7fffffff / 64) / (D * esz);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// a * b without int64 overflow; returns false when the product exceeds lim.
bool mul_ok(int64_t a, int64_t b, int64_t lim, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > lim / a) return false;
    *out = a * b;
    return true;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, int64_t bytes) {
    const uintptr_t lo = (uintptr_t)p;
    return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

}  // namespace

int kda::wait_spin_limit() {
    const char *e = getenv("KDA_WAIT_SPIN_LIMIT");
    if (e && *e) {
        char *end = nullptr;
        const long v = strtol(e, &end, 10);
        if (end && *end == 0 && v >= 0 && v <= (1L << 30)) return (int)v;
    }
    return 1 << 22;
}

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_str(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is negative or too large";
        case KDA_ERR_UNSUPPORTED:
            return "KDA_ERR_UNSUPPORTED: dtype / head size / chunk / split not supported";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: a pointer is not 16-byte aligned";
        case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error";
        default: return "unknown kda_status";
    }
}

size_t kda_prefill_workspace_size(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                                  int64_t dv, int32_t chunk) {
    (void)dtype; (void)B; (void)T; (void)H; (void)dk; (void)dv; (void)chunk;
    return 0;
}

}  // extern "C"

namespace {

// Shared validation and dispatch of the prefill entry points.  `cu` == NULL:
// dense [B, T, H, d]; otherwise B packed sequences over T tokens.
size_t order_bytes(int64_t N) {
    return N > 1 && N <= kda::kMaxOrderSeqs ? (size_t)((N * 4 + 255) / 256 * 256) : 0;
}

kda_status prefill_impl(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        int32_t chunk, const int64_t *cu, const void *q, const void *k,
                        const void *v, const void *z, const void *beta, const float *A,
                        const float *S0, void *o, float *S_T, int32_t ckpt_every,
                        float *ckpt, int64_t n_ckpt, void *workspace, size_t workspace_bytes,
                        void *stream, int32_t dv_per_block, int mode = 0,
                        bool check_only = false, bool ckpt_blocked = false,
                        bool scratch_ranking = false, int32_t *order_scratch = nullptr) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || n_ckpt < 0 || ckpt_every < 0)
        return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv || (dk != 16 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 64) return KDA_ERR_UNSUPPORTED;
    if (ckpt_every > 0 && ckpt_every % chunk != 0) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk;
    const int64_t esz = dtype == KDA_BF16 ? 2 : 4;
    const int64_t ntok_seqs = cu ? 1 : B;   // the token axis is shared when packed
    int64_t bt, bth, nin, nstate, bh, nck = 0;
    if (!mul_ok(ntok_seqs, T, kMaxElems, &bt) || !mul_ok(bt, H, kMaxElems, &bth) ||
        !mul_ok(bth, D, kMaxElems / 4, &nin) || !mul_ok(B, H, kMaxElems, &bh) ||
        !mul_ok(bh, D * D, kMaxElems / 4, &nstate))
        return KDA_ERR_SHAPE;
    int64_t nckh = 0;
    if (ckpt_every > 0 && (!mul_ok(n_ckpt, H, kMaxElems, &nckh) ||
                           !mul_ok(nckh, D * D, kMaxElems / 4, &nck)))
        return KDA_ERR_SHAPE;
    // grid size: at most 4096 work-items per head, and a dispatch counts
    // work-items in 32 bits
    if (bh > (int64_t)(0xffffffffu / 4096)) return KDA_ERR_SHAPE;
    if (!tile_rows_fit(H, D, esz)) return KDA_ERR_SHAPE;
    const bool want_ckpt = ckpt_every > 0 && n_ckpt > 0;
    int dvb = dv_per_block;
    if (dvb == 0) {
        dvb = kda::prefill_default_dv_per_block(dtype, B, H, D, chunk);
        if (want_ckpt && !kda::prefill16_supported(dtype, D, chunk, dvb) &&
            !kda::prefill_ckpt_supported(dtype, D, chunk, dvb))
            dvb /= 2;
    }
    const bool role_split = kda::prefill16_supported(dtype, D, chunk, dvb);
    if (dvb <= 0 || D % dvb != 0 || (!role_split && !kda::prefill_supported(dtype, D, chunk, dvb)))
        return KDA_ERR_UNSUPPORTED;
    if (want_ckpt && !role_split && !kda::prefill_ckpt_supported(dtype, D, chunk, dvb))
        return KDA_ERR_UNSUPPORTED;
    // mode 1 writes final states only (o is neither read nor written)
    if (mode != 0 && (mode != 1 || !role_split || dvb != 64))
        return KDA_ERR_UNSUPPORTED;
    if (ckpt_blocked && want_ckpt && !role_split) return KDA_ERR_UNSUPPORTED;
    if (!A || !S_T) return KDA_ERR_NULL;
    if (bth > 0 && (!q || !k || !v || !z || !beta || (mode == 0 && !o))) return KDA_ERR_NULL;
    if (ckpt_every > 0 && n_ckpt > 0 && !ckpt) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, z, beta, A, S0, o, S_T, ckpt};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    if (cu && ((uintptr_t)cu & 7u) != 0) return KDA_ERR_MISALIGNED;
    // longest-first order of packed sequences: in the caller's workspace, or
    // in the library's static scratch (order_scratch, kMaxOrderSeqs entries)
    const size_t need_ws = cu && H > 0 && !scratch_ranking ? order_bytes(B) : 0;
    const bool rank = cu && H > 0 && order_bytes(B) > 0;
    if (need_ws > 0 && (!workspace || workspace_bytes < need_ws)) return KDA_ERR_WORKSPACE;
    if (need_ws > 0 && !aligned16(workspace)) return KDA_ERR_MISALIGNED;
    const Range rq = range_of(q, nin * esz), rk = range_of(k, nin * esz),
                rv = range_of(v, nin * esz), rz = range_of(z, nin * esz),
                rb = range_of(beta, bth * esz), rA = range_of(A, H * 4),
                rS0 = range_of(S0, nstate * 4), ro = range_of(mode == 0 ? o : nullptr, nin * esz),
                rST = range_of(S_T, nstate * 4),
                rcu = range_of(cu, cu ? (B + 1) * 8 : 0),
                rws = range_of(need_ws > 0 ? workspace : nullptr, (int64_t)need_ws),
                rck = range_of(ckpt_every > 0 ? ckpt : nullptr, nck * 4);
    const Range ins[] = {rq, rk, rv, rz, rb, rA, rcu};
    for (const Range &r : ins)
        if (overlaps(ro, r) || overlaps(rST, r) || overlaps(rck, r)) return KDA_ERR_ALIAS;
    if (overlaps(ro, rS0) || overlaps(ro, rST) || overlaps(rck, rS0) || overlaps(rck, ro) ||
        overlaps(rck, rST))
        return KDA_ERR_ALIAS;
    if (overlaps(rST, rS0) && (const void *)S_T != (const void *)S0) return KDA_ERR_ALIAS;
    {
        const Range all[] = {rq, rk, rv, rz, rb, rA, rS0, ro, rST, rcu, rck};
        for (const Range &r : all)
            if (overlaps(rws, r)) return KDA_ERR_ALIAS;
    }
    if (bh == 0 || check_only) return KDA_OK;

    kda::PrefillArgs a;
    a.dtype = dtype; a.B = B; a.T = T; a.H = H; a.D = D; a.chunk = chunk;
    a.dv_per_block = dvb;
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.A = A; a.S0 = S0;
    a.o = mode == 0 ? o : nullptr; a.S_T = S_T;
    a.cu_seqlens = cu;
    a.order = nullptr;
    if (rank) {
        int32_t *order = scratch_ranking ? order_scratch : static_cast<int32_t *>(workspace);
        if (!order) return KDA_ERR_NULL;
        if (kda::launch_seq_order(cu, B, T, order, (hipStream_t)stream) != hipSuccess)
            return KDA_ERR_HIP;
        a.order = order;
    }
    a.ckpt_every = ckpt_every > 0 && n_ckpt > 0 ? ckpt_every : 0;
    a.ckpt = a.ckpt_every > 0 ? ckpt : nullptr;
    a.ckpt_blocked = ckpt_blocked;
    a.n_ckpt = n_ckpt;
    a.mode = mode;
    a.stream = (hipStream_t)stream;
    const hipError_t err = role_split ? kda::launch_prefill16(a) : kda::launch_prefill(a);
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status kda_prefill_ex(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                          int32_t chunk, const void *q, const void *k, const void *v,
                          const void *z, const void *beta, const float *A, const float *S0,
                          void *o, float *S_T, void *workspace, size_t workspace_bytes,
                          void *stream, int32_t dv_per_block) {
    (void)workspace;
    (void)workspace_bytes;
    return prefill_impl(dtype, B, T, H, dk, dv, chunk, nullptr, q, k, v, z, beta, A, S0, o, S_T,
                        0, nullptr, 0, nullptr, 0, stream, dv_per_block);
}

size_t kda_prefill_varlen_workspace_size(int64_t N) { return order_bytes(N); }

kda_status kda_prefill_varlen(int dtype, int64_t N, int64_t T_total, int64_t H, int64_t dk,
                              int64_t dv, int32_t chunk, const int64_t *cu_seqlens,
                              const void *q, const void *k, const void *v, const void *z,
                              const void *beta, const float *A, const float *S0, void *o,
                              float *S_T, int32_t ckpt_every, float *ckpt, int64_t n_ckpt,
                              void *workspace, size_t workspace_bytes, void *stream,
                              int32_t dv_per_block) {
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    return prefill_impl(dtype, N, T_total, H, dk, dv, chunk, cu_seqlens, q, k, v, z, beta, A,
                        S0, o, S_T, ckpt_every, ckpt, n_ckpt, workspace, workspace_bytes, stream,
                        dv_per_block);
}

}  // extern "C"

namespace {

// Scratch of kda_prefill_varlen_noalloc: the longest-first ranking of up to
// kMaxOrderSeqs packed sequences (32 KiB on every device the library runs
// on, held until the process ends).  Host code never uses this name as an
// address: each device's copy is looked up once with hipGetSymbolAddress
// (that device current) and only that pointer is passed to kernels.
static __device__ __align__(256) int32_t scratch[kda::kMaxOrderSeqs];

constexpr int kScratchDevices = 256;
std::mutex g_scratch_mu;
int32_t *g_scratch_ptr[kScratchDevices] = {};

// This device's copy of `scratch`, set up on the first call on the device.
kda_status scratch_of_current_device(int32_t **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return KDA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<int32_t *>(p);
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_varlen_noalloc(int dtype, int64_t N, int64_t T_total, int64_t H,
                                      int64_t dk, int64_t dv, int32_t chunk,
                                      const int64_t *cu_seqlens, const void *q, const void *k,
                                      const void *v, const void *z, const void *beta,
                                      const float *A, const float *S0, void *o, float *S_T,
                                      int32_t ckpt_every, float *ckpt, int64_t n_ckpt,
                                      void *stream, int32_t dv_per_block) {
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    if (N > kda::kMaxOrderSeqs) return KDA_ERR_WORKSPACE;   // beyond the static scratch
    // every other check first, so that an invalid call touches nothing
    const kda_status st = prefill_impl(dtype, N, T_total, H, dk, dv, chunk, cu_seqlens, q, k, v,
                                       z, beta, A, S0, o, S_T, ckpt_every, ckpt, n_ckpt, nullptr,
                                       0, stream, dv_per_block, 0, /*check_only=*/true,
                                       false, /*scratch_ranking=*/true);
    if (st != KDA_OK) return st;
    int32_t *order = nullptr;
    const kda_status ss = scratch_of_current_device(&order);
    if (ss != KDA_OK) return ss;
    return prefill_impl(dtype, N, T_total, H, dk, dv, chunk, cu_seqlens, q, k, v, z, beta, A, S0,
                        o, S_T, ckpt_every, ckpt, n_ckpt, nullptr, 0, stream, dv_per_block, 0,
                        false, false, true, order);
}

kda_status kda_prefill(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                       int32_t chunk, const void *q, const void *k, const void *v,
                       const void *z, const void *beta, const float *A, const float *S0,
                       void *o, float *S_T, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return kda_prefill_ex(dtype, B, T, H, dk, dv, chunk, q, k, v, z, beta, A, S0, o, S_T,
                          workspace, workspace_bytes, stream, 0);
}

kda_status kda_decode_step(int dtype, int64_t B, int64_t H, int64_t dk, int64_t dv,
                           const void *q, const void *k, const void *v, const void *z,
                           const void *beta, const float *A, float *S, void *o,
                           void *stream) {
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv || !kda::decode_supported(dtype, dk)) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk;
    const int64_t esz = dtype == KDA_BF16 ? 2 : 4;
    int64_t bh, nin, nstate;
    if (!mul_ok(B, H, kMaxElems, &bh) || !mul_ok(bh, D, kMaxElems / 4, &nin) ||
        !mul_ok(bh, D * D, kMaxElems / 4, &nstate))
        return KDA_ERR_SHAPE;
    if (bh > (int64_t)(0xffffffffu / 512)) return KDA_ERR_SHAPE;   // 512 work-items per head
    if (!A) return KDA_ERR_NULL;
    if (bh > 0 && (!q || !k || !v || !z || !beta || !S || !o)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, z, beta, A, S, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const Range rq = range_of(q, nin * esz), rk = range_of(k, nin * esz),
                rv = range_of(v, nin * esz), rz = range_of(z, nin * esz),
                rb = range_of(beta, bh * esz), rA = range_of(A, H * 4),
                rS = range_of(S, nstate * 4), ro = range_of(o, nin * esz);
    const Range others[] = {rq, rk, rv, rz, rb, rA, rS};
    for (const Range &r : others)
        if (overlaps(ro, r)) return KDA_ERR_ALIAS;
    const Range ins[] = {rq, rk, rv, rz, rb, rA};
    for (const Range &r : ins)
        if (overlaps(rS, r)) return KDA_ERR_ALIAS;
    if (bh == 0) return KDA_OK;

    kda::DecodeArgs a{};
    a.dtype = dtype; a.B = B; a.H = H; a.D = D;
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.A = A; a.S = S; a.o = o;
    a.conv = 0;
    a.stream = (hipStream_t)stream;
    return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"

// ------------------------------------------------------------ prologue ----

namespace {

size_t round256(int64_t bytes) { return (size_t)((bytes + 255) / 256 * 256); }

// Checked prologue parameters of one call.
struct ConvSpec {
    int W, act;
    float eps;
    const float *w[3];
    const void *sin[3];
    void *sout[3];
    Range rw[3], rsin[3], rsout[3];
};

// Validates the prologue parameters and state arrays of a call over B
// sequences of H heads (d = D channels per head).  `need_state_in`: the state
// array is required (decode).  Fills `cs` on success.
kda_status conv_check(int dtype, int64_t B, int64_t H, int64_t D, const kda_short_conv *conv,
                      const void *const *state_in, void *const *state_out, bool need_state_in,
                      ConvSpec *cs) {
    if (!conv) return KDA_ERR_NULL;
    if (conv->width < 1 || conv->width > 4 || conv->reserved != 0) return KDA_ERR_UNSUPPORTED;
    if (conv->activation != KDA_ACT_NONE && conv->activation != KDA_ACT_SILU)
        return KDA_ERR_UNSUPPORTED;
    if (!(conv->eps >= 0.0f) || !(conv->eps <= 3.4e38f)) return KDA_ERR_UNSUPPORTED;
    if (!kda::conv_supported(dtype, D)) return KDA_ERR_UNSUPPORTED;
    const int W = conv->width;
    const int64_t esz = dtype == KDA_BF16 ? 2 : 4;
    int64_t bw, bwh, nst;
    if (!mul_ok(B, W - 1, kMaxElems, &bw) || !mul_ok(bw, H, kMaxElems, &bwh) ||
        !mul_ok(bwh, D, kMaxElems / 4, &nst) || !tile_rows_fit(H, D, esz))
        return KDA_ERR_SHAPE;
    cs->W = W;
    cs->act = conv->activation;
    cs->eps = conv->eps;
    cs->w[0] = conv->wq; cs->w[1] = conv->wk; cs->w[2] = conv->wv;
    const bool states = W > 1;
    for (int i = 0; i < 3; ++i) {
        cs->sin[i] = states && state_in ? state_in[i] : nullptr;
        cs->sout[i] = states && state_out ? state_out[i] : nullptr;
    }
    if (H > 0)
        for (int i = 0; i < 3; ++i)
            if (!cs->w[i]) return KDA_ERR_NULL;
    if (states && B > 0 && H > 0) {
        if (need_state_in && !state_in) return KDA_ERR_NULL;
        for (int i = 0; i < 3; ++i) {
            if (state_in && !cs->sin[i]) return KDA_ERR_NULL;
            if (state_out && !cs->sout[i]) return KDA_ERR_NULL;
        }
    }
    for (int i = 0; i < 3; ++i) {
        const void *ptrs[] = {cs->w[i], cs->sin[i], cs->sout[i]};
        for (const void *p : ptrs)
            if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
        cs->rw[i] = range_of(cs->w[i], H * D * W * 4);
        cs->rsin[i] = range_of(cs->sin[i], nst * esz);
        cs->rsout[i] = range_of(cs->sout[i], nst * esz);
    }
    // state outputs must not overlap each other, the taps or the state inputs
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
            if (i != j && overlaps(cs->rsout[i], cs->rsout[j])) return KDA_ERR_ALIAS;
            if (overlaps(cs->rsout[i], cs->rw[j])) return KDA_ERR_ALIAS;
            if (!need_state_in && overlaps(cs->rsout[i], cs->rsin[j])) return KDA_ERR_ALIAS;
        }
    return KDA_OK;
}

// Sizes the prologue kernel can address: (tile + 3) token rows in 32-bit
// buffer offsets, and the grid (256 work-items per workgroup, counted in 32
// bits by a dispatch).
bool conv_sizes_ok(int dtype, int64_t B, int64_t T, int64_t H, int64_t D) {
    const int64_t esz = dtype == KDA_BF16 ? 2 : 4;
    const int64_t tt = kda::conv_tile_tokens(dtype, D);
    if (H * D * esz * (tt + 3) >= ((int64_t)1 << 31)) return false;
    const int64_t ntile = T > 0 ? (T + tt - 1) / tt : 1;
    const int64_t nslab = (H * (D / 8) + 63) / 64;
    int64_t n1, n2;
    return mul_ok(B, nslab, kMaxElems, &n1) && mul_ok(n1, (ntile + 3) / 4, kMaxElems, &n2) &&
           n2 < ((int64_t)1 << 32) / 256;
}

kda::ConvNormArgs conv_args(int dtype, int64_t B, int64_t T, int64_t H, int64_t D,
                            const ConvSpec &cs, const void *const x[3], void *const y[3],
                            void *stream) {
    kda::ConvNormArgs a{};
    a.dtype = dtype; a.B = B; a.T = T; a.H = H; a.D = D;
    for (int i = 0; i < 3; ++i) {
        a.t[i].x = x[i];
        a.t[i].w = cs.w[i];
        a.t[i].sin = cs.sin[i];
        a.t[i].y = y[i];
        a.t[i].sout = cs.sout[i];
        a.t[i].norm = i < 2;
    }
    a.W = cs.W; a.act = cs.act; a.eps = cs.eps;
    a.stream = (hipStream_t)stream;
    return a;
}

}  // namespace

extern "C" {

kda_status kda_conv_norm(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                         const kda_short_conv *conv, const void *q, const void *k,
                         const void *v, const void *const *state_in, void *const *state_out,
                         void *q_out, void *k_out, void *v_out, void *stream) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk, esz = dtype == KDA_BF16 ? 2 : 4;
    ConvSpec cs;
    const kda_status st = conv_check(dtype, B, H, D, conv, state_in, state_out, false, &cs);
    if (st != KDA_OK) return st;
    int64_t bt, bth, nin;
    if (!mul_ok(B, T, kMaxElems, &bt) || !mul_ok(bt, H, kMaxElems, &bth) ||
        !mul_ok(bth, D, kMaxElems / 4, &nin))
        return KDA_ERR_SHAPE;
    if (!conv_sizes_ok(dtype, B, T, H, D)) return KDA_ERR_SHAPE;
    if (nin > 0 && (!q || !k || !v || !q_out || !k_out || !v_out)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, q_out, k_out, v_out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const Range rin[] = {range_of(q, nin * esz), range_of(k, nin * esz), range_of(v, nin * esz),
                         cs.rw[0], cs.rw[1], cs.rw[2], cs.rsin[0], cs.rsin[1], cs.rsin[2]};
    const Range rout[] = {range_of(q_out, nin * esz), range_of(k_out, nin * esz),
                          range_of(v_out, nin * esz), cs.rsout[0], cs.rsout[1], cs.rsout[2]};
    for (int i = 0; i < 6; ++i) {
        for (const Range &r : rin)
            if (overlaps(rout[i], r)) return KDA_ERR_ALIAS;
        for (int j = 0; j < 6; ++j)
            if (i != j && overlaps(rout[i], rout[j])) return KDA_ERR_ALIAS;
    }
    if (B == 0 || H == 0) return KDA_OK;
    const void *x[3] = {q, k, v};
    void *y[3] = {q_out, k_out, v_out};
    const kda::ConvNormArgs a = conv_args(dtype, B, T, H, D, cs, x, y, stream);
    return kda::launch_conv_norm(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_conv_norm_varlen(int dtype, int64_t N, int64_t T_total, int64_t H, int64_t dk,
                                int64_t dv, const int64_t *cu_seqlens, const kda_short_conv *conv,
                                const void *q, const void *k, const void *v,
                                const void *const *state_in, void *const *state_out,
                                void *q_out, void *k_out, void *v_out, void *stream) {
    if (N < 0 || T_total < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk, esz = dtype == KDA_BF16 ? 2 : 4;
    ConvSpec cs;
    const kda_status st = conv_check(dtype, N, H, D, conv, state_in, state_out, false, &cs);
    if (st != KDA_OK) return st;
    int64_t th, nin;
    if (!mul_ok(T_total, H, kMaxElems, &th) || !mul_ok(th, D, kMaxElems / 4, &nin))
        return KDA_ERR_SHAPE;
    if (!conv_sizes_ok(dtype, 1, T_total, H, D)) return KDA_ERR_SHAPE;
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 7u) != 0) return KDA_ERR_MISALIGNED;
    if (nin > 0 && (!q || !k || !v || !q_out || !k_out || !v_out)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, q_out, k_out, v_out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const Range rin[] = {range_of(q, nin * esz), range_of(k, nin * esz), range_of(v, nin * esz),
                         cs.rw[0], cs.rw[1], cs.rw[2], cs.rsin[0], cs.rsin[1], cs.rsin[2],
                         range_of(cu_seqlens, N > 0 ? (N + 1) * 8 : 0)};
    const Range rout[] = {range_of(q_out, nin * esz), range_of(k_out, nin * esz),
                          range_of(v_out, nin * esz), cs.rsout[0], cs.rsout[1], cs.rsout[2]};
    for (int i = 0; i < 6; ++i) {
        for (const Range &r : rin)
            if (overlaps(rout[i], r)) return KDA_ERR_ALIAS;
        for (int j = 0; j < 6; ++j)
            if (i != j && overlaps(rout[i], rout[j])) return KDA_ERR_ALIAS;
    }
    if (N == 0 || H == 0) return KDA_OK;
    const void *x[3] = {q, k, v};
    void *y[3] = {q_out, k_out, v_out};
    kda::ConvNormArgs a = conv_args(dtype, 1, T_total, H, D, cs, x, y, stream);
    a.cu = cu_seqlens;
    a.N = N;
    return kda::launch_conv_norm(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_prefill_conv_workspace_size(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                                       int64_t dv, int32_t chunk) {
    (void)chunk;
    if ((dtype != KDA_F32 && dtype != KDA_BF16) || B < 0 || T < 0 || H < 0 || dk <= 0 ||
        dv <= 0)
        return 0;
    const int64_t esz = dtype == KDA_BF16 ? 2 : 4;
    int64_t bt, bth, nk, nv;
    if (!mul_ok(B, T, kMaxElems, &bt) || !mul_ok(bt, H, kMaxElems, &bth) ||
        !mul_ok(bth, dk, kMaxElems / 4, &nk) || !mul_ok(bth, dv, kMaxElems / 4, &nv))
        return 0;
    return 2 * round256(nk * esz) + round256(nv * esz);
}

kda_status kda_prefill_conv(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                            int32_t chunk, const kda_short_conv *conv, const void *q,
                            const void *k, const void *v, const void *z, const void *beta,
                            const float *A, const void *const *state_in,
                            void *const *state_out, const float *S0, void *o, float *S_T,
                            void *workspace, size_t workspace_bytes, void *stream,
                            int32_t dv_per_block) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk, esz = dtype == KDA_BF16 ? 2 : 4;
    ConvSpec cs;
    kda_status st = conv_check(dtype, B, H, D, conv, state_in, state_out, false, &cs);
    if (st != KDA_OK) return st;
    int64_t bt, bth, nin;
    if (!mul_ok(B, T, kMaxElems, &bt) || !mul_ok(bt, H, kMaxElems, &bth) ||
        !mul_ok(bth, D, kMaxElems / 4, &nin))
        return KDA_ERR_SHAPE;
    if (!conv_sizes_ok(dtype, B, T, H, D)) return KDA_ERR_SHAPE;
    const size_t need = kda_prefill_conv_workspace_size(dtype, B, T, H, dk, dv, chunk);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (workspace && !aligned16(workspace)) return KDA_ERR_MISALIGNED;
    char *ws = static_cast<char *>(workspace);
    void *qh = need > 0 ? ws : nullptr;
    void *kh = need > 0 ? ws + round256(nin * esz) : nullptr;
    void *vh = need > 0 ? ws + 2 * round256(nin * esz) : nullptr;
    // the recurrence's own checks, on the prologue's outputs, before any launch
    st = prefill_impl(dtype, B, T, H, dk, dv, chunk, nullptr, qh, kh, vh, z, beta, A, S0, o, S_T,
                      0, nullptr, 0, nullptr, 0, stream, dv_per_block, 0, true);
    if (st != KDA_OK) return st;
    if (nin > 0 && (!q || !k || !v)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const int64_t bh = B * H;
    const Range rws = range_of(need > 0 ? workspace : nullptr, (int64_t)need);
    const Range rin[] = {range_of(q, nin * esz), range_of(k, nin * esz), range_of(v, nin * esz),
                         range_of(z, nin * esz), range_of(beta, bth * esz), range_of(A, H * 4),
                         range_of(S0, bh * D * D * 4), cs.rw[0], cs.rw[1], cs.rw[2],
                         cs.rsin[0], cs.rsin[1], cs.rsin[2]};
    const Range rout[] = {range_of(o, nin * esz), range_of(S_T, bh * D * D * 4), rws,
                          cs.rsout[0], cs.rsout[1], cs.rsout[2]};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 13; ++j) {
            // S_T == S0 is the allowed in-place carry of the recurrent state
            if (i == 1 && j == 6 && (const void *)S_T == (const void *)S0) continue;
            if (overlaps(rout[i], rin[j])) return KDA_ERR_ALIAS;
        }
        for (int j = 0; j < 6; ++j)
            if (i != j && overlaps(rout[i], rout[j])) return KDA_ERR_ALIAS;
    }
    if (bh == 0) return KDA_OK;
    const void *x[3] = {q, k, v};
    void *y[3] = {qh, kh, vh};
    const kda::ConvNormArgs a = conv_args(dtype, B, T, H, D, cs, x, y, stream);
    if (kda::launch_conv_norm(a) != hipSuccess) return KDA_ERR_HIP;
    return prefill_impl(dtype, B, T, H, dk, dv, chunk, nullptr, qh, kh, vh, z, beta, A, S0, o,
                        S_T, 0, nullptr, 0, nullptr, 0, stream, dv_per_block);
}

kda_status kda_decode_step_conv(int dtype, int64_t B, int64_t H, int64_t dk, int64_t dv,
                                const kda_short_conv *conv, const void *q, const void *k,
                                const void *v, const void *z, const void *beta, const float *A,
                                void *const *state, float *S, void *o, void *stream) {
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv || !kda::decode_supported(dtype, dk)) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk, esz = dtype == KDA_BF16 ? 2 : 4;
    ConvSpec cs;
    // the states are read and written in place: pass them as input and output
    kda_status st = conv_check(dtype, B, H, D, conv, state, state, true, &cs);
    if (st != KDA_OK) return st;
    int64_t bh, nin, nstate;
    if (!mul_ok(B, H, kMaxElems, &bh) || !mul_ok(bh, D, kMaxElems / 4, &nin) ||
        !mul_ok(bh, D * D, kMaxElems / 4, &nstate))
        return KDA_ERR_SHAPE;
    if (bh > (int64_t)(0xffffffffu / 512)) return KDA_ERR_SHAPE;   // 512 work-items per head
    if (!A) return KDA_ERR_NULL;
    if (bh > 0 && (!q || !k || !v || !z || !beta || !S || !o)) return KDA_ERR_NULL;
    const void *ptrs[] = {q, k, v, z, beta, A, S, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const Range rin[] = {range_of(q, nin * esz), range_of(k, nin * esz), range_of(v, nin * esz),
                         range_of(z, nin * esz), range_of(beta, bh * esz), range_of(A, H * 4),
                         cs.rw[0], cs.rw[1], cs.rw[2]};
    const Range rout[] = {range_of(o, nin * esz), range_of(S, nstate * 4), cs.rsin[0],
                          cs.rsin[1], cs.rsin[2]};
    for (int i = 0; i < 5; ++i) {
        for (const Range &r : rin)
            if (overlaps(rout[i], r)) return KDA_ERR_ALIAS;
        for (int j = 0; j < 5; ++j)
            if (i != j && overlaps(rout[i], rout[j])) return KDA_ERR_ALIAS;
    }
    if (bh == 0) return KDA_OK;
    kda::DecodeArgs a{};
    a.dtype = dtype; a.B = B; a.H = H; a.D = D;
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.A = A; a.S = S; a.o = o;
    a.conv = 1;
    a.wq = cs.w[0]; a.wk = cs.w[1]; a.wv = cs.w[2];
    a.cq = const_cast<void *>(cs.sin[0]);
    a.ck = const_cast<void *>(cs.sin[1]);
    a.cv = const_cast<void *>(cs.sin[2]);
    a.W = cs.W; a.act = cs.act; a.eps = cs.eps;
    a.stream = (hipStream_t)stream;
    return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"

// ------------------------------------------------------- sequence split ----

namespace {

constexpr int kMaxSegments = 1024;

// Segment length: ceil(T / P) rounded up to a whole chunk, so that every
// segment boundary is a chunk boundary of the unsplit run.
int64_t split_len(int64_t T, int P, int chunk) {
    const int64_t L = (T + P - 1) / P;
    return (L + chunk - 1) / chunk * chunk;
}

struct SplitLayout {
    size_t cu, first, M, N, S, total;   // byte offsets into the workspace, and its size
};

bool split_layout(int64_t B, int64_t H, int64_t D, int P, SplitLayout *lay) {
    int64_t n, nh, ne;
    if (!mul_ok(B, P, kMaxElems, &n) || !mul_ok(n, H, kMaxElems, &nh) ||
        !mul_ok(nh, D * D, kMaxElems / 16, &ne))
        return false;
    lay->cu = 0;
    lay->first = round256((n + 1) * 8);
    lay->M = lay->first + round256(n * 8);   // three rank lists: B * (2P - 2) <= 2n entries
    lay->N = lay->M + round256(ne * 4);
    lay->S = lay->N + round256(ne * 4);
    lay->total = lay->S + round256(ne * 4);
    return true;
}

// Arguments of one prefill run over segments of a split call (whose
// arguments were validated on entry): `nseq` segments of the packing `cu`,
// rank r running segment order[r]; S0, S_T, S_T2 indexed by segment.  Chunk
// 16 runs the role-split kernel at 64 columns per workgroup, chunk 64 the
// general kernel at 128.
kda::PrefillArgs split_args(int chunk, int64_t nseq, int64_t Ttot, int64_t H, const int64_t *cu,
                            const int32_t *order, const void *q, const void *k, const void *v,
                            const void *z, const void *beta, const float *A, const float *S0,
                            void *o, float *S_T, float *S_T2, int mode, hipStream_t stream) {
    kda::PrefillArgs a;
    a.dtype = KDA_BF16; a.B = nseq; a.T = Ttot; a.H = H; a.D = 128; a.chunk = chunk;
    a.dv_per_block = chunk == 16 ? 64 : 128;
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.A = A; a.S0 = S0;
    a.o = o; a.S_T = S_T; a.S_T2 = S_T2;
    a.cu_seqlens = cu;
    a.order = order;
    a.ckpt_every = 0; a.ckpt = nullptr; a.n_ckpt = 0;
    a.mode = mode;
    a.stream = stream;
    return a;
}

}  // namespace

extern "C" {

size_t kda_prefill_split_workspace_size(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                                        int64_t dv, int32_t chunk, int32_t segments) {
    (void)T;
    if (dtype != KDA_BF16 || dk != 128 || dv != 128 || (chunk != 16 && chunk != 64) || B < 0 ||
        H < 0 || segments < 1 || segments > kMaxSegments)
        return 0;
    if (segments == 1) return 0;
    SplitLayout lay;
    return split_layout(B, H, dk, segments, &lay) ? lay.total : 0;
}

kda_status kda_prefill_split(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             int32_t chunk, int32_t segments, const void *q, const void *k,
                             const void *v, const void *z, const void *beta, const float *A,
                             const float *S0, void *o, float *S_T, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (segments < 1 || segments > kMaxSegments) return KDA_ERR_UNSUPPORTED;
    if (dtype != KDA_BF16 || dk != 128 || dv != 128 || (chunk != 16 && chunk != 64))
        return KDA_ERR_UNSUPPORTED;
    const int dvb = chunk == 16 ? 64 : 128;
    // every check of the plain call on the caller's arguments
    kda_status st = prefill_impl(dtype, B, T, H, dk, dv, chunk, nullptr, q, k, v, z, beta, A, S0,
                                 o, S_T, 0, nullptr, 0, nullptr, 0, stream, dvb, 0, true);
    if (st != KDA_OK) return st;
    const int P = segments;
    if (P == 1)
        return prefill_impl(dtype, B, T, H, dk, dv, chunk, nullptr, q, k, v, z, beta, A, S0, o,
                            S_T, 0, nullptr, 0, nullptr, 0, stream, dvb);
    SplitLayout lay;
    if (!split_layout(B, H, dk, P, &lay)) return KDA_ERR_SHAPE;
    // segments; the passes' grids hold at most 4096 work-items per (segment,
    // head) unit, and a dispatch counts work-items in 32 bits
    int64_t nseg;
    if (!mul_ok(B, P, (int64_t)(0xffffffffu / 4096) / (H > 0 ? H : 1), &nseg)) return KDA_ERR_SHAPE;
    if (!workspace || workspace_bytes < lay.total) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
    {
        const int64_t esz = 2, D = dk;
        const Range rws = range_of(workspace, (int64_t)lay.total);
        const Range all[] = {range_of(q, B * T * H * D * esz), range_of(k, B * T * H * D * esz),
                             range_of(v, B * T * H * D * esz), range_of(z, B * T * H * D * esz),
                             range_of(beta, B * T * H * esz), range_of(A, H * 4),
                             range_of(S0, B * H * D * D * 4), range_of(o, B * T * H * D * esz),
                             range_of(S_T, B * H * D * D * 4)};
        for (const Range &r : all)
            if (overlaps(rws, r)) return KDA_ERR_ALIAS;
    }
    if (B * H == 0) return KDA_OK;
    char *ws = static_cast<char *>(workspace);
    int64_t *cu = reinterpret_cast<int64_t *>(ws + lay.cu);
    int32_t *lists = reinterpret_cast<int32_t *>(ws + lay.first);
    float *Mb = reinterpret_cast<float *>(ws + lay.M);
    float *Nb = reinterpret_cast<float *>(ws + lay.N);
    float *Sb = reinterpret_cast<float *>(ws + lay.S);   // start states, by segment
    const hipStream_t s = (hipStream_t)stream;
    const int64_t L = split_len(T, P, chunk);
    const int64_t Ttot = B * T;   // [B, T, H, d] read as the packing [B*T, H, d]
    const int64_t per = H * dk * dk;   // one segment's states
    if (kda::launch_split_setup(cu, lists, S0, Sb, B, T, L, P, H, (int)dk, s) != hipSuccess)
        return KDA_ERR_HIP;
    // (1) one launch: the first segment of each sequence from S0 (its final
    // state is the second segment's start), beside the maps M (from I, v as
    // zero) and offsets N (from 0) of the segments between first and last
    const kda::PrefillArgs a0 = split_args(chunk, B, Ttot, H, cu, lists, q, k, v, z, beta, A,
                                           S0 ? Sb : nullptr, o, Sb + per, nullptr, 0, s);
    if (chunk == 16) {   // M and N on one prep (role-split kernel, mode 2)
        const kda::PrefillArgs a2 = split_args(chunk, B * (P - 2), Ttot, H, cu, lists + B, q, k,
                                               v, z, beta, A, nullptr, nullptr, Mb, Nb, 2, s);
        if (kda::launch_prefill16_split_head(a0, a2) != hipSuccess) return KDA_ERR_HIP;
    } else {             // N (mode 1 from zero) and M (mode 3) as runs of their own
        const kda::PrefillArgs a[3] = {
            a0,
            split_args(chunk, B * (P - 2), Ttot, H, cu, lists + B, q, k, v, z, beta, A, nullptr,
                       nullptr, Nb, nullptr, 1, s),
            split_args(chunk, B * (P - 2), Ttot, H, cu, lists + B, q, k, v, z, beta, A, nullptr,
                       nullptr, Mb, nullptr, 3, s)};
        if (kda::launch_prefill_multi(a) != hipSuccess) return KDA_ERR_HIP;
    }
    // (2) start states of segments 2 .. P-1
    if (kda::launch_split_scan(Mb, Nb, Sb, B, H, P, (int)dk, s) != hipSuccess)
        return KDA_ERR_HIP;
    // (3) segments 1 .. P-1 from their start states; final states go to Mb
    const kda::PrefillArgs a3 = split_args(chunk, B * (P - 1), Ttot, H, cu, lists + B + B * (P - 2),
                                           q, k, v, z, beta, A, Sb, o, Mb, nullptr, 0, s);
    if ((chunk == 16 ? kda::launch_prefill16(a3) : kda::launch_prefill(a3)) != hipSuccess)
        return KDA_ERR_HIP;
    return kda::launch_split_gather(Mb, S_T, B, H, P, (int)dk, s) == hipSuccess ? KDA_OK
                                                                                : KDA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------- backward --

namespace {

constexpr int kBwdChunk = 16;

struct BwdLayout {
    size_t o, S_T, ckpt, prep, part, dA, dsp, total;   // byte offsets, and the size
};

bool bwd_layout(int dtype, int64_t B, int64_t T, int64_t H, int64_t D, BwdLayout *lay) {
    const int64_t esz = dtype == KDA_BF16 ? 2 : 4;
    const int64_t nchunk = (T + kBwdChunk - 1) / kBwdChunk, nfull = T / kBwdChunk;
    int64_t bt, bth, nin, bh, units, nst, nck, nprep, npart, ndsp;
    if (!mul_ok(B, T, kMaxElems, &bt) || !mul_ok(bt, H, kMaxElems, &bth) ||
        !mul_ok(bth, D, kMaxElems / 16, &nin) || !mul_ok(B, H, kMaxElems, &bh) ||
        !mul_ok(bh, D * D, kMaxElems / 16, &nst) || !mul_ok(bh, nchunk, kMaxElems, &units) ||
        !mul_ok(bh * nfull, D * D, kMaxElems / 16, &nck) ||
        !mul_ok(units, (int64_t)kda::bwd_prep_floats(D), kMaxElems / 16, &nprep) ||
        !mul_ok(units, (int64_t)kda::bwd_part_floats(D), kMaxElems / 16, &npart) ||
        !mul_ok(units, (int64_t)kda::bwd_dsp_bytes(dtype, D), kMaxElems / 16, &ndsp))
        return false;
    // the MFMA backward (bf16, d = 128) reruns the forward for its states only
    const bool mfma = kda::bwd_dsp_bytes(dtype, D) > 0;
    lay->o = 0;
    lay->S_T = mfma ? 0 : round256(nin * esz);
    lay->ckpt = lay->S_T + round256(nst * 4);
    // the MFMA backward (bf16, d = 128) keeps its checkpoints in bf16
    lay->prep = lay->ckpt + round256(nck * (mfma ? 2 : 4));
    lay->part = lay->prep + round256(nprep * 4);
    lay->dA = lay->part + round256(npart * 4);
    lay->dsp = lay->dA + round256(units * 4);
    lay->total = lay->dsp + round256(ndsp);
    return true;
}

}  // namespace

extern "C" {

size_t kda_prefill_bwd_workspace_size(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                                      int64_t dv) {
    if ((dtype != KDA_F32 && dtype != KDA_BF16) || dk != dv || (dk != 16 && dk != 128) ||
        B < 0 || T < 0 || H < 0)
        return 0;
    BwdLayout lay;
    return bwd_layout(dtype, B, T, H, dk, &lay) ? lay.total : 0;
}

}  // extern "C"

namespace {

// The backward on `stream`; with a second caller stream `side` (not NULL and
// not `stream`), the bf16 d = 128 path runs its prep kernel there, beside the
// forward rerun, forked from and joined back to `stream` with two events made
// for this call (destroyed once enqueued; HIP frees them when they complete).
kda_status bwd_impl(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                    const void *q, const void *k, const void *v, const void *z,
                    const void *beta, const float *A, const float *S0, const void *dO,
                    const float *dS_T, float *dq, float *dk_out, float *dv_out,
                    float *dz, float *dbeta, float *dA, float *dS0, void *workspace,
                    size_t workspace_bytes, void *stream, void *side) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (dk != dv || (dk != 16 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    const int64_t D = dk, esz = dtype == KDA_BF16 ? 2 : 4;
    BwdLayout lay;
    if (!bwd_layout(dtype, B, T, H, D, &lay)) return KDA_ERR_SHAPE;
    const int64_t bh = B * H, nchunk = (T + kBwdChunk - 1) / kBwdChunk;
    // grid sizes: the per-chunk kernels launch up to 1024 work-items per chunk
    // and a dispatch counts work-items in 32 bits (the bound is ~4.2 M
    // chunk-heads, past any workspace that fits in HBM)
    if (bh > 0x7fffffff / 8 || bh * nchunk > (int64_t)(0xffffffffu / 1024)) return KDA_ERR_SHAPE;
    if (!tile_rows_fit(H, D, esz)) return KDA_ERR_SHAPE;
    const int64_t bth = B * T * H, nin = bth * D, nst = bh * D * D;
    if (!A || !dA) return KDA_ERR_NULL;
    if (bh > 0 && (!dS0)) return KDA_ERR_NULL;
    if (bth > 0 && (!q || !k || !v || !z || !beta || !dO || !dq || !dk_out || !dv_out || !dz ||
                    !dbeta))
        return KDA_ERR_NULL;
    if (bh > 0 && (!workspace || workspace_bytes < lay.total)) return KDA_ERR_WORKSPACE;
    const void *ptrs[] = {q, k, v, z, beta, A, S0, dO, dS_T, dq, dk_out, dv_out, dz, dbeta,
                          dA, dS0, bh > 0 ? workspace : nullptr};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
    const Range ins[] = {range_of(q, nin * esz), range_of(k, nin * esz), range_of(v, nin * esz),
                         range_of(z, nin * esz), range_of(beta, bth * esz), range_of(A, H * 4),
                         range_of(S0, nst * 4), range_of(dO, nin * esz),
                         range_of(dS_T, nst * 4)};
    const Range outs[] = {range_of(dq, nin * 4), range_of(dk_out, nin * 4),
                          range_of(dv_out, nin * 4), range_of(dz, nin * 4),
                          range_of(dbeta, bth * 4), range_of(dA, H * 4), range_of(dS0, nst * 4),
                          range_of(bh > 0 ? workspace : nullptr, (int64_t)lay.total)};
    const int nout = sizeof(outs) / sizeof(outs[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return KDA_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j])) return KDA_ERR_ALIAS;
    }
    if (H == 0) return KDA_OK;   // every output is empty
    char *ws = static_cast<char *>(workspace);
    const hipStream_t s = (hipStream_t)stream;
    const int64_t nfull = T / kBwdChunk;
    float *ckpt = bh > 0 ? reinterpret_cast<float *>(ws + lay.ckpt) : nullptr;
    // bf16 d = 128 (MFMA path): the rerun writes states only (no o), its
    // checkpoints in the 4-row block layout the backward reads
    const bool mfma = kda::bwd_dsp_bytes(dtype, D) > 0;
    // forward with a checkpoint at every chunk boundary
    auto rerun = [&](void *on, bool check_only) {
        return prefill_impl(dtype, B, T, H, dk, dv, kBwdChunk, nullptr, q, k, v, z, beta, A, S0,
                            mfma ? nullptr : ws + lay.o, reinterpret_cast<float *>(ws + lay.S_T),
                            nfull > 0 ? kBwdChunk : 0, ckpt, B * nfull, nullptr, 0, on,
                            mfma ? 64 : 0, mfma ? 1 : 0, check_only, mfma);
    };
    kda::BwdArgs a;
    a.dtype = dtype; a.B = B; a.T = T; a.H = H; a.D = D; a.nchunk = nchunk;
    a.q = q; a.k = k; a.v = v; a.z = z; a.beta = beta; a.dO = dO;
    a.A = A; a.S0 = S0; a.dST = dS_T; a.ckpt = ckpt;
    a.prep = bh > 0 ? reinterpret_cast<float *>(ws + lay.prep) : nullptr;
    a.part = bh > 0 ? reinterpret_cast<float *>(ws + lay.part) : nullptr;
    a.dA_part = bh > 0 ? reinterpret_cast<float *>(ws + lay.dA) : nullptr;
    a.dsp = bh > 0 && lay.total > lay.dsp ? static_cast<void *>(ws + lay.dsp) : nullptr;
    a.dq = dq; a.dk = dk_out; a.dv = dv_out; a.dz = dz; a.dbeta = dbeta; a.dA = dA; a.dS0 = dS0;
    a.stream = s;
    if (!mfma || bth == 0 || !side || side == stream) {
        if (bth > 0) {
            const kda_status st = rerun(stream, false);
            if (st != KDA_OK) return st;
        }
        return kda::launch_bwd(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // fork: the rerun here (launched first and behind no event wait, so that
    // its 192 large workgroups get their CUs before prep's many small ones),
    // prep on the side stream; join before the dS recurrence (run beside the
    // rerun, two latency-bound chains slow each other)
    {
        const kda_status chk = rerun(nullptr, true);   // validation only, before any launch
        if (chk != KDA_OK) return chk;
    }
    const hipStream_t ss = (hipStream_t)side;
    hipEvent_t fork = nullptr, join = nullptr;
    if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess) return KDA_ERR_HIP;
    if (hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess) {
        (void)hipEventDestroy(fork);
        return KDA_ERR_HIP;
    }
    kda_status st = KDA_OK;
    if (hipEventRecord(fork, s) != hipSuccess) st = KDA_ERR_HIP;
    if (st == KDA_OK) st = rerun(stream, false);
    kda::BwdArgs af = a;
    af.stream = ss;
    if (st == KDA_OK &&
        (hipStreamWaitEvent(ss, fork, 0) != hipSuccess || kda::launch_bwd_front(af) != hipSuccess ||
         hipEventRecord(join, ss) != hipSuccess || hipStreamWaitEvent(s, join, 0) != hipSuccess))
        st = KDA_ERR_HIP;
    (void)hipEventDestroy(fork);
    (void)hipEventDestroy(join);
    if (st != KDA_OK) return st;
    return kda::launch_bwd_back(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status kda_prefill_bwd(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           const void *q, const void *k, const void *v, const void *z,
                           const void *beta, const float *A, const float *S0, const void *dO,
                           const float *dS_T, float *dq, float *dk_out, float *dv_out,
                           float *dz, float *dbeta, float *dA, float *dS0, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return bwd_impl(dtype, B, T, H, dk, dv, q, k, v, z, beta, A, S0, dO, dS_T, dq, dk_out, dv_out,
                    dz, dbeta, dA, dS0, workspace, workspace_bytes, stream, nullptr);
}

kda_status kda_prefill_bwd_ex(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              const void *q, const void *k, const void *v, const void *z,
                              const void *beta, const float *A, const float *S0, const void *dO,
                              const float *dS_T, float *dq, float *dk_out, float *dv_out,
                              float *dz, float *dbeta, float *dA, float *dS0, void *workspace,
                              size_t workspace_bytes, void *stream, void *side_stream) {
    return bwd_impl(dtype, B, T, H, dk, dv, q, k, v, z, beta, A, S0, dO, dS_T, dq, dk_out, dv_out,
                    dz, dbeta, dA, dS0, workspace, workspace_bytes, stream, side_stream);
}

}  // extern "C"
