/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) on AMD Instinct
 * MI355X (gfx950).
 *
 * KDA is the gated delta-rule recurrence of "Kimi K3 Open Weights: What Is
 * Actually New In Its 2.8 Trillion Parameter Architecture" (shivasnotes.com),
 * section 1 "Kimi Delta Attention is a real new kernel family":
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *     alpha_t = exp(g_t),  g_t = g_min * sigma(e^{A_h} z_t),  g_min = -5
 *
 * per batch entry b and head h.  S_t has dk key rows and dv value columns;
 * alpha_t is a per-key-channel vector scaling S's rows; sigma is the logistic
 * function.  The same section splits the work into a chunked-parallel prefill
 * (the tokens of a chunk handled together) and a fused recurrent one-token
 * decode step whose state persists between calls.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer on the current HIP device; the
 *    caller owns all memory and every stream.  The library allocates no device
 *    memory.  Its only state across calls is the per-device address of the
 *    static scratch of kda_prefill_varlen_noalloc, set once per device; calls
 *    are thread-safe and re-entrant (except that noalloc calls overlapping on
 *    one GPU share that scratch).
 *  - Layouts are dense row-major:
 *        q, k, z : [B, T, H, dk]        v, o : [B, T, H, dv]
 *        beta    : [B, T, H]            A    : [H]  (fp32)
 *        S0, S_T : [B, H, dk, dv]  (fp32; key rows, value columns)
 *    Decode drops the T axis.  q, k, v, z, beta and o use `dtype`; A and every
 *    state tensor are fp32.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns without waiting.  All argument checks run before anything is
 *    enqueued: on any error status nothing is launched and no output is
 *    written.  A failed launch returns KDA_ERR_HIP.
 *  - Pointers must be 16-byte aligned.  Sizes are int64.
 *  - Supported: dtype in {KDA_F32, KDA_BF16}; dk == dv in {16, 128}; prefill
 *    chunk in {16, 64}, except fp32 with dk = 128, which runs chunk 16 only
 *    (its chunk-64 tiles do not fit in LDS).  Anything else returns
 *    KDA_ERR_UNSUPPORTED.
 *  - Numerics: fp32 accumulation and an fp32 state.  bf16 outputs are rounded
 *    to nearest even.  NaN/Inf inputs are not checked and propagate.  Results
 *    are bitwise reproducible run to run (no atomics in the arithmetic).
 *  - Internal waits are bounded.  The prefill kernels hand chunks between
 *    waves of a workgroup through LDS counters; a wave that waits longer than
 *    its bound (2^22 sleeps, about a tenth of a second; never seen) gives up,
 *    and every state column it may have corrupted is then written to S_T as
 *    NaN, so a give-up never passes for a valid result (o of those columns is
 *    then unreliable as well).  The environment variable KDA_WAIT_SPIN_LIMIT,
 *    read at each launch, lowers the bound for testing.
 *  - Preconditions (not checked): q and k are L2-normalised over dk (the
 *    caller's Q/K normalisation; the chunkwise rescaling relies on |k_d| <= 1
 *    for its bf16 range), beta is used as given.  The *_conv entry points
 *    take raw q, k, v instead and run the layer's prologue (short
 *    convolutions and the q/k normalisation) themselves.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 8

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                    */
    KDA_ERR_SHAPE = 2,       /* a size is negative, or a product of sizes (B*H,
                              * element counts, or a launch's work-items, which a
                              * dispatch counts in 32 bits: B*H heads above ~1 M
                              * for prefill, ~8.4 M for decode, B*H*ceil(T/16)
                              * above ~4.2 M for the backward) is too large, or
                              * 64 tokens' rows (64*H*d elements) of the
                              * prefill, prologue or backward inputs pass
                              * 2^31 bytes (bf16, d = 128: H above 131,071)    */
    KDA_ERR_UNSUPPORTED = 3, /* dtype / head size / chunk outside the set      */
    KDA_ERR_MISALIGNED = 4,  /* a pointer is not 16-byte aligned               */
    KDA_ERR_ALIAS = 5,       /* outputs overlap inputs (other than S_T == S0)  */
    KDA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required     */
    KDA_ERR_HIP = 7          /* the HIP runtime reported an error              */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *kda_status_str(int status);

/* Bytes of device workspace kda_prefill needs for these sizes (0 means none:
 * NULL may then be passed).  Returns 0 for unsupported arguments too. */
size_t kda_prefill_workspace_size(int dtype, int64_t B, int64_t T, int64_t H,
                                  int64_t dk, int64_t dv, int32_t chunk);

/*
 * Chunkwise prefill over T tokens (the prefill half of the prefill/decode
 * split in the section cited above).  Tokens are grouped into chunks of
 * `chunk`; within a chunk all interactions run as dense tiles, between chunks
 * the state is carried.  A last partial chunk is allowed (any T >= 0).
 *
 *   in : q, k, z [B,T,H,dk], v [B,T,H,dv], beta [B,T,H] (dtype); A [H] fp32;
 *        S0 [B,H,dk,dv] fp32, or NULL for a zero initial state.
 *   out: o [B,T,H,dv] (dtype) -- o_t = S_t^T q_t, the raw read, no scale;
 *        S_T [B,H,dk,dv] fp32 -- the state after token T-1 (S0 when T = 0).
 *        S_T may be the same pointer as S0 (in-place state carry); any other
 *        overlap between an output and an input is KDA_ERR_ALIAS.
 *   workspace: device memory of at least kda_prefill_workspace_size(...)
 *        bytes (may be NULL when that size is 0).
 * The result depends on `chunk` only through floating-point rounding.
 */
kda_status kda_prefill(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                       int64_t dv, int32_t chunk,
                       const void *q, const void *k, const void *v, const void *z,
                       const void *beta, const float *A, const float *S0,
                       void *o, float *S_T,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Same as kda_prefill, with the number of value columns each workgroup owns
 * fixed by the caller (`dv_per_block` in {16, 32, 64, 128}, dividing dv; 0
 * picks automatically).  Value columns of the state evolve independently, so
 * every choice gives the same result up to rounding order; it only changes
 * how the work is spread over the GPU.  With dk = 128, chunk 64 runs 32, 64
 * or 128 columns per workgroup (bf16 only; 0 picks 128); other values return
 * KDA_ERR_UNSUPPORTED.
 */
kda_status kda_prefill_ex(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                          int64_t dv, int32_t chunk,
                          const void *q, const void *k, const void *v, const void *z,
                          const void *beta, const float *A, const float *S0,
                          void *o, float *S_T,
                          void *workspace, size_t workspace_bytes, void *stream,
                          int32_t dv_per_block);

/*
 * Prefill over N variable-length sequences packed along one token axis, with
 * optional state checkpoints.  The KDA state persists per request and layer,
 * and a reused prefix is only valid together with the KDA state checkpoint
 * taken at the same token boundary ("Kimi K3 Open Weights: What Is
 * Actually New ...", section "Why '104B active' still understates the systems
 * problem"); this entry point produces those checkpoints as it goes.
 *
 *   cu_seqlens : DEVICE int64 [N+1], 8-byte aligned.  Sequence i is tokens
 *                [cu_seqlens[i], cu_seqlens[i+1]) of the packing.  Expected:
 *                cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T_total
 *                (not checked on the host; the kernels clamp every range into
 *                [0, T_total], so malformed offsets cannot cause an access
 *                outside the tensors).
 *   in : q, k, z [T_total,H,dk], v [T_total,H,dv], beta [T_total,H] (dtype);
 *        A [H] fp32; S0 [N,H,dk,dv] fp32 per sequence, or NULL (zeros).
 *   out: o [T_total,H,dv] (dtype); S_T [N,H,dk,dv] fp32, the state after each
 *        sequence's last token (S_T may be S0 itself).
 *   ckpt_every : 0 for no checkpoints, else a positive multiple of `chunk`.
 *        For sequence i of length L_i, checkpoint j = 1 .. floor(L_i /
 *        ckpt_every) is the state after token j*ckpt_every - 1 of the
 *        sequence, written to row  R_i + j - 1  of ckpt [n_ckpt,H,dk,dv]
 *        (fp32), where R_i = sum over earlier sequences of floor(L / ckpt_every).
 *        Rows at or beyond n_ckpt are not written.  ckpt must not overlap any
 *        other argument.
 *   workspace: device memory of at least kda_prefill_varlen_workspace_size(N)
 *        bytes, 16-byte aligned (NULL allowed when that size is 0).  The call
 *        ranks the sequences longest first there, and the kernels dispatch
 *        the long sequences first, which balances the load of a mixed batch.
 *        Its contents are scratch; calls sharing a workspace must not overlap.
 * All other conventions (dtype, sizes, alignment, aliasing, errors, the
 * dv_per_block split) are those of kda_prefill_ex; each sequence's result is
 * that of kda_prefill on the sequence alone.
 */
kda_status kda_prefill_varlen(int dtype, int64_t N, int64_t T_total, int64_t H,
                              int64_t dk, int64_t dv, int32_t chunk,
                              const int64_t *cu_seqlens,
                              const void *q, const void *k, const void *v, const void *z,
                              const void *beta, const float *A, const float *S0,
                              void *o, float *S_T,
                              int32_t ckpt_every, float *ckpt, int64_t n_ckpt,
                              void *workspace, size_t workspace_bytes,
                              void *stream, int32_t dv_per_block);

/* Bytes of device workspace kda_prefill_varlen needs for N sequences (0 for
 * N <= 1, and above 8192 sequences, which run in sequence order). */
size_t kda_prefill_varlen_workspace_size(int64_t N);

/*
 * kda_prefill_varlen for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call without a workspace argument.  The longest-first
 * ranking of the sequences goes to a static scratch array inside the library
 * (32 KiB per GPU, for at most 8192 sequences, set up on the first call on
 * each device and held until the process ends); nothing is allocated.
 *   N > 8192 returns KDA_ERR_WORKSPACE (beyond the scratch); every other
 *   argument, check and result is that of kda_prefill_varlen (bit for bit).
 * All calls on one GPU share that GPU's scratch: calls that overlap in time on
 * one GPU (different streams, threads) race and must be serialised by the
 * caller.  The scratch needs no clearing: each call writes every rank it
 * reads, before reading it, in stream order.
 */
kda_status kda_prefill_varlen_noalloc(int dtype, int64_t N, int64_t T_total, int64_t H,
                                      int64_t dk, int64_t dv, int32_t chunk,
                                      const int64_t *cu_seqlens,
                                      const void *q, const void *k, const void *v,
                                      const void *z, const void *beta, const float *A,
                                      const float *S0, void *o, float *S_T,
                                      int32_t ckpt_every, float *ckpt, int64_t n_ckpt,
                                      void *stream, int32_t dv_per_block);

/*
 * Prefill of long sequences split into `segments` parallel pieces.
 *
 * The recurrence is affine in the state, so over a segment S_end = M S_start
 * + N (M: the product of the segment's transitions (I - beta k k^T)Diag(alpha),
 * N: its final state from a zero start).  Splitting a sequence and combining
 * the pieces through these maps is the sequence-parallel form of the same
 * section's recurrence; here it runs inside one GPU to occupy it when B*H
 * alone cannot (a head share of a long context: e.g. H = 16, T = 2^20).  Each
 * sequence is cut into `segments` pieces of L = ceil(T / segments) tokens
 * rounded up to a whole chunk (trailing pieces may be empty); the call runs
 * (1) in one launch, the prefill of each sequence's first piece from S0 and M
 * and N of every piece between the first and the last (chunk 16: M and N of a
 * piece share one pass over its per-chunk preparation; chunk 64: they are
 * runs of their own), (2) the pieces' start states by the scan
 * S_{j+1} = M_j S_j + N_j in fp32, (3) every other piece from its start
 * state.  It costs about two prefills of work spread over B*H*segments
 * units (chunk 64: up to three).
 *
 * Arguments and results as kda_prefill (o, S_T identical in meaning; S_T may
 * be S0).  Supported: bf16, dk = dv = 128, chunk 16 or 64,
 * 1 <= segments <= 1024 (1: the plain prefill).  workspace:
 * kda_prefill_split_workspace_size bytes,
 * 16-byte aligned, not overlapping any other argument; scratch (calls sharing
 * it must not overlap).  The result equals the unsplit call's up to rounding
 * (the start states pass through bf16-rounded products once more).
 */
kda_status kda_prefill_split(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                             int64_t dv, int32_t chunk, int32_t segments,
                             const void *q, const void *k, const void *v, const void *z,
                             const void *beta, const float *A, const float *S0,
                             void *o, float *S_T,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace kda_prefill_split needs (0 for segments == 1 and for
 * unsupported arguments). */
size_t kda_prefill_split_workspace_size(int dtype, int64_t B, int64_t T, int64_t H,
                                        int64_t dk, int64_t dv, int32_t chunk,
                                        int32_t segments);

/*
 * Backward of the prefill: gradients of a loss L through the recurrence of
 * section 1, in the chunked-parallel form that the K3 coverage page
 * (nishifamily.com/k3, innovation table, row "Kimi Delta Attention (linear)")
 * names as the next KDA primitive after the serving form.
 *
 *   in : q, k, z [B,T,H,dk], v [B,T,H,dv], beta [B,T,H] (dtype), A [H] fp32,
 *        S0 [B,H,dk,dv] fp32 or NULL (zeros) -- the forward call's inputs;
 *        dO [B,T,H,dv] (dtype) = dL/do; dS_T [B,H,dk,dv] fp32 = dL/dS_T, or
 *        NULL (zero).
 *   out (all fp32): dq, dk, dz [B,T,H,dk]; dv [B,T,H,dv]; dbeta [B,T,H];
 *        dA [H] (summed over b, t and key channels); dS0 [B,H,dk,dv].
 *        Every output is written in full (dS0 also when S0 is NULL).
 *   workspace: kda_prefill_bwd_workspace_size bytes, 16-byte aligned; scratch
 *        (calls sharing it must not overlap).
 *
 * The call reruns the forward with a state checkpoint every 16 tokens, then
 * works chunk by chunk in reverse: per 16-token chunk the S-independent
 * factors in parallel, the state gradient carried backwards over the chunks
 * (one workgroup per (b, h, 64 value columns)), and the per-token gradients
 * in parallel again.  For bf16 inputs with dk = dv = 128 the state-gradient
 * chain and the value-column contractions run on bf16 matrix-core tiles with
 * fp32 accumulation (the forward's operand precision; the forward rerun's
 * state checkpoints and the per-chunk dL/dS' hand-off between them are kept
 * in bf16 in the workspace); every other case, and all per-token work, is
 * fp32.  No atomics, so results are bitwise reproducible.
 * Every kernel runs on `stream`, in order (see kda_prefill_bwd_ex for an
 * overlapped variant).
 * Supported: dtype in {KDA_F32, KDA_BF16}, dk == dv in {16, 128}.  Outputs
 * must not overlap one another, any input or the workspace.  Errors as
 * kda_prefill_ex.
 */
kda_status kda_prefill_bwd(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                           int64_t dv,
                           const void *q, const void *k, const void *v, const void *z,
                           const void *beta, const float *A, const float *S0,
                           const void *dO, const float *dS_T,
                           float *dq, float *dk_out, float *dv_out, float *dz,
                           float *dbeta, float *dA, float *dS0,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill_bwd with a second stream of the caller's (`side_stream`, on the
 * same device; NULL or equal to `stream` gives kda_prefill_bwd itself).  On
 * the bf16 dk = dv = 128 path the per-chunk prep kernel, which reads no state
 * checkpoint, then runs on `side_stream` beside the forward rerun on
 * `stream`: forked after the work already on `stream`, joined back before the
 * state-gradient chain, with two events created for the call and destroyed
 * once enqueued.  Results are identical bit for bit.  All work stays ordered
 * after earlier work on `stream`, later work on `stream` sees every output,
 * and nothing else is enqueued on `side_stream` (work queued there after the
 * call may run before the call's prep finishes; it never runs alongside
 * earlier work on `stream` that the call depends on).  Use one side stream
 * per concurrent call.
 */
kda_status kda_prefill_bwd_ex(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                              int64_t dv,
                              const void *q, const void *k, const void *v, const void *z,
                              const void *beta, const float *A, const float *S0,
                              const void *dO, const float *dS_T,
                              float *dq, float *dk_out, float *dv_out, float *dz,
                              float *dbeta, float *dA, float *dS0,
                              void *workspace, size_t workspace_bytes, void *stream,
                              void *side_stream);

/* Bytes of workspace kda_prefill_bwd needs (0 for unsupported arguments). */
size_t kda_prefill_bwd_workspace_size(int dtype, int64_t B, int64_t T, int64_t H,
                                      int64_t dk, int64_t dv);

/*
 * One fused recurrent decode step for B sequences (the decode half of the
 * same section's prefill/decode split: the state is updated once per token
 * and layer and persists between calls).
 *
 *   in : q, k, z [B,H,dk], v [B,H,dv], beta [B,H] (dtype); A [H] fp32.
 *   in/out: S [B,H,dk,dv] fp32 -- read once and overwritten with S_t.
 *   out: o [B,H,dv] (dtype), o = S_t^T q.  o must not overlap any input or S.
 * Each state entry is read once and written once per call.
 */
kda_status kda_decode_step(int dtype, int64_t B, int64_t H, int64_t dk, int64_t dv,
                           const void *q, const void *k, const void *v, const void *z,
                           const void *beta, const float *A,
                           float *S, void *o, void *stream);

/* ------------------------------------------------------------------------
 * The layer prologue: short convolutions and Q/K normalisation.
 *
 * "Kimi K3 Open Weights: What Is Actually New ...", section 1, lists short
 * convolutions and Q/K normalisation among the steps of a KDA prefill and
 * says one-token decode keeps a convolution state persistent beside the
 * recurrent state; section "Why '104B active' still understates the systems
 * problem" counts that short-convolution state per request and layer.  The
 * page gives no width, activation or normalisation guard; this library reads
 * the steps as follows (each choice a parameter where one exists):
 *
 *   1. q, k and v each pass through their own causal depthwise convolution
 *      over the tokens of a sequence, channel c of token t being
 *          y_t[c] = sum_{j=0}^{W-1} w[c][j] * x_{t-(W-1)+j}[c]
 *      (tap W-1 weighs the current token).  Tokens before the segment come
 *      from the convolution state: the last W-1 RAW inputs of the sequence,
 *      oldest first; a fresh sequence uses zeros.
 *   2. Optionally y <- y * logistic(y) (KDA_ACT_SILU).
 *   3. q and k are L2-normalised per token and head over their dk channels:
 *      x <- x / sqrt(sum_c x[c]^2 + eps).  v is not normalised.
 *   4. z and beta bypass the prologue.
 * The recurrence then runs on the results exactly as in kda_prefill /
 * kda_decode_step.
 *
 * Convolution-state layout: one tensor per input, [B, W-1, H, d] in `dtype`
 * (the raw inputs themselves, so the state is exact).  States are passed as a
 * HOST array of three device pointers {q state, k state, v state}.  With
 * W = 1 the states are empty and the arrays are not read.
 * ------------------------------------------------------------------------ */

typedef enum kda_activation {
    KDA_ACT_NONE = 0,
    KDA_ACT_SILU = 1
} kda_activation;

/* Prologue parameters (a host struct; the taps are device memory). */
typedef struct kda_short_conv {
    int32_t width;       /* W, taps per channel, 1..4                         */
    int32_t activation;  /* KDA_ACT_NONE or KDA_ACT_SILU                      */
    float eps;           /* normalisation guard, finite and >= 0              */
    int32_t reserved;    /* must be 0                                         */
    const float *wq;     /* [H, dk, W] fp32, taps of q's channels             */
    const float *wk;     /* [H, dk, W] fp32                                   */
    const float *wv;     /* [H, dv, W] fp32                                   */
} kda_short_conv;

/*
 * The prologue alone over a segment of T tokens:
 *   in : q, k [B,T,H,dk], v [B,T,H,dv] raw (dtype); conv (host, non-NULL);
 *        state_in: NULL (zero states) or 3 device pointers [B,W-1,H,d].
 *   out: q_out, k_out [B,T,H,dk] (normalised), v_out [B,T,H,dv] (dtype,
 *        rounded once from fp32); state_out: NULL (not written) or 3 device
 *        pointers receiving the states after the segment (T = 0 copies
 *        state_in).
 * No output may overlap an input or another output (KDA_ERR_ALIAS).  Other
 * conventions as kda_prefill; supported for the same dtypes and dk == dv in
 * {16, 128}.  Invalid width / activation / eps / reserved: KDA_ERR_UNSUPPORTED.
 */
kda_status kda_conv_norm(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                         int64_t dv, const kda_short_conv *conv,
                         const void *q, const void *k, const void *v,
                         const void *const *state_in, void *const *state_out,
                         void *q_out, void *k_out, void *v_out, void *stream);

/*
 * The prologue over N packed variable-length sequences (the layout of
 * kda_prefill_varlen: cu_seqlens device int64 [N+1], 8-byte aligned; tokens
 * [cu_seqlens[i], cu_seqlens[i+1]) belong to sequence i; offsets are clamped
 * into [0, T_total]).  q, k, v, q_out, k_out, v_out: [T_total, H, d]; the
 * convolution states are per sequence, [N, W-1, H, d] each: a token's taps
 * never reach into another sequence, they read its sequence's state_in rows
 * (or zeros) instead, and state_out receives each sequence's last W-1 raw
 * inputs.  Each sequence's result equals kda_conv_norm on that sequence
 * alone.  Other conventions as kda_conv_norm.
 */
kda_status kda_conv_norm_varlen(int dtype, int64_t N, int64_t T_total, int64_t H, int64_t dk,
                                int64_t dv, const int64_t *cu_seqlens,
                                const kda_short_conv *conv,
                                const void *q, const void *k, const void *v,
                                const void *const *state_in, void *const *state_out,
                                void *q_out, void *k_out, void *v_out, void *stream);

/* Bytes of device workspace kda_prefill_conv needs (the prologue's outputs:
 * three [B,T,H,d] tensors in dtype, each rounded up to 256 bytes). */
size_t kda_prefill_conv_workspace_size(int dtype, int64_t B, int64_t T, int64_t H,
                                       int64_t dk, int64_t dv, int32_t chunk);

/*
 * Prologue + chunkwise prefill: kda_conv_norm of the raw q, k, v into the
 * workspace, then kda_prefill_ex on the results.  Arguments as in those two
 * calls; workspace (16-byte aligned, at least
 * kda_prefill_conv_workspace_size bytes) must not overlap any other argument,
 * and state_out must not overlap state_in.  Every check of both steps runs
 * before the first launch.
 */
kda_status kda_prefill_conv(int dtype, int64_t B, int64_t T, int64_t H, int64_t dk,
                            int64_t dv, int32_t chunk, const kda_short_conv *conv,
                            const void *q, const void *k, const void *v, const void *z,
                            const void *beta, const float *A,
                            const void *const *state_in, void *const *state_out,
                            const float *S0, void *o, float *S_T,
                            void *workspace, size_t workspace_bytes, void *stream,
                            int32_t dv_per_block);

/*
 * One decode step with the prologue fused in: q, k, v [B,H,d] are the raw
 * inputs of the new token; `state` (3 device pointers, required when W > 1)
 * holds each sequence's convolution states and is updated in place (shifted
 * by one token), as S is.  The result is that of kda_conv_norm over the one
 * token followed by kda_decode_step.  State tensors must not overlap each
 * other, an input, S or o.
 */
kda_status kda_decode_step_conv(int dtype, int64_t B, int64_t H, int64_t dk, int64_t dv,
                                const kda_short_conv *conv,
                                const void *q, const void *k, const void *v, const void *z,
                                const void *beta, const float *A,
                                void *const *state, float *S, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
