// kda_launch.h -- host-side launchers behind the C ABI (internal).
//
// The C entry points (kda_api.hip) validate every argument and then call one
// of these; they only pick a kernel instantiation, size the grid and enqueue
// it.  They return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace kda {

struct PrefillArgs {
    int dtype;          // KDA_F32 / KDA_BF16
    int64_t B, T, H, D; // dk == dv == D; B sequences (dense: of T tokens each)
    int chunk;
    int dv_per_block;   // value columns per workgroup (16 * waves)
    const void *q, *k, *v, *z, *beta;
    const float *A, *S0;
    void *o;
    float *S_T;
    float *S_T2 = nullptr;   // mode 2: the offsets N
    // Packed variable-length mode: sequence b holds tokens
    // [cu_seqlens[b], cu_seqlens[b+1]) of a [T, H, d] packing (T = total
    // tokens).  NULL: dense [B, T, H, d].
    const int64_t *cu_seqlens;
    // Optional longest-first order of the sequences (device int32 [B]): rank r
    // runs sequence order[r].  NULL: sequence order.
    const int32_t *order;
    // State checkpoints: every ckpt_every tokens of a sequence (0 = none),
    // rows of ckpt [n_ckpt, H, D, D] in sequence order.
    int ckpt_every;
    float *ckpt;
    int64_t n_ckpt;
    // Checkpoint layout: false -- fp32 row-major [D][D]; true -- bf16 in 4-row
    // blocks, state element (d, j) at ((d/4)*D + j)*4 + d%4 (the backward's own
    // rerun; role-split kernel only).
    bool ckpt_blocked = false;
    // 0: the prefill.  1: final states only (o not written).  2: the affine
    // state map S_end = M S_start + N of each sequence in one pass (M to S_T,
    // N -- the final state from S0, or zero -- to S_T2; o not written).
    // 3: M alone (the state starts at the identity, v is read as zero; M to
    // S_T; o not written).  Modes 1 and 2 run on the role-split kernel at 64
    // columns (checkpoints in mode 1 only); modes 1 and 3 on the general kernel
    // through launch_prefill_multi.
    int mode = 0;
    hipStream_t stream;
};

// Short causal convolution of one of q, k, v (prologue of a layer).
struct ConvTensor {
    const void *x;        // raw input [B, T, H, D]
    const float *w;       // taps [H, D, W]
    const void *sin;      // convolution state in [B, W-1, H, D], or NULL (zeros)
    void *y;              // output [B, T, H, D]
    void *sout;           // convolution state out, or NULL
    int norm;             // L2-normalize each token's head row
};

struct ConvNormArgs {
    int dtype;
    int64_t B, T, H, D;
    ConvTensor t[3];      // q, k, v
    int W;                // taps, 1..4
    int act;              // 0: none, 1: SiLU
    float eps;
    // Packed sequences (cu != NULL): N sequences over the T-token axis (B = 1);
    // states are [N, W-1, H, D].
    const int64_t *cu = nullptr;
    int64_t N = 0;
    int64_t ntile = 0, ngroup = 0;   // set by the launcher
    hipStream_t stream;
};

bool conv_supported(int dtype, int64_t D);
// Tokens per wave tile of the prologue kernel.
int conv_tile_tokens(int dtype, int64_t D);
hipError_t launch_conv_norm(const ConvNormArgs &a);

struct DecodeArgs {
    int dtype;
    int64_t B, H, D;
    const void *q, *k, *v, *z, *beta;
    const float *A;
    float *S;
    void *o;
    // Fused prologue (conv != 0): taps wq, wk, wv [H, D, W] and the persistent
    // convolution states cq, ck, cv [B, W-1, H, D] (updated in place).
    int conv;
    const float *wq, *wk, *wv;
    void *cq, *ck, *cv;
    int W, act;
    float eps;
    hipStream_t stream;
};

// Whether an instantiation exists for (dtype, D, chunk, dv_per_block).
bool prefill_supported(int dtype, int64_t D, int chunk, int dv_per_block);
// Default value columns per workgroup for these sizes.
int prefill_default_dv_per_block(int dtype, int64_t B, int64_t H, int64_t D, int chunk);
hipError_t launch_prefill(const PrefillArgs &a);
// Three general-kernel runs (bf16, d = 128, 64-token chunks, 128 columns per
// workgroup, modes 0, 1 or 3, no checkpoints) in one launch.
hipError_t launch_prefill_multi(const PrefillArgs *a);
// Whether the general kernel takes state checkpoints for this configuration.
bool prefill_ckpt_supported(int dtype, int64_t D, int chunk, int dv_per_block);
// Role-split variant for bf16, D = 128, chunk 16 (kda_prefill16.hip).
bool prefill16_supported(int dtype, int64_t D, int chunk, int dv_per_block);
hipError_t launch_prefill16(const PrefillArgs &a);
// One launch of the role-split kernel running a0 (mode 0) and a2 (mode 2,
// 64 columns, same H) side by side: the first pass of a sequence split.
hipError_t launch_prefill16_split_head(const PrefillArgs &a0, const PrefillArgs &a2);

// Longest-first ranking of packed sequences (device): order[rank] = sequence.
// Only used for 1 < N <= kMaxOrderSeqs.
constexpr int64_t kMaxOrderSeqs = 8192;
hipError_t launch_seq_order(const int64_t *cu, int64_t N, int64_t T, int32_t *order,
                            hipStream_t stream);

// Sequence split (kda_split.hip), P >= 2 segments per sequence.  Setup: the
// segment offsets cu [B*P + 1] and three rank lists in `lists`: the first
// segment of each sequence [B], the middle ones (1 .. P-2) [B*(P-2)], and
// all but the first [B*(P-1)]; with S0 given, S0[b] is copied to
// Sstart[b*P] (the first segment's start state).  Scan: from Sstart[b*P+1]
// (the first segment's final state), Sstart[b*P+j+1] = M_j Sstart[b*P+j] +
// N_j for j = 1 .. P-2.  Gather: S_T[b] = Sseg[b*P + P-1].
hipError_t launch_split_setup(int64_t *cu, int32_t *lists, const float *S0, float *Sstart,
                              int64_t B, int64_t T, int64_t L, int P, int64_t H, int D,
                              hipStream_t stream);
hipError_t launch_split_scan(const float *M, const float *N, float *Sstart, int64_t B,
                             int64_t H, int P, int D, hipStream_t stream);
hipError_t launch_split_gather(const float *Sseg, float *S_T, int64_t B, int64_t H, int P, int D,
                               hipStream_t stream);

// Sleeps a role-split kernel's slot wait takes before it gives up (and
// poisons the affected state columns with NaN): 2^22 by default, or the value
// of the environment variable KDA_WAIT_SPIN_LIMIT (a testing knob: a host-side
// test forces give-ups with a tiny limit, every kernel still exits normally).
int wait_spin_limit();

bool decode_supported(int dtype, int64_t D);
hipError_t launch_decode(const DecodeArgs &a);

// Chunk-parallel backward of the prefill (16-token chunks).  Inputs as in the
// prefill; dO in the input dtype, dST (dL/dS_T) fp32 or NULL (zero).  ckpt
// holds the forward's state checkpoints every 16 tokens ([B*(T/16), H, D, D]);
// prep, part and dA_part are workspace.  Gradients are fp32.
struct BwdArgs {
    int dtype;
    int64_t B, T, H, D;
    int64_t nchunk;     // ceil(T / 16)
    const void *q, *k, *v, *z, *beta, *dO;
    const float *A, *S0, *dST, *ckpt;
    float *prep, *part, *dA_part;
    void *dsp;          // incoming dS' of every chunk, bf16 [B, H, nchunk, D, D] (MFMA path), or NULL
    float *dq, *dk, *dv, *dz, *dbeta, *dA, *dS0;
    hipStream_t stream;
};
size_t bwd_prep_floats(int64_t D);   // per (b, h, chunk)
size_t bwd_part_floats(int64_t D);   // per (b, h, chunk), all column slices
size_t bwd_dsp_bytes(int dtype, int64_t D);   // per (b, h, chunk): 2*D*D on the MFMA path, else 0
hipError_t launch_bwd(const BwdArgs &a);
// the MFMA path (bf16, d = 128) in two halves: prep, which reads no state
// checkpoint and may run beside the forward rerun, then the rest
hipError_t launch_bwd_front(const BwdArgs &a);
hipError_t launch_bwd_back(const BwdArgs &a);

}  // namespace kda
