// kda_split.hip -- one long sequence as several segments run in parallel (gfx950).
//
// The recurrence is affine in the state: over a segment, S_end = M S_start + N,
// where N is the segment's final state from S_start = 0 and M (dk x dk) the
// product of its per-token transitions (I - beta k k^T) Diag(alpha).  So a
// sequence of T tokens can run as P segments at once: (1) in one launch, the
// prefill of the first segment from the sequence's start state and, beside
// it, M and N of every segment between the first and the last (the prefill
// kernel's state-map mode: M from the identity with v read as zero, N from
// zero, on shared prep); (2) the other segments' true start states by the
// scan S_{j+1} = M_j S_j + N_j, starting from the first segment's final
// state; (3) the prefill of every other segment from its start state (the
// packed-sequence path).  With H heads, P segments make 2 H (P - 1)
// workgroups per pass.  This is the sequence-parallel
// combine of the sharding design, done inside one GPU: it turns B*H units of
// sequential work into B*H*P when B*H is too small to fill the chip (a head
// share of a million-token context has 16 heads for 256 compute units).
//
// This file holds the small kernels around the two prefill passes: the
// segment offsets and the rank lists of the passes, the copy of the start
// states, the scan, and the gather of the last segment's final state.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// cu[i] for the B*P segments: sequence b, segment j covers tokens
// [b*T + min(j*L, T), b*T + min((j+1)*L, T)) of the [B*T, H, d] packing.
// The rank lists (segment indices b*P + j): lists[0 .. B) the first segments
// (j = 0), then B*(P-2) middle ones (j = 1 .. P-2), then B*(P-1) ones with
// j = 1 .. P-1.
__global__ void kda_split_offsets_kernel(int64_t *cu, int32_t *lists, int64_t B, int64_t T,
                                         int64_t L, int P) {
    const int64_t n = B * P, nmid = B * (P - 2), nrest = B * (P - 1);
    const int64_t total = n + 1 > B + nmid + nrest ? n + 1 : B + nmid + nrest;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i <= n) {
            const int64_t b = i / P, j = i % P;
            const int64_t t = j * L < T ? j * L : T;
            cu[i] = i == n ? B * T : b * T + t;
        }
        if (i < B) lists[i] = (int32_t)(i * P);
        if (i < nmid) lists[B + i] = (int32_t)((i / (P - 2)) * P + 1 + i % (P - 2));
        if (i < nrest) lists[B + nmid + i] = (int32_t)((i / (P - 1)) * P + 1 + i % (P - 1));
    }
}

// Sstart[b*P, h] = S0[b, h] (fp32 D x D per head).
__global__ void kda_split_copy_start_kernel(const float *__restrict__ S0,
                                            float *__restrict__ Sstart, int64_t B, int64_t H,
                                            int P, int D) {
    const int64_t per = H * (int64_t)D * D;
    const int64_t total = B * per;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x)
        Sstart[(i / per) * P * per + i % per] = S0[i];
}

// Start states of segments 2 .. P-1.  One workgroup per (b, h, 32-column
// slice): S = Sstart[b*P + 1, h][:, cols] (the first segment's final state);
// for j = 1 .. P-2: S <- M_j S + N_j, Sstart[b*P + j + 1, h][:, cols] = S,
// in fp32.  S lives in LDS; thread t computes row t / 2,
// columns 16 (t % 2) .. +15 of the slice (D = 128, 256 threads).
constexpr int kScanCols = 32;
__global__ __launch_bounds__(256) void kda_split_scan_kernel(const float *__restrict__ M,
                                                             const float *__restrict__ N,
                                                             float *__restrict__ Sstart,
                                                             int64_t H, int P) {
    constexpr int D = 128, NC = kScanCols;
    __shared__ float sS[D][NC + 1];
    const int64_t x = blockIdx.x;
    const int cs = (int)(x % (D / NC));
    const int64_t bh = x / (D / NC);
    const int64_t b = bh / H, h = bh % H;
    const int c0 = cs * NC;
    const int tid = threadIdx.x;
    const int r0 = tid / 2;             // rows r0 (and the thread's 16 columns)
    const int cq = (tid % 2) * 16;      // column offset within the slice
    // the first segment's final state: the second segment's start
    {
        const int64_t u1 = (b * P + 1) * H + h;
        for (int i = tid; i < D * NC; i += 256) {
            const int r = i / NC, c = i % NC;
            sS[r][c] = Sstart[(u1 * D + r) * D + c0 + c];
        }
    }
    __syncthreads();
    for (int j = 1; j + 1 < P; ++j) {
        const int64_t u = (b * P + j) * H + h;   // (segment, head) unit
        // row r0 of M_j S + N_j, columns cq .. cq+15
        float acc[16];
        const float *Nr = N + (u * D + r0) * D + c0 + cq;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[c] = Nr[c];
        const float *Mr = M + (u * D + r0) * D;
        for (int k = 0; k < D; ++k) {
            const float m = Mr[k];
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[c] = fmaf(m, sS[k][cq + c], acc[c]);
        }
        __syncthreads();   // every thread has read sS for this step
#pragma unroll
        for (int c = 0; c < 16; ++c) sS[r0][cq + c] = acc[c];
        // and the start state of segment j + 1
        float *Sn = Sstart + ((u + H) * D + r0) * D + c0 + cq;
#pragma unroll
        for (int c = 0; c < 16; ++c) Sn[c] = acc[c];
        __syncthreads();
    }
}

// S_T[b, h] = Sseg[b*P + P - 1, h]
__global__ void kda_split_gather_kernel(const float *__restrict__ Sseg, float *__restrict__ S_T,
                                        int64_t B, int64_t H, int P, int D) {
    const int64_t per = H * (int64_t)D * D;
    const int64_t total = B * per;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / per, rest = i % per;
        S_T[i] = Sseg[(b * P + P - 1) * per + rest];
    }
}

static unsigned grid_for(int64_t n, int threads) {
    int64_t g = (n + threads - 1) / threads;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

hipError_t launch_split_setup(int64_t *cu, int32_t *lists, const float *S0, float *Sstart,
                              int64_t B, int64_t T, int64_t L, int P, int64_t H, int D,
                              hipStream_t stream) {
    if (P < 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_split_offsets_kernel, dim3(grid_for(B * P + 1, 256)), dim3(256), 0,
                       stream, cu, lists, B, T, L, P);
    if (S0)
        hipLaunchKernelGGL(kda_split_copy_start_kernel, dim3(grid_for(B * H * D * D, 256)),
                           dim3(256), 0, stream, S0, Sstart, B, H, P, D);
    return hipGetLastError();
}

hipError_t launch_split_scan(const float *M, const float *N, float *Sstart, int64_t B,
                             int64_t H, int P, int D, hipStream_t stream) {
    if (D != 128) return hipErrorInvalidValue;
    if (P < 3 || B * H == 0) return hipSuccess;   // no segment between the first and the last
    hipLaunchKernelGGL(kda_split_scan_kernel, dim3((unsigned)(B * H * (D / kScanCols))), dim3(256),
                       0, stream, M, N, Sstart, H, P);
    return hipGetLastError();
}

hipError_t launch_split_gather(const float *Sseg, float *S_T, int64_t B, int64_t H, int P, int D,
                               hipStream_t stream) {
    hipLaunchKernelGGL(kda_split_gather_kernel, dim3(grid_for(B * H * D * D, 256)), dim3(256), 0,
                       stream, Sseg, S_T, B, H, P, D);
    return hipGetLastError();
}

}  // namespace kda
