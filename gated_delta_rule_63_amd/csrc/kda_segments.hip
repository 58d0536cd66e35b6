// kda_segments.hip -- the combine step of the intra-GPU segment scan.
//
// The state map of a slice of a chain is affine in the state it starts from:
// S_end = Pmap S_start + R, with Pmap (K x K) the slice's transition (its end
// state from the identity with v = 0) and R its end state from zero. With the
// first slice run for real, the start state of the next slice is one such
// product; the slices after it can then be run, in parallel, from their true
// start states. This file holds the product; the slices run in the fused
// kernel (kda_fused_pipe.hip, task table).
#include "kda_launch.h"

namespace kda {
namespace seg {

constexpr int D = 128;
constexpr int CB = 16;   // output columns per workgroup

// S_out = Pmap S_in + R for one (sequence, head) and 16 columns, fp32. Thread t
// owns row t / 2 and columns 8 (t % 2) .. +7 of the block; S_in's columns are
// staged in LDS.
__global__ __launch_bounds__(256) void affine_combine_kernel(const float* Pm, const float* Sin, const float* R,
                                                             float* Sout) {
    const long long off = (long long)blockIdx.x * D * D;
    const int cb = blockIdx.y * CB;
    __shared__ float sS[D][CB + 1];
    for (int i = threadIdx.x; i < D * CB; i += 256) {
        const int k = i / CB, c = i % CB;
        sS[k][c] = Sin[off + (long long)k * D + cb + c];
    }
    __syncthreads();
    const int r = threadIdx.x >> 1, c0 = 8 * (threadIdx.x & 1);
    const long long ro = off + (long long)r * D + cb + c0;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = R[ro + j];
    const float* prow = Pm + off + (long long)r * D;
    for (int k = 0; k < D; ++k) {
        const float p = prow[k];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(p, sS[k][c0 + j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) Sout[ro + j] = acc[j];
}

}  // namespace seg

hipError_t launch_affine_combine(const float* Pmap, const float* S_in, const float* R, float* S_out,
                                 int nchains, hipStream_t stream) {
    if (nchains <= 0) return hipSuccess;
    hipLaunchKernelGGL(seg::affine_combine_kernel, dim3(nchains, seg::D / seg::CB), dim3(256), 0, stream,
                       Pmap, S_in, R, S_out);
    return hipGetLastError();
}

}  // namespace kda
