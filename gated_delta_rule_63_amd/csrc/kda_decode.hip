// kda_decode.hip -- one KDA recurrence step per (sequence, head): the decode
// step that follows a prefill (one new token per sequence).
//
//   S' = Diag(exp g) S,   e = v - S'^T k,   S'' = S' + beta k e^T,   o = S''^T q
//
// The state is the whole cost: 64 KiB read and 64 KiB written per (sequence,
// head), against 1.3 KB of token inputs, so the kernel is HBM-bound and is
// organised for one coalesced pass over S. A (sequence, head) is split over
// CB workgroups of 128 / CB columns (CB = 4 when there are few sequences, so
// that enough workgroups stream the state; 1 otherwise), each of 256 / CB
// threads; thread t holds rows 16*(t/CG) .. +15 of four columns in registers
// (CG = 32 / CB column groups of four). The two column sums (S'^T k and
// S'^T q) are reduced across the eight row groups through LDS; then
//   o = S'^T q + beta e (k . q)
// needs no second pass, and each thread writes back exactly the block it read
// (so the state may be updated in place).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace decode {

constexpr int RG = 8;            // row groups of 16 rows

template <bool F32, int CB>
__global__ __launch_bounds__(256 / CB) void kda_decode_kernel(FwdArgs a) {
    constexpr int NT = 256 / CB;           // threads per workgroup
    constexpr int CG = 32 / CB;            // column groups of 4 columns
    const int nh = blockIdx.x / CB;        // sequence * H + head
    if (nh >= a.nchains) return;
    const int n = nh / a.H, h = nh % a.H;
    const int t = threadIdx.x, cg = t % CG, rg = t / CG;
    const long long tok = ((long long)n * a.H + h) * D;   // [N, 1, H, 128] inputs
    const long long sb = (long long)nh * D * D;           // [N, H, 128, 128] state

    __shared__ float sk[D], sq[D], sgam[D];
    __shared__ float4 pk[RG][CG], pq[RG][CG];
    __shared__ float pkq[RG];
    for (int i = t; i < D; i += NT) {
        sk[i] = ld_in<F32>(a.k, tok + i);
        sq[i] = ld_in<F32>(a.q, tok + i);
        sgam[i] = expf(a.scalar_gate ? a.g[(long long)n * a.H + h] : a.g[tok + i]);
    }
    // this thread's block of the state
    float4 s[16];
    const int v0 = (blockIdx.x % CB) * (D / CB) + 4 * cg;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int c = 16 * rg + r;
        s[r] = a.h0 ? *reinterpret_cast<const float4*>(a.h0 + sb + (long long)c * D + v0) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    // decay, then the partial column sums over this thread's 16 rows
    float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), aq = ak;
    float kq = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int c = 16 * rg + r;
        const float gm = sgam[c], kc = sk[c], qc = sq[c];
        s[r].x *= gm; s[r].y *= gm; s[r].z *= gm; s[r].w *= gm;
        ak.x += s[r].x * kc; ak.y += s[r].y * kc; ak.z += s[r].z * kc; ak.w += s[r].w * kc;
        aq.x += s[r].x * qc; aq.y += s[r].y * qc; aq.z += s[r].z * qc; aq.w += s[r].w * qc;
        kq += kc * qc;
    }
    pk[rg][cg] = ak;
    pq[rg][cg] = aq;
    if (cg == 0) pkq[rg] = kq;
    __syncthreads();
    float4 K = pk[0][cg], Q = pq[0][cg];
    float kqt = pkq[0];
#pragma unroll
    for (int i = 1; i < RG; ++i) {
        const float4 x = pk[i][cg], y = pq[i][cg];
        K.x += x.x; K.y += x.y; K.z += x.z; K.w += x.w;
        Q.x += y.x; Q.y += y.y; Q.z += y.z; Q.w += y.w;
        kqt += pkq[i];
    }
    const float beta = a.beta[(long long)n * a.H + h];
    const float4 e = make_float4(ld_in<F32>(a.v, tok + v0) - K.x, ld_in<F32>(a.v, tok + v0 + 1) - K.y,
                                 ld_in<F32>(a.v, tok + v0 + 2) - K.z, ld_in<F32>(a.v, tok + v0 + 3) - K.w);
    const float4 be = make_float4(beta * e.x, beta * e.y, beta * e.z, beta * e.w);
    if (rg == 0)
        *reinterpret_cast<float4*>(a.o + tok + v0) =
            make_float4(Q.x + be.x * kqt, Q.y + be.y * kqt, Q.z + be.z * kqt, Q.w + be.w * kqt);
    if (a.hT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = 16 * rg + r;
            const float kc = sk[c];
            *reinterpret_cast<float4*>(a.hT + sb + (long long)c * D + v0) =
                make_float4(s[r].x + kc * be.x, s[r].y + kc * be.y, s[r].z + kc * be.z, s[r].w + kc * be.w);
        }
    }
}

}  // namespace decode

hipError_t launch_decode(const FwdArgs& a, bool f32_inputs, hipStream_t stream) {
    if (a.nchains == 0) return hipSuccess;
    // few (sequence, head) pairs: four workgroups each, so that four times as
    // many workgroups stream the state
    const bool split = a.nchains < 512;
    const dim3 grid(split ? 4 * a.nchains : a.nchains);
    if (f32_inputs) {
        if (split) hipLaunchKernelGGL((decode::kda_decode_kernel<true, 4>), grid, dim3(64), 0, stream, a);
        else hipLaunchKernelGGL((decode::kda_decode_kernel<true, 1>), grid, dim3(256), 0, stream, a);
    } else {
        if (split) hipLaunchKernelGGL((decode::kda_decode_kernel<false, 4>), grid, dim3(64), 0, stream, a);
        else hipLaunchKernelGGL((decode::kda_decode_kernel<false, 1>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kda
