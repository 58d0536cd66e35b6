// kda_segments.hip -- the combine step of the intra-GPU segment scan.
//
// The state map of a slice of a chain is affine in the state it starts from:
// S_end = Pmap S_start + R, with Pmap (K x K) the slice's transition (its end
// state from the identity with v = 0) and R its end state from zero. With the
// first slice run for real, the start state of the next slice is one such
// product; the slices after it can then be run, in parallel, from their true
// start states. The outputs are affine in the start state as well: a slice's o
// from its true start state S is its o from zero plus S^T ell_t per token,
// with ell_t the o of the same slice run from the identity with v = 0. This
// file holds the product and that correction; the slices run in the fused
// kernel (kda_fused_pipe.hip, task table).
#include "kda_device.h"
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

// x = hi + lo for a pair of floats: hi is x cut to bf16 (x - hi is exact), lo
// that remainder rounded to bf16; together about 16 significant bits.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
    const bf16x2 l = {(__bf16)(x0 - __uint_as_float(u0 & 0xffff0000u)), (__bf16)(x1 - __uint_as_float(u1 & 0xffff0000u))};
    lo = __builtin_bit_cast(uint32_t, l);
}

constexpr int TB = 256;   // tokens per workgroup: four steps of the four waves' 16 tokens

// o[n, t, h, :] += S^T ell[n, t - e0, h, :] for one (row n, head h) and TB
// tokens t of [t0, t1); ell holds tokens e0 .. T - 1 of each row. ell (A operand: 16 tokens x 32 channels per MFMA) and S (B
// operand: 32 channels x 16 columns) each enter as two bf16 terms, three MFMA
// terms with fp32 accumulation onto o. S is staged once per workgroup in LDS
// as the B operands of its eight 16-column tiles and four 32-channel steps,
// one 16-byte piece per lane, so each lane reads its own piece.
__global__ __launch_bounds__(256) void state_correction_kernel(const float* __restrict__ S,
                                                              const float* __restrict__ ell, float* __restrict__ o,
                                                              int T, int H, int t0, int t1, int e0) {
    __shared__ uint4 Bh[8][4][64], Bl[8][4][64];
    const int chain = blockIdx.y, n = chain / H, h = chain % H;
    const int Tc = t1 - t0;
    const float* Sc = S + (size_t)chain * D * D;
    for (int p = threadIdx.x; p < 8 * 4 * 64; p += 256) {
        const int c = p >> 8, kk = (p >> 6) & 3, ln = p & 63;
        const int col = 16 * c + (ln & 15), r0 = 32 * kk + 8 * (ln >> 4);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            split_pair(Sc[(size_t)(r0 + 2 * i) * D + col], Sc[(size_t)(r0 + 2 * i + 1) * D + col], hi[i], lo[i]);
        Bh[c][kk][ln] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        Bl[c][kk][ln] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
    const size_t ts = (size_t)H * D;   // elements per token
    const float* erow = ell + ((size_t)n * (T - e0) + (t0 - e0)) * ts + (size_t)h * D;
    float* orow = o + ((size_t)n * T + t0) * ts + (size_t)h * D;
    for (int step = 0; step < TB / 64; ++step) {
        const int tt = blockIdx.x * TB + 64 * step + 16 * wave;   // first of this wave's 16 tokens
        if (tt >= Tc) break;
        // A: token tt + l16, channels 32kk + 8grp .. 32kk + 8grp + 7
        bf16x8 Ah[4], Al[4];
        const int ta = tt + l16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
            if (ta < Tc) {
                const float4* src = reinterpret_cast<const float4*>(erow + (size_t)ta * ts + 32 * kk + 8 * grp);
                x0 = src[0];
                x1 = src[1];
            }
            uint32_t hi[4], lo[4];
            split_pair(x0.x, x0.y, hi[0], lo[0]);
            split_pair(x0.z, x0.w, hi[1], lo[1]);
            split_pair(x1.x, x1.y, hi[2], lo[2]);
            split_pair(x1.z, x1.w, hi[3], lo[3]);
            Ah[kk] = __builtin_bit_cast(bf16x8, hi);
            Al[kk] = __builtin_bit_cast(bf16x8, lo);
        }
        // accumulators: o of tokens tt + 4grp + j, columns 16c + l16
        f32x4 acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tr = tt + 4 * grp + j;
                acc[c][j] = tr < Tc ? orow[(size_t)tr * ts + 16 * c + l16] : 0.f;
            }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const bf16x8 bh = __builtin_bit_cast(bf16x8, Bh[c][kk][lane]);
                const bf16x8 bl = __builtin_bit_cast(bf16x8, Bl[c][kk][lane]);
                acc[c] = mfma16(Ah[kk], bh, acc[c]);
                acc[c] = mfma16(Ah[kk], bl, acc[c]);
                acc[c] = mfma16(Al[kk], bh, acc[c]);
            }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float v[4] = {acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tr = tt + 4 * grp + j;
                if (tr < Tc) orow[(size_t)tr * ts + 16 * c + l16] = v[j];
            }
        }
    }
}

}  // namespace seg

hipError_t launch_state_correction(const float* S, const float* ell, float* o, int B, int T, int H, int t0,
                                   int t1, int e0, hipStream_t stream) {
    const int Tc = t1 - t0;
    if (B <= 0 || H <= 0 || Tc <= 0) return hipSuccess;
    hipLaunchKernelGGL(seg::state_correction_kernel, dim3((Tc + seg::TB - 1) / seg::TB, B * H), dim3(256), 0, stream,
                       S, ell, o, T, H, t0, t1, e0);
    return hipGetLastError();
}

hipError_t launch_affine_combine(const float* Pmap, const float* S_in, const float* R, float* S_out,
                                 int nchains, hipStream_t stream) {
    if (nchains <= 0) return hipSuccess;
    hipLaunchKernelGGL(seg::affine_combine_kernel, dim3(nchains, seg::D / seg::CB), dim3(256), 0, stream,
                       Pmap, S_in, R, S_out);
    return hipGetLastError();
}

}  // namespace kda
