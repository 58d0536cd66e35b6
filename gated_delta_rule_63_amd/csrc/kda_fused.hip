// kda_fused.hip -- the fused chunked KDA forward for gfx950.
//
// One workgroup owns one (sequence, head, V-block) chain and walks its chunks
// in order. Per chunk of C = 32 tokens it
//   (1) scans the log-gate within each 16-token sub-block and forms the gated
//       key/query factors (per-chunk cumulative log-gate scan);
//   (2) builds the beta-weighted strictly-lower gated K K^T (A) and the lower
//       gated Q K^T (M) on MFMA, and solves T = (I + A)^{-1} by forward
//       substitution on the A tile staged in LDS;
//   (3) advances the 128 x 16-per-wave fp32 state on MFMA:
//           E = V - (K*gamma) S,  Delta = T Diag(beta) E,
//           S <- Diag(gamma_last) S + (K*exp(Gamma_last - Gamma))^T Delta;
//   (4) writes O = (Q*gamma) S + M Delta before the update.
// These are the four steps of the chunked prefill; the pages credit a chunked
// two-kernel CUTLASS design on Hopper (toolarium.ru page, section
// "Где ограничения прямо сейчас"). Here all four run in one kernel so each
// input byte crosses HBM once, because MI355X's ratio of matrix throughput to
// HBM bandwidth makes this path bandwidth-bound.
//
// Gating factors are referenced to the middle of each 16-token sub-block, so
// for g >= -5 every factor lies in [e^-40, e^40] and stays a normal fp32/bf16
// number (the pages' reason for short chunks: the bf16 numeric range).
//
// Precision. bf16 inputs: the gated K K^T / Q K^T blocks use two-term bf16
// splits (3 MFMAs per product, fp32 range); (K*gamma) S and (Q*gamma) S use
// fp16 operands; T Diag(beta) E, M Delta and Kt^T Delta split their V-scale
// operands into fp16 hi + lo. fp32 inputs: A and M on fp32 MFMA and every
// other product split into fp16 hi + lo on both sides.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace fused {

constexpr int C = 32;          // chunk length
constexpr int NW = 4;          // waves per workgroup, each owns 16 V columns
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int VB = 16 * NW;    // V columns per workgroup
constexpr int P = D / VB;      // workgroups per (sequence, head)
constexpr int LDP = D + 8;     // padded row of a 2-byte [row][128] array
constexpr int LDF = D + 4;     // padded row of a 4-byte [row][128] array
constexpr int TP = C + 8;      // padded row of a 2-byte [row][32] array
constexpr int LDA = C + 4;     // padded row of the fp32 A tile
static_assert(NT == 2 * D, "the scan maps one thread to each (channel, 16-token sub-block)");
static_assert(C == 32, "the sub-block bookkeeping below is written for two 16-token sub-blocks");

template <bool F32> struct AMStore;
template <> struct AMStore<true> {   // fp32 operands for 16x16x4 fp32 MFMA
    float Ka[C][LDF], Qa[C][LDF], Kb[C][LDF], Kr[16][LDF];
};
template <> struct AMStore<false> {  // [hi, lo] bf16 operands
    __bf16 Ka[2][C][LDP], Qa[2][C][LDP], Kb[2][C][LDP], Kr[2][16][LDP];
};

template <bool F32> struct alignas(16) Smem {
    AMStore<F32> am;
    _Float16 Kg[F32 ? 2 : 1][C][LDP];   // K * exp(Gamma), channels permuted in 32-groups
    _Float16 Qg[F32 ? 2 : 1][C][LDP];   // Q * exp(Gamma), same order
    _Float16 KtT[2][D][TP];             // (K * exp(Gamma_last - Gamma))^T, [hi, lo][channel][kperm(token)]
    float A[C][LDA];                    // beta-weighted strictly-lower gated K K^T
    _Float16 Tm[2][C][TP];              // (I + A)^{-1}, [hi, lo][row][kperm(col)]
    _Float16 M[2][C][TP];               // lower gated Q K^T, [hi, lo][row][kperm(col)]
    float gl[D];                        // exp(Gamma_last), the chunk's decay per channel
    float beta[C];
    float tot[2][D];                    // sum of g over each sub-block
    float mid1[D];                      // Gamma(token 23) - Gamma(token 15)
};

template <bool F32>
__device__ __forceinline__ float ex(float x) {
    if constexpr (F32) return expf(x);
    else return __expf(x);
}

template <bool F32>
__global__ __launch_bounds__(NT, 1) void kda_fwd_fused(FwdArgs a) {
    __shared__ Smem<F32> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;

    // Workgroup -> chain. Dispatch round-robins workgroups over the 8 XCDs, so
    // the P V-blocks of one (sequence, head) take ids congruent mod 8 and land on
    // one XCD, where they share the q/k/g lines in that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, rest = bid >> 3;
    const int vblk = rest % P;
    const int chain = (rest / P) * 8 + xcd;
    if (chain >= a.nchains) return;
    const int n = chain / a.H, h = chain % a.H;
    int row, t0, t1;
    if (a.cu) { row = 0; t0 = a.cu[n]; t1 = a.cu[n + 1]; }
    else      { row = n; t0 = 0;       t1 = a.T; }
    const long long ts = (long long)a.H * D;                       // elements per token
    const long long base = (long long)row * a.T * ts + (long long)h * D;
    const int vc = vblk * VB + wave * 16 + l16;                     // this lane's V column
    const long long sbase = ((long long)n * a.H + h) * D * D;

    f32x4 S[8];                                  // rows 16m + 4grp + j, column vc
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            S[m][j] = a.h0 ? a.h0[sbase + (long long)(16 * m + 4 * grp + j) * D + vc] : 0.f;

    const int pc = tid & (D - 1), pb = tid >> 7;   // scan thread: channel, sub-block

    for (int cs = t0; cs < t1; cs += C) {
        const int nv = min(C, t1 - cs);

        // ---- (1) gate scan and gated factors for (channel pc, tokens 16pb .. 16pb+15)
        float kv[16], qv[16], L[16];
        {
            float run = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rr = 16 * pb + j;
                float gv = 0.f, k_ = 0.f, q_ = 0.f;
                if (rr < nv) {
                    const long long idx = base + (long long)(cs + rr) * ts + pc;
                    gv = a.g[idx];
                    k_ = ld_in<F32>(a.k, idx);
                    q_ = ld_in<F32>(a.q, idx);
                }
                run += gv;
                L[j] = run;
                kv[j] = k_;
                qv[j] = q_;
            }
        }
        if (tid < C)
            sm.beta[tid] = tid < nv ? a.beta[((long long)row * a.T + cs + tid) * a.H + h] : 0.f;
        sm.tot[pb][pc] = L[15];
        if (pb == 1) sm.mid1[pc] = L[7];
        __syncthreads();
        {
            const float tot0 = sm.tot[0][pc], tot1 = sm.tot[1][pc];
            if (pb == 1) sm.gl[pc] = ex<F32>(tot0 + tot1);
            const float start = pb ? tot0 : 0.f;        // Gamma at the end of the previous sub-block
            const float after = pb ? 0.f : tot1;        // decay from this sub-block's end to the chunk's end
            const float krs = pb ? 0.f : sm.mid1[pc];   // off-diagonal column factor reference shift
            const int pcp = (pc & ~31) | kperm(pc & 31);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int rr = 16 * pb + j;
                const float e1 = ex<F32>(L[j] - L[7]);             // row factor, mid-block reference
                const float e2 = ex<F32>(L[7] - L[j]);             // column factor, diagonal blocks
                const float eg = ex<F32>(start + L[j]);            // exp(Gamma_r), from the chunk start
                const float et = ex<F32>(L[15] - L[j] + after);    // exp(Gamma_last - Gamma_r)
                const float ka = kv[j] * e1, qa = qv[j] * e1, kb = kv[j] * e2;
                const float kg = kv[j] * eg, qg = qv[j] * eg, kt = kv[j] * et;
                if constexpr (F32) {
                    sm.am.Ka[rr][pc] = ka;
                    sm.am.Qa[rr][pc] = qa;
                    sm.am.Kb[rr][pc] = kb;
                    if (pb == 0) sm.am.Kr[j][pc] = kv[j] * ex<F32>(L[15] - L[j] + krs);
                    split16(kg, sm.Kg[0][rr][pcp], sm.Kg[1][rr][pcp]);
                    split16(qg, sm.Qg[0][rr][pcp], sm.Qg[1][rr][pcp]);
                } else {
                    splitbf(ka, sm.am.Ka[0][rr][pc], sm.am.Ka[1][rr][pc]);
                    splitbf(qa, sm.am.Qa[0][rr][pc], sm.am.Qa[1][rr][pc]);
                    splitbf(kb, sm.am.Kb[0][rr][pc], sm.am.Kb[1][rr][pc]);
                    if (pb == 0) {
                        const float kr = kv[j] * ex<F32>(L[15] - L[j] + krs);
                        splitbf(kr, sm.am.Kr[0][j][pc], sm.am.Kr[1][j][pc]);
                    }
                    sm.Kg[0][rr][pcp] = (_Float16)kg;
                    sm.Qg[0][rr][pcp] = (_Float16)qg;
                }
                split16(kt, sm.KtT[0][pc][kperm(rr)], sm.KtT[1][pc][kperm(rr)]);
            }
        }
        __syncthreads();

        // ---- (2a) A and M on 16 x 16 blocks: (0,0), (1,1) diagonal, (1,0) below
        {
            // wave 0: A00, A10   wave 1: A11   wave 2: M00, M10   wave 3: M11
            const bool isM = wave >= 2;
            const int ntile = (wave & 1) ? 1 : 2;
            for (int ti = 0; ti < ntile; ++ti) {
                const int rb = (wave & 1) ? 1 : ti;       // row block
                const int cb = (wave & 1) ? 1 : 0;        // column block
                const bool diag = (rb == cb);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (F32) {
                    const float* ro = isM ? &sm.am.Qa[16 * rb + l16][0] : &sm.am.Ka[16 * rb + l16][0];
                    const float* co = diag ? &sm.am.Kb[16 * cb + l16][0] : &sm.am.Kr[l16][0];
#pragma unroll 8
                    for (int kk = 0; kk < D / 4; ++kk)
                        acc = mfma16x4(ro[4 * kk + grp], co[4 * kk + grp], acc);
                } else {
#pragma unroll
                    for (int kk = 0; kk < D / 32; ++kk) {
                        const int off = 32 * kk + 8 * grp;
                        bf16x8 rh, rl, ch, cl;
                        if (isM) {
                            rh = lds_vec<bf16x8>(&sm.am.Qa[0][16 * rb + l16][off]);
                            rl = lds_vec<bf16x8>(&sm.am.Qa[1][16 * rb + l16][off]);
                        } else {
                            rh = lds_vec<bf16x8>(&sm.am.Ka[0][16 * rb + l16][off]);
                            rl = lds_vec<bf16x8>(&sm.am.Ka[1][16 * rb + l16][off]);
                        }
                        if (diag) {
                            ch = lds_vec<bf16x8>(&sm.am.Kb[0][16 * cb + l16][off]);
                            cl = lds_vec<bf16x8>(&sm.am.Kb[1][16 * cb + l16][off]);
                        } else {
                            ch = lds_vec<bf16x8>(&sm.am.Kr[0][l16][off]);
                            cl = lds_vec<bf16x8>(&sm.am.Kr[1][l16][off]);
                        }
                        acc = mfma16(rh, ch, acc);
                        acc = mfma16(rh, cl, acc);
                        acc = mfma16(rl, ch, acc);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rb + 4 * grp + j, i = 16 * cb + l16;
                    if (!isM) {
                        sm.A[r][i] = (i < r) ? sm.beta[r] * acc[j] : 0.f;
                    } else {
                        const float val = (i <= r) ? acc[j] : 0.f;
                        split16(val, sm.M[0][r][kperm(i)], sm.M[1][r][kperm(i)]);
                    }
                }
            }
            // the zero upper-right blocks
            if (wave == 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sm.A[4 * grp + j][16 + l16] = 0.f;
            } else if (wave == 3) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sm.M[0][4 * grp + j][kperm(16 + l16)] = (_Float16)0.f;
                    sm.M[1][4 * grp + j][kperm(16 + l16)] = (_Float16)0.f;
                }
            }
        }
        __syncthreads();

        // ---- (2b) T = (I + A)^{-1}: lane j computes column j by forward substitution
        if (wave == 0) {
            const int j = lane & (C - 1);
            float x[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) s -= sm.A[r][i] * x[i];
                x[r] = s;
            }
            if (lane < C) {
#pragma unroll
                for (int r = 0; r < C; ++r) split16(x[r], sm.Tm[0][r][kperm(j)], sm.Tm[1][r][kperm(j)]);
            }
        }
        __syncthreads();

        // ---- (3)+(4) state-side products for this wave's 16 columns
        {
            f16x8 SBh[4], SBl[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (F32) {
                        const half2s u = split16(S[2 * kk][j]), w = split16(S[2 * kk + 1][j]);
                        SBh[kk][j] = u.hi;
                        SBl[kk][j] = u.lo;
                        SBh[kk][4 + j] = w.hi;
                        SBl[kk][4 + j] = w.lo;
                    } else {
                        SBh[kk][j] = (_Float16)S[2 * kk][j];
                        SBh[kk][4 + j] = (_Float16)S[2 * kk + 1][j];
                    }
                }
            f32x4 Pt[2], Ot[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                Pt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                Ot[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int off = 32 * kk + 8 * grp;
                    const f16x8 kg = lds_vec<f16x8>(&sm.Kg[0][16 * t + l16][off]);
                    const f16x8 qg = lds_vec<f16x8>(&sm.Qg[0][16 * t + l16][off]);
                    Pt[t] = mfma16(kg, SBh[kk], Pt[t]);
                    Ot[t] = mfma16(qg, SBh[kk], Ot[t]);
                    if constexpr (F32) {
                        const f16x8 kgl = lds_vec<f16x8>(&sm.Kg[1][16 * t + l16][off]);
                        const f16x8 qgl = lds_vec<f16x8>(&sm.Qg[1][16 * t + l16][off]);
                        Pt[t] = mfma16(kg, SBl[kk], Pt[t]);
                        Pt[t] = mfma16(kgl, SBh[kk], Pt[t]);
                        Ot[t] = mfma16(qg, SBl[kk], Ot[t]);
                        Ot[t] = mfma16(qgl, SBh[kk], Ot[t]);
                    }
                }
            }
            // beta (V - P) as a split B operand over the chunk's 32 tokens
            f16x8 BEh, BEl;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 16 * t + 4 * grp + j;
                    const float vv = rr < nv ? ld_in<F32>(a.v, base + (long long)(cs + rr) * ts + vc) : 0.f;
                    const half2s u = split16(sm.beta[rr] * (vv - Pt[t][j]));
                    BEh[4 * t + j] = u.hi;
                    BEl[4 * t + j] = u.lo;
                }
            // Delta = T beta (V - P)
            f32x4 Dt[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f16x8 th = lds_vec<f16x8>(&sm.Tm[0][16 * t + l16][8 * grp]);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(th, BEh, acc);
                acc = mfma16(th, BEl, acc);
                if constexpr (F32) {
                    const f16x8 tl = lds_vec<f16x8>(&sm.Tm[1][16 * t + l16][8 * grp]);
                    acc = mfma16(tl, BEh, acc);
                }
                Dt[t] = acc;
            }
            f16x8 DBh, DBl;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2s u = split16(Dt[t][j]);
                    DBh[4 * t + j] = u.hi;
                    DBl[4 * t + j] = u.lo;
                }
            // O = (Q*gamma) S + M Delta
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f16x8 mh = lds_vec<f16x8>(&sm.M[0][16 * t + l16][8 * grp]);
                const f16x8 ml = lds_vec<f16x8>(&sm.M[1][16 * t + l16][8 * grp]);
                f32x4 acc = Ot[t];
                acc = mfma16(mh, DBh, acc);
                acc = mfma16(mh, DBl, acc);
                acc = mfma16(ml, DBh, acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 16 * t + 4 * grp + j;
                    if (rr < nv) a.o[base + (long long)(cs + rr) * ts + vc] = acc[j];
                }
            }
            // S <- Diag(gamma_last) S + Kt^T Delta
#pragma unroll
            for (int m = 0; m < 8; ++m) {
#pragma unroll
                for (int j = 0; j < 4; ++j) S[m][j] *= sm.gl[16 * m + 4 * grp + j];
                const f16x8 kh = lds_vec<f16x8>(&sm.KtT[0][16 * m + l16][8 * grp]);
                const f16x8 kl = lds_vec<f16x8>(&sm.KtT[1][16 * m + l16][8 * grp]);
                S[m] = mfma16(kh, DBh, S[m]);
                S[m] = mfma16(kh, DBl, S[m]);
                S[m] = mfma16(kl, DBh, S[m]);
            }
        }
        __syncthreads();
    }

    if (a.hT) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a.hT[sbase + (long long)(16 * m + 4 * grp + j) * D + vc] = S[m][j];
    }
}

}  // namespace fused

int fused_workgroups(int nchains) {
    const int groups = (nchains + 7) / 8;
    return groups * 8 * fused::P;
}

hipError_t launch_fwd_fused(const FwdArgs& a, bool f32_inputs, hipStream_t stream) {
    const int grid = fused_workgroups(a.nchains);
    if (grid == 0) return hipSuccess;
    if (f32_inputs)
        hipLaunchKernelGGL(fused::kda_fwd_fused<true>, dim3(grid), dim3(fused::NT), 0, stream, a);
    else
        hipLaunchKernelGGL(fused::kda_fwd_fused<false>, dim3(grid), dim3(fused::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
