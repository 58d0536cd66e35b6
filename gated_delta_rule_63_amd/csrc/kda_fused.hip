// kda_fused.hip -- the fused chunked KDA forward for gfx950.
//
// One workgroup owns one (sequence, head, V-block) chain and walks its chunks
// in order. Per chunk of C = 32 tokens it
//   (1) scans the log-gate within each 16-token sub-block and forms the gated
//       key/query factors (per-chunk cumulative log-gate scan);
//   (2) builds the beta-weighted strictly-lower gated K K^T (A) and the lower
//       gated Q K^T (M) on MFMA, and solves T = (I + A)^{-1}: forward
//       substitution for the two 16 x 16 diagonal blocks on the A tile staged
//       in LDS, then T10 = -T11 A10 T00 on fp32 MFMA;
//   (3) advances the 128 x 16-per-wave fp32 state on MFMA:
//           E = V - (K*gamma) S,  Delta = T Diag(beta) E,
//           S <- Diag(gamma_last) S + (K*exp(Gamma_last - Gamma))^T Delta;
//   (4) writes O = (Q*gamma) S + M Delta before the update.
// These are the four steps of the chunked prefill; the pages credit a chunked
// two-kernel CUTLASS design on Hopper (toolarium.ru page, section
// "Где ограничения прямо сейчас"). Here all four run in one kernel so each
// input byte crosses HBM once, because MI355X's ratio of matrix throughput to
// HBM bandwidth makes this path bandwidth-bound. The next chunk's inputs are
// fetched into registers while the current chunk computes.
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
constexpr int LDV = VB + 4;    // padded row of the staged V tile
static_assert(NT == 4 * (D / 2), "the scan maps one thread to each (channel pair, 8-token quarter)");
static_assert(C == 32, "the sub-block bookkeeping below is written for two 16-token sub-blocks");
static_assert(NT * 8 == C * VB, "one 8-element slice of the V tile per thread");

template <bool F32> struct alignas(16) Smem {
    float Ka[C][LDF];                   // k * exp(Gamma_r - Gamma_mid(block))    row factors
    float Qa[C][LDF];                   // q * exp(Gamma_r - Gamma_mid(block))
    float Kb[C][LDF];                   // k * exp(Gamma_mid(block) - Gamma_r)    column factors
    float Kr[16][LDF];                  // block-0 keys referenced to block 1's middle
    _Float16 Kg[F32 ? 2 : 1][C][LDP];   // K * exp(Gamma), channels permuted in 32-groups
    _Float16 Qg[F32 ? 2 : 1][C][LDP];   // Q * exp(Gamma), same order
    _Float16 KtT[2][D][TP];             // (K * exp(Gamma_last - Gamma))^T, [hi, lo][channel][kperm(token)]
    float A[C][LDA];                    // beta-weighted strictly-lower gated K K^T
    float Tf[2][16][17];                // fp32 inverses of the two diagonal blocks of I + A
    _Float16 Tm[2][C][TP];              // (I + A)^{-1}, [hi, lo][row][kperm(col)]
    _Float16 M[2][C][TP];               // lower gated Q K^T, [hi, lo][row][kperm(col)]
    float V[C][LDV];                    // this workgroup's V columns of the chunk
    float gl[D];                        // exp(Gamma_last), the chunk's decay per channel
    float beta[C];
    float qtot[4][D];                   // sum of g over each 8-token quarter
};

template <bool F32>
__device__ __forceinline__ float ex(float x) {
    if constexpr (F32) return expf(x);
    else return __expf(x);
}

// Registers of one chunk's inputs for thread (channel pair cp, quarter qq).
template <bool F32> struct Fetch;
template <> struct Fetch<false> {
    float2 g[8];
    uint32_t k[8], q[8];   // two bf16 each
    uint4 v;               // eight bf16 of the V tile
    float beta;
};
template <> struct Fetch<true> {
    float2 g[8], k[8], q[8];
    float4 v0, v1;
    float beta;
};

__device__ __forceinline__ float2 bf2(uint32_t u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

template <bool F32>
__device__ __forceinline__ void fetch(Fetch<F32>& f, const FwdArgs& a, long long base, long long ts,
                                      int row, int h, int cs, int nv, int cp, int qq, int tid, int vcol0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int rr = 8 * qq + t;
        if (rr < nv) {
            const long long idx = base + (long long)(cs + rr) * ts + 2 * cp;
            f.g[t] = *reinterpret_cast<const float2*>(a.g + idx);
            if constexpr (F32) {
                f.k[t] = *reinterpret_cast<const float2*>(static_cast<const float*>(a.k) + idx);
                f.q[t] = *reinterpret_cast<const float2*>(static_cast<const float*>(a.q) + idx);
            } else {
                f.k[t] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.k) + idx);
                f.q[t] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + idx);
            }
        } else {
            f.g[t] = make_float2(0.f, 0.f);
            if constexpr (F32) { f.k[t] = make_float2(0.f, 0.f); f.q[t] = make_float2(0.f, 0.f); }
            else { f.k[t] = 0u; f.q[t] = 0u; }
        }
    }
    f.beta = (tid < nv) ? a.beta[((long long)row * a.T + cs + tid) * a.H + h] : 0.f;
    const int vr = tid >> 3, vc = (tid & 7) * 8;
    if (vr < nv) {
        const long long vi = base + (long long)(cs + vr) * ts + vcol0 + vc;
        if constexpr (F32) {
            f.v0 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + vi);
            f.v1 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + vi + 4);
        } else {
            f.v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + vi);
        }
    } else {
        if constexpr (F32) { f.v0 = make_float4(0.f, 0.f, 0.f, 0.f); f.v1 = f.v0; }
        else f.v = make_uint4(0u, 0u, 0u, 0u);
    }
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
    const int vcol0 = vblk * VB;
    const int vc = vcol0 + wave * 16 + l16;                         // this lane's V column
    const long long sbase = ((long long)n * a.H + h) * D * D;

    f32x4 S[8];                                  // rows 16m + 4grp + j, column vc
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            S[m][j] = a.h0 ? a.h0[sbase + (long long)(16 * m + 4 * grp + j) * D + vc] : 0.f;

    const int cp = tid & 63, qq = tid >> 6;      // scan thread: channel pair, 8-token quarter
    const int b = qq >> 1, half = qq & 1;        // its 16-token sub-block and half of it

    Fetch<F32> nxt;
    if (t0 < t1) fetch<F32>(nxt, a, base, ts, row, h, t0, min(C, t1 - t0), cp, qq, tid, vcol0);

    for (int cs = t0; cs < t1; cs += C) {
        const int nv = min(C, t1 - cs);
        const Fetch<F32> cur = nxt;
        if (cs + C < t1) fetch<F32>(nxt, a, base, ts, row, h, cs + C, min(C, t1 - cs - C), cp, qq, tid, vcol0);

        // ---- (1) gate scan and gated factors for channels 2cp, 2cp+1, tokens 8qq .. 8qq+7
        float L[2][8];
        {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                r0 += cur.g[t].x;
                r1 += cur.g[t].y;
                L[0][t] = r0;
                L[1][t] = r1;
            }
            *reinterpret_cast<float2*>(&sm.qtot[qq][2 * cp]) = make_float2(r0, r1);
        }
        if (tid < C) sm.beta[tid] = cur.beta;
        {
            const int vr = tid >> 3, vcc = (tid & 7) * 8;
            float vv[8];
            if constexpr (F32) {
                vv[0] = cur.v0.x; vv[1] = cur.v0.y; vv[2] = cur.v0.z; vv[3] = cur.v0.w;
                vv[4] = cur.v1.x; vv[5] = cur.v1.y; vv[6] = cur.v1.z; vv[7] = cur.v1.w;
            } else {
                const float2 p0 = bf2(cur.v.x), p1 = bf2(cur.v.y), p2 = bf2(cur.v.z), p3 = bf2(cur.v.w);
                vv[0] = p0.x; vv[1] = p0.y; vv[2] = p1.x; vv[3] = p1.y;
                vv[4] = p2.x; vv[5] = p2.y; vv[6] = p3.x; vv[7] = p3.y;
            }
            *reinterpret_cast<float4*>(&sm.V[vr][vcc]) = make_float4(vv[0], vv[1], vv[2], vv[3]);
            *reinterpret_cast<float4*>(&sm.V[vr][vcc + 4]) = make_float4(vv[4], vv[5], vv[6], vv[7]);
        }
        __syncthreads();
        {
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                const int c = 2 * cp + ch;
                const float qt0 = sm.qtot[0][c], qt1 = sm.qtot[1][c], qt2 = sm.qtot[2][c], qt3 = sm.qtot[3][c];
                const float tot0 = qt0 + qt1, tot1 = qt2 + qt3;
                const float L7 = b ? qt2 : qt0;                // sub-block middle (end of its first quarter)
                const float L15 = b ? tot1 : tot0;
                const float off = half ? L7 : 0.f;             // scan offset of this quarter in its sub-block
                const float start = b ? tot0 : 0.f;            // Gamma at the end of the previous sub-block
                const float after = b ? 0.f : tot1;            // decay from this sub-block's end to the chunk end
                const float c1 = ex<F32>(start + L7);          // exp(Gamma_mid)                -> K*gamma, Q*gamma
                const float c2 = ex<F32>(L15 - L7 + after);    // exp(Gamma_last - Gamma_mid)   -> Kt
                const float c3 = ex<F32>(L15 - L7 + qt2);      // block 0 -> block 1's middle   -> Kr
                if (qq == 0) sm.gl[c] = ex<F32>(tot0 + tot1);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int rr = 8 * qq + t;
                    const float d = L[ch][t] + off - L7;        // Gamma_r - Gamma_mid, |d| <= 8 * 5
                    const float e1 = ex<F32>(d), e2 = ex<F32>(-d);
                    float kv, qv;
                    if constexpr (F32) { kv = ch ? cur.k[t].y : cur.k[t].x; qv = ch ? cur.q[t].y : cur.q[t].x; }
                    else { kv = ch ? bf2(cur.k[t]).y : bf2(cur.k[t]).x; qv = ch ? bf2(cur.q[t]).y : bf2(cur.q[t]).x; }
                    const float ka = kv * e1, qa = qv * e1, kb = kv * e2;
                    sm.Ka[rr][c] = ka;
                    sm.Qa[rr][c] = qa;
                    sm.Kb[rr][c] = kb;
                    if (b == 0) sm.Kr[rr][c] = kb * c3;
                    const float kg = ka * c1, qg = qa * c1, kt = kb * c2;
                    const int cpos = (c & ~31) | kperm(c & 31);
                    if constexpr (F32) {
                        split16(kg, sm.Kg[0][rr][cpos], sm.Kg[1][rr][cpos]);
                        split16(qg, sm.Qg[0][rr][cpos], sm.Qg[1][rr][cpos]);
                    } else {
                        sm.Kg[0][rr][cpos] = (_Float16)kg;
                        sm.Qg[0][rr][cpos] = (_Float16)qg;
                    }
                    split16(kt, sm.KtT[0][c][kperm(rr)], sm.KtT[1][c][kperm(rr)]);
                }
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
                const float* ro = isM ? &sm.Qa[16 * rb + l16][0] : &sm.Ka[16 * rb + l16][0];
                const float* co = diag ? &sm.Kb[16 * cb + l16][0] : &sm.Kr[l16][0];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (F32) {
#pragma unroll 8
                    for (int kk = 0; kk < D / 4; ++kk)
                        acc = mfma16x4(ro[4 * kk + grp], co[4 * kk + grp], acc);
                } else {
#pragma unroll
                    for (int kk = 0; kk < D / 32; ++kk) {
                        const int off = 32 * kk + 8 * grp;
                        const float4 r0 = lds_vec<float4>(ro + off), r1 = lds_vec<float4>(ro + off + 4);
                        const float4 c0 = lds_vec<float4>(co + off), c1 = lds_vec<float4>(co + off + 4);
                        const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                        bf16x8 rh, rl, ch, cl;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const __bf16 a_hi = cvtbf_once(rv[j]);
                            rh[j] = a_hi;
                            rl[j] = (__bf16)(rv[j] - (float)a_hi);
                            const __bf16 b_hi = cvtbf_once(cv[j]);
                            ch[j] = b_hi;
                            cl[j] = (__bf16)(cv[j] - (float)b_hi);
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
            // the zero upper-right blocks of M and of T
            if (wave == 3) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sm.M[0][4 * grp + j][kperm(16 + l16)] = (_Float16)0.f;
                    sm.M[1][4 * grp + j][kperm(16 + l16)] = (_Float16)0.f;
                    sm.Tm[0][4 * grp + j][kperm(16 + l16)] = (_Float16)0.f;
                    sm.Tm[1][4 * grp + j][kperm(16 + l16)] = (_Float16)0.f;
                }
            }
        }
        __syncthreads();

        // ---- (2b) T = (I + A)^{-1}
        if (wave == 0) {
            // diagonal blocks: lane (block bb, column j) forward-substitutes column j
            const int bb = (lane >> 4) & 1, j = l16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float* arow = &sm.A[16 * bb + r][16 * bb];
                float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < r; i += 2) {
                    s0 -= arow[i] * x[i];
                    if (i + 1 < r) s1 -= arow[i + 1] * x[i + 1];
                }
                x[r] = s0 + s1;
            }
            if (lane < 32) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sm.Tf[bb][r][j] = x[r];
                    split16(x[r], sm.Tm[0][16 * bb + r][kperm(16 * bb + j)], sm.Tm[1][16 * bb + r][kperm(16 * bb + j)]);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            // T10 = -T11 (A10 T00) on fp32 MFMA. Y = A10 T00 lands in accumulator
            // layout (rows 4grp + jj); fed back as a B operand with the reduction
            // index of step jj taken as {4g + jj : g = 0..3}.
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                Y = mfma16x4(sm.A[16 + l16][4 * kk + grp], sm.Tf[0][4 * kk + grp][l16], Y);
            f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Z = mfma16x4(sm.Tf[1][l16][4 * grp + jj], Y[jj], Z);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                split16(-Z[jj], sm.Tm[0][16 + 4 * grp + jj][kperm(l16)], sm.Tm[1][16 + 4 * grp + jj][kperm(l16)]);
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
                    const half2s u = split16(sm.beta[rr] * (sm.V[rr][wave * 16 + l16] - Pt[t][j]));
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
