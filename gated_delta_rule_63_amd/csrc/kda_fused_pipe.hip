// kda_fused_pipe.hip -- the pipelined fused chunked KDA forward for gfx950
// (bf16 q/k/v).
//
// Same arithmetic as the serial kernel (kda_fused_serial.hip), organised as a
// two-stage pipeline inside each workgroup:
//   * NS "state" waves each own 16 V columns of the 128 x 128 fp32 state of one
//     (sequence, head) and run only the sequential, MFMA-bound part for chunk i:
//        P = (K*gamma) S,  Delta = (I + A)^{-1} Diag(beta) (V - P),
//        O = (Q*gamma) S + M Delta,  S <- Diag(gamma_last) S + Kt^T Delta;
//   * NH "helper" waves prepare chunk i+1 at the same time: the per-chunk
//     cumulative log-gate scan, the gated factors, the gated K K^T (A) and
//     Q K^T (M) blocks on MFMA, and the inverses of the diagonal blocks of
//     I + A; they write the state waves' operands into the other half of a
//     double-buffered LDS area.
// One workgroup barrier per chunk hands the buffers over. The two points where
// the helpers need each other's results inside a chunk use an LDS counter
// that only the helpers wait on, so the state waves never stall there.
// The split into a chunk-parallel preparation and a sequential recurrence is
// the pages' two-kernel design (toolarium.ru page, section "Где ограничения
// прямо сейчас"); here the two run concurrently on one CU so that each input
// byte crosses HBM once.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace pipe {

constexpr int C = 32;          // chunk length (two 16-token sub-blocks)
constexpr int NS = 4;          // state waves, 16 V columns each
constexpr int NH = 8;          // helper waves
constexpr int NT = 64 * (NS + NH);
constexpr int VB = 16 * NS;    // V columns per workgroup
constexpr int P = D / VB;      // workgroups per (sequence, head)
constexpr int TS = C / NH;     // tokens per helper segment
constexpr int LDP = D + 8;     // padded row of a 2-byte [row][128] array
constexpr int TP = C + 8;      // padded row of a 2-byte [row][32] array
constexpr int LDA = 16 + 4;    // padded row of an fp32 16 x 16 tile
constexpr float LOG2E = 1.4426950408889634f;

// 2^x as one v_exp_f32. Every argument here lies within [-60, 60] (log2 units
// of a 16-token decay span with g >= -5), far from fp32's denormal range, so
// the library's range handling around the instruction is not needed.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
static_assert(NH * 64 * TS * 2 == C * D, "one (channel pair, segment) per helper thread");
static_assert(16 % TS == 0 && 8 % TS == 0, "segments must not straddle a sub-block or its middle");
static_assert(NH == 4 || NH >= 6, "A/M tile assignments exist for four or six-plus helper waves");

// Operands of one chunk for the state waves (double-buffered).
struct alignas(16) Ops {
    _Float16 Kg[C][LDP];        // K * exp(Gamma), channels permuted in 32-groups
    _Float16 Qg[C][LDP];        // Q * exp(Gamma), same order
    _Float16 KtT[2][D][TP];     // (K * exp(Gamma_last - Gamma))^T, [hi, lo][channel][kperm(token)]
    _Float16 Tm[C][TP];         // block-diagonal (I + A)^{-1}, [row][kperm(col)]
    _Float16 A10[16][TP];       // A rows 16-31, cols 0-15, [row][kperm(col)]
    _Float16 M[2][C][TP];       // lower gated Q K^T, [hi, lo][row][kperm(col)]
    float gl[D];                // exp(Gamma_last), the chunk's decay per channel
    float beta[C];
};

struct alignas(16) Smem {
    Ops op[2];
    __bf16 Ka[C][LDP];          // k * exp(Gamma_r - Gamma_mid(block)) (A needs only bf16)
    __bf16 Qa[2][C][LDP];       // q * exp(Gamma_r - Gamma_mid(block))
    __bf16 Kb[2][C][LDP];       // k * exp(Gamma_mid(block) - Gamma_r)
    __bf16 Kr[2][16][LDP];      // block-0 keys referenced to block 1's middle
    float Ad[2][16][LDA];       // diagonal blocks of A for the forward substitution
    float qtot[NH][D];          // sum of g * log2(e) over each helper segment
    uint32_t hcount;            // helper-only barrier counter
};

// Helper-only barrier: an LDS counter that every helper wave bumps and then
// waits on. The wait is bounded; under correct use it never runs out.
__device__ __forceinline__ void helper_sync(uint32_t* cnt, uint32_t& target, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    target += NH;
    for (uint32_t spin = 0; spin < (1u << 20); ++spin) {
        if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ float2 bf2(uint32_t u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

// One helper thread's share of a chunk: channels 2cp, 2cp+1 of tokens seg*TS .. +TS.
// Loads are unconditional from a clamped (valid) token so that no load sits
// behind a branch that would make the compiler wait for it on the spot;
// tokens past the chunk's end are zeroed where the values are used.
struct HFetch {
    float2 g[TS];
    uint32_t k[TS], q[TS];
    float beta;
};

__device__ __forceinline__ void hfetch(HFetch& f, const FwdArgs& a, long long cbase, long long cbeta,
                                       uint32_t ts, uint32_t off0, int nv, int seg, int ht) {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + cbase;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + cbase;
    const float* gp = a.g + cbase;
#pragma unroll
    for (int t = 0; t < TS; ++t) {
        const int rc = min(seg * TS + t, nv - 1);
        const uint32_t o = off0 + (uint32_t)rc * ts;
        f.g[t] = *reinterpret_cast<const float2*>(gp + o);
        f.k[t] = *reinterpret_cast<const uint32_t*>(kp + o);
        f.q[t] = *reinterpret_cast<const uint32_t*>(qp + o);
    }
    f.beta = a.beta[cbeta + (uint32_t)min(ht, nv - 1) * (uint32_t)a.H];
}

// Forward substitution of one unit-lower-triangular 16 x 16 block: lane j
// (of 16) returns column j of (I + Ablk)^{-1}. The lower triangle is read into
// registers first (36 broadcast 16-byte reads), so the 16 dependent row steps
// wait on FMAs only, not on LDS round trips.
__device__ __forceinline__ void tri_inverse16(const float (*Ablk)[LDA], int j, float x[16]) {
    float4 ar[16][4];
#pragma unroll
    for (int r = 1; r < 16; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (4 * q < r) ar[r][q] = *reinterpret_cast<const float4*>(&Ablk[r][4 * q]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) {
            const float4 v4 = ar[r][i >> 2];
            const float av = (i & 3) == 0 ? v4.x : (i & 3) == 1 ? v4.y : (i & 3) == 2 ? v4.z : v4.w;
            if (i & 1) s1 -= av * x[i];
            else s0 -= av * x[i];
        }
        x[r] = s0 + s1;
    }
}

// Helpers: prepare the operands of one chunk from the fetched registers.
__device__ __forceinline__ void prepare(Smem& sm, Ops& op, HFetch& f, int nv, int hw, int lane,
                                        int ht, uint32_t& htarget, bool fetch_next,
                                        const FwdArgs& a, long long nbase, long long nbeta, uint32_t ts,
                                        uint32_t off, int nnv) {
    const int cp = ht & 63, seg = ht >> 6;
    const int b = (seg * TS) >> 4;                 // sub-block of this segment
    const int l16 = lane & 15, grp = lane >> 4;

    // (1a) local scan in log2 units
    float L[2][TS];
    float kv[2][TS], qv[2][TS];
    {
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            const bool ok = seg * TS + t < nv;
            r0 += ok ? f.g[t].x * LOG2E : 0.f;
            r1 += ok ? f.g[t].y * LOG2E : 0.f;
            L[0][t] = r0;
            L[1][t] = r1;
            const float2 k2 = bf2(ok ? f.k[t] : 0u), q2 = bf2(ok ? f.q[t] : 0u);
            kv[0][t] = k2.x; kv[1][t] = k2.y;
            qv[0][t] = q2.x; qv[1][t] = q2.y;
        }
        *reinterpret_cast<float2*>(&sm.qtot[seg][2 * cp]) = make_float2(r0, r1);
    }
    if (ht < C) op.beta[ht] = (ht < nv) ? f.beta : 0.f;
    helper_sync(&sm.hcount, htarget, lane);
    // the fetched registers are consumed: fetch the chunk after this one
    if (fetch_next) hfetch(f, a, nbase, nbeta, ts, off, nnv, seg, ht);

    // (1b) gated factors
    {
        constexpr int SPB = 16 / TS;               // segments per sub-block
        constexpr int MIDSEG = 8 / TS - 1;         // last segment of a sub-block's first half
        float d[2][TS], c1[2], c2[2], c3[2];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const int c = 2 * cp + ch;
            float tot0 = 0.f, tot1 = 0.f, L7b0 = 0.f, L7b1 = 0.f, pre = 0.f;
#pragma unroll
            for (int s = 0; s < NH; ++s) {
                const float v = sm.qtot[s][c];
                if (s < SPB) { tot0 += v; if (s <= MIDSEG) L7b0 += v; }
                else { tot1 += v; if (s - SPB <= MIDSEG) L7b1 += v; }
                if (s < seg && s >= b * SPB) pre += v;      // earlier segments of this sub-block
            }
            const float L7 = b ? L7b1 : L7b0;
            const float L15 = b ? tot1 : tot0;
            const float start = b ? tot0 : 0.f;
            const float after = b ? 0.f : tot1;
            c1[ch] = ex2(start + L7);                // exp(Gamma_mid)              -> K*gamma, Q*gamma
            c2[ch] = ex2(L15 - L7 + after);          // exp(Gamma_last - Gamma_mid) -> Kt
            c3[ch] = ex2(L15 - L7 + L7b1);           // block 0 -> block 1's middle -> Kr
            if (seg == 0) op.gl[c] = ex2(tot0 + tot1);
#pragma unroll
            for (int t = 0; t < TS; ++t) d[ch][t] = L[ch][t] + pre - L7;
        }
        const int cpos = ((2 * cp) & ~31) | kperm((2 * cp) & 31);
        float ktp[TS], ktq[TS];
#pragma unroll
        for (int t = 0; t < TS; t += 2) {
            float kt[2][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int rr = seg * TS + t + u;
                float ka[2], qa[2], kb[2];
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    const float e1 = ex2(d[ch][t + u]), e2 = ex2(-d[ch][t + u]);
                    ka[ch] = kv[ch][t + u] * e1;
                    qa[ch] = qv[ch][t + u] * e1;
                    kb[ch] = kv[ch][t + u] * e2;
                    kt[u][ch] = kb[ch] * c2[ch];
                }
                uint32_t hi, lo;
                {
                    const bf16x2 kah = {(__bf16)ka[0], (__bf16)ka[1]};
                    *reinterpret_cast<bf16x2*>(&sm.Ka[rr][2 * cp]) = kah;
                }
                split_bf16x2(qa[0], qa[1], hi, lo);
                *reinterpret_cast<uint32_t*>(&sm.Qa[0][rr][2 * cp]) = hi;
                *reinterpret_cast<uint32_t*>(&sm.Qa[1][rr][2 * cp]) = lo;
                split_bf16x2(kb[0], kb[1], hi, lo);
                *reinterpret_cast<uint32_t*>(&sm.Kb[0][rr][2 * cp]) = hi;
                *reinterpret_cast<uint32_t*>(&sm.Kb[1][rr][2 * cp]) = lo;
                if (b == 0) {
                    split_bf16x2(kb[0] * c3[0], kb[1] * c3[1], hi, lo);
                    *reinterpret_cast<uint32_t*>(&sm.Kr[0][rr][2 * cp]) = hi;
                    *reinterpret_cast<uint32_t*>(&sm.Kr[1][rr][2 * cp]) = lo;
                }
                *reinterpret_cast<uint32_t*>(&op.Kg[rr][cpos]) = pack_f16(ka[0] * c1[0], ka[1] * c1[1]);
                *reinterpret_cast<uint32_t*>(&op.Qg[rr][cpos]) = pack_f16(qa[0] * c1[0], qa[1] * c1[1]);
            }
            // K^T: tokens come in pairs here and in quads below
            ktp[t] = kt[0][0]; ktp[t + 1] = kt[1][0];
            ktq[t] = kt[0][1]; ktq[t + 1] = kt[1][1];
        }
        // tokens seg*TS .. seg*TS+3 occupy four contiguous kperm positions: 8-byte stores
        static_assert(TS == 4, "the K^T store below writes one 4-token group per channel");
        const int tp = kperm(seg * TS);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const float* kq = ch ? ktq : ktp;
            uint32_t h01, l01, h23, l23;
            split_f16x2(kq[0], kq[1], h01, l01);
            split_f16x2(kq[2], kq[3], h23, l23);
            *reinterpret_cast<uint2*>(&op.KtT[0][2 * cp + ch][tp]) = make_uint2(h01, h23);
            *reinterpret_cast<uint2*>(&op.KtT[1][2 * cp + ch][tp]) = make_uint2(l01, l23);
        }
    }
    helper_sync(&sm.hcount, htarget, lane);

    // (2) A and M blocks on MFMA; the diagonal blocks of A are inverted by the
    // wave that built them.
    //   six or more helpers:  hw 0: A00 -> T00  1: A11 -> T11  2: A10  3: M10  4: M00  5: M11
    //   four helpers:         hw 0: A00 -> T00  1: A11 -> T11  2: A10, M10    3: M00, M11
    constexpr int NTILE = (NH >= 6) ? 1 : 2;
    for (int ti = 0; ti < NTILE; ++ti) {
        int tile;                                  // 0 A00, 1 A11, 2 A10, 3 M10, 4 M00, 5 M11
        if constexpr (NH >= 6) tile = hw;
        else tile = (hw < 2) ? (ti == 0 ? hw : 6) : (hw == 2 ? 2 + ti : 4 + ti);
        if (tile >= 6) continue;
        const bool isM = tile >= 3;
        const int rb = (tile == 0 || tile == 4) ? 0 : 1;
        const int cb = (tile == 2 || tile == 3) ? 0 : rb;
        const bool diag = (rb == cb);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = acc, acc3 = acc;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const int off32 = 32 * kk + 8 * grp;
            const int rrow = 16 * rb + l16;
            const bf16x8 ch = lds_vec<bf16x8>(diag ? &sm.Kb[0][16 * cb + l16][off32] : &sm.Kr[0][l16][off32]);
            if (isM) {   // M feeds the output directly: two-term split on both sides
                const bf16x8 rh = lds_vec<bf16x8>(&sm.Qa[0][rrow][off32]);
                const bf16x8 rl = lds_vec<bf16x8>(&sm.Qa[1][rrow][off32]);
                const bf16x8 cl = lds_vec<bf16x8>(diag ? &sm.Kb[1][16 * cb + l16][off32] : &sm.Kr[1][l16][off32]);
                acc = mfma16(rh, ch, acc);      // three independent chains
                acc2 = mfma16(rh, cl, acc2);
                acc3 = mfma16(rl, ch, acc3);
            } else {     // A only conditions the solve: bf16 operands
                acc = mfma16(lds_vec<bf16x8>(&sm.Ka[rrow][off32]), ch, acc);
            }
        }
        if (isM) {
            acc += acc2 + acc3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rb + 4 * grp + j, i = 16 * cb + l16;
                const float val = (i <= r) ? acc[j] : 0.f;
                split16(val, op.M[0][r][kperm(i)], op.M[1][r][kperm(i)]);
                if (rb == 0) {
                    op.M[0][r][kperm(16 + l16)] = (_Float16)0.f;
                    op.M[1][r][kperm(16 + l16)] = (_Float16)0.f;
                }
            }
        } else if (!diag) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * grp + j;
                op.A10[r][kperm(l16)] = (_Float16)(op.beta[16 + r] * acc[j]);
                op.A10[r][kperm(16 + l16)] = (_Float16)0.f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * grp + j;
                sm.Ad[rb][r][l16] = (l16 < r) ? op.beta[16 * rb + r] * acc[j] : 0.f;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            float x[16];
            tri_inverse16(sm.Ad[rb], l16, x);
            if (grp == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    op.Tm[16 * rb + r][kperm(16 * rb + l16)] = (_Float16)x[r];
                    op.Tm[16 * rb + r][kperm(16 * (1 - rb) + l16)] = (_Float16)0.f;
                }
            }
        }
    }
}

__global__ __launch_bounds__(NT, 1) void kda_fwd_pipe(FwdArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    const bool is_state = wave < NS;

    const int bid = blockIdx.x;
    const int xcd = bid & 7, rest = bid >> 3;
    const int vblk = rest % P;
    const int chain = (rest / P) * 8 + xcd;
    if (chain >= a.nchains) return;
    const int n = chain / a.H, h = chain % a.H;
    int row, t0, t1;
    if (a.cu) { row = 0; t0 = a.cu[n]; t1 = a.cu[n + 1]; }
    else      { row = n; t0 = 0;       t1 = a.T; }
    const int nch = (t1 - t0 + C - 1) / C;
    const uint32_t ts = (uint32_t)a.H * D;
    const long long base = (long long)row * a.T * ts + (long long)h * D;
    const long long bbase = (long long)row * a.T * a.H + h;
    const long long sbase = ((long long)n * a.H + h) * D * D;

    if (tid == 0) sm.hcount = 0u;
    __syncthreads();

    // ---------------- state-wave registers
    const int vc = vblk * VB + wave * 16 + l16;                     // state lane's V column
    const uint32_t vofs = (uint32_t)(4 * grp) * ts + vc;            // (row 4grp, column vc) in a chunk
    f32x4 S[8];
    uint32_t vcur[8], vnxt[8];
    // ---------------- helper registers
    const int ht = tid - 64 * NS, hw = wave - NS;
    const uint32_t hoff = 2 * (ht & 63);                           // channel pair offset
    uint32_t htarget = 0;
    HFetch f;

    // V of this lane's column for the chunk's tokens 16t + 4grp + j, as raw bf16
    // bits from clamped rows; converted and masked where used.
    auto vfetch = [&](uint32_t* dst, int cidx) {
        const int cs = t0 + cidx * C;
        const int nv = min(C, t1 - cs);
        const uint16_t* vp = static_cast<const uint16_t*>(a.v) + base + (long long)cs * ts;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rc = min(16 * t + 4 * grp + j, nv - 1);
                dst[4 * t + j] = vp[(uint32_t)rc * ts + vc];
            }
    };

    // Both roles execute the same number of workgroup barriers: two before the
    // chunk loop and one per chunk.
    if (is_state) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[m][j] = a.h0 ? a.h0[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] : 0.f;
        if (nch > 0) vfetch(vcur, 0);
        __syncthreads();
        for (int ci = 0; ci < nch; ++ci) {
            const int cs = t0 + ci * C;
            const int nv = min(C, t1 - cs);
                const Ops& op = sm.op[ci & 1];
                if (ci + 1 < nch) vfetch(vnxt, ci + 1);
                f16x8 SBh[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        SBh[kk][j] = (_Float16)S[2 * kk][j];
                        SBh[kk][4 + j] = (_Float16)S[2 * kk + 1][j];
                    }
                f32x4 Pt[2], Ot[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    Pt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    Ot[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int off = 32 * kk + 8 * grp;
                        Pt[t] = mfma16(lds_vec<f16x8>(&op.Kg[16 * t + l16][off]), SBh[kk], Pt[t]);
                        Ot[t] = mfma16(lds_vec<f16x8>(&op.Qg[16 * t + l16][off]), SBh[kk], Ot[t]);
                    }
                }
                float be[2][4];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        be[t][j] = op.beta[16 * t + 4 * grp + j] * (__uint_as_float(vcur[4 * t + j] << 16) - Pt[t][j]);
                // Delta0 = T00 bE0
                const f16x8 Z8 = {0, 0, 0, 0, 0, 0, 0, 0};
                f16x8 Bh = Z8, Bl = Z8;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2s u = split16(be[0][j]);
                    Bh[j] = u.hi;
                    Bl[j] = u.lo;
                }
                f32x4 D0 = {0.f, 0.f, 0.f, 0.f};
                {
                    const f16x8 th = lds_vec<f16x8>(&op.Tm[l16][8 * grp]);
                    D0 = mfma16(th, Bh, D0);
                    D0 = mfma16(th, Bl, D0);
                }
                f16x8 DBh = Z8, DBl = Z8;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2s u = split16(D0[j]);
                    DBh[j] = u.hi;
                    DBl[j] = u.lo;
                }
                // Delta1 = T11 (bE1 - A10 Delta0)
                f32x4 X = {0.f, 0.f, 0.f, 0.f};
                {
                    const f16x8 ah = lds_vec<f16x8>(&op.A10[l16][8 * grp]);
                    X = mfma16(ah, DBh, X);
                    X = mfma16(ah, DBl, X);
                }
                Bh = Z8;
                Bl = Z8;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2s u = split16(be[1][j] - X[j]);
                    Bh[4 + j] = u.hi;
                    Bl[4 + j] = u.lo;
                }
                f32x4 D1 = {0.f, 0.f, 0.f, 0.f};
                {
                    const f16x8 th = lds_vec<f16x8>(&op.Tm[16 + l16][8 * grp]);
                    D1 = mfma16(th, Bh, D1);
                    D1 = mfma16(th, Bl, D1);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2s u = split16(D1[j]);
                    DBh[4 + j] = u.hi;
                    DBl[4 + j] = u.lo;
                }
                // O = (Q*gamma) S + M Delta
                float* och = a.o + base + (long long)cs * ts;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const f16x8 mh = lds_vec<f16x8>(&op.M[0][16 * t + l16][8 * grp]);
                    const f16x8 ml = lds_vec<f16x8>(&op.M[1][16 * t + l16][8 * grp]);
                    f32x4 acc = Ot[t];
                    acc = mfma16(mh, DBh, acc);
                    acc = mfma16(mh, DBl, acc);
                    acc = mfma16(ml, DBh, acc);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (16 * t + 4 * grp + j < nv) och[vofs + (uint32_t)(16 * t + j) * ts] = acc[j];
                }
                // S <- Diag(gamma_last) S + Kt^T Delta
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const float4 g4 = lds_vec<float4>(&op.gl[16 * m + 4 * grp]);
                    S[m][0] *= g4.x;
                    S[m][1] *= g4.y;
                    S[m][2] *= g4.z;
                    S[m][3] *= g4.w;
                    const f16x8 kh = lds_vec<f16x8>(&op.KtT[0][16 * m + l16][8 * grp]);
                    const f16x8 kl = lds_vec<f16x8>(&op.KtT[1][16 * m + l16][8 * grp]);
                    S[m] = mfma16(kh, DBh, S[m]);
                    S[m] = mfma16(kh, DBl, S[m]);
                    S[m] = mfma16(kl, DBh, S[m]);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) vcur[j] = vnxt[j];
            __syncthreads();
        }
        if (a.hT) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a.hT[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] = S[m][j];
        }
    } else {
        if (nch > 0) {
            hfetch(f, a, base + (long long)t0 * ts, bbase + (long long)t0 * a.H, ts, hoff, min(C, t1 - t0), ht >> 6, ht);
            const bool more = nch > 1;
            prepare(sm, sm.op[0], f, min(C, t1 - t0), hw, lane, ht, htarget, more, a,
                    base + (long long)(t0 + C) * ts, bbase + (long long)(t0 + C) * a.H, ts, hoff,
                    more ? min(C, t1 - t0 - C) : 0);
        }
        __syncthreads();
        for (int ci = 0; ci < nch; ++ci) {
            const int cs = t0 + ci * C;
            if (ci + 1 < nch) {
                // registers of chunk ci+1 were fetched during the previous prepare()
                const int ncs = cs + C;
                const bool more = ci + 2 < nch;
                const long long nb = base + (long long)(ncs + C) * ts, nbb = bbase + (long long)(ncs + C) * a.H;
                const int nnv = more ? min(C, t1 - ncs - C) : 0;
                prepare(sm, sm.op[(ci + 1) & 1], f, min(C, t1 - ncs), hw, lane, ht, htarget, more, a, nb, nbb, ts,
                        hoff, nnv);
            }
            __syncthreads();
        }
    }
}
}  // namespace pipe

int pipe_workgroups(int nchains) {
    const int groups = (nchains + 7) / 8;
    return groups * 8 * pipe::P;
}

hipError_t launch_fwd_pipe(const FwdArgs& a, hipStream_t stream) {
    const int grid = pipe_workgroups(a.nchains);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(pipe::kda_fwd_pipe, dim3(grid), dim3(pipe::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
