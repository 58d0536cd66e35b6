// kda_fused_serial.hip -- the fused chunked KDA forward for gfx950, one phase at a time.
// It serves fp32 inputs; bf16 inputs take the pipelined kernel (kda_fused_pipe.hip).
//
// One workgroup owns one (sequence, head, V-block) chain and walks its chunks
// in order. Per chunk of C = 32 tokens (two 16-token sub-blocks) it
//   (1) scans the log-gate within each sub-block and forms the gated key/query
//       factors (per-chunk cumulative log-gate scan);
//   (2) builds the beta-weighted strictly-lower gated K K^T (A) and the lower
//       gated Q K^T (M) on MFMA, and inverts the two 16 x 16 diagonal blocks
//       of I + A by forward substitution on tiles staged in LDS;
//   (3) advances the 128 x 16-per-wave fp32 state on MFMA:
//           E = V - (K*gamma) S,   Delta = (I + A)^{-1} Diag(beta) E   (block
//           forward substitution: Delta0 = T00 bE0, Delta1 = T11 (bE1 - A10 Delta0)),
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
// number (the pages' reason for short chunks: the bf16 numeric range). The
// scan runs in log2 units so every exponential is one v_exp_f32.
//
// Precision. bf16 inputs: the gated K K^T / Q K^T blocks use two-term bf16
// splits (3 MFMAs per product, fp32 range); (K*gamma) S and (Q*gamma) S use
// fp16 operands; the V-scale operands of the Delta solve, of M Delta and of
// Kt^T Delta are split into fp16 hi + lo. fp32 inputs: A and M on fp32 MFMA
// and every other product split into fp16 hi + lo on both sides.
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
constexpr int LDA = 16 + 4;    // padded row of an fp32 16 x 16 tile
constexpr int LDV = VB + 4;    // padded row of the staged V tile
constexpr float LOG2E = 1.4426950408889634f;
static_assert(NT == 4 * (D / 2), "the scan maps one thread to each (channel pair, 8-token quarter)");
static_assert(C == 32, "the sub-block bookkeeping below is written for two 16-token sub-blocks");
static_assert(NT * 8 == C * VB, "one 8-element slice of the V tile per thread");

// A/M operands: fp32 for the fp32-MFMA path, [hi, lo] bf16 otherwise.
template <bool F32> struct AMStore;
template <> struct AMStore<true> {
    float Ka[C][LDF], Qa[C][LDF], Kb[C][LDF], Kr[16][LDF];
};
template <> struct AMStore<false> {
    __bf16 Ka[2][C][LDP], Qa[2][C][LDP], Kb[2][C][LDP], Kr[2][16][LDP];
};

template <bool F32> struct alignas(16) Smem {
    AMStore<F32> am;                    // Ka, Qa: row factors  k, q * exp(Gamma_r - Gamma_mid)
                                        // Kb: column factors   k * exp(Gamma_mid - Gamma_r)
                                        // Kr: block-0 keys referenced to block 1's middle
    _Float16 Kg[F32 ? 2 : 1][C][LDP];   // K * exp(Gamma), channels permuted in 32-groups
    _Float16 Qg[F32 ? 2 : 1][C][LDP];   // Q * exp(Gamma), same order
    _Float16 KtT[2][D][TP];             // (K * exp(Gamma_last - Gamma))^T, [hi, lo][channel][kperm(token)]
    float Ad[2][16][LDA];               // diagonal blocks of A for the forward substitution
    _Float16 A10[2][16][TP];            // A block (rows 16-31, cols 0-15), [hi, lo][row][kperm(col)]
    _Float16 Tm[2][C][TP];              // block-diagonal (I + A)^{-1}, [hi, lo][row][kperm(col)]
    _Float16 M[2][C][TP];               // lower gated Q K^T, [hi, lo][row][kperm(col)]
    float V[C][LDV];                    // this workgroup's V columns of the chunk
    float gl[D];                        // exp(Gamma_last), the chunk's decay per channel
    float beta[C];
    float qtot[4][D];                   // sum of g * log2(e) over each 8-token quarter
};

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

// Per-thread constant offsets (elements) of its loads within a chunk.
struct Offs {
    uint32_t gk;   // (8qq) * ts + 2cp : q, k, g of token 8qq, channels 2cp, 2cp+1
    uint32_t v;    // (tid >> 3) * ts + vcol0 + (tid & 7) * 8 : V tile slice
};

// Raw buffer access to the rows of one chunk of a [row][...] tensor: the
// resource starts at the chunk's first element for this head and ends after
// the last valid row's `valid_elems` elements, so reads of rows past the end
// return zero. Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* p, long long elem_off, int elem_bytes, int nv,
                                                            uint32_t row_elems, int valid_elems) {
    const char* base = static_cast<const char*>(p) + elem_off * elem_bytes;
    const int nbytes = nv > 0 ? ((nv - 1) * (int)row_elems + valid_elems) * elem_bytes : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nbytes, 0x00020000);
}

// Rows past the chunk's valid rows read as zero through bounded buffer
// resources: the loads need no branch and no select, so they stay in flight
// until the next chunk consumes them, and the fetched values stay in registers.
template <bool F32>
__device__ __forceinline__ void fetch(Fetch<F32>& f, const FwdArgs& a, long long cbase, long long cbeta,
                                      uint32_t ts, const Offs& of, int nv, int qq, int tid) {
    constexpr int EB = F32 ? 4 : 2;   // bytes per q, k, v element
    const auto rk = rows_rsrc(a.k, cbase, EB, nv, ts, D);
    const auto rq = rows_rsrc(a.q, cbase, EB, nv, ts, D);
    const auto rg = a.scalar_gate ? rows_rsrc(a.g, cbeta, 4, nv, (uint32_t)a.H, 1) : rows_rsrc(a.g, cbase, 4, nv, ts, D);
    const auto rb = rows_rsrc(a.beta, cbeta, 4, nv, (uint32_t)a.H, 1);
    const auto rv = rows_rsrc(a.v, cbase, EB, nv, ts, D);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t o = of.gk + (uint32_t)t * ts;   // element offset of (token 8qq + t, channel 2cp)
        if (a.scalar_gate) {
            const float gs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       rg, (uint32_t)(8 * qq + t) * (uint32_t)a.H * 4u, 0, 0));
            f.g[t] = make_float2(gs, gs);
        } else {
            f.g[t] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rg, 4u * o, 0, 0));
        }
        if constexpr (F32) {
            f.k[t] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rk, 4u * o, 0, 0));
            f.q[t] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rq, 4u * o, 0, 0));
        } else {
            f.k[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, 2u * o, 0, 0);
            f.q[t] = __builtin_amdgcn_raw_buffer_load_b32(rq, 2u * o, 0, 0);
        }
    }
    f.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)tid * (uint32_t)a.H * 4u, 0, 0));
    if constexpr (F32) {
        f.v0 = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rv, 4u * of.v, 0, 0));
        f.v1 = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rv, 4u * (of.v + 4), 0, 0));
    } else {
        f.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, 2u * of.v, 0, 0));
    }
}

// Forward substitution of one unit-lower-triangular 16 x 16 block: lane j
// (of 16) returns column j of (I + Ablk)^{-1}; Ablk rows are read from LDS.
__device__ __forceinline__ void tri_inverse16(const float (*Ablk)[LDA], int j, float x[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float s0 = (r == j) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i + 1 < r; i += 2) {
            const float2 a2 = *reinterpret_cast<const float2*>(&Ablk[r][i]);
            s0 -= a2.x * x[i];
            s1 -= a2.y * x[i + 1];
        }
        if (r & 1) s0 -= Ablk[r][r - 1] * x[r - 1];
        x[r] = s0 + s1;
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
    const uint32_t ts = (uint32_t)a.H * D;                          // elements per token
    const long long base = (long long)row * a.T * ts + (long long)h * D;
    const long long bbase = (long long)row * a.T * a.H + h;         // beta of (row, t = 0, h)
    const int vcol0 = vblk * VB;
    const int vc = vcol0 + wave * 16 + l16;                         // this lane's V column
    const long long sbase = ((long long)n * a.H + h) * D * D;

    f32x4 S[8];                                  // rows 16m + 4grp + j, column vc
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            S[m][j] = a.h0 ? a.h0[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] : 0.f;

    const int cp = tid & 63, qq = tid >> 6;      // scan thread: channel pair, 8-token quarter
    const int b = qq >> 1, half = qq & 1;        // its 16-token sub-block and half of it
    Offs of;
    of.gk = (uint32_t)(8 * qq) * ts + 2 * cp;
    of.v = (uint32_t)(tid >> 3) * ts + vcol0 + (tid & 7) * 8;
    const uint32_t ooff = (uint32_t)(4 * grp) * ts + vc;           // o: this lane's (row 4grp, column vc)

    Fetch<F32> f;
    if (t0 < t1) fetch<F32>(f, a, base + (long long)t0 * ts, bbase + (long long)t0 * a.H, ts, of, min(C, t1 - t0), qq, tid);

    for (int cs = t0; cs < t1; cs += C) {
        const int nv = min(C, t1 - cs);

        // ---- (1) gate scan (log2 units) over tokens 8qq .. 8qq+7, channels 2cp, 2cp+1
        float L[2][8];
        {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                r0 += f.g[t].x * LOG2E;
                r1 += f.g[t].y * LOG2E;
                L[0][t] = r0;
                L[1][t] = r1;
            }
            *reinterpret_cast<float2*>(&sm.qtot[qq][2 * cp]) = make_float2(r0, r1);
        }
        if (tid < C) sm.beta[tid] = f.beta;
        {
            const int vr = tid >> 3, vcc = (tid & 7) * 8;
            float4 w0, w1;
            if constexpr (F32) {
                w0 = f.v0;
                w1 = f.v1;
            } else {
                const float2 p0 = bf2(f.v.x), p1 = bf2(f.v.y), p2 = bf2(f.v.z), p3 = bf2(f.v.w);
                w0 = make_float4(p0.x, p0.y, p1.x, p1.y);
                w1 = make_float4(p2.x, p2.y, p3.x, p3.y);
            }
            *reinterpret_cast<float4*>(&sm.V[vr][vcc]) = w0;
            *reinterpret_cast<float4*>(&sm.V[vr][vcc + 4]) = w1;
        }
        float kv[2][8], qv[2][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (F32) {
                kv[0][t] = f.k[t].x; kv[1][t] = f.k[t].y; qv[0][t] = f.q[t].x; qv[1][t] = f.q[t].y;
            } else {
                const float2 kk2 = bf2(f.k[t]), qq2 = bf2(f.q[t]);
                kv[0][t] = kk2.x; kv[1][t] = kk2.y; qv[0][t] = qq2.x; qv[1][t] = qq2.y;
            }
        }
        __syncthreads();
        // the registers are consumed: fetch the next chunk while this one computes
        if (cs + C < t1)
            fetch<F32>(f, a, base + (long long)(cs + C) * ts, bbase + (long long)(cs + C) * a.H, ts, of,
                       min(C, t1 - cs - C), qq, tid);
        {
            float d[2][8], c1[2], c2[2], c3[2];
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
                c1[ch] = exp2f(start + L7);                    // exp(Gamma_mid)               -> K*gamma, Q*gamma
                c2[ch] = exp2f(L15 - L7 + after);              // exp(Gamma_last - Gamma_mid)  -> Kt
                c3[ch] = exp2f(L15 - L7 + qt2);                // block 0 -> block 1's middle  -> Kr
                if (qq == 0) sm.gl[c] = exp2f(tot0 + tot1);
#pragma unroll
                for (int t = 0; t < 8; ++t) d[ch][t] = L[ch][t] + off - L7;   // |d| <= 8 * 5 * log2(e)
            }
            const int cpos = ((2 * cp) & ~31) | kperm((2 * cp) & 31);     // channel pair position in Kg/Qg
#pragma unroll
            for (int t = 0; t < 8; t += 2) {
                float ka[2][2], qa[2][2], kb[2][2], kt[2][2];     // [token][channel]
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch) {
                        const float e1 = exp2f(d[ch][t + u]), e2 = exp2f(-d[ch][t + u]);
                        ka[u][ch] = kv[ch][t + u] * e1;
                        qa[u][ch] = qv[ch][t + u] * e1;
                        kb[u][ch] = kv[ch][t + u] * e2;
                        kt[u][ch] = kb[u][ch] * c2[ch];
                    }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int rr = 8 * qq + t + u;
                    if constexpr (F32) {
                        *reinterpret_cast<float2*>(&sm.am.Ka[rr][2 * cp]) = make_float2(ka[u][0], ka[u][1]);
                        *reinterpret_cast<float2*>(&sm.am.Qa[rr][2 * cp]) = make_float2(qa[u][0], qa[u][1]);
                        *reinterpret_cast<float2*>(&sm.am.Kb[rr][2 * cp]) = make_float2(kb[u][0], kb[u][1]);
                        if (b == 0)
                            *reinterpret_cast<float2*>(&sm.am.Kr[rr][2 * cp]) =
                                make_float2(kb[u][0] * c3[0], kb[u][1] * c3[1]);
                        uint32_t hi, lo;
                        split_f16x2(ka[u][0] * c1[0], ka[u][1] * c1[1], hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.Kg[0][rr][cpos]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.Kg[1][rr][cpos]) = lo;
                        split_f16x2(qa[u][0] * c1[0], qa[u][1] * c1[1], hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.Qg[0][rr][cpos]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.Qg[1][rr][cpos]) = lo;
                    } else {
                        uint32_t hi, lo;
                        split_bf16x2(ka[u][0], ka[u][1], hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.am.Ka[0][rr][2 * cp]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.am.Ka[1][rr][2 * cp]) = lo;
                        split_bf16x2(qa[u][0], qa[u][1], hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.am.Qa[0][rr][2 * cp]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.am.Qa[1][rr][2 * cp]) = lo;
                        split_bf16x2(kb[u][0], kb[u][1], hi, lo);
                        *reinterpret_cast<uint32_t*>(&sm.am.Kb[0][rr][2 * cp]) = hi;
                        *reinterpret_cast<uint32_t*>(&sm.am.Kb[1][rr][2 * cp]) = lo;
                        if (b == 0) {
                            split_bf16x2(kb[u][0] * c3[0], kb[u][1] * c3[1], hi, lo);
                            *reinterpret_cast<uint32_t*>(&sm.am.Kr[0][rr][2 * cp]) = hi;
                            *reinterpret_cast<uint32_t*>(&sm.am.Kr[1][rr][2 * cp]) = lo;
                        }
                        *reinterpret_cast<uint32_t*>(&sm.Kg[0][rr][cpos]) = pack_f16(ka[u][0] * c1[0], ka[u][1] * c1[1]);
                        *reinterpret_cast<uint32_t*>(&sm.Qg[0][rr][cpos]) = pack_f16(qa[u][0] * c1[0], qa[u][1] * c1[1]);
                    }
                }
                // Kt^T: tokens rr, rr+1 sit next to each other in kperm order
                const int tp = kperm(8 * qq + t);
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    uint32_t hi, lo;
                    split_f16x2(kt[0][ch], kt[1][ch], hi, lo);
                    *reinterpret_cast<uint32_t*>(&sm.KtT[0][2 * cp + ch][tp]) = hi;
                    *reinterpret_cast<uint32_t*>(&sm.KtT[1][2 * cp + ch][tp]) = lo;
                }
            }
        }
        __syncthreads();

        // ---- (2) A and M blocks; each diagonal block of A is inverted by the wave that built it.
        // wave 0: A00 -> T00   wave 1: A11 -> T11   wave 2: A10, M10   wave 3: M00, M11
        {
            const int ntile = (wave >= 2) ? 2 : 1;
            for (int ti = 0; ti < ntile; ++ti) {
                const bool isM = (wave == 3) || (wave == 2 && ti == 1);
                const int rb = (wave == 0) ? 0 : (wave == 3 ? ti : 1);
                const int cb = (wave == 2) ? 0 : rb;
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
                        const int rrow = 16 * rb + l16;
                        const bf16x8 rh = lds_vec<bf16x8>(isM ? &sm.am.Qa[0][rrow][off] : &sm.am.Ka[0][rrow][off]);
                        const bf16x8 rl = lds_vec<bf16x8>(isM ? &sm.am.Qa[1][rrow][off] : &sm.am.Ka[1][rrow][off]);
                        const bf16x8 ch = lds_vec<bf16x8>(diag ? &sm.am.Kb[0][16 * cb + l16][off] : &sm.am.Kr[0][l16][off]);
                        const bf16x8 cl = lds_vec<bf16x8>(diag ? &sm.am.Kb[1][16 * cb + l16][off] : &sm.am.Kr[1][l16][off]);
                        acc = mfma16(rh, ch, acc);
                        acc = mfma16(rh, cl, acc);
                        acc = mfma16(rl, ch, acc);
                    }
                }
                if (isM) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 16 * rb + 4 * grp + j, i = 16 * cb + l16;
                        const float val = (i <= r) ? acc[j] : 0.f;
                        split16(val, sm.M[0][r][kperm(i)], sm.M[1][r][kperm(i)]);
                        if (rb == 0) {   // zero upper-right block of M
                            sm.M[0][r][kperm(16 + l16)] = (_Float16)0.f;
                            sm.M[1][r][kperm(16 + l16)] = (_Float16)0.f;
                        }
                    }
                } else if (!diag) {      // A10 as an fp16 [hi, lo] operand over the block-0 token slots
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * grp + j;
                        split16(sm.beta[16 + r] * acc[j], sm.A10[0][r][kperm(l16)], sm.A10[1][r][kperm(l16)]);
                        sm.A10[0][r][kperm(16 + l16)] = (_Float16)0.f;
                        sm.A10[1][r][kperm(16 + l16)] = (_Float16)0.f;
                    }
                } else {                 // diagonal block: stage, then invert in this wave
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * grp + j;
                        sm.Ad[rb][r][l16] = (l16 < r) ? sm.beta[16 * rb + r] * acc[j] : 0.f;
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    float x[16];
                    tri_inverse16(sm.Ad[rb], l16, x);
                    if (grp == 0) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            split16(x[r], sm.Tm[0][16 * rb + r][kperm(16 * rb + l16)],
                                    sm.Tm[1][16 * rb + r][kperm(16 * rb + l16)]);
                            sm.Tm[0][16 * rb + r][kperm(16 * (1 - rb) + l16)] = (_Float16)0.f;
                            sm.Tm[1][16 * rb + r][kperm(16 * (1 - rb) + l16)] = (_Float16)0.f;
                        }
                    }
                }
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
            // beta (V - P) for both token tiles
            float be[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 16 * t + 4 * grp + j;
                    be[t][j] = sm.beta[rr] * (sm.V[rr][wave * 16 + l16] - Pt[t][j]);
                }
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
                const f16x8 th = lds_vec<f16x8>(&sm.Tm[0][l16][8 * grp]);
                D0 = mfma16(th, Bh, D0);
                D0 = mfma16(th, Bl, D0);
                if constexpr (F32) D0 = mfma16(lds_vec<f16x8>(&sm.Tm[1][l16][8 * grp]), Bh, D0);
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
                const f16x8 ah = lds_vec<f16x8>(&sm.A10[0][l16][8 * grp]);
                X = mfma16(ah, DBh, X);
                X = mfma16(ah, DBl, X);
                if constexpr (F32) X = mfma16(lds_vec<f16x8>(&sm.A10[1][l16][8 * grp]), DBh, X);
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
                const f16x8 th = lds_vec<f16x8>(&sm.Tm[0][16 + l16][8 * grp]);
                D1 = mfma16(th, Bh, D1);
                D1 = mfma16(th, Bl, D1);
                if constexpr (F32) D1 = mfma16(lds_vec<f16x8>(&sm.Tm[1][16 + l16][8 * grp]), Bh, D1);
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
                const f16x8 mh = lds_vec<f16x8>(&sm.M[0][16 * t + l16][8 * grp]);
                const f16x8 ml = lds_vec<f16x8>(&sm.M[1][16 * t + l16][8 * grp]);
                f32x4 acc = Ot[t];
                acc = mfma16(mh, DBh, acc);
                acc = mfma16(mh, DBl, acc);
                acc = mfma16(ml, DBh, acc);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rr = 16 * t + 4 * grp + j;
                    if (rr < nv) och[ooff + (uint32_t)(16 * t + j) * ts] = acc[j];
                }
            }
            // S <- Diag(gamma_last) S + Kt^T Delta
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float4 g4 = lds_vec<float4>(&sm.gl[16 * m + 4 * grp]);
                S[m][0] *= g4.x;
                S[m][1] *= g4.y;
                S[m][2] *= g4.z;
                S[m][3] *= g4.w;
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
                a.hT[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] = S[m][j];
    }
}

}  // namespace fused

int serial_workgroups(int nchains) {
    const int groups = (nchains + 7) / 8;
    return groups * 8 * fused::P;
}

hipError_t launch_fwd_serial(const FwdArgs& a, bool f32_inputs, hipStream_t stream) {
    const int grid = serial_workgroups(a.nchains);
    if (grid == 0) return hipSuccess;
    if (f32_inputs)
        hipLaunchKernelGGL(fused::kda_fwd_fused<true>, dim3(grid), dim3(fused::NT), 0, stream, a);
    else
        hipLaunchKernelGGL(fused::kda_fwd_fused<false>, dim3(grid), dim3(fused::NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
