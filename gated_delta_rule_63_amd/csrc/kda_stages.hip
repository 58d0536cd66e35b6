// kda_stages.hip -- the chunked KDA forward as separately launchable stages.
//
// The same four steps the fused kernels run, each as its own kernel that
// reads and writes its intermediates in device memory, in plain fp32:
//   a0 chunk map       slot -> (sequence, first token, valid tokens) from cu_seqlens
//   a1 gate scan       Gamma_r = sum_{j<=r} g_j within each chunk; gamma_last = exp(Gamma_last)
//   a2 intra-chunk     A = strict-lower(Diag(beta) (K K^T gated)), Tinv = (I + A)^{-1},
//                      W = Tinv Diag(beta) (K*gamma), U = Tinv Diag(beta) V,
//                      Kt = K*exp(Gamma_last - Gamma), Qg = Q*gamma, M = lower(Q K^T gated)
//   a3 recurrence      per (sequence, head, V-block), chunk by chunk:
//                      h_c = S; Delta = U - W S; S <- Diag(gamma_last) S + Kt^T Delta; hT = S
//   a4 output          O = Qg h_c + M Delta
// The pages describe the method's forward as a chunked two-kernel design
// (toolarium.ru page, section "Где ограничения прямо сейчас"); these stages
// make every intermediate observable, which is what the stage tests and the
// stage-by-stage timing use. The fused kernels are the product's hot path.
#include "kda_device.h"
#include "kda_stages.h"
#include "kda_launch.h"

namespace kda {
namespace stages {

constexpr int C = kStageChunk;

// ---------------------------------------------------------------- a0 chunk map
// One workgroup. Without cu_seqlens the sequences are the B rows of T tokens.
// Slots beyond the last chunk get length 0 (the grid is sized for the worst case).
__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* cu, int N, int B, int T, int nslots,
                                                         int32_t* map, int32_t* seqinfo) {
    __shared__ int32_t base[1025];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int s0 = 0; s0 < N; s0 += 1024) {
        const int n = s0 + tid;
        int len = 0;
        if (n < N) len = cu ? (cu[n + 1] - cu[n]) : T;
        const int nc = (len + C - 1) / C;
        base[tid + 1] = nc;
        if (tid == 0) base[0] = carry;
        __syncthreads();
        // inclusive scan of base[1..1024] (Hillis-Steele), then add the carry in base[0]
        for (int off = 1; off < 1024; off <<= 1) {
            const int v = (tid >= off) ? base[tid + 1 - off] : 0;
            __syncthreads();
            base[tid + 1] += v;
            __syncthreads();
        }
        const int first = base[0] + base[tid + 1] - nc;   // this sequence's first slot
        if (n < N) {
            const int t0 = cu ? cu[n] : 0;
            seqinfo[2 * n] = first;
            seqinfo[2 * n + 1] = nc;
            for (int c = 0; c < nc; ++c) {
                const int s = first + c;
                map[4 * s + 0] = n;
                map[4 * s + 1] = t0 + c * C;                  // first token (within the row)
                map[4 * s + 2] = min(C, len - c * C);         // valid tokens
                map[4 * s + 3] = cu ? 0 : n;                  // batch row
            }
        }
        __syncthreads();
        if (tid == 0) carry = base[0] + base[1024];
        __syncthreads();
    }
    // empty slots
    const int used = carry;
    for (int s = used + tid; s < nslots; s += 1024) {
        map[4 * s + 0] = -1;
        map[4 * s + 1] = 0;
        map[4 * s + 2] = 0;
        map[4 * s + 3] = 0;
    }
}

struct Slot {
    int seq, t0, nv, row;
};
__device__ __forceinline__ Slot slot_of(const int32_t* map, int s) {
    const int4 m = reinterpret_cast<const int4*>(map)[s];
    return Slot{m.x, m.y, m.z, m.w};
}

__device__ __forceinline__ float ld(const void* p, long long i, bool f32) {
    if (f32) return static_cast<const float*>(p)[i];
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}

// ---------------------------------------------------------------- a1 gate scan
// grid (slot, head), 128 threads = channels.
__global__ __launch_bounds__(D) void gate_scan_kernel(StageArgs a) {
    const Slot sl = slot_of(a.map, blockIdx.x);
    const int h = blockIdx.y, c = threadIdx.x;
    if (sl.nv <= 0) return;
    const long long ts = (long long)a.H * D;
    const long long base = ((long long)sl.row * a.T + sl.t0) * ts + (long long)h * D + c;
    float run = 0.f;
    for (int r = 0; r < sl.nv; ++r) {
        run += a.g[base + r * ts];
        a.Gamma[base + r * ts] = run;
    }
    a.gl[((long long)blockIdx.x * a.H + h) * D + c] = expf(run);
}

// ---------------------------------------------------------------- a2 intra-chunk
// grid (slot, head), 256 threads. All fp32 in LDS.
__global__ __launch_bounds__(256) void intra_kernel(StageArgs a) {
    const Slot sl = slot_of(a.map, blockIdx.x);
    const int h = blockIdx.y, tid = threadIdx.x;
    if (sl.nv <= 0) return;
    __shared__ float sK[C][D + 1], sQ[C][D + 1], sG[C][D + 1];
    __shared__ float sA[C][C + 1], sT[C][C + 1], sB[C];
    const int n = sl.nv;
    const long long ts = (long long)a.H * D;
    const long long base = ((long long)sl.row * a.T + sl.t0) * ts + (long long)h * D;
    const long long bbase = ((long long)sl.row * a.T + sl.t0) * a.H + h;
    for (int i = tid; i < C * D; i += 256) {
        const int r = i / D, c = i % D;
        const bool ok = r < n;
        sK[r][c] = ok ? ld(a.k, base + r * ts + c, a.f32) : 0.f;
        sQ[r][c] = ok ? ld(a.q, base + r * ts + c, a.f32) : 0.f;
        sG[r][c] = ok ? a.Gamma[base + r * ts + c] : 0.f;
    }
    if (tid < C) sB[tid] = tid < n ? a.beta[bbase + (long long)tid * a.H] : 0.f;
    __syncthreads();
    // A (strictly lower, beta-weighted) and M (lower incl. diagonal)
    for (int e = tid; e < C * C; e += 256) {
        const int r = e / C, i = e % C;
        float sa = 0.f, sm = 0.f;
        if (i <= r && r < n) {
            for (int c = 0; c < D; ++c) {
                const float gate = expf(sG[r][c] - sG[i][c]);      // exponent <= 0
                sa += sK[r][c] * sK[i][c] * gate;
                sm += sQ[r][c] * sK[i][c] * gate;
            }
        }
        sA[r][i] = (i < r) ? sB[r] * sa : 0.f;
        if (r < n) a.M[((long long)(blockIdx.x * a.H + h) * C + r) * C + i] = (i <= r) ? sm : 0.f;
        else a.M[((long long)(blockIdx.x * a.H + h) * C + r) * C + i] = 0.f;
    }
    __syncthreads();
    // Tinv = (I + A)^{-1}: thread j < C forward-substitutes column j
    if (tid < C) {
        const int j = tid;
        for (int r = 0; r < C; ++r) {
            float s = (r == j) ? 1.f : 0.f;
            for (int i = 0; i < r; ++i) s -= sA[r][i] * sT[i][j];
            sT[r][j] = s;
        }
    }
    __syncthreads();
    // Kt = K*exp(Gamma_last - Gamma), Qg = Q*gamma (raw K, Q still in LDS)
    for (int e = tid; e < C * D; e += 256) {
        const int r = e / D, c = e % D;
        if (r >= n) continue;
        const long long o = base + r * ts + c;
        a.Kt[o] = sK[r][c] * expf(sG[n - 1][c] - sG[r][c]);
        a.Qg[o] = sQ[r][c] * expf(sG[r][c]);
    }
    __syncthreads();
    // reuse the tiles: sK <- Diag(beta) (K*gamma), sQ <- Diag(beta) V
    for (int e = tid; e < C * D; e += 256) {
        const int r = e / D, c = e % D;
        const bool ok = r < n;
        sK[r][c] = ok ? sB[r] * sK[r][c] * expf(sG[r][c]) : 0.f;
        sQ[r][c] = ok ? sB[r] * ld(a.v, base + r * ts + c, a.f32) : 0.f;
    }
    __syncthreads();
    // W = Tinv Diag(beta) (K*gamma), U = Tinv Diag(beta) V
    for (int e = tid; e < C * D; e += 256) {
        const int r = e / D, c = e % D;
        if (r >= n) continue;
        float w = 0.f, u = 0.f;
        for (int i = 0; i <= r; ++i) {
            w += sT[r][i] * sK[i][c];
            u += sT[r][i] * sQ[i][c];
        }
        a.W[base + r * ts + c] = w;
        a.U[base + r * ts + c] = u;
    }
}

// ---------------------------------------------------------------- a3 recurrence
// grid (sequence * head, 8 V-blocks of 16 columns), 256 threads. S block [128][16]
// lives in LDS; each thread owns 8 of its entries.
constexpr int RVB = 16;
__global__ __launch_bounds__(256) void recurrence_kernel(StageArgs a) {
    const int chain = blockIdx.x, vb = blockIdx.y, tid = threadIdx.x;
    const int n = chain / a.H, h = chain % a.H;
    __shared__ float sS[D][RVB + 1], sW[C][D + 1], sKt[C][D + 1], sD[C][RVB + 1], sgl[D];
    const int first = a.seqinfo[2 * n], nch = a.seqinfo[2 * n + 1];
    const long long sb = ((long long)n * a.H + h) * D * D;
    for (int e = tid; e < D * RVB; e += 256) {
        const int kk = e / RVB, v = e % RVB;
        sS[kk][v] = a.h0 ? a.h0[sb + kk * D + vb * RVB + v] : 0.f;
    }
    const long long ts = (long long)a.H * D;
    for (int ci = 0; ci < nch; ++ci) {
        const int s = first + ci;
        const Slot sl = slot_of(a.map, s);
        const long long base = ((long long)sl.row * a.T + sl.t0) * ts + (long long)h * D;
        __syncthreads();
        for (int e = tid; e < C * D; e += 256) {
            const int r = e / D, c = e % D;
            const bool ok = r < sl.nv;
            sW[r][c] = ok ? a.W[base + r * ts + c] : 0.f;
            sKt[r][c] = ok ? a.Kt[base + r * ts + c] : 0.f;
        }
        if (tid < D) sgl[tid] = a.gl[((long long)s * a.H + h) * D + tid];
        // h_c = S (state entering the chunk)
        for (int e = tid; e < D * RVB; e += 256) {
            const int kk = e / RVB, v = e % RVB;
            a.hc[(((long long)s * a.H + h) * D + kk) * D + vb * RVB + v] = sS[kk][v];
        }
        __syncthreads();
        // Delta = U - W S
        for (int e = tid; e < C * RVB; e += 256) {
            const int r = e / RVB, v = e % RVB;
            float acc = 0.f;
            if (r < sl.nv) {
                acc = a.U[base + r * ts + vb * RVB + v];
                for (int kk = 0; kk < D; ++kk) acc -= sW[r][kk] * sS[kk][v];
                a.Delta[base + r * ts + vb * RVB + v] = acc;
            }
            sD[r][v] = acc;
        }
        __syncthreads();
        // S <- Diag(gamma_last) S + Kt^T Delta
        for (int e = tid; e < D * RVB; e += 256) {
            const int kk = e / RVB, v = e % RVB;
            float acc = sgl[kk] * sS[kk][v];
            for (int r = 0; r < C; ++r) acc += sKt[r][kk] * sD[r][v];
            sS[kk][v] = acc;
        }
    }
    __syncthreads();
    if (a.hT)
        for (int e = tid; e < D * RVB; e += 256) {
            const int kk = e / RVB, v = e % RVB;
            a.hT[sb + kk * D + vb * RVB + v] = sS[kk][v];
        }
}

// ---------------------------------------------------------------- a4 output
// grid (slot, head), 256 threads: O = Qg h_c + M Delta.
__global__ __launch_bounds__(256) void output_kernel(StageArgs a) {
    const Slot sl = slot_of(a.map, blockIdx.x);
    const int h = blockIdx.y, tid = threadIdx.x;
    if (sl.nv <= 0) return;
    __shared__ float sQ[C][D + 1], sM[C][C + 1], sH[D][33];
    __shared__ float sDl[C][33];
    const long long ts = (long long)a.H * D;
    const long long base = ((long long)sl.row * a.T + sl.t0) * ts + (long long)h * D;
    const long long hcb = ((long long)blockIdx.x * a.H + h) * D * D;
    for (int e = tid; e < C * D; e += 256) {
        const int r = e / D, c = e % D;
        sQ[r][c] = r < sl.nv ? a.Qg[base + r * ts + c] : 0.f;
    }
    for (int e = tid; e < C * C; e += 256) sM[e / C][e % C] = a.M[((long long)(blockIdx.x * a.H + h) * C) * C + e];
    for (int v0 = 0; v0 < D; v0 += 32) {
        __syncthreads();
        for (int e = tid; e < D * 32; e += 256) sH[e / 32][e % 32] = a.hc[hcb + (long long)(e / 32) * D + v0 + e % 32];
        for (int e = tid; e < C * 32; e += 256) {
            const int r = e / 32;
            sDl[r][e % 32] = r < sl.nv ? a.Delta[base + r * ts + v0 + e % 32] : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < C * 32; e += 256) {
            const int r = e / 32, v = e % 32;
            if (r >= sl.nv) continue;
            float acc = 0.f;
            for (int kk = 0; kk < D; ++kk) acc += sQ[r][kk] * sH[kk][v];
            for (int i = 0; i <= r; ++i) acc += sM[r][i] * sDl[i][v];
            a.o[base + r * ts + v0 + v] = acc;
        }
    }
}

}  // namespace stages

hipError_t launch_chunk_map(const StageArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(stages::chunk_map_kernel, dim3(1), dim3(1024), 0, s, a.cu, a.N, a.B, a.T, a.nslots,
                       a.map, a.seqinfo);
    return hipGetLastError();
}
hipError_t launch_gate_scan(const StageArgs& a, hipStream_t s) {
    if (a.nslots == 0) return hipSuccess;
    hipLaunchKernelGGL(stages::gate_scan_kernel, dim3(a.nslots, a.H), dim3(D), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_intra(const StageArgs& a, hipStream_t s) {
    if (a.nslots == 0) return hipSuccess;
    hipLaunchKernelGGL(stages::intra_kernel, dim3(a.nslots, a.H), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_recurrence(const StageArgs& a, hipStream_t s) {
    if (a.N * a.H == 0) return hipSuccess;
    hipLaunchKernelGGL(stages::recurrence_kernel, dim3(a.N * a.H, D / stages::RVB), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_output(const StageArgs& a, hipStream_t s) {
    if (a.nslots == 0) return hipSuccess;
    hipLaunchKernelGGL(stages::output_kernel, dim3(a.nslots, a.H), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
