// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation on
// the host, then kernel launches on the caller's stream.
#include "../../include/kda.h"

#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "kda_launch.h"
#include "kda_stages.h"

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

// Size limits, so that no index or byte count below overflows: at most 2^46
// elements per [B, T, H, 128] tensor and fewer than 2^27 (sequence, head)
// chains. Tested without overflowing (each factor is below 2^31).
bool sizes_ok(const kda_desc_t* d) {
    const long long tok = (long long)d->B * d->T;   // < 2^62
    if (tok > (((long long)1 << 46) / 128) / d->H) return false;
    return (long long)d->num_seqs * d->H <= INT_MAX / 16;
}

kda_status_t check(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   const int32_t* cu_seqlens, const void* o, const kda_desc_t* d) {
    if (!d) return KDA_ERR_NULL;
    if (d->B < 1 || d->T < 0 || d->H < 1 || d->K < 1 || d->V < 1) return KDA_ERR_SHAPE;
    if (d->K != 128 || d->V != 128) return KDA_ERR_UNSUPPORTED;
    if (d->in_dtype != KDA_BF16 && d->in_dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (d->out_dtype != KDA_BF16 && d->out_dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (d->out_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (cu_seqlens) {
        if (d->B != 1 || d->num_seqs < 0) return KDA_ERR_SHAPE;
    } else if (d->num_seqs != d->B) {
        return KDA_ERR_SHAPE;
    }
    if (!sizes_ok(d)) return KDA_ERR_SHAPE;
    const long long tok = (long long)d->B * d->T;
    if (tok > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    return KDA_OK;
}

// Shape-only validation shared by the staged entry points.
kda_status_t check_desc(const kda_desc_t* d, bool varlen) {
    if (!d) return KDA_ERR_NULL;
    if (d->B < 1 || d->T < 0 || d->H < 1 || d->K < 1 || d->V < 1) return KDA_ERR_SHAPE;
    if (d->K != 128 || d->V != 128) return KDA_ERR_UNSUPPORTED;
    if (d->in_dtype != KDA_BF16 && d->in_dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (d->out_dtype != KDA_BF16 && d->out_dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (d->out_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (varlen ? (d->B != 1 || d->num_seqs < 0) : (d->num_seqs != d->B)) return KDA_ERR_SHAPE;
    if (!sizes_ok(d)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device, read once per device (the attribute
// cannot change while the process runs; concurrent first calls store the
// same value).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

kda::FwdArgs fwd_args(const void* q, const void* k, const void* v, const float* g, const float* beta,
                      const int32_t* cu_seqlens, const float* h0, void* o, float* hT, const kda_desc_t* d) {
    kda::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu = cu_seqlens;
    a.h0 = h0;
    a.o = static_cast<float*>(o);
    a.hT = hT;
    a.B = d->B;
    a.T = d->T;
    a.H = d->H;
    a.N = d->num_seqs;
    a.nchains = d->num_seqs * d->H;
    a.scalar_gate = 0;
    a.ntasks = 0;
    return a;
}

constexpr int kMinSlice = 4096;   // tokens per slice before a chain is cut into three

// Few long chains (fixed-length, bf16): the chip holds far more workgroups
// than the chains fill, and each chain is a long sequential walk. A slice's
// state map and its outputs are affine in the state it starts from, so a
// chain is cut into slices of whole chunks, each later slice run from zero and
// from the identity alongside the first. Two routes:
//   S slices in one pass (desc->workspace of multi_slice_workspace_bytes):
//     one launch runs slice 0 for real and every later slice j from zero (o
//     into o, end state R_j) and from the identity with v = 0 (its o, ell,
//     into the workspace; its end state is Pmap_j), one workgroup per run, so
//     that all 2S - 1 runs of every chain fit on the chip together (S = 4 for
//     32 chains on 256 CUs). Then S_{j+1} = Pmap_j S_j + R_j in turn (the last
//     one is hT), and o of slice j += S_j^T ell per token. The critical path
//     is 1/S of a chain plus a streaming pass over the later slices' o.
//   three slices (less workspace, or none: 256 KiB per chain, allocated on
//     the stream when not given): pass 1 runs slice 0 for real and slice 1
//     from zero and from the identity; a combine forms slice 2's start state;
//     pass 2 reruns slice 1 and runs slice 2 from their true start states.
//     Two thirds of a chain on the critical path.
bool use_slices(long long nchains, const kda_desc_t* d, bool varlen, int cus) {
    return d->in_dtype == KDA_BF16 && !varlen && d->T >= 3 * kMinSlice && 6LL * nchains <= cus;
}

// Workspace of the three-slice route: four fp32 states per chain (S1, R1, Pmap1, S2).
size_t slice_workspace_bytes(long long nchains) { return (size_t)nchains * 4 * 128 * 128 * sizeof(float); }

// Slice count of the one-pass route: each slice after the first runs twice,
// one workgroup per run, and the 2S - 1 runs of all chains must fit on the
// chip at once; each slice keeps at least kMinSlice tokens. At least 2.
constexpr int kMaxSlices = (kda::kMaxTasks + 1) / 2;
int multi_slice_count(long long nchains, int T, int cus) {
    if (nchains <= 0) return 2;
    long long n = (cus / nchains + 1) / 2;
    n = std::min<long long>(n, kMaxSlices);
    n = std::min<long long>(n, T / kMinSlice);
    return (int)std::max<long long>(n, 2);
}

// First token of slice j of S (whole chunks; slice S starts at T).
int slice_begin(int T, int S, int j) { return j >= S ? T : (int)(((long long)j * T / S) / 32 * 32); }

// Workspace of the one-pass route: three fp32 states per chain and later
// slice (its start state S_j, R_j and Pmap_j) and ell, fp32
// [B, T - (first token of slice 1), H, 128].
size_t multi_slice_workspace_bytes(const kda_desc_t* d, int S) {
    const size_t states = (size_t)d->B * d->H * 3 * (S - 1) * 128 * 128 * sizeof(float);
    return states + (size_t)d->B * (d->T - slice_begin(d->T, S, 1)) * d->H * 128 * sizeof(float);
}

hipError_t run_multi_slices(const kda::FwdArgs& a, const kda_desc_t* d, int S, int cus, hipStream_t s) {
    const size_t per = (size_t)a.nchains * 128 * 128;
    float* const ws = static_cast<float*>(d->workspace);
    const auto start = [&](int j) { return ws + (size_t)(j - 1) * per; };            // S_j, slice j's start state
    const auto zero = [&](int j) { return ws + (size_t)(S - 1 + j - 1) * per; };      // R_j, slice j from zero
    const auto pmap = [&](int j) { return ws + (size_t)(2 * (S - 1) + j - 1) * per; };  // Pmap_j
    float* ell = ws + (size_t)3 * (S - 1) * per;                                     // o of the identity runs
    const int T = d->T, b1 = slice_begin(T, S, 1);
    kda::FwdArgs p = a;
    p.ntasks = 2 * S - 1;
    p.nchains = p.ntasks * a.nchains;
    p.task[0] = {0, b1, a.h0, start(1), 0};
    for (int j = 1; j < S; ++j) {
        const int t0 = slice_begin(T, S, j), t1 = slice_begin(T, S, j + 1);
        p.task[2 * j - 1] = {t0, t1, nullptr, zero(j), 0};
        p.task[2 * j] = {t0, t1, nullptr, pmap(j), kda::TASK_ZERO_V | kda::TASK_IDENTITY_H0, ell, b1, T - b1};
    }
    hipError_t e = kda::launch_fwd_pipe(p, cus, s);
    // the later slices' start states in turn; the last combine is the final state
    for (int j = 1; j < S && e == hipSuccess; ++j) {
        float* out = j + 1 < S ? start(j + 1) : a.hT;
        if (out) e = kda::launch_affine_combine(pmap(j), start(j), zero(j), out, a.nchains, s);
    }
    for (int j = 1; j < S && e == hipSuccess; ++j)
        e = kda::launch_state_correction(start(j), ell, a.o, a.N, T, a.H, slice_begin(T, S, j),
                                         slice_begin(T, S, j + 1), b1, s);
    return e;
}

hipError_t run_slices(const kda::FwdArgs& a, const kda_desc_t* d, int cus, hipStream_t s) {
    // the output correction reads ell in 16-byte pieces
    const int S = multi_slice_count(a.nchains, d->T, cus);
    if (d->workspace && d->workspace_bytes >= multi_slice_workspace_bytes(d, S) && aligned16(d->workspace))
        return run_multi_slices(a, d, S, cus, s);
    const size_t per = (size_t)a.nchains * 128 * 128;
    const size_t bytes = slice_workspace_bytes(a.nchains);
    void* ws = nullptr;
    bool owned = false;
    if (d->workspace && d->workspace_bytes >= bytes) {
        ws = d->workspace;
    } else {
        if (hipMallocAsync(&ws, bytes, s) != hipSuccess) {
            (void)hipGetLastError();
            return kda::launch_fwd_pipe(a, cus, s);   // no room: one pass over whole chains
        }
        owned = true;
    }
    float* S1 = static_cast<float*>(ws);   // state after slice 0
    float* R1 = S1 + per;                   // slice 1 from zero
    float* P1 = R1 + per;                   // slice 1's transition map
    float* S2 = P1 + per;                   // state after slice 1
    const int T = d->T;
    const int s1 = (T / 3) / 32 * 32, s2 = (2 * T / 3) / 32 * 32;
    kda::FwdArgs p1 = a;
    p1.ntasks = 3;
    p1.nchains = 3 * a.nchains;
    p1.task[0] = {0, s1, a.h0, S1, 0};
    p1.task[1] = {s1, s2, nullptr, R1, kda::TASK_NO_OUTPUT};
    p1.task[2] = {s1, s2, nullptr, P1, kda::TASK_NO_OUTPUT | kda::TASK_ZERO_V | kda::TASK_IDENTITY_H0};
    hipError_t e = kda::launch_fwd_pipe(p1, cus, s);
    if (e == hipSuccess) e = kda::launch_affine_combine(P1, S1, R1, S2, a.nchains, s);
    if (e == hipSuccess) {
        kda::FwdArgs p2 = a;
        p2.ntasks = 2;
        p2.nchains = 2 * a.nchains;
        p2.task[0] = {s1, s2, S1, nullptr, 0};
        p2.task[1] = {s2, T, S2, a.hT, 0};
        e = kda::launch_fwd_pipe(p2, cus, s);
    }
    if (owned) {
        const hipError_t ef = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = ef;
    }
    return e;
}

// The two-kernel form: operand records in desc->workspace when it is large
// enough, else in a stream-ordered allocation freed on the same stream.
kda_status_t run_two_pass(const kda::FwdArgs& a, const kda_desc_t* d, int cus, hipStream_t s) {
    const size_t bytes = kda::two_pass_workspace(a.nchains, d->T);
    void* ws = nullptr;
    bool owned = false;
    if (d->workspace && d->workspace_bytes >= bytes) {
        ws = d->workspace;
    } else if (bytes > 0) {
        if (hipMallocAsync(&ws, bytes, s) != hipSuccess) {
            (void)hipGetLastError();
            return KDA_ERR_WORKSPACE;
        }
        owned = true;
    }
    hipError_t e = kda::launch_fwd_two_pass(a, ws, cus, s);
    if (owned) {
        const hipError_t ef = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = ef;
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Chooses the kernel for a forward pass (kda_fwd and kda_gdn_fwd).
kda_status_t run_fwd(const kda::FwdArgs& a, const kda_desc_t* desc, const void* o, const float* h0,
                     const float* hT, bool varlen, void* stream) {
    if (a.nchains == 0) return KDA_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool f32 = desc->in_dtype == KDA_F32;
    hipError_t e;
    const int cus = device_cus();
    if (desc->T == 1 && !varlen && aligned16(o) && aligned16(h0) && aligned16(hT))
        e = kda::launch_decode(a, f32, s);   // one token per sequence: a single recurrence step
    else if (use_slices(a.nchains, desc, varlen, cus))
        e = run_slices(a, desc, cus, s);
    else
        e = f32 ? kda::launch_fwd_serial(a, true, s) : kda::launch_fwd_pipe(a, cus, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Layout of the staged path's workspace. Whether the descriptor is varlen is
// not part of kda_desc_t, so the slot count covers both cases: the larger of
// B*ceil(T/32) and ceil(T/32) + N.
kda_status_t layout(const kda_desc_t* d, kda_staged_layout_t* L) {
    const kda_status_t st = check_desc(d, d && d->num_seqs != d->B);
    if (st != KDA_OK) return st;
    const long long C = kda::kStageChunk;
    const long long nchunk = (d->T + C - 1) / C;
    const long long nslots = std::max((long long)d->B * nchunk, nchunk + d->num_seqs);
    if (nslots > INT_MAX / 4) return KDA_ERR_SHAPE;
    const size_t tok = (size_t)d->B * d->T * d->H * 128 * sizeof(float);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    L->nslots = (int32_t)nslots;
    L->chunk = (int32_t)C;
    L->map = take((size_t)nslots * 4 * sizeof(int32_t));
    L->seqinfo = take((size_t)std::max(d->num_seqs, 1) * 2 * sizeof(int32_t));
    L->Gamma = take(tok);
    L->gl = take((size_t)nslots * d->H * 128 * sizeof(float));
    L->W = take(tok);
    L->U = take(tok);
    L->Kt = take(tok);
    L->Qg = take(tok);
    L->M = take((size_t)nslots * d->H * C * C * sizeof(float));
    L->hc = take((size_t)nslots * d->H * 128 * 128 * sizeof(float));
    L->Delta = take(tok);
    L->total = off;
    return KDA_OK;
}

// StageArgs pointing into the caller's workspace.
kda_status_t stage_args(const kda_desc_t* d, const int32_t* cu, kda::StageArgs* a) {
    kda_staged_layout_t L;
    const kda_status_t st = layout(d, &L);
    if (st != KDA_OK) return st;
    if (!d->workspace || d->workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
    char* w = static_cast<char*>(d->workspace);
    *a = kda::StageArgs{};
    a->cu = cu;
    a->map = reinterpret_cast<int32_t*>(w + L.map);
    a->seqinfo = reinterpret_cast<int32_t*>(w + L.seqinfo);
    a->Gamma = reinterpret_cast<float*>(w + L.Gamma);
    a->gl = reinterpret_cast<float*>(w + L.gl);
    a->W = reinterpret_cast<float*>(w + L.W);
    a->U = reinterpret_cast<float*>(w + L.U);
    a->Kt = reinterpret_cast<float*>(w + L.Kt);
    a->Qg = reinterpret_cast<float*>(w + L.Qg);
    a->M = reinterpret_cast<float*>(w + L.M);
    a->hc = reinterpret_cast<float*>(w + L.hc);
    a->Delta = reinterpret_cast<float*>(w + L.Delta);
    a->B = d->B;
    a->T = d->T;
    a->H = d->H;
    a->N = d->num_seqs;
    a->nslots = L.nslots;
    a->f32 = d->in_dtype == KDA_F32;
    return KDA_OK;
}

kda_status_t hip_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }


}  // namespace

namespace kda {

size_t fwd_workspace_bytes(const kda_desc_t* desc, bool smallest) {
    if (!desc) return 0;
    // shape validation only: stand-in pointers, never dereferenced
    static const float dummy = 0.f;
    const float* p = &dummy;
    // without cu_seqlens num_seqs == B; only then can the slice routes run
    const bool maybe_fixed = desc->num_seqs == desc->B;
    const int32_t* cu = maybe_fixed ? nullptr : reinterpret_cast<const int32_t*>(p);
    if (check(p, p, p, p, p, cu, p, desc) != KDA_OK) return 0;
    if (desc->T == 1) return 0;   // the decode route
    const long long nchains = (long long)desc->num_seqs * desc->H;
    if (!maybe_fixed || !use_slices(nchains, desc, false, device_cus())) return 0;
    const int S = multi_slice_count(nchains, desc->T, device_cus());
    const size_t one_pass = multi_slice_workspace_bytes(desc, S), three = slice_workspace_bytes(nchains);
    return smallest ? std::min(one_pass, three) : one_pass;
}

}  // namespace kda

extern "C" {

const char* kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "inconsistent sizes";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration (K and V must be 128; o must be fp32)";
        case KDA_ERR_DTYPE: return "unknown dtype code";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP launch or runtime error";
    }
    return "unknown status";
}

int32_t kda_version(void) { return kVersion; }

kda_status_t kda_fwd_check(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu_seqlens, const float* h0,
                           const void* o, const float* hT, const kda_desc_t* desc) {
    (void)h0;
    (void)hT;
    return check(q, k, v, g, beta, cu_seqlens, o, desc);
}

kda_status_t kda_fwd(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                     float* hT, const kda_desc_t* desc, void* stream) {
    const kda_status_t st = check(q, k, v, g, beta, cu_seqlens, o, desc);
    if (st != KDA_OK) return st;
    const kda::FwdArgs a = fwd_args(q, k, v, g, beta, cu_seqlens, h0, o, hT, desc);
    return run_fwd(a, desc, o, h0, hT, cu_seqlens != nullptr, stream);
}

kda_status_t kda_gdn_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                         float* hT, const kda_desc_t* desc, void* stream) {
    const kda_status_t st = check(q, k, v, g, beta, cu_seqlens, o, desc);
    if (st != KDA_OK) return st;
    kda::FwdArgs a = fwd_args(q, k, v, g, beta, cu_seqlens, h0, o, hT, desc);
    a.scalar_gate = 1;
    return run_fwd(a, desc, o, h0, hT, cu_seqlens != nullptr, stream);
}

kda_status_t kda_fwd_kernel(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                            float* hT, const kda_desc_t* desc, int32_t kernel, void* stream) {
    const kda_status_t st = check(q, k, v, g, beta, cu_seqlens, o, desc);
    if (st != KDA_OK) return st;
    const bool f32 = desc->in_dtype == KDA_F32;
    if (kernel < KDA_KERNEL_AUTO || kernel > KDA_KERNEL_TWO_PASS) return KDA_ERR_UNSUPPORTED;
    if (f32 && kernel != KDA_KERNEL_AUTO && kernel != KDA_KERNEL_SERIAL) return KDA_ERR_UNSUPPORTED;
    if (kernel == KDA_KERNEL_TWO_PASS && cu_seqlens) return KDA_ERR_UNSUPPORTED;
    const kda::FwdArgs a = fwd_args(q, k, v, g, beta, cu_seqlens, h0, o, hT, desc);
    if (kernel == KDA_KERNEL_AUTO) return run_fwd(a, desc, o, h0, hT, cu_seqlens != nullptr, stream);
    if (a.nchains == 0) return KDA_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (kernel == KDA_KERNEL_TWO_PASS) return run_two_pass(a, desc, device_cus(), s);
    hipError_t e;
    if (kernel == KDA_KERNEL_PIPE) e = kda::launch_fwd_pipe(a, device_cus(), s);
    else if (kernel == KDA_KERNEL_SERIAL) e = kda::launch_fwd_serial(a, f32, s);
    else e = kda::launch_fwd_chunk16(a, s);
    return hip_status(e);
}

size_t kda_fwd_kernel_workspace_size(const kda_desc_t* desc, int32_t kernel) {
    if (!desc || kernel != KDA_KERNEL_TWO_PASS) return 0;
    if (check_desc(desc, desc->num_seqs != desc->B) != KDA_OK) return 0;
    return kda::two_pass_workspace(desc->num_seqs * desc->H, desc->T);   // sizes checked above
}

kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* state_in, void* o, float* state_out,
                             const kda_desc_t* desc, void* stream) {
    if (!desc) return KDA_ERR_NULL;
    if (desc->T != 1 || desc->num_seqs != desc->B) return KDA_ERR_SHAPE;
    const kda_status_t st = check(q, k, v, g, beta, nullptr, o, desc);
    if (st != KDA_OK) return st;
    if (!aligned16(o) || !aligned16(state_in) || !aligned16(state_out)) return KDA_ERR_UNSUPPORTED;
    const kda::FwdArgs a = fwd_args(q, k, v, g, beta, nullptr, state_in, o, state_out, desc);
    const hipError_t e = kda::launch_decode(a, desc->in_dtype == KDA_F32, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_staged_layout(const kda_desc_t* desc, kda_staged_layout_t* out) {
    if (!out) return KDA_ERR_NULL;
    return layout(desc, out);
}

size_t kda_staged_workspace_size(const kda_desc_t* desc) {
    kda_staged_layout_t L;
    return layout(desc, &L) == KDA_OK ? L.total : 0;
}

size_t kda_fwd_workspace_size(const kda_desc_t* desc) { return kda::fwd_workspace_bytes(desc, false); }

kda_status_t kda_stage_chunk_map(const int32_t* cu_seqlens, const kda_desc_t* desc, void* stream) {
    if (desc && cu_seqlens == nullptr && desc->num_seqs != desc->B) return KDA_ERR_SHAPE;
    kda::StageArgs a;
    const kda_status_t st = stage_args(desc, cu_seqlens, &a);
    if (st != KDA_OK) return st;
    if (cu_seqlens && desc->B != 1) return KDA_ERR_SHAPE;
    return hip_status(kda::launch_chunk_map(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_stage_gate_scan(const float* g, const kda_desc_t* desc, void* stream) {
    kda::StageArgs a;
    const kda_status_t st = stage_args(desc, nullptr, &a);
    if (st != KDA_OK) return st;
    if (!g && desc->T > 0) return KDA_ERR_NULL;
    a.g = g;
    return hip_status(kda::launch_gate_scan(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_stage_intra(const void* q, const void* k, const void* v, const float* beta,
                             const kda_desc_t* desc, void* stream) {
    kda::StageArgs a;
    const kda_status_t st = stage_args(desc, nullptr, &a);
    if (st != KDA_OK) return st;
    if ((!q || !k || !v || !beta) && desc->T > 0) return KDA_ERR_NULL;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    return hip_status(kda::launch_intra(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_stage_recurrence(const float* h0, float* hT, const kda_desc_t* desc, void* stream) {
    kda::StageArgs a;
    const kda_status_t st = stage_args(desc, nullptr, &a);
    if (st != KDA_OK) return st;
    a.h0 = h0;
    a.hT = hT;
    return hip_status(kda::launch_recurrence(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_stage_output(void* o, const kda_desc_t* desc, void* stream) {
    kda::StageArgs a;
    const kda_status_t st = stage_args(desc, nullptr, &a);
    if (st != KDA_OK) return st;
    if (!o && desc->T > 0) return KDA_ERR_NULL;
    a.o = static_cast<float*>(o);
    return hip_status(kda::launch_output(a, static_cast<hipStream_t>(stream)));
}

kda_status_t kda_fwd_staged(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, const float* h0, void* o,
                            float* hT, const kda_desc_t* desc, void* stream) {
    kda_status_t st = check(q, k, v, g, beta, cu_seqlens, o, desc);
    if (st != KDA_OK) return st;
    kda::StageArgs a;
    st = stage_args(desc, cu_seqlens, &a);
    if (st != KDA_OK) return st;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.h0 = h0;
    a.hT = hT;
    a.o = static_cast<float*>(o);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = kda::launch_chunk_map(a, s);
    if (e == hipSuccess) e = kda::launch_gate_scan(a, s);
    if (e == hipSuccess) e = kda::launch_intra(a, s);
    if (e == hipSuccess) e = kda::launch_recurrence(a, s);
    if (e == hipSuccess) e = kda::launch_output(a, s);
    return hip_status(e);
}

}  // extern "C"
