// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation on
// the host, then kernel launches on the caller's stream.
#include "../../include/kda.h"

#include <limits.h>

#include "kda_launch.h"

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

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
    const long long tok = (long long)d->B * d->T;
    if (tok * d->H * 128 > (long long)1 << 46) return KDA_ERR_SHAPE;
    if ((long long)d->num_seqs * d->H > INT_MAX / 16) return KDA_ERR_SHAPE;
    if (tok > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    return KDA_OK;
}

}  // namespace

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
    a.B = desc->B;
    a.T = desc->T;
    a.H = desc->H;
    a.N = desc->num_seqs;
    a.nchains = desc->num_seqs * desc->H;
    if (a.nchains == 0) return KDA_OK;
    const hipError_t e = desc->in_dtype == KDA_F32
                             ? kda::launch_fwd_serial(a, true, static_cast<hipStream_t>(stream))
                             : kda::launch_fwd_pipe(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_fwd_workspace_size(const kda_desc_t* desc) {
    if (check(reinterpret_cast<const void*>(1), reinterpret_cast<const void*>(1),
              reinterpret_cast<const void*>(1), reinterpret_cast<const float*>(1),
              reinterpret_cast<const float*>(1), nullptr, reinterpret_cast<const void*>(1),
              desc) != KDA_OK &&
        !(desc && desc->B == 1))
        return 0;
    return 0;
}

}  // extern "C"
