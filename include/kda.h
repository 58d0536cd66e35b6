/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention chunked prefill.
 *
 * The operation. KDA is a refinement of Gated DeltaNet with fine-grained,
 * channel-wise gating (toolarium.ru page "FlashKDA: Moonshot открыла ядра Kimi
 * Delta Attention для H20", section "Почему это новость про инфраструктуру";
 * donniechu.com page "FlashKDA ... Kimi Delta Attention", section "Số liệu kỹ
 * thuật"). Per sequence and head, with a state S in R^{K x V}:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                       (updated state, no 1/sqrt(K) scale)
 *
 * g is the per-channel log-decay, already computed by the caller (the pages
 * name the gate's parameters A_log, dt_bias and lower_bound but not its
 * formula). The interface follows the pages' description of flash_kda.fwd():
 * batch, variable-length sequences through cu_seqlens, and initial/final
 * recurrent states; head dimension K = V = 128 only; bfloat16 + float32
 * (donniechu.com page, sections "Số liệu kỹ thuật" and "Hạn chế & điều kiện").
 *
 * Layouts. Row-major, innermost dimension last, all buffers contiguous:
 *     q, k, v   [B, T, H, 128]  in_dtype (bf16 or fp32)
 *     g         [B, T, H, 128]  fp32, expected in [-5, 0]
 *     beta      [B, T, H]       fp32
 *     cu_seqlens int32 [N + 1]  device memory, cu[0] = 0, non-decreasing, cu[N] = T
 *     h0, hT    [N, H, 128, 128] fp32, the state as S[k][v]
 *     o         [B, T, H, 128]  fp32
 * With cu_seqlens == NULL there are N = B sequences of T tokens (one per batch
 * row). With cu_seqlens, B must be 1 and sequence n is tokens [cu[n], cu[n+1]).
 * Chunks restart at every sequence start.
 *
 * Ownership and asynchrony. The caller owns every buffer; the library keeps no
 * pointer after a call returns. All device work is enqueued on `stream` (a
 * hipStream_t; NULL is the default stream); no call synchronises the device
 * or copies device memory to the host.
 *
 * Aliasing. h0 == hT (the same pointer) is allowed: each state tile is read
 * before it is overwritten by the workgroup that owns it. Any other overlap
 * between outputs and inputs is undefined.
 *
 * Errors. Argument errors are found on the host before anything is enqueued;
 * the call then returns a negative status and has no side effects. A failed
 * launch returns KDA_ERR_HIP. Contents of cu_seqlens are not checked (they live
 * on the device): invalid offsets are undefined behaviour.
 *
 * Edge cases. T = 0 or zero-length sequences are allowed: such a sequence has
 * no output rows and hT = h0 (or 0 without h0).
 *
 * Threads. Every entry point is thread-safe and keeps no global mutable state.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,         /* a required pointer is NULL                      */
    KDA_ERR_SHAPE = -2,        /* inconsistent sizes (B, T, H, N, cu_seqlens use) */
    KDA_ERR_UNSUPPORTED = -3,  /* valid request outside what is built (K, V != 128) */
    KDA_ERR_DTYPE = -4,        /* unknown or unsupported dtype code                */
    KDA_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required       */
    KDA_ERR_HIP = -6           /* a HIP launch or runtime call failed              */
} kda_status_t;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype_t;

typedef struct kda_desc {
    int32_t B, T, H, K, V;   /* K and V must both be 128                                 */
    int32_t num_seqs;        /* N: equals B without cu_seqlens; count of sequences with it */
    int32_t in_dtype;        /* kda_dtype_t of q, k, v                                    */
    int32_t out_dtype;       /* kda_dtype_t of o; only KDA_F32 is built                   */
    void* workspace;         /* device scratch for the staged path (kda_fwd_staged)       */
    size_t workspace_bytes;  /* its size; kda_fwd itself needs none                       */
} kda_desc_t;

/* Text for a status code (static storage, never NULL). */
const char* kda_status_string(kda_status_t s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t kda_version(void);

/* Validates a descriptor and the pointer set of kda_fwd without launching
 * anything (host only; usable without a GPU). Returns KDA_OK or the error
 * kda_fwd would return. */
kda_status_t kda_fwd_check(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu_seqlens, const float* h0,
                           const void* o, const float* hT, const kda_desc_t* desc);

/* The chunked KDA forward (prefill): o for every token and, when hT != NULL,
 * the final state of every (sequence, head). h0 == NULL starts from zero.
 * Runs as one fused kernel per (sequence, head, V-block) that reads every
 * input once; it needs no workspace. */
kda_status_t kda_fwd(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const int32_t* cu_seqlens, const float* h0,
                     void* o, float* hT, const kda_desc_t* desc, void* stream);

/* Bytes of workspace kda_fwd_staged needs for this descriptor (0 on error). */
size_t kda_fwd_workspace_size(const kda_desc_t* desc);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
