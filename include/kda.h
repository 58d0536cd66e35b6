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
 * Graph capture. Every call may be recorded into a HIP graph on `stream`: the
 * library launches kernels only (no memset, no host synchronisation). The one
 * allocation, kda_fwd's slice workspace for few long chains, is skipped when
 * desc->workspace is large enough; kda_fwd_kernel with KDA_KERNEL_TWO_PASS
 * likewise.
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
 * Operand domain. The bf16 kernels round the state S and the gated operands
 * K*exp(Gamma), Q*exp(Gamma) and K*exp(Gamma_last - Gamma) (Gamma the in-chunk
 * cumulative gate, so these factors are at most 1 in magnitude) to fp16 for
 * their matrix products, keep every product's accumulation and the state
 * itself in fp32, and split the gated key and query factors of the intra-chunk
 * blocks into two bf16 terms (fp32 range). The results meet the tolerance of
 * the tests (2e-2 of RMS(o), 1e-2 of RMS(hT)) when
 *   - every state entry, h0 included, stays below 65504 in magnitude at every
 *     32-token chunk boundary, and the entries of q and k are below 65504;
 *   - g lies in [-5, 0] (the factors of a 32-token chunk then stay within
 *     e^-80 .. e^75); a gate below about -5.4 sustained over 16 tokens
 *     overflows them to inf/NaN, and g > 0 is a growing state;
 *   - beta lies in [0, 1] and the keys are L2-normalised per token and head.
 * The last condition keeps the state bounded: each step (I - beta k k^T)
 * Diag(exp g) is then a contraction, so an entry of S grows by at most
 * beta |v| per token and forgets at the gate's rate. The fp32 path (fp32
 * q, k, v) uses two-term fp16 operands and has the same domain.
 *
 * Threads. Every entry point is thread-safe; the only global state is a cache
 * of each device's compute-unit count, written atomically.
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
    void* workspace;         /* optional device scratch; kda_fwd_workspace_size() says how much   */
    size_t workspace_bytes;  /* kda_fwd needs (often 0), kda_staged_workspace_size() the staged path */
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
 * input once. With T == 1 and no cu_seqlens (one token per batch row) and
 * 16-byte aligned o, h0, hT, it runs the decode kernel of kda_decode_step
 * instead.
 * Few long chains (bf16, no cu_seqlens, T >= 12288, at most one chain per six
 * compute units) are cut into slices of whole 32-token chunks. A slice's end
 * state and its outputs are affine in the state it starts from (S_end =
 * Pmap S_start + R; o = o from zero + S_start^T ell, with ell the slice's
 * output from the identity with v = 0), so later slices are run from zero and
 * from the identity alongside the first. Two routes:
 *  - one pass: with desc->workspace of at least kda_fwd_workspace_size(desc)
 *    bytes, 16-byte aligned. S slices, S the largest number (at most 4, each
 *    at least 4096 tokens) for which the 2S - 1 runs of every (sequence, head)
 *    fit on the device's compute units at one workgroup each; slice j starts
 *    at token j T / S rounded down to a multiple of 32. One launch runs them
 *    all (its end states and ell into the workspace), then S_{j+1} =
 *    Pmap_j S_j + R_j in turn (the last is hT) and each later slice's o is
 *    corrected by S_j^T ell. Workspace: three fp32 states per (sequence, head)
 *    and later slice, and ell, fp32 [B, T - T1, H, 128] with T1 the first
 *    token of slice 1;
 *  - three slices: with a smaller workspace of at least 256 KiB per
 *    (sequence, head), or none (then a stream-ordered allocation of that size
 *    on `stream`, freed on the same stream; if that allocation fails, the
 *    chains run whole): two passes of a third of the length each.
 * Every other case needs no workspace. */
kda_status_t kda_fwd(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const int32_t* cu_seqlens, const float* h0,
                     void* o, float* hT, const kda_desc_t* desc, void* stream);

/* Bytes of device workspace kda_fwd (and kda_gdn_fwd) takes for this
 * descriptor on the current device with its one-pass slice route for few long
 * chains (bf16, T >= 12288, at most one chain per six compute units of the
 * current device, no cu_seqlens): 196,608 per (sequence, head) and later
 * slice plus 512 * B * (T - T1) * H, with the slice count and T1 as described
 * at kda_fwd (T = 131072, H = 32 on 256 compute units: four slices, 18 MiB +
 * 1.5 GiB); else 0. A workspace of 262,144 per (sequence, head) up to this
 * size runs the three-slice route without allocating.
 * The descriptor does not say whether cu_seqlens will be passed; with B ==
 * num_seqs == 1 the fixed-length answer is returned, which is never smaller
 * than what a varlen call needs. 0 also for an invalid descriptor. Host only;
 * reads the device's compute-unit count once. */
size_t kda_fwd_workspace_size(const kda_desc_t* desc);

/* ---------------------------------------------------------------------------
 * kda_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Arguments,
 * layouts, results and errors as kda_fwd; desc->workspace is ignored. The
 * slice routes' workspace comes from a static device array of
 * kda_fwd_noalloc_max_workspace() bytes (8 MiB) that each GPU holds from the
 * first call on it until the process ends: the one-pass slice route when
 * kda_fwd_workspace_size(desc) fits there, else the three-slice route (256 KiB
 * per sequence-head: up to 32). A descriptor whose three-slice workspace does
 * not fit either returns KDA_ERR_WORKSPACE before anything is enqueued. No
 * hipMalloc, hipFree or other allocating call is made.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams or host threads, or with the array still in use by an
 * earlier call's kernels on another stream) race and give undefined results.
 * Calls ordered on one stream are safe. */
kda_status_t kda_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, const float* h0,
                             void* o, float* hT, const kda_desc_t* desc, void* stream);

/* Size in bytes of kda_fwd_noalloc's static workspace. */
size_t kda_fwd_noalloc_max_workspace(void);

/* ---------------------------------------------------------------------------
 * Gated DeltaNet forward: the same recurrence with one scalar gate per
 * (token, head) instead of one per channel. KDA is presented as Gated DeltaNet
 * refined with channel-wise gating, and the pages benchmark FlashKDA against a
 * "gdn" kernel (toolarium.ru page, section "Почему это новость про
 * инфраструктуру" and its H20 benchmark table).
 *
 *     S_t = (I - beta_t k_t k_t^T) exp(g_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t
 *
 * Arguments, layouts, aliasing, routing and errors exactly as kda_fwd, except
 *     g  [B, T, H] fp32, one natural-log decay per (token, head), in [-5, 0].
 * The result equals kda_fwd with g repeated over the 128 channels, bit for
 * bit; the gate costs 4 bytes per token-head instead of 512. */
kda_status_t kda_gdn_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const int32_t* cu_seqlens, const float* h0,
                         void* o, float* hT, const kda_desc_t* desc, void* stream);

/* ---------------------------------------------------------------------------
 * One forward kernel by name, for comparisons and ablations. Arguments,
 * layouts, aliasing and errors as kda_fwd; `kernel` is a kda_kernel_t.
 *   KDA_KERNEL_AUTO     what kda_fwd runs (including its decode and slice routes).
 *   KDA_KERNEL_PIPE     32-token chunks; helper waves form chunk i+1's operands
 *                       while state waves advance chunk i (bf16 inputs only).
 *   KDA_KERNEL_SERIAL   32-token chunks; the four steps of a chunk (gate scan,
 *                       A/M blocks and inverse, state products, output) one after
 *                       another in four waves. kda_fwd uses it for fp32 inputs.
 *   KDA_KERNEL_CHUNK16  as SERIAL with 16-token chunks: one 16 x 16 block per
 *                       chunk, the chunk length FlashKDA's v1 chose for its bf16
 *                       range and cheap inverse (toolarium.ru page, section "Где
 *                       ограничения прямо сейчас"); bf16 inputs only.
 *   KDA_KERNEL_TWO_PASS PIPE's work as two kernels, the split the same section
 *                       credits to FlashKDA: a chunk-parallel preparation writes
 *                       every chunk's operands to device memory, then the
 *                       recurrence reads them back. Same values as PIPE, bit for
 *                       bit. bf16 inputs, no cu_seqlens. Needs
 *                       kda_fwd_kernel_workspace_size() bytes of device memory:
 *                       desc->workspace when at least that large, else a
 *                       stream-ordered allocation on `stream`, freed on it
 *                       (KDA_ERR_WORKSPACE if that fails).
 * All give the same result within rounding (no kernel changes the method).
 * An unknown value, a bf16-only kernel with fp32 inputs, or TWO_PASS with
 * cu_seqlens is KDA_ERR_UNSUPPORTED. Only TWO_PASS uses a workspace. */
typedef enum {
    KDA_KERNEL_AUTO = 0,
    KDA_KERNEL_PIPE = 1,
    KDA_KERNEL_SERIAL = 2,
    KDA_KERNEL_CHUNK16 = 3,
    KDA_KERNEL_TWO_PASS = 4
} kda_kernel_t;

/* Bytes of device workspace kda_fwd_kernel needs for `kernel` (0 when it
 * needs none or the descriptor is invalid). TWO_PASS: one 53,248-byte record
 * per (sequence, head, 32-token chunk). */
size_t kda_fwd_kernel_workspace_size(const kda_desc_t* desc, int32_t kernel);

kda_status_t kda_fwd_kernel(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, const float* h0,
                            void* o, float* hT, const kda_desc_t* desc, int32_t kernel,
                            void* stream);

/* ---------------------------------------------------------------------------
 * Decode step: one new token for each of N sequences, i.e. one step of the
 * recurrence above per (sequence, head), applied to a state carried over from
 * a prefill (the pages list decode as the next, not yet tuned, part of the
 * interface: toolarium.ru page, section "Где ограничения прямо сейчас";
 * donniechu.com page, section "Hạn chế & điều kiện").
 *
 *     S' = (I - beta k k^T) Diag(exp(g)) S + beta k v^T,    o = S'^T q
 *
 * desc: B = num_seqs = N, T = 1, H, K = V = 128, in_dtype bf16 or fp32,
 * out_dtype fp32; desc->workspace is ignored.
 *     q, k, v   [N, 1, H, 128]   in_dtype
 *     g         [N, 1, H, 128]   fp32
 *     beta      [N, 1, H]        fp32
 *     state_in  [N, H, 128, 128] fp32 (NULL: zero state)
 *     o         [N, 1, H, 128]   fp32
 *     state_out [N, H, 128, 128] fp32 (NULL: not written)
 * state_in == state_out (the same pointer) updates the state in place. o,
 * state_in and state_out must be 16-byte aligned (KDA_ERR_UNSUPPORTED
 * otherwise). Errors as for kda_fwd; T != 1 or num_seqs != B is
 * KDA_ERR_SHAPE. One workgroup per (sequence, head); the state is read and
 * written once (HBM-bound). */
kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* state_in, void* o, float* state_out,
                             const kda_desc_t* desc, void* stream);

/* ---------------------------------------------------------------------------
 * Staged path. The same chunked forward as four kernels (plus a chunk map)
 * that keep every intermediate in a caller-owned device workspace
 * (desc->workspace, desc->workspace_bytes), all in fp32 with 32-token chunks.
 * It is slower than kda_fwd (it writes and re-reads the intermediates) and
 * exists so that each step can be run, checked and timed on its own. The
 * pages describe the method's forward as a chunked two-kernel design
 * (toolarium.ru page, section "Где ограничения прямо сейчас").
 *
 * Workspace contents, at the byte offsets kda_staged_layout reports:
 *   map      int32 [nslots][4]  (sequence, first token, valid tokens, batch row);
 *                               unused slots have sequence -1 and 0 tokens
 *   seqinfo  int32 [N][2]       (first slot, chunk count) per sequence
 *   Gamma    fp32 [B,T,H,128]   in-chunk cumulative sum of g (a1)
 *   gl       fp32 [nslots,H,128] exp(Gamma at the chunk's last token) (a1)
 *   W, U, Kt, Qg  fp32 [B,T,H,128]  (a2): W = (I+A)^{-1} Diag(beta)(K*exp Gamma),
 *                               U = (I+A)^{-1} Diag(beta) V, Kt = K*exp(Gamma_last-Gamma),
 *                               Qg = Q*exp(Gamma)
 *   M        fp32 [nslots,H,32,32]  lower-triangular gated Q K^T (a2)
 *   hc       fp32 [nslots,H,128,128] state entering each chunk (a3)
 *   Delta    fp32 [B,T,H,128]   U - W h_c (a3)
 * A workspace is used by one call sequence at a time.
 * ------------------------------------------------------------------------- */
typedef struct kda_staged_layout {
    int32_t nslots;   /* chunk slots: B*ceil(T/32), or ceil(T/32) + N with cu_seqlens */
    int32_t chunk;    /* 32 */
    size_t map, seqinfo, Gamma, gl, W, U, Kt, Qg, M, hc, Delta;   /* byte offsets */
    size_t total;     /* bytes */
} kda_staged_layout_t;

/* Fills *out for this descriptor (host only). */
kda_status_t kda_staged_layout(const kda_desc_t* desc, kda_staged_layout_t* out);

/* Bytes of workspace the staged path needs for this descriptor (0 on error):
 * kda_staged_layout()'s total. */
size_t kda_staged_workspace_size(const kda_desc_t* desc);

/* a0: chunk map from cu_seqlens (NULL: B rows of T tokens), built on the device. */
kda_status_t kda_stage_chunk_map(const int32_t* cu_seqlens, const kda_desc_t* desc, void* stream);
/* a1: per-chunk cumulative log-gate scan (needs a0). */
kda_status_t kda_stage_gate_scan(const float* g, const kda_desc_t* desc, void* stream);
/* a2: intra-chunk step: gated K K^T, its unit-lower-triangular inverse, W, U, Kt, Qg, M (needs a1). */
kda_status_t kda_stage_intra(const void* q, const void* k, const void* v, const float* beta,
                             const kda_desc_t* desc, void* stream);
/* a3: inter-chunk recurrence per (sequence, head, 16-column V-block): h_c, Delta, hT (needs a2). */
kda_status_t kda_stage_recurrence(const float* h0, float* hT, const kda_desc_t* desc, void* stream);
/* a4: output O = Qg h_c + M Delta (needs a3). */
kda_status_t kda_stage_output(void* o, const kda_desc_t* desc, void* stream);

/* a0..a4 in order: the same contract as kda_fwd, plus the workspace. */
kda_status_t kda_fwd_staged(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const int32_t* cu_seqlens, const float* h0,
                            void* o, float* hT, const kda_desc_t* desc, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
