// kda_launch.h -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct kda_desc;

namespace kda {

// Device workspace kda_fwd uses for this descriptor: the one-pass slice route's
// (what kda_fwd_workspace_size reports), or with `smallest` the least any
// route takes without allocating (the three-slice route's when that is
// smaller). 0 where no route needs any, and for an invalid descriptor.
size_t fwd_workspace_bytes(const struct kda_desc* desc, bool smallest);

// Arguments of the fused forward kernel. Layouts are those of include/kda.h.
// One slice of every chain of a fixed-length batch: tokens [t_begin, t_end)
// of each row, from its own initial state into its own final state.
enum : int {
    TASK_IDENTITY_H0 = 1,   // start from the identity (the state is then the slice's transition map)
    TASK_ZERO_V = 2,        // v read as zero
    TASK_NO_OUTPUT = 4,     // o not written
};
struct FwdTask {
    int t_begin, t_end;
    const float* h0;        // [N, H, K, V] or nullptr (zero), unless TASK_IDENTITY_H0
    float* hT;              // [N, H, K, V] or nullptr
    int flags;
    // nullptr: o goes to FwdArgs::o. Else to this [N, o_T, H, V] buffer, whose
    // token 0 is token o_t0 of the row (the task writes tokens t - o_t0).
    float* o;
    int o_t0, o_T;
};
constexpr int kMaxTasks = 7;   // slice runs per chain in one launch: 1 + 2 * 3

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;      // [B, T, H, K], or [B, T, H] when scalar_gate
    const float* beta;
    const int32_t* cu;   // device cu_seqlens or nullptr
    const float* h0;     // nullptr: zero initial state
    float* o;
    float* hT;           // nullptr: final state not written
    int B, T, H, N;
    int nchains;         // N * H
    int scalar_gate;     // 1: one gate per (token, head) (Gated DeltaNet)
    // ntasks > 0 (fixed-length batches only): chain c runs task c / (N * H) on
    // (sequence, head) c % (N * H); nchains = ntasks * N * H, and h0/hT above
    // are unused.
    int ntasks;
    FwdTask task[kMaxTasks];
};

// S_out = Pmap S_in + R per (sequence, head): the state at the end of a slice
// from its transition map Pmap (K x K) and its zero-start end state R (K x V).
hipError_t launch_affine_combine(const float* Pmap, const float* S_in, const float* R, float* S_out,
                                 int nchains, hipStream_t stream);

// o[n, t, h, :] += S[n H + h]^T ell[n, t - e0, h, :] for t in [t0, t1), every
// row n < B and head h: the part of a slice's output due to its start state S,
// from ell, the output of the same slice run from the identity with v = 0.
// o is [B, T, H, V], ell [B, T - e0, H, K] (tokens e0 .. T - 1, e0 <= t0), S
// [B H, K, V], all fp32.
hipError_t launch_state_correction(const float* S, const float* ell, float* o, int B, int T, int H, int t0,
                                   int t1, int e0, hipStream_t stream);

// One phase at a time (both input dtypes); used for fp32 inputs.
int serial_workgroups(int nchains);
hipError_t launch_fwd_serial(const FwdArgs& a, bool f32_inputs, hipStream_t stream);
// Helper waves prepare chunk i+1 while state waves advance chunk i (bf16 inputs).
// The chain is split over 128 / (16 * state_waves) workgroups; state_waves is
// 4, 2 or 1, the largest that still fills `cus` compute units, or 8 (one
// workgroup per chain) when two workgroups per chain would not fit on them.
int pipe_state_waves(int nchains, int cus);
int pipe_workgroups(int nchains, int state_waves);
hipError_t launch_fwd_pipe(const FwdArgs& a, int cus, hipStream_t stream);
// The one-phase-at-a-time kernel with 16-token chunks (bf16 inputs): the
// chunk-length ablation.
hipError_t launch_fwd_chunk16(const FwdArgs& a, hipStream_t stream);
// The pipelined kernel's work as two kernels (fixed-length bf16 batches): a
// chunk-parallel preparation that writes every chunk's operands to
// `workspace` (two_pass_workspace bytes), then the recurrence that reads them.
size_t two_pass_workspace(int nchains, int T);
hipError_t launch_fwd_two_pass(const FwdArgs& a, void* workspace, int cus, hipStream_t stream);
// One recurrence step per (sequence, head) (T = 1, no cu): the decode step.
// o, h0 and hT must be 16-byte aligned.
hipError_t launch_decode(const FwdArgs& a, bool f32_inputs, hipStream_t stream);

}  // namespace kda
