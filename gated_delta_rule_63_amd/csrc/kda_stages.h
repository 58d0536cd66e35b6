// kda_stages.h -- host/device interface of the stage kernels (kda_stages.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kStageChunk = 32;   // chunk length of the staged path

// Layouts: q, k, v, g, Gamma, W, U, Kt, Qg, Delta, o are [B, T, H, 128];
// beta [B, T, H]; map int32 [nslots][4] = (sequence, first token, valid tokens,
// batch row); seqinfo int32 [N][2] = (first slot, chunk count); gl [nslots, H, 128];
// M [nslots, H, 32, 32]; hc [nslots, H, 128, 128] (state entering each chunk);
// h0, hT [N, H, 128, 128].
struct StageArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu;
    int32_t* map;
    int32_t* seqinfo;
    float* Gamma;
    float* gl;
    float* W;
    float* U;
    float* Kt;
    float* Qg;
    float* M;
    float* hc;
    float* Delta;
    const float* h0;
    float* hT;
    float* o;
    int B, T, H, N, nslots;
    bool f32;   // q, k, v are fp32 (else bf16)
};

hipError_t launch_chunk_map(const StageArgs& a, hipStream_t s);
hipError_t launch_gate_scan(const StageArgs& a, hipStream_t s);
hipError_t launch_intra(const StageArgs& a, hipStream_t s);
hipError_t launch_recurrence(const StageArgs& a, hipStream_t s);
hipError_t launch_output(const StageArgs& a, hipStream_t s);

}  // namespace kda
