// Host-only stand-ins for the kernel launchers of libkda (the .hip files), so
// that kda_api.cpp can be built with g++ and run under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU. Every launcher
// records its arguments and returns hipSuccess; nothing touches device memory.
#include "stub_log.h"

namespace kda {

std::vector<StubCall> g_calls;

static void rec(const char* what, const FwdArgs* a) {
    StubCall c;
    c.what = what;
    if (a) c.args = *a;
    g_calls.push_back(c);
}

hipError_t launch_affine_combine(const float*, const float*, const float*, float*, int, hipStream_t) {
    rec("affine_combine", nullptr);
    return hipSuccess;
}
hipError_t launch_state_correction(const float*, const float*, float*, int, int, int, int, int, int, hipStream_t) {
    rec("state_correction", nullptr);
    return hipSuccess;
}
int serial_workgroups(int nchains) { return nchains * 2; }
hipError_t launch_fwd_serial(const FwdArgs& a, bool, hipStream_t) { rec("serial", &a); return hipSuccess; }
int pipe_state_waves(int nchains, int cus) { return nchains * 8 <= cus ? 1 : nchains * 4 <= cus ? 2 : 4; }
int pipe_workgroups(int nchains, int state_waves) { return (nchains + 7) / 8 * 8 * (128 / (16 * state_waves)); }
hipError_t launch_fwd_pipe(const FwdArgs& a, int, hipStream_t) { rec("pipe", &a); return hipSuccess; }
hipError_t launch_fwd_chunk16(const FwdArgs& a, hipStream_t) { rec("chunk16", &a); return hipSuccess; }
size_t two_pass_workspace(int nchains, int T) { return (size_t)nchains * ((T + 31) / 32) * 53248; }
hipError_t launch_fwd_two_pass(const FwdArgs& a, void*, int, hipStream_t) { rec("two_pass", &a); return hipSuccess; }
hipError_t launch_decode(const FwdArgs& a, bool, hipStream_t) { rec("decode", &a); return hipSuccess; }
hipError_t launch_chunk_map(const StageArgs&, hipStream_t) { rec("stage", nullptr); return hipSuccess; }
hipError_t launch_gate_scan(const StageArgs&, hipStream_t) { rec("stage", nullptr); return hipSuccess; }
hipError_t launch_intra(const StageArgs&, hipStream_t) { rec("stage", nullptr); return hipSuccess; }
hipError_t launch_recurrence(const StageArgs&, hipStream_t) { rec("stage", nullptr); return hipSuccess; }
hipError_t launch_output(const StageArgs&, hipStream_t) { rec("stage", nullptr); return hipSuccess; }

}  // namespace kda
