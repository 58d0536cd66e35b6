// Drives the host side of the C ABI (kda_api.cpp) through its validation and
// routing paths with the kernel launchers stubbed out: argument errors, size
// limits, workspace queries and the slice route's task table. Built with
// -fsanitize=address,undefined by tests/test_sanitize.py; exits non-zero on the
// first failed expectation.
#include <stdio.h>
#include <string.h>

#include <climits>

#include "../../include/kda.h"
#include "stub_log.h"

static int failures = 0;
#define EXPECT(c)                                                          \
    do {                                                                   \
        if (!(c)) {                                                        \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static kda_desc_t desc(int B, int T, int H, int N = -1, int in_dt = KDA_BF16) {
    kda_desc_t d;
    memset(&d, 0, sizeof d);
    d.B = B; d.T = T; d.H = H; d.K = 128; d.V = 128;
    d.num_seqs = N < 0 ? B : N;
    d.in_dtype = in_dt; d.out_dtype = KDA_F32;
    return d;
}

int main() {
    // stand-ins for device pointers: never dereferenced by the host code
    static float buf[64];
    const void* P = buf;
    float* F = buf;
    const int32_t* CU = reinterpret_cast<const int32_t*>(buf);

    for (int s = -8; s <= 1; ++s) EXPECT(kda_status_string((kda_status_t)s) != nullptr);
    EXPECT(kda_version() == 100);

    kda_desc_t d = desc(1, 64, 2);
    EXPECT(kda_fwd_check(P, P, P, F, F, nullptr, nullptr, P, nullptr, &d) == KDA_OK);
    EXPECT(kda_fwd_check(P, P, P, F, F, nullptr, nullptr, P, nullptr, nullptr) == KDA_ERR_NULL);
    EXPECT(kda_fwd_check(nullptr, P, P, F, F, nullptr, nullptr, P, nullptr, &d) == KDA_ERR_NULL);
    d.K = 64;
    EXPECT(kda_fwd_check(P, P, P, F, F, nullptr, nullptr, P, nullptr, &d) == KDA_ERR_UNSUPPORTED);
    d = desc(1, 64, 2); d.in_dtype = 9;
    EXPECT(kda_fwd_check(P, P, P, F, F, nullptr, nullptr, P, nullptr, &d) == KDA_ERR_DTYPE);
    d = desc(2, 64, 2, 3);
    EXPECT(kda_fwd_check(P, P, P, F, F, CU, nullptr, P, nullptr, &d) == KDA_ERR_SHAPE);
    // size limits: products that would overflow 32-bit arithmetic are refused
    d = desc(INT_MAX, INT_MAX, INT_MAX);
    EXPECT(kda_fwd_check(P, P, P, F, F, nullptr, nullptr, P, nullptr, &d) == KDA_ERR_SHAPE);
    d = desc(1, 16, INT_MAX, INT_MAX);
    EXPECT(kda_fwd_check(P, P, P, F, F, CU, nullptr, P, nullptr, &d) == KDA_ERR_SHAPE);
    d = desc(1, -1, 2);
    EXPECT(kda_fwd_check(P, P, P, F, F, nullptr, nullptr, P, nullptr, &d) == KDA_ERR_SHAPE);
    EXPECT(kda_fwd_workspace_size(&d) == 0 && kda_staged_workspace_size(&d) == 0);
    d = desc(INT_MAX, INT_MAX, INT_MAX);
    EXPECT(kda_fwd_workspace_size(&d) == 0 && kda_staged_workspace_size(&d) == 0);
    EXPECT(kda_fwd_kernel_workspace_size(&d, KDA_KERNEL_TWO_PASS) == 0);
    kda_staged_layout_t L;
    EXPECT(kda_staged_layout(&d, &L) == KDA_ERR_SHAPE);
    EXPECT(kda_staged_layout(nullptr, &L) == KDA_ERR_NULL);
    d = desc(1, 64, 2);
    EXPECT(kda_staged_layout(&d, nullptr) == KDA_ERR_NULL);

    // no GPU here: the compute-unit count falls back to 256
    d = desc(1, 8192, 96);
    EXPECT(kda_fwd_workspace_size(&d) == 0);
    d = desc(1, 131072, 32);
    EXPECT(kda_fwd_workspace_size(&d) == ((size_t)18 << 20) + ((size_t)3 << 29));   // one pass, four slices

    // a valid call launches (stubbed) kernels with consistent arguments
    kda::g_calls.clear();
    d = desc(1, 8192, 96);
    EXPECT(kda_fwd(P, P, P, F, F, nullptr, nullptr, F, F, &d, nullptr) == KDA_OK);
    EXPECT(kda::g_calls.size() == 1 && strcmp(kda::g_calls[0].what, "pipe") == 0);
    EXPECT(kda::g_calls[0].args.nchains == 96 && kda::g_calls[0].args.ntasks == 0);

    // the one-pass route with a caller workspace of kda_fwd_workspace_size: four
    // slices of 32768 tokens in one launch (seven tasks: slice 0 for real, then
    // each later slice from zero and from the identity, the identity runs' o
    // into the workspace after nine states per chain), the combines into S2,
    // S3 and hT, one output correction per later slice
    static float ws_stand_in[4];
    kda::g_calls.clear();
    d = desc(1, 131072, 32);
    d.workspace = ws_stand_in;
    d.workspace_bytes = kda_fwd_workspace_size(&d);
    EXPECT(kda_fwd(P, P, P, F, F, nullptr, F, F, F, &d, nullptr) == KDA_OK);
    EXPECT(kda::g_calls.size() == 7);
    if (kda::g_calls.size() == 7) {
        const kda::FwdArgs& p = kda::g_calls[0].args;
        for (int c = 1; c <= 3; ++c) EXPECT(strcmp(kda::g_calls[c].what, "affine_combine") == 0);
        for (int c = 4; c <= 6; ++c) EXPECT(strcmp(kda::g_calls[c].what, "state_correction") == 0);
        EXPECT(p.ntasks == 7 && p.nchains == 7 * 32);
        EXPECT(p.task[0].t_begin == 0 && p.task[0].t_end == 32768 && p.task[0].o == nullptr);
        for (int j = 1; j < 4; ++j) {
            const kda::FwdTask& z = p.task[2 * j - 1];
            const kda::FwdTask& e = p.task[2 * j];
            EXPECT(z.t_begin == 32768 * j && z.t_end == 32768 * (j + 1) && z.o == nullptr && z.flags == 0);
            EXPECT(e.t_begin == 32768 * j && e.t_end == 32768 * (j + 1));
            EXPECT(e.o == ws_stand_in + 9 * 32 * 128 * 128 && e.o_t0 == 32768 && e.o_T == 98304 &&
                   e.flags == (kda::TASK_ZERO_V | kda::TASK_IDENTITY_H0));
        }
    }

    // the three-slice route with a smaller caller workspace (four states per
    // chain): pass 1 (three tasks), combine, pass 2 (two tasks)
    kda::g_calls.clear();
    d.workspace_bytes = (size_t)32 * 4 * 128 * 128 * 4;
    EXPECT(kda_fwd(P, P, P, F, F, nullptr, F, F, F, &d, nullptr) == KDA_OK);
    EXPECT(kda::g_calls.size() == 3);
    if (kda::g_calls.size() == 3) {
        const kda::FwdArgs& p1 = kda::g_calls[0].args;
        const kda::FwdArgs& p2 = kda::g_calls[2].args;
        EXPECT(strcmp(kda::g_calls[1].what, "affine_combine") == 0);
        EXPECT(p1.ntasks == 3 && p1.nchains == 96 && p2.ntasks == 2 && p2.nchains == 64);
        EXPECT(p1.task[0].t_begin == 0 && p1.task[0].t_end == 43680);
        EXPECT(p1.task[1].t_begin == 43680 && p1.task[1].t_end == 87360);
        EXPECT(p2.task[1].t_begin == 87360 && p2.task[1].t_end == 131072);
        EXPECT(p1.task[0].t_end % 32 == 0 && p1.task[1].t_end % 32 == 0);
    }

    // varlen, decode and empty work
    kda::g_calls.clear();
    d = desc(1, 8192, 96, 6);
    EXPECT(kda_fwd(P, P, P, F, F, CU, F, F, F, &d, nullptr) == KDA_OK);
    d = desc(4, 1, 8);
    EXPECT(kda_decode_step(P, P, P, F, F, F, F, F, &d, nullptr) == KDA_OK);
    // T = 0 still launches: every final state is written (h0, or zero)
    d = desc(1, 0, 8);
    EXPECT(kda_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, F, &d, nullptr)
           == KDA_OK);
    d = desc(1, 64, 8, 0);
    EXPECT(kda_fwd(P, P, P, F, F, CU, nullptr, F, nullptr, &d, nullptr) == KDA_OK);   // no sequences: nothing
    EXPECT(kda::g_calls.size() == 3 && strcmp(kda::g_calls[0].what, "pipe") == 0 &&
           strcmp(kda::g_calls[1].what, "decode") == 0 && strcmp(kda::g_calls[2].what, "pipe") == 0);
    if (kda::g_calls.size() == 3) EXPECT(kda::g_calls[2].args.T == 0 && kda::g_calls[2].args.nchains == 8);

    // kernels by name
    d = desc(1, 256, 2, -1, KDA_F32);
    EXPECT(kda_fwd_kernel(P, P, P, F, F, nullptr, nullptr, F, nullptr, &d, KDA_KERNEL_PIPE, nullptr)
           == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_fwd_kernel(P, P, P, F, F, nullptr, nullptr, F, nullptr, &d, 99, nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_fwd_kernel(P, P, P, F, F, nullptr, nullptr, F, nullptr, &d, KDA_KERNEL_SERIAL, nullptr) == KDA_OK);

    // staged path: workspace required and sized by the layout
    d = desc(1, 100, 2, 3);
    EXPECT(kda_staged_layout(&d, &L) == KDA_OK && L.nslots == 4 + 3 && L.total == kda_staged_workspace_size(&d));
    EXPECT(kda_fwd_staged(P, P, P, F, F, CU, nullptr, F, nullptr, &d, nullptr) == KDA_ERR_WORKSPACE);

    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("api driver: all expectations met\n");
    return 0;
}
