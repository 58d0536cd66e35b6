// What the stand-in launchers (launch_stubs.cpp) record.
#pragma once
#include <vector>

#include "../../gated_delta_rule_63_amd/csrc/kda_launch.h"
#include "../../gated_delta_rule_63_amd/csrc/kda_stages.h"

namespace kda {
struct StubCall {
    const char* what = "";
    FwdArgs args{};
};
extern std::vector<StubCall> g_calls;
}  // namespace kda
