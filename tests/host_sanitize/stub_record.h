// What the stand-in launchers of hip_stubs.cpp saw (host-only sanitizer build).
#pragma once

#include "la_gdn_internal.h"

struct StubRecord {
    int pipeline_calls = 0;
    int cu64_calls = 0;
    int sbwd_calls = 0;
    int bwd_calls = 0;
    bool last_summary = false;
    la::Prob last{};
    la::Ws last_ws{};
};

extern StubRecord g_stub;
