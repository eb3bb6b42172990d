// Launchers shared between the library's sources (no validation: callers
// check their arguments first).
#pragma once

#include "common.hpp"

namespace kvcc {

// Per-head selection as kv_select, with optional per-head lengths n_head
// (overriding ctx) and, when k_zero_ok, BUDGET_K heads whose k is <= 0
// keeping nothing.
void select_launch(const float* scores, const int32_t* ctx, const int32_t* n_head, int B,
                   int Hkv, int N_max, const kv_budget& bud, bool k_zero_ok,
                   int32_t* kept_idx, int32_t* kept_count, hipStream_t st,
                   const char* timer_name);

}  // namespace kvcc
