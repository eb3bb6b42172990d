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

// Host validation of a budget (kv_select's rules): KV_OK or a kv_status.
int check_budget(const kv_budget& bu);

// Selection from the top-digit key histogram [B*Hkv][KEY_BINS] that the
// score kernels build (kv_score_select): the budgets select_hist_budget
// accepts (explicit k or kept fraction, no protected tokens), one workgroup
// per head for N_max <= 32768 (select_hist_eligible, select_hist_launch),
// the part path's launches 1-4 above (select_parts_launch with head_hist).
// Same kept indices and counts as select_launch.
bool select_hist_budget(const kv_budget& bud);
bool select_hist_eligible(const kv_budget& bud, int N_max);
void select_hist_launch(const float* scores, const int32_t* ctx, const uint32_t* hist, int B,
                        int Hkv, int N_max, const kv_budget& bud, int32_t* kept_idx,
                        int32_t* kept_count, hipStream_t st);

// The part path of kv_select for heads above 32768 tokens under a count
// budget: its workspace size, and the launch (false if it does not apply).
// head_hist: the score pass's top-digit histogram, for budgets that
// select_hist_budget accepts (launch 0 is then skipped), or null.
size_t select_part_workspace(int B, int Hkv, int N_max);
bool select_parts_launch(const float* scores, const int32_t* ctx, int B, int Hkv, int N_max,
                         const kv_budget& bud, int32_t* kept_idx, int32_t* kept_count,
                         void* workspace, size_t workspace_bytes, hipStream_t st,
                         const uint32_t* head_hist = nullptr);

}  // namespace kvcc
