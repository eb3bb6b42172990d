// Opt-in per-kernel timing: when enabled, every kernel the library launches
// (or only those of one name) carries a start/stop hipEvent pair that its
// dispatch stamps (see launch() in common.hpp).
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace kvcc {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
  int32_t grid, block;   // workgroups and threads per workgroup of the launch
};

std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;
bool g_enabled = false;
std::string g_only;   // record only launches of this name (empty: all)

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool timing_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled || (!g_only.empty() && g_only != name)) return false;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) {
    if (a) g_pool.push_back(a);
    if (b) g_pool.push_back(b);
    return false;
  }
  *start = a;
  *stop = b;
  return true;
}

void timing_done(const char* name, hipEvent_t start, hipEvent_t stop, dim3 grid, dim3 block) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back(Record{name, start, stop, (int32_t)(grid.x * grid.y * grid.z),
                             (int32_t)(block.x * block.y * block.z)});
}

}  // namespace kvcc

using namespace kvcc;

extern "C" int kv_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Record& r : g_records) {
    (void)hipEventSynchronize(r.stop);
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
  g_enabled = on != 0;
  return KV_OK;
}

extern "C" int kv_timing_only(const char* name) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_only = name ? name : "";
  return KV_OK;
}

extern "C" int kv_timing_read(kv_kernel_time* out, int max_entries) {
  if (!out && max_entries > 0) return -KV_ERR_NULL;
  std::vector<kv_kernel_time> acc;
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Record& r : g_records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return -KV_ERR_LAUNCH;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -KV_ERR_LAUNCH;
    size_t i = 0;
    for (; i < acc.size(); ++i)
      if (strncmp(acc[i].name, r.name, sizeof(acc[i].name)) == 0) break;
    if (i == acc.size()) {
      kv_kernel_time t;
      memset(&t, 0, sizeof(t));
      strncpy(t.name, r.name, sizeof(t.name) - 1);
      acc.push_back(t);
    }
    acc[i].launches += 1;
    acc[i].total_ms += ms;
    acc[i].grid = r.grid;     // the last launch's shape
    acc[i].block = r.block;
  }
  const int n = (int)acc.size();
  for (int i = 0; i < n && i < max_entries; ++i) out[i] = acc[i];
  return n;
}
