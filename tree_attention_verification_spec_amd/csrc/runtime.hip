// Status strings, launch status, tuning overrides and per-kernel event timing for libspectree.
#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.h"

extern "C" const char* spec_strerror(int s) {
  switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EUNSUPPORTED: return "unsupported configuration";
    case SPEC_EWORKSPACE: return "workspace missing or too small";
    case SPEC_EHIP: return "HIP runtime error";
    case SPEC_ESCRATCH: return "request exceeds the fixed scratch array";
  }
  return "unknown status";
}

namespace spectree {
namespace {

struct Record {
  std::string name;
  hipEvent_t start;
  hipEvent_t stop;
};

std::mutex g_mu;
bool g_enabled = false;
std::vector<Record> g_records;

thread_local hipError_t t_launch = hipSuccess;

std::atomic<int> g_knobs[kKnobCount];
bool init_knobs() {
  for (auto& k : g_knobs) k.store(INT_MIN);
  return true;
}
const bool g_knobs_ready = init_knobs();

const char* const kKnobNames[kKnobCount] = {
  "attn_cb", "attn_waves", "attn_splits", "attn_lpt", "attn_prio", "attn_lazy",
  "verify_chunk", "verify_store_w", "verify_rows_list",
  "res_rowblocks", "lm_rowblocks", "walk_parts", "walk_spin",
};

}  // namespace

void note_launch(hipError_t r) {
  if (r != hipSuccess) {
    if (t_launch == hipSuccess) t_launch = r;
    (void)hipGetLastError();     // the error is reported through this call's status
  }
}

spec_status launch_status() {
  const hipError_t r = t_launch;
  t_launch = hipSuccess;
  return r == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int tuning(Knob k, int fallback) {
  const int v = g_knobs[k].load(std::memory_order_relaxed);
  return v == INT_MIN ? fallback : v;
}

bool prof_pair(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_enabled) return false;
  Record r{name, nullptr, nullptr};
  if (hipEventCreate(&r.start) != hipSuccess) return false;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return false;
  }
  g_records.push_back(r);
  *start = r.start;
  *stop = r.stop;
  return true;
}

}  // namespace spectree

extern "C" void spec_prof_enable(int on) {
  std::lock_guard<std::mutex> lock(spectree::g_mu);
  spectree::g_enabled = on != 0;
}

extern "C" void spec_prof_reset(void) {
  std::lock_guard<std::mutex> lock(spectree::g_mu);
  for (auto& r : spectree::g_records) {
    (void)hipEventSynchronize(r.stop);
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  spectree::g_records.clear();
}

extern "C" int spec_prof_read(const char* name, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lock(spectree::g_mu);
  double total = 0.0;
  int64_t n = 0;
  for (auto& r : spectree::g_records) {
    if (r.name != name) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      total += ms;
      ++n;
    }
  }
  if (total_ms) *total_ms = total;
  if (launches) *launches = n;
  return n > 0 ? 0 : -1;
}

extern "C" int spec_internal_tune(const char* name, int value) {
  if (!name) return -1;
  for (int k = 0; k < spectree::kKnobCount; ++k) {
    if (std::strcmp(name, spectree::kKnobNames[k]) == 0) {
      spectree::g_knobs[k].store(value < 0 ? INT_MIN : value);
      return 0;
    }
  }
  return -1;
}
