// Optional per-kernel timing with HIP events.  When enabled, every kernel
// launch of the library is bracketed by two events recorded on the launch
// stream; dspark_profile_get sums the elapsed times per kernel kind.
#include <mutex>
#include <vector>

#include "dspark.h"
#include "launch.hpp"

namespace dspark {

namespace {

const char* const kNames[kProfKinds] = {
    "tile_pass_sample", "tile_pass_greedy", "tile_pass_overlap", "tile_pass_bias", "draft_select",
    "verify_init",      "target_stats",     "verify_decide",     "residual_stats", "residual_select",
    "survival_conf",    "survival_tnorm",   "survival_finish",   "schedule",   "confidence",   "rnn_cell",
    "draft_resident",
};

struct Record {
  int kind;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;
size_t g_used = 0;

hipEvent_t take_event() {
  if (g_used == g_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_used++];
}

}  // namespace

thread_local int g_suppress = 0;

ProfSuppress::ProfSuppress() { ++g_suppress; }
ProfSuppress::~ProfSuppress() { --g_suppress; }

ProfScope::ProfScope(hipStream_t s, int kind) : stream_(s), index_(-1) {
  if (g_suppress) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return;
  if (hipEventRecord(a, s) != hipSuccess) return;
  g_records.push_back(Record{kind, a, b});
  index_ = (int)g_records.size() - 1;
}

void ProfScope::discard() {
  if (index_ < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (index_ < (int)g_records.size()) g_records[index_].kind = -1;
}

ProfScope::~ProfScope() {
  if (index_ < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (index_ < (int)g_records.size()) (void)hipEventRecord(g_records[index_].stop, stream_);
}

}  // namespace dspark

using namespace dspark;

extern "C" {

dspark_status dspark_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (const Record& r : g_records) (void)hipEventSynchronize(r.stop);
  g_records.clear();
  g_used = 0;
  g_on = on != 0;
  return DSPARK_OK;
}

int dspark_profile_kinds(void) { return kProfKinds; }

dspark_status dspark_profile_get(int kind, const char** name, long long* launches, double* total_ms) {
  if (kind < 0 || kind >= kProfKinds) return DSPARK_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_mu);
  long long n = 0;
  double ms = 0.0;
  for (const Record& r : g_records) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return DSPARK_ERR_HIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return DSPARK_ERR_HIP;
    ms += t;
    ++n;
  }
  if (name) *name = kNames[kind];
  if (launches) *launches = n;
  if (total_ms) *total_ms = ms;
  return DSPARK_OK;
}

}  // extern "C"
