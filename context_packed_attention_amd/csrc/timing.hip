// Optional per-kernel timing with HIP events on each launch's own stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "internal.h"

namespace cpattn {

namespace {
struct Rec {
  const char* name;
  hipEvent_t a, b;
};
std::atomic<bool> g_on{false};  // read by every launch, so atomic even though recording is single-threaded
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_all() {
  for (auto& r : g_recs) {
    if (r.a) g_free.push_back(r.a);
    if (r.b) g_free.push_back(r.b);
  }
  g_recs.clear();
}
}  // namespace

// launches being captured into a graph are not timed
static bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

void timing_begin(hipStream_t st, const char* name) {
  if (!g_on || capturing(st)) return;
  Rec r{name, take_event(), take_event()};
  if (r.a) (void)hipEventRecord(r.a, st);
  g_recs.push_back(r);
}

void timing_end(hipStream_t st) {
  if (!g_on || g_recs.empty() || capturing(st)) return;
  Rec& r = g_recs.back();
  if (r.b) (void)hipEventRecord(r.b, st);
}

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_attn_status cp_attn_timing_enable(int32_t on) {
  if (on) recycle_all();
  g_on = on != 0;
  return CP_ATTN_OK;
}

extern "C" int32_t cp_attn_timing_read(char* names, int32_t name_len, double* total_ms, int64_t* launches,
                                       int32_t max) {
  std::map<std::string, std::pair<double, int64_t>> agg;
  std::vector<std::string> order;
  for (auto& r : g_recs) {
    if (!r.a || !r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) {
      recycle_all();
      return -1;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      recycle_all();
      return -1;
    }
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {ms, 1};
    } else {
      it->second.first += ms;
      it->second.second += 1;
    }
  }
  int32_t n = 0;
  for (const auto& nm : order) {
    if (n >= max) break;
    if (names && name_len > 0) {
      std::strncpy(names + (size_t)n * name_len, nm.c_str(), name_len - 1);
      names[(size_t)n * name_len + name_len - 1] = 0;
    }
    if (total_ms) total_ms[n] = agg[nm].first;
    if (launches) launches[n] = agg[nm].second;
    ++n;
  }
  recycle_all();
  return n;
}
