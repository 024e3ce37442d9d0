// Error reporting, version and the launch profiler of the kdtopk C ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "kd_internal.h"

static thread_local char g_msg[512] = "";

kd_status kd_fail(kd_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

extern "C" const char* kd_last_error(void) { return g_msg; }

extern "C" const char* kd_version(void) { return "kdtopk 0.1 (gfx950)"; }

namespace {
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRec> g_prof;
}  // namespace

bool kd_prof_active() { return g_prof_on; }

void kd_prof_record(const char* name, hipStream_t stream, bool begin) {
  if (begin) {
    ProfRec r{name, nullptr, nullptr};
    if (hipEventCreate(&r.a) != hipSuccess) return;
    if (hipEventCreate(&r.b) != hipSuccess || hipEventRecord(r.a, stream) != hipSuccess) {
      // an unusable record is dropped: the launch is simply not timed
      (void)hipEventDestroy(r.a);
      if (r.b) (void)hipEventDestroy(r.b);
      return;
    }
    g_prof.push_back(r);
  } else if (!g_prof.empty() && g_prof.back().name == name && g_prof.back().b) {
    ProfRec& r = g_prof.back();
    if (hipEventRecord(r.b, stream) != hipSuccess) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
      g_prof.pop_back();
    }
  }
}

extern "C" kd_status kd_profile_begin(void) {
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  g_prof_on = true;
  return KD_OK;
}

extern "C" int32_t kd_profile_end(int32_t max_kernels, const char** names, float* total_ms, int32_t* launches) {
  g_prof_on = false;
  std::vector<const char*> nm;
  std::vector<double> ms;
  std::vector<int32_t> cnt;
  for (auto& r : g_prof) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) t = 0.f;
    size_t i = 0;
    for (; i < nm.size(); ++i)
      if (strcmp(nm[i], r.name) == 0) break;
    if (i == nm.size()) {
      nm.push_back(r.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += t;
    cnt[i] += 1;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  const int32_t n = (int32_t)nm.size();
  for (int32_t i = 0; i < n && i < max_kernels; ++i) {
    if (names) names[i] = nm[i];
    if (total_ms) total_ms[i] = (float)ms[i];
    if (launches) launches[i] = cnt[i];
  }
  return n;
}
