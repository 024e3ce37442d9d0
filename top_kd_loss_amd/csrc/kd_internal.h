// Host-side helpers shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/kdtopk.h"

// Record a formatted message for kd_last_error() and return `code`.
kd_status kd_fail(kd_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Arrays that the kernels read or write with 16-byte vector accesses (the
// GEMM operands, dh, dW and the workspace) must be 16-byte aligned.
static inline bool kd_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Launch profiler: while kd_profile_begin() is active on this thread, each
// scope records a pair of HIP events around one kernel launch on `stream`.
bool kd_prof_active();
void kd_prof_record(const char* name, hipStream_t stream, bool begin);

struct KdProfScope {
  const char* name;
  hipStream_t stream;
  bool on;
  KdProfScope(const char* n, hipStream_t s) : name(n), stream(s), on(kd_prof_active()) {
    if (on) kd_prof_record(name, stream, true);
  }
  ~KdProfScope() {
    if (on) kd_prof_record(name, stream, false);
  }
};



// Kernel launch on `stream`, bracketed by profiler events when profiling is on.
#define KD_LAUNCH(kern, grid, block, shm, stream, ...)                 \
  do {                                                                 \
    KdProfScope kd_ps_(#kern, stream);                                 \
    hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);   \
  } while (0)
