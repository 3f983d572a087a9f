// Event timing of the apply launches (see launch.hpp).  Off by default;
// enabled only by muon_kernel_timing for benchmarks.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace muon {

namespace {

struct TimerState {
  std::mutex mu;
  bool on = false;
  bool created = false;
  hipEvent_t ev[2 * kTimerPairs];
  double alg[kTimerPairs], exec[kTimerPairs];
  int n = 0;          // pairs recorded since the last read
  bool open = false;  // a begin without its end yet
};
TimerState g_t;

}  // namespace

void timer_begin(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_t.mu);
  if (!g_t.on || g_t.n >= kTimerPairs) return;
  if (hipEventRecord(g_t.ev[2 * g_t.n], st) == hipSuccess) g_t.open = true;
}

void timer_end(hipStream_t st, double alg_flops, double exec_flops) {
  std::lock_guard<std::mutex> lk(g_t.mu);
  if (!g_t.on || !g_t.open) return;
  g_t.open = false;
  if (hipEventRecord(g_t.ev[2 * g_t.n + 1], st) != hipSuccess) return;
  g_t.alg[g_t.n] = alg_flops;
  g_t.exec[g_t.n] = exec_flops;
  ++g_t.n;
}

hipError_t timer_enable(bool on) {
  std::lock_guard<std::mutex> lk(g_t.mu);
  if (on && !g_t.created) {
    for (int i = 0; i < 2 * kTimerPairs; ++i)
      if (hipError_t e = hipEventCreate(&g_t.ev[i]); e != hipSuccess) return e;
    g_t.created = true;
  }
  g_t.on = on;
  g_t.open = false;
  return hipSuccess;
}

hipError_t timer_read(double* ms, int64_t* launches, double* alg_flops, double* exec_flops) {
  std::lock_guard<std::mutex> lk(g_t.mu);
  double t = 0.0, a = 0.0, x = 0.0;
  for (int i = 0; i < g_t.n; ++i) {
    if (hipError_t e = hipEventSynchronize(g_t.ev[2 * i + 1]); e != hipSuccess) return e;
    float f = 0.f;
    if (hipError_t e = hipEventElapsedTime(&f, g_t.ev[2 * i], g_t.ev[2 * i + 1]); e != hipSuccess) return e;
    t += f;
    a += g_t.alg[i];
    x += g_t.exec[i];
  }
  *ms = t;
  *launches = g_t.n;
  *alg_flops = a;
  *exec_flops = x;
  g_t.n = 0;
  return hipSuccess;
}

}  // namespace muon
