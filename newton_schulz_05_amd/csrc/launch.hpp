// Host-side launch interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "plan.hpp"

namespace muon {

// One chunk of the multi-launch path (MFMA bf16 or fp32).
struct LargeArgs {
  MatTable tab;
  StepScalars sc;
  LargeLayout L;
  void* ws;          // base of the chunk region in the workspace
  int count;
  int64_t m, n, mp, np;
  int tile;          // bf16 GEMM tile (128 or 256)
  int cus;           // compute units of the device (one 256-tile workgroup each)
  bool bf16;
  bool whole;        // bf16 path: all NS steps in one group
  bool precise;      // bf16 path: split m x m chain with lo planes
  bool x0_lo;        // bf16 muon_step: X_0 carries its lo plane
  // a second stream on the device with events that fork work onto it and
  // join it back, or null (every launch on the launch stream)
  hipStream_t side;
  hipEvent_t ev_fork, ev_join;
};

// u32 indices, in the workspace's sync region, of the skinny path's timeout
// flag and of the launch counter that numbers launches recorded into a graph
constexpr int kSyncErrWord = 2040;
constexpr int kSyncEpochWord = 2044;
// Exchange epochs: launches numbered on the host take [1, 2^26); launches
// numbered by the device counter (graph capture) take 2^26 + (count mod 2^26).
constexpr uint32_t kDeviceEpochBit = 1u << 26;

// One chunk of the persistent skinny path.
struct SkinnyArgs {
  MatTable tab;
  StepScalars sc;
  int count;
  int m;
  int64_t n;
  int slabs;
  int64_t slab_w;
  float* part;       // published slab partials
  uint32_t* sync;    // timeout flag
  unsigned spin_limit;
  uint32_t epoch;    // distinct per launch: tags the published partials
  const uint32_t* epoch_dev;  // if set, the epoch is read from here (graph capture)
  uint32_t* host_flag;        // host-visible word set on a timed-out wait, or null
  uint8_t* lobuf;             // muon_step: lo codes of U, 16 bytes per lane and block
};

hipError_t run_large(const LargeArgs& a, hipStream_t st);

// Optional timing of the MFMA path's apply launches (the dominant kernel of
// large workloads) with HIP events on the launch stream, for benchmarks.
// While enabled, every apply (its main launch and a partial-round launch, if
// any) is bracketed by an event pair, up to kTimerPairs pairs.
constexpr int kTimerPairs = 4096;
void timer_begin(hipStream_t st);
void timer_end(hipStream_t st, double alg_flops, double exec_flops);
// enable (creating the events on first use) or disable; read drains and
// resets the totals: host waits for the recorded events
hipError_t timer_enable(bool on);
hipError_t timer_read(double* ms, int64_t* launches, double* alg_flops, double* exec_flops);
hipError_t run_skinny(const SkinnyArgs& a, hipStream_t st);
int skinny_max_blocks_per_cu();
// one-thread kernel: counter <- counter + 1 (numbers the next skinny launch)
hipError_t run_epoch_bump(uint32_t* counter, hipStream_t st);

// W[i] <- W[i] (1 - lr wd) - lr scale O[i], i < len (one rank's shard of a parameter).
hipError_t run_shard_update(void* w, bool bf16, const float* o, int64_t len, float lr, float wd, float scale,
                            hipStream_t st);

// AdamW over a list of 1-D tensors (pointer table in the kernel arguments).
constexpr int kAdamMaxTensors = 32;       // tensors per launch
constexpr int64_t kAdamChunk = 2048;      // elements per workgroup
struct AdamTable {
  void* p[kAdamMaxTensors];
  const void* g[kAdamMaxTensors];
  float* m[kAdamMaxTensors];
  float* v[kAdamMaxTensors];
  int64_t numel[kAdamMaxTensors];
  int32_t first_block[kAdamMaxTensors + 1];  // prefix sums of ceil(numel / kAdamChunk)
  int32_t n;
};
struct AdamScalars {
  float lr, b1, b2, eps, wd, step_size, bc2_sqrt;  // step_size = lr / (1 - b1^t), bc2_sqrt = sqrt(1 - b2^t)
};
hipError_t run_adamw(const AdamTable& t, const AdamScalars& s, bool bf16, hipStream_t st);

}  // namespace muon
