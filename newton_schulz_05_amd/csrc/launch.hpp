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
  bool bf16;
};

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
  uint32_t epoch;    // distinct per call: tags the published partials
};

hipError_t run_large(const LargeArgs& a, hipStream_t st);
hipError_t run_skinny(const SkinnyArgs& a, hipStream_t st);
int skinny_max_blocks_per_cu();

}  // namespace muon
