// Argument validation of the C ABI entry points.  Pure C++ (no HIP calls),
// so the checks build with g++ for the host tests as well.  Each function
// returns MUON_OK, or an error status with `detail` filled, before anything
// is enqueued; none of them touches device memory.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/muon.h"
#include "plan.hpp"

namespace muon {

// Largest number of NS steps accepted by muon_step / muon_ns.
constexpr int32_t kMaxNsSteps = 16;

muon_status check_shapes(const Plan& P, const muon_shape* shapes, int32_t n_params, std::string* detail);
muon_status check_ptrs(const void* const* ptrs, int32_t n, const char* what, std::string* detail);
muon_status check_workspace(const Plan& P, const void* workspace, size_t bytes, std::string* detail);
muon_status check_coeffs(float a, float b, float c, int32_t ns_steps, std::string* detail);

// Everything muon_step checks before it looks at the device.
muon_status validate_step(const Plan* P, void* const* params, const void* const* grads, void* const* moms,
                          const muon_shape* shapes, int32_t n_params, float lr, float mu, int32_t nesterov,
                          float wd, float a, float b, float c, int32_t ns_steps, float scale,
                          const void* workspace, size_t workspace_bytes, std::string* detail);

// Everything muon_ns checks before it looks at the device.
muon_status validate_ns(const Plan* P, const void* const* in, float* const* out, const muon_shape* shapes,
                        int32_t n_params, float a, float b, float c, int32_t ns_steps, const void* workspace,
                        size_t workspace_bytes, std::string* detail);

// muon_shard_update's checks; *nothing_to_do is set when len == 0.
muon_status validate_shard_update(const void* w_shard, muon_dtype dt, const float* o_full, int64_t offset,
                                  int64_t len, float lr, float wd, float scale, bool* nothing_to_do,
                                  std::string* detail);

// muon_adamw_step's checks.
muon_status validate_adamw(void* const* params, const void* const* grads, float* const* exp_avg,
                           float* const* exp_avg_sq, const int64_t* numels, int32_t n, muon_dtype dt, float lr,
                           float b1, float b2, float eps, float wd, int64_t step, std::string* detail);

}  // namespace muon
