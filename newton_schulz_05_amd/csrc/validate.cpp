// Argument validation of the C ABI entry points (see validate.hpp).
#include "validate.hpp"

#include <cmath>

namespace muon {

namespace {

bool finite(float x) { return std::isfinite(x); }

muon_status fail(muon_status s, std::string* detail, const std::string& d) {
  *detail = d;
  return s;
}

}  // namespace

muon_status check_shapes(const Plan& P, const muon_shape* shapes, int32_t n_params, std::string* detail) {
  if (n_params != (int32_t)P.shapes.size())
    return fail(MUON_ERR_PLAN_MISMATCH, detail,
                "n_params " + std::to_string(n_params) + " != plan's " + std::to_string(P.shapes.size()));
  if (!shapes) return fail(MUON_ERR_INVALID_ARG, detail, "shapes is null");
  for (int32_t i = 0; i < n_params; ++i) {
    const muon_shape& a = shapes[i];
    const muon_shape& b = P.shapes[i];
    if (a.batch != b.batch || a.rows != b.rows || a.cols != b.cols)
      return fail(MUON_ERR_PLAN_MISMATCH, detail, "shape of parameter " + std::to_string(i) + " differs from the plan");
  }
  return MUON_OK;
}

muon_status check_ptrs(const void* const* ptrs, int32_t n, const char* what, std::string* detail) {
  if (!ptrs) return fail(MUON_ERR_INVALID_ARG, detail, std::string(what) + " array is null");
  for (int32_t i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(MUON_ERR_INVALID_ARG, detail, std::string(what) + "[" + std::to_string(i) + "] is null");
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 15u) != 0)
      return fail(MUON_ERR_ALIGNMENT, detail,
                  std::string(what) + "[" + std::to_string(i) + "] is not 16-byte aligned");
  }
  return MUON_OK;
}

muon_status check_workspace(const Plan& P, const void* workspace, size_t bytes, std::string* detail) {
  if (!workspace) return fail(MUON_ERR_WORKSPACE, detail, "workspace is null");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MUON_ERR_WORKSPACE, detail, "workspace is not 256-byte aligned");
  if (bytes < P.ws_bytes)
    return fail(MUON_ERR_WORKSPACE, detail,
                "workspace has " + std::to_string(bytes) + " bytes, needs " + std::to_string(P.ws_bytes));
  return MUON_OK;
}

muon_status check_coeffs(float a, float b, float c, int32_t ns_steps, std::string* detail) {
  if (!finite(a) || !finite(b) || !finite(c)) return fail(MUON_ERR_INVALID_ARG, detail, "NS coefficients must be finite");
  if (ns_steps < 0 || ns_steps > kMaxNsSteps)
    return fail(MUON_ERR_INVALID_ARG, detail, "ns_steps must be in 0.." + std::to_string(kMaxNsSteps));
  return MUON_OK;
}

muon_status validate_step(const Plan* P, void* const* params, const void* const* grads, void* const* moms,
                          const muon_shape* shapes, int32_t n_params, float lr, float mu, int32_t nesterov,
                          float wd, float a, float b, float c, int32_t ns_steps, float scale,
                          const void* workspace, size_t workspace_bytes, std::string* detail) {
  if (!P) return fail(MUON_ERR_INVALID_ARG, detail, "null plan");
  muon_status s = check_shapes(*P, shapes, n_params, detail);
  if (s != MUON_OK) return s;
  if ((s = check_ptrs((const void* const*)params, n_params, "param_ptrs", detail)) != MUON_OK) return s;
  if ((s = check_ptrs(grads, n_params, "grad_ptrs", detail)) != MUON_OK) return s;
  if ((s = check_ptrs((const void* const*)moms, n_params, "mom_ptrs", detail)) != MUON_OK) return s;
  if (!finite(lr) || !finite(mu) || !finite(wd) || !finite(scale))
    return fail(MUON_ERR_INVALID_ARG, detail, "lr, mu, wd and scale must be finite");
  if (nesterov != 0 && nesterov != 1) return fail(MUON_ERR_INVALID_ARG, detail, "nesterov must be 0 or 1");
  if ((s = check_coeffs(a, b, c, ns_steps, detail)) != MUON_OK) return s;
  return check_workspace(*P, workspace, workspace_bytes, detail);
}

muon_status validate_ns(const Plan* P, const void* const* in, float* const* out, const muon_shape* shapes,
                        int32_t n_params, float a, float b, float c, int32_t ns_steps, const void* workspace,
                        size_t workspace_bytes, std::string* detail) {
  if (!P) return fail(MUON_ERR_INVALID_ARG, detail, "null plan");
  muon_status s = check_shapes(*P, shapes, n_params, detail);
  if (s != MUON_OK) return s;
  if ((s = check_ptrs(in, n_params, "in_ptrs", detail)) != MUON_OK) return s;
  if ((s = check_ptrs((const void* const*)out, n_params, "out_ptrs", detail)) != MUON_OK) return s;
  if ((s = check_coeffs(a, b, c, ns_steps, detail)) != MUON_OK) return s;
  return check_workspace(*P, workspace, workspace_bytes, detail);
}

muon_status validate_shard_update(const void* w_shard, muon_dtype dt, const float* o_full, int64_t offset,
                                  int64_t len, float lr, float wd, float scale, bool* nothing_to_do,
                                  std::string* detail) {
  *nothing_to_do = false;
  if (dt != MUON_F32 && dt != MUON_BF16) return fail(MUON_ERR_DTYPE, detail, "dt must be MUON_F32 or MUON_BF16");
  if (offset < 0 || len < 0) return fail(MUON_ERR_INVALID_ARG, detail, "offset and len must be >= 0");
  if (!finite(lr) || !finite(wd) || !finite(scale))
    return fail(MUON_ERR_INVALID_ARG, detail, "lr, wd and scale must be finite");
  if (len == 0) {
    *nothing_to_do = true;
    return MUON_OK;
  }
  if (!w_shard || !o_full) return fail(MUON_ERR_INVALID_ARG, detail, "null w_shard or o_full");
  if (len > (int64_t(1) << 40) || offset > (int64_t(1) << 40))
    return fail(MUON_ERR_SHAPE, detail, "offset or len too large");
  const uintptr_t es = (dt == MUON_BF16) ? 2 : 4;
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(w_shard);
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(o_full) + uintptr_t(offset) * 4;
  if (w0 < o0 + uintptr_t(len) * 4 && o0 < w0 + uintptr_t(len) * es)
    return fail(MUON_ERR_INVALID_ARG, detail, "w_shard and o_full overlap");
  return MUON_OK;
}

muon_status validate_adamw(void* const* params, const void* const* grads, float* const* exp_avg,
                           float* const* exp_avg_sq, const int64_t* numels, int32_t n, muon_dtype dt, float lr,
                           float b1, float b2, float eps, float wd, int64_t step, std::string* detail) {
  if (dt != MUON_F32 && dt != MUON_BF16) return fail(MUON_ERR_DTYPE, detail, "dt must be MUON_F32 or MUON_BF16");
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, detail, "n must be >= 0");
  if (n > 0 && (!params || !grads || !exp_avg || !exp_avg_sq || !numels))
    return fail(MUON_ERR_INVALID_ARG, detail, "null pointer array");
  if (!finite(lr) || !finite(b1) || !finite(b2) || !finite(eps) || !finite(wd))
    return fail(MUON_ERR_INVALID_ARG, detail, "lr, b1, b2, eps and wd must be finite");
  if (!(b1 >= 0.f && b1 < 1.f && b2 >= 0.f && b2 < 1.f))
    return fail(MUON_ERR_INVALID_ARG, detail, "b1 and b2 must be in [0, 1)");
  if (!(eps > 0.f)) return fail(MUON_ERR_INVALID_ARG, detail, "eps must be > 0");
  if (step < 1) return fail(MUON_ERR_INVALID_ARG, detail, "step must be >= 1");
  for (int32_t i = 0; i < n; ++i) {
    if (numels[i] < 0) return fail(MUON_ERR_SHAPE, detail, "numels[" + std::to_string(i) + "] < 0");
    if (numels[i] == 0) continue;
    if (numels[i] > (int64_t(1) << 40)) return fail(MUON_ERR_SHAPE, detail, "tensor too large");
    const void* ptrs[4] = {params[i], grads[i], exp_avg[i], exp_avg_sq[i]};
    for (const void* q : ptrs) {
      if (!q) return fail(MUON_ERR_INVALID_ARG, detail, "null tensor pointer at " + std::to_string(i));
      if (reinterpret_cast<uintptr_t>(q) % 4 != 0)
        return fail(MUON_ERR_ALIGNMENT, detail, "tensor " + std::to_string(i) + " not 4-byte aligned");
    }
  }
  return MUON_OK;
}

}  // namespace muon
