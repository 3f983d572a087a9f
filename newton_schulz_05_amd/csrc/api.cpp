// C ABI entry points (include/muon.h): validation, per-chunk descriptor
// tables, and the launch sequence on the caller's stream.  No device memory is
// allocated or freed here and the host never waits for the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "launch.hpp"
#include "plan.hpp"

struct muon_plan_s {
  muon::Plan p;
};

namespace {

thread_local std::string g_detail;

muon_status fail(muon_status s, const std::string& d) {
  g_detail = d;
  return s;
}

constexpr unsigned kSpinLimit = 1u << 20;  // bounded barrier wait (polls, about a second)
std::atomic<unsigned> g_spin_limit{kSpinLimit};

// Distinct number per skinny launch (modulo 2^26): tags the kernel's published
// partials, so words left by an earlier launch in the same workspace are never
// mistaken for new ones.  Launches recorded into a graph are numbered on the
// device instead (kDeviceEpochBit range), since a replay repeats the kernel
// arguments.
std::atomic<uint32_t> g_epoch{1};

uint32_t next_epoch() {
  uint32_t e = g_epoch.fetch_add(1) & (muon::kDeviceEpochBit - 1);
  if (e == 0) e = g_epoch.fetch_add(1) & (muon::kDeviceEpochBit - 1);  // tag 0 marks unwritten words
  return e;
}

bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

// Compute-unit count of the current device, per device id.
std::mutex g_cu_mu;
std::vector<int> g_cus;  // -1 = not queried

muon_status device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if (int(g_cus.size()) <= dev) g_cus.resize(dev + 1, -1);
  if (g_cus[dev] < 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(MUON_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
    g_cus[dev] = n;
  }
  *cus = g_cus[dev];
  return MUON_OK;
}

// Co-resident workgroup capacity of the skinny kernel on the current device.
muon_status skinny_capacity(int* cap) {
  int cus = 0;
  if (muon_status s = device_cus(&cus); s != MUON_OK) return s;
  *cap = cus * muon::skinny_max_blocks_per_cu();
  return MUON_OK;
}

bool finite(float x) { return std::isfinite(x); }

muon_status check_shapes(const muon::Plan& P, const muon_shape* shapes, int32_t n_params) {
  if (n_params != (int32_t)P.shapes.size())
    return fail(MUON_ERR_PLAN_MISMATCH, "n_params " + std::to_string(n_params) + " != plan's " +
                                            std::to_string(P.shapes.size()));
  if (!shapes) return fail(MUON_ERR_INVALID_ARG, "shapes is null");
  for (int32_t i = 0; i < n_params; ++i) {
    const muon_shape& a = shapes[i];
    const muon_shape& b = P.shapes[i];
    if (a.batch != b.batch || a.rows != b.rows || a.cols != b.cols)
      return fail(MUON_ERR_PLAN_MISMATCH, "shape of parameter " + std::to_string(i) + " differs from the plan");
  }
  return MUON_OK;
}

muon_status check_ptrs(const void* const* ptrs, int32_t n, const char* what) {
  if (!ptrs) return fail(MUON_ERR_INVALID_ARG, std::string(what) + " array is null");
  for (int32_t i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(MUON_ERR_INVALID_ARG, std::string(what) + "[" + std::to_string(i) + "] is null");
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & 15u) != 0)
      return fail(MUON_ERR_ALIGNMENT, std::string(what) + "[" + std::to_string(i) + "] is not 16-byte aligned");
  }
  return MUON_OK;
}

size_t elem_size(muon_dtype d) { return d == MUON_BF16 ? 2 : 4; }

// Enqueue every chunk of every group.  `w`, `g`, `m` are per-parameter device
// pointers (m may be null for muon_ns).
muon_status run_all(const muon::Plan& P, void* const* w, const void* const* g, void* const* m,
                    const muon::StepScalars& sc, void* workspace, hipStream_t st) {
  using namespace muon;
  uint8_t* ws = (uint8_t*)workspace;
  const size_t pes = elem_size(P.param_dt);
  for (const Group& grp : P.groups) {
    if (grp.path == PATH_SKINNY) {
      int cap = 0;
      muon_status s = skinny_capacity(&cap);
      if (s != MUON_OK) return s;
      if (int64_t(grp.max_chunk) * grp.slabs > cap)
        return fail(MUON_ERR_HIP, "device holds only " + std::to_string(cap) +
                                      " co-resident workgroups of the skinny kernel; a chunk needs " +
                                      std::to_string(int64_t(grp.max_chunk) * grp.slabs));
    }
    for (const Chunk& ch : grp.chunks) {
      MatTable tab;
      std::memset(&tab, 0, sizeof(tab));
      for (int32_t q = 0; q < ch.count; ++q) {
        const MatEntry& me = P.mats[grp.mats[ch.first + q]];
        const size_t off = size_t(me.e) * size_t(me.rows) * size_t(me.cols);
        const size_t wes = (sc.mode == 1) ? 4 : pes;  // muon_ns writes fp32 O
        tab.e[q].w = (uint8_t*)w[me.param] + off * wes;
        tab.e[q].g = (const uint8_t*)g[me.param] + off * pes;
        tab.e[q].m = m ? (float*)m[me.param] + off : nullptr;
        tab.tr[q] = me.tr ? 1 : 0;
      }
      hipError_t e = hipSuccess;
      if (grp.path == PATH_SKINNY) {
        SkinnyArgs a;
        a.tab = tab;
        a.sc = sc;
        a.count = ch.count;
        a.m = int(grp.m);
        a.n = grp.n;
        a.slabs = grp.slabs;
        a.slab_w = grp.slab_w;
        a.part = (float*)(ws + P.ws_dyn_off);
        a.sync = (uint32_t*)(ws + P.ws_sync_off);
        a.spin_limit = g_spin_limit.load();
        a.epoch = 0;
        a.epoch_dev = nullptr;
        if (capturing(st)) {
          uint32_t* counter = a.sync + muon::kSyncEpochWord;
          e = muon::run_epoch_bump(counter, st);
          a.epoch_dev = counter;
        } else {
          a.epoch = next_epoch();
        }
        if (e == hipSuccess) e = run_skinny(a, st);
      } else {
        LargeArgs a;
        a.tab = tab;
        a.sc = sc;
        a.L = large_layout(grp, ch.count, P.param_dt);
        a.ws = ws + P.ws_dyn_off;
        a.count = ch.count;
        a.m = grp.m;
        a.n = grp.n;
        a.mp = grp.mp;
        a.np = grp.np;
        a.tile = grp.tile;
        a.bf16 = (grp.path == PATH_MFMA);
        a.grouped = grp.grouped;
        if (muon_status s = device_cus(&a.cus); s != MUON_OK) return s;
        e = run_large(a, st);
      }
      if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    }
  }
  return MUON_OK;
}

muon_status check_workspace(const muon::Plan& P, void* workspace, size_t bytes) {
  if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is null");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MUON_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (bytes < P.ws_bytes)
    return fail(MUON_ERR_WORKSPACE, "workspace has " + std::to_string(bytes) + " bytes, needs " +
                                        std::to_string(P.ws_bytes));
  return MUON_OK;
}

muon_status check_coeffs(float a, float b, float c, int32_t ns_steps) {
  if (!finite(a) || !finite(b) || !finite(c)) return fail(MUON_ERR_INVALID_ARG, "NS coefficients must be finite");
  if (ns_steps < 0 || ns_steps > 16) return fail(MUON_ERR_INVALID_ARG, "ns_steps must be in 0..16");
  return MUON_OK;
}

}  // namespace

extern "C" {

muon_status muon_plan_create(const muon_shape* shapes, int32_t n_params, muon_dtype param_dt,
                             muon_dtype grad_dt, muon_dtype mom_dt, muon_plan* out) {
  if (!out) return fail(MUON_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  muon::Plan P;
  std::string d;
  muon_status s = muon::build_plan(shapes, n_params, param_dt, grad_dt, mom_dt, &P, &d);
  if (s != MUON_OK) return fail(s, d);
  muon_plan h = new (std::nothrow) muon_plan_s;
  if (!h) return fail(MUON_ERR_INVALID_ARG, "out of host memory");
  h->p = std::move(P);
  *out = h;
  return MUON_OK;
}

void muon_plan_destroy(muon_plan plan) { delete plan; }

muon_status muon_plan_workspace_bytes(muon_plan plan, size_t* bytes) {
  if (!plan || !bytes) return fail(MUON_ERR_INVALID_ARG, "null argument");
  *bytes = plan->p.ws_bytes;
  return MUON_OK;
}

muon_status muon_plan_num_groups(muon_plan plan, int32_t* n_groups) {
  if (!plan || !n_groups) return fail(MUON_ERR_INVALID_ARG, "null argument");
  *n_groups = (int32_t)plan->p.groups.size();
  return MUON_OK;
}

muon_status muon_plan_group_info(muon_plan plan, int32_t g, int64_t* m, int64_t* n, int64_t* count,
                                 int64_t* n_transposed, int64_t* n_chunks) {
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "null plan");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(MUON_ERR_INVALID_ARG, "group index out of range");
  const muon::Group& G = plan->p.groups[g];
  if (m) *m = G.m;
  if (n) *n = G.n;
  if (count) *count = (int64_t)G.mats.size();
  if (n_transposed) *n_transposed = G.n_tr;
  if (n_chunks) *n_chunks = (int64_t)G.chunks.size();
  return MUON_OK;
}

muon_status muon_plan_num_matrices(muon_plan plan, int64_t* n) {
  if (!plan || !n) return fail(MUON_ERR_INVALID_ARG, "null plan or output pointer");
  *n = (int64_t)plan->p.mats.size();
  return MUON_OK;
}

muon_status muon_plan_assign(muon_plan plan, int32_t n_ranks, int32_t* owner, int64_t n_owner,
                             double* rank_cost) {
  if (!plan || !owner) return fail(MUON_ERR_INVALID_ARG, "null plan or owner array");
  if (n_ranks < 1) return fail(MUON_ERR_INVALID_ARG, "n_ranks must be >= 1");
  if (n_owner != (int64_t)plan->p.mats.size())
    return fail(MUON_ERR_INVALID_ARG, "n_owner must equal the plan's number of matrices (" +
                                          std::to_string(plan->p.mats.size()) + ")");
  std::vector<int32_t> own;
  std::vector<double> cost;
  muon::assign_greedy(plan->p, n_ranks, &own, &cost);
  std::memcpy(owner, own.data(), own.size() * sizeof(int32_t));
  if (rank_cost) std::memcpy(rank_cost, cost.data(), cost.size() * sizeof(double));
  return MUON_OK;
}

muon_status muon_shard_update(void* w_shard, muon_dtype dt, const float* o_full, int64_t offset, int64_t len,
                              float lr, float wd, float scale, void* stream) {
  if (dt != MUON_F32 && dt != MUON_BF16) return fail(MUON_ERR_DTYPE, "dt must be MUON_F32 or MUON_BF16");
  if (offset < 0 || len < 0) return fail(MUON_ERR_INVALID_ARG, "offset and len must be >= 0");
  if (!finite(lr) || !finite(wd) || !finite(scale)) return fail(MUON_ERR_INVALID_ARG, "lr, wd and scale must be finite");
  if (len == 0) return MUON_OK;
  if (!w_shard || !o_full) return fail(MUON_ERR_INVALID_ARG, "null w_shard or o_full");
  const size_t es = (dt == MUON_BF16) ? 2 : 4;
  const char* w0 = (const char*)w_shard;
  const char* o0 = (const char*)(o_full + offset);
  if (w0 < o0 + size_t(len) * 4 && o0 < w0 + size_t(len) * es)
    return fail(MUON_ERR_INVALID_ARG, "w_shard and o_full overlap");
  hipError_t e = muon::run_shard_update(w_shard, dt == MUON_BF16, o_full + offset, len, lr, wd, scale,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return MUON_OK;
}

muon_status muon_adamw_step(void* const* params, const void* const* grads, float* const* exp_avg,
                            float* const* exp_avg_sq, const int64_t* numels, int32_t n, muon_dtype dt,
                            float lr, float b1, float b2, float eps, float wd, int64_t step, void* stream) {
  if (dt != MUON_F32 && dt != MUON_BF16) return fail(MUON_ERR_DTYPE, "dt must be MUON_F32 or MUON_BF16");
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (!params || !grads || !exp_avg || !exp_avg_sq || !numels))
    return fail(MUON_ERR_INVALID_ARG, "null pointer array");
  if (!finite(lr) || !finite(b1) || !finite(b2) || !finite(eps) || !finite(wd))
    return fail(MUON_ERR_INVALID_ARG, "lr, b1, b2, eps and wd must be finite");
  if (!(b1 >= 0.f && b1 < 1.f && b2 >= 0.f && b2 < 1.f)) return fail(MUON_ERR_INVALID_ARG, "b1 and b2 must be in [0, 1)");
  if (!(eps > 0.f)) return fail(MUON_ERR_INVALID_ARG, "eps must be > 0");
  if (step < 1) return fail(MUON_ERR_INVALID_ARG, "step must be >= 1");
  for (int32_t i = 0; i < n; ++i) {
    if (numels[i] < 0) return fail(MUON_ERR_SHAPE, "numels[" + std::to_string(i) + "] < 0");
    if (numels[i] == 0) continue;
    const void* ptrs[4] = {params[i], grads[i], exp_avg[i], exp_avg_sq[i]};
    for (const void* q : ptrs)
      if (!q) return fail(MUON_ERR_INVALID_ARG, "null tensor pointer at " + std::to_string(i));
      else if ((uintptr_t)q % 4 != 0) return fail(MUON_ERR_ALIGNMENT, "tensor " + std::to_string(i) + " not 4-byte aligned");
    if (numels[i] > (int64_t(1) << 40)) return fail(MUON_ERR_SHAPE, "tensor too large");
  }
  // step size and bias corrections in double, rounded once to fp32
  const double t = double(step);
  muon::AdamScalars sc;
  sc.lr = lr; sc.b1 = b1; sc.b2 = b2; sc.eps = eps; sc.wd = wd;
  sc.step_size = float(double(lr) / (1.0 - std::pow(double(b1), t)));
  sc.bc2_sqrt = float(std::sqrt(1.0 - std::pow(double(b2), t)));
  const hipStream_t st = (hipStream_t)stream;
  muon::AdamTable tab;
  tab.n = 0;
  tab.first_block[0] = 0;
  auto flush = [&]() -> hipError_t {
    if (tab.n == 0) return hipSuccess;
    hipError_t e = muon::run_adamw(tab, sc, dt == MUON_BF16, st);
    tab.n = 0;
    tab.first_block[0] = 0;
    return e;
  };
  for (int32_t i = 0; i < n; ++i) {
    if (numels[i] == 0) continue;
    int64_t done = 0;
    while (done < numels[i]) {  // a tensor larger than one launch's block budget is split
      const int64_t room = (int64_t(1) << 30) - tab.first_block[tab.n];
      if (tab.n == muon::kAdamMaxTensors || room < 1) {
        if (hipError_t e = flush(); e != hipSuccess) return fail(MUON_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
        continue;
      }
      const int64_t take = std::min<int64_t>(numels[i] - done, room * muon::kAdamChunk);
      const size_t es = (dt == MUON_BF16) ? 2 : 4;
      tab.p[tab.n] = (char*)params[i] + done * es;
      tab.g[tab.n] = (const char*)grads[i] + done * es;
      tab.m[tab.n] = exp_avg[i] + done;
      tab.v[tab.n] = exp_avg_sq[i] + done;
      tab.numel[tab.n] = take;
      tab.first_block[tab.n + 1] = tab.first_block[tab.n] + int32_t((take + muon::kAdamChunk - 1) / muon::kAdamChunk);
      tab.n++;
      done += take;
    }
  }
  if (hipError_t e = flush(); e != hipSuccess) return fail(MUON_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return MUON_OK;
}

muon_status muon_workspace_status(muon_plan plan, void* workspace, size_t workspace_bytes, void* stream,
                                  int32_t* timed_out) {
  if (!plan || !timed_out) return fail(MUON_ERR_INVALID_ARG, "null plan or output pointer");
  const muon::Plan& P = plan->p;
  muon_status s = check_workspace(P, workspace, workspace_bytes);
  if (s != MUON_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  uint32_t* flag = (uint32_t*)((uint8_t*)workspace + P.ws_sync_off) + muon::kSyncErrWord;
  uint32_t h = 0;
  if (hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(MUON_ERR_HIP, "reading the workspace flag failed");
  *timed_out = h ? 1 : 0;
  if (h) {
    const uint32_t zero = 0;
    if (hipMemcpyAsync(flag, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return fail(MUON_ERR_HIP, "clearing the workspace flag failed");
  }
  return MUON_OK;
}

void muon_set_wait_limit(uint32_t polls) { g_spin_limit.store(polls ? polls : kSpinLimit); }

muon_status muon_step(muon_plan plan, void* const* param_ptrs, const void* const* grad_ptrs,
                      void* const* mom_ptrs, const muon_shape* shapes, int32_t n_params, float lr,
                      float mu, int32_t nesterov, float wd, float a, float b, float c, int32_t ns_steps,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "null plan");
  const muon::Plan& P = plan->p;
  muon_status s = check_shapes(P, shapes, n_params);
  if (s != MUON_OK) return s;
  if ((s = check_ptrs((const void* const*)param_ptrs, n_params, "param_ptrs")) != MUON_OK) return s;
  if ((s = check_ptrs(grad_ptrs, n_params, "grad_ptrs")) != MUON_OK) return s;
  if ((s = check_ptrs((const void* const*)mom_ptrs, n_params, "mom_ptrs")) != MUON_OK) return s;
  if (!finite(lr) || !finite(mu) || !finite(wd) || !finite(scale))
    return fail(MUON_ERR_INVALID_ARG, "lr, mu, wd and scale must be finite");
  if (nesterov != 0 && nesterov != 1) return fail(MUON_ERR_INVALID_ARG, "nesterov must be 0 or 1");
  if ((s = check_coeffs(a, b, c, ns_steps)) != MUON_OK) return s;
  if ((s = check_workspace(P, workspace, workspace_bytes)) != MUON_OK) return s;
  muon::StepScalars sc{lr, mu, wd, scale, a, b, c, nesterov, ns_steps, 0};
  return run_all(P, param_ptrs, grad_ptrs, mom_ptrs, sc, workspace, (hipStream_t)stream);
}

muon_status muon_ns(muon_plan plan, const void* const* in_ptrs, float* const* out_ptrs,
                    const muon_shape* shapes, int32_t n_params, float a, float b, float c,
                    int32_t ns_steps, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "null plan");
  const muon::Plan& P = plan->p;
  muon_status s = check_shapes(P, shapes, n_params);
  if (s != MUON_OK) return s;
  if ((s = check_ptrs(in_ptrs, n_params, "in_ptrs")) != MUON_OK) return s;
  if ((s = check_ptrs((const void* const*)out_ptrs, n_params, "out_ptrs")) != MUON_OK) return s;
  if ((s = check_coeffs(a, b, c, ns_steps)) != MUON_OK) return s;
  if ((s = check_workspace(P, workspace, workspace_bytes)) != MUON_OK) return s;
  muon::StepScalars sc{0.f, 0.f, 0.f, 1.f, a, b, c, 0, ns_steps, 1};
  return run_all(P, (void* const*)out_ptrs, in_ptrs, nullptr, sc, workspace, (hipStream_t)stream);
}

const char* muon_status_str(muon_status s) {
  switch (s) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
    case MUON_ERR_SHAPE: return "MUON_ERR_SHAPE";
    case MUON_ERR_DTYPE: return "MUON_ERR_DTYPE";
    case MUON_ERR_PLAN_MISMATCH: return "MUON_ERR_PLAN_MISMATCH";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
    case MUON_ERR_ALIGNMENT: return "MUON_ERR_ALIGNMENT";
  }
  return "MUON_ERR_UNKNOWN";
}

const char* muon_last_error_detail(void) { return g_detail.c_str(); }

int32_t muon_version(void) { return 100; }

}  // extern "C"
