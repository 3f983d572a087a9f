// C ABI entry points (include/muon.h): validation, per-chunk descriptor
// tables, and the launch sequence on the caller's stream.  The step entry
// points allocate and free no device memory and never wait for the device;
// the only allocation is one 4-byte pinned host word per device, made on the
// first eager step (the skinny path's timeout report).  A plan with MFMA
// groups also creates, on its first eager step on a device, one stream and
// two events there (the side stream of small groups' product chains), and
// releases them when it is destroyed.
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
#include "validate.hpp"

// A second stream on one device with the events that fork work onto it from
// the launch stream and join it back (kernels' launches, not the results,
// depend on it: see ns_group_bf16).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;  // creation attempted (it is not retried after a failure)
};
constexpr int kMaxDevices = 64;

struct muon_plan_s {
  muon::Plan p;
  SideStream side[kMaxDevices];  // per device, made on the plan's first eager step there
  ~muon_plan_s() {
    bool any = false;
    for (const SideStream& ss : side) any = any || ss.s || ss.fork || ss.join;
    if (!any) return;  // no HIP call for a plan that never made one
    int cur = -1;
    const bool have = hipGetDevice(&cur) == hipSuccess;
    for (int d = 0; d < kMaxDevices; ++d) {
      SideStream& ss = side[d];
      if (!ss.s && !ss.fork && !ss.join) continue;
      if (hipSetDevice(d) != hipSuccess) continue;
      // the host waits for the stream's queued work, so nothing still
      // queued anywhere refers to the events when they go
      if (ss.s) (void)hipStreamSynchronize(ss.s);
      if (ss.join) (void)hipEventDestroy(ss.join);
      if (ss.fork) (void)hipEventDestroy(ss.fork);
      if (ss.s) (void)hipStreamDestroy(ss.s);
    }
    if (have) (void)hipSetDevice(cur);
  }
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

// Per-device state: compute units, the skinny kernel's co-resident
// capacity, and a host-visible word (pinned host memory) that a skinny
// workgroup sets when one of its waits times out.
struct DevState {
  int index = -1;                 // device ordinal
  int cus = -1;
  int skinny_cap = -1;
  uint32_t* host_flag = nullptr;  // hipHostMalloc'd, 4 bytes; null until first eager step
  bool flag_tried = false;
  void* scratch = nullptr;        // device address of this device's copy of `scratch`
};
std::mutex g_dev_mu;
DevState g_dev[kMaxDevices];  // fixed storage: looking a device up allocates nothing

// Queries the current device once and returns its state.  `allow_alloc`: the
// host-visible flag may be allocated (never while the stream is captured).
muon_status device_state(bool allow_alloc, DevState* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_ERR_HIP, "device index beyond the library's table");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevState& d = g_dev[dev];
  if (d.cus < 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(MUON_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
    const int per_cu = muon::skinny_max_blocks_per_cu();
    if (per_cu <= 0) return fail(MUON_ERR_HIP, "occupancy query of the skinny kernel failed");
    d.cus = n;
    d.skinny_cap = n * per_cu;
  }
  if (allow_alloc && !d.flag_tried) {
    d.flag_tried = true;
    void* p = nullptr;
    if (hipHostMalloc(&p, sizeof(uint32_t), hipHostMallocDefault) == hipSuccess && p) {
      *(volatile uint32_t*)p = 0u;
      d.host_flag = (uint32_t*)p;
    }
  }
  *out = d;
  out->index = dev;
  return MUON_OK;
}

// Whether small groups may run a product chain on a plan's side stream
// (muon_set_side_stream; on by default).
std::atomic<bool> g_side_enabled{true};

// The plan's side stream on the current device, made on first use when
// `allow_alloc` (never while `st` is being captured: a recorded step keeps
// every launch on the captured stream), or null.  Plans without MFMA groups
// never make one.
SideStream* side_stream(muon_plan plan, const DevState& dev, hipStream_t st, bool allow_alloc) {
  if (!plan || !g_side_enabled.load() || capturing(st)) return nullptr;
  SideStream& ss = plan->side[dev.index];
  if (!ss.tried && allow_alloc) {
    ss.tried = true;
    bool mfma = false;
    for (const muon::Group& grp : plan->p.groups) mfma = mfma || grp.path == muon::PATH_MFMA;
    if (mfma) {
      // default priority, and not synchronised with the null stream (the
      // events order it against the launch stream)
      const bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess &&
                      hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess &&
                      hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
      if (!ok) {
        if (ss.join) (void)hipEventDestroy(ss.join);
        if (ss.fork) (void)hipEventDestroy(ss.fork);
        if (ss.s) (void)hipStreamDestroy(ss.s);
        ss = SideStream{};
        ss.tried = true;
        (void)hipGetLastError();  // the failure changes nothing but the schedule
      }
    }
  }
  return ss.s ? &ss : nullptr;
}

// Reads and clears the host-visible timeout word of the current device.
bool take_timeout(const DevState& d) {
  if (!d.host_flag) return false;
  return __atomic_exchange_n(d.host_flag, 0u, __ATOMIC_ACQ_REL) != 0u;
}

// Device checks done before anything is enqueued: every skinny chunk must
// fit the device's co-resident capacity.
muon_status check_device(const muon::Plan& P, const DevState& d) {
  for (const muon::Group& grp : P.groups) {
    if (grp.path != muon::PATH_SKINNY) continue;
    const int64_t need = int64_t(grp.max_chunk) * grp.slabs;
    if (need > d.skinny_cap)
      return fail(MUON_ERR_HIP, "device holds only " + std::to_string(d.skinny_cap) +
                                    " co-resident workgroups of the skinny kernel; a chunk needs " +
                                    std::to_string(need));
  }
  return MUON_OK;
}

size_t elem_size(muon_dtype d) { return d == MUON_BF16 ? 2 : 4; }

// Enqueue every chunk of every group (arguments already validated).  `w`,
// `g`, `m` are per-parameter device pointers (m may be null for muon_ns).
muon_status run_all(const muon::Plan& P, void* const* w, const void* const* g, void* const* m,
                    const muon::StepScalars& sc, void* workspace, hipStream_t st, const DevState& dev,
                    const SideStream* side) {
  using namespace muon;
  uint8_t* ws = (uint8_t*)workspace;
  const size_t pes = elem_size(P.param_dt);
  const bool cap = capturing(st);
  for (const Group& grp : P.groups) {
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
        a.host_flag = dev.host_flag;
        a.lobuf = ws + P.ws_dyn_off + skinny_lo_offset(grp, ch.count);
        if (cap) {
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
        a.whole = grp.whole;
        a.precise = grp.precise;
        a.x0_lo = a.bf16 && sc.mode == 0;  // muon_ns inputs are bf16 already: no lo part
        a.cus = dev.cus;
        a.side = side ? side->s : nullptr;
        a.ev_fork = side ? side->fork : nullptr;
        a.ev_join = side ? side->join : nullptr;
        e = run_large(a, st);
      }
      if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    }
  }
  return MUON_OK;
}

// Device checks, the timeout report of earlier calls, then the launches.
// `allow_alloc`: the host-visible timeout word and the plan's side stream may
// be made (first eager call); `plan` null: no side stream.
muon_status enqueue(muon_plan plan, const muon::Plan& P, void* const* w, const void* const* g, void* const* m,
                    const muon::StepScalars& sc, void* workspace, hipStream_t st, bool allow_alloc = true) {
  DevState dev;
  if (muon_status s = device_state(allow_alloc && !capturing(st), &dev); s != MUON_OK) return s;
  if (muon_status s = check_device(P, dev); s != MUON_OK) return s;
  if (take_timeout(dev))
    return fail(MUON_ERR_TIMEOUT, "an earlier skinny-path launch on this device timed out waiting for its "
                                  "workgroups; its W (or O) was left partly unwritten and its momenta were "
                                  "updated (nothing was enqueued by this call)");
  const SideStream* side = side_stream(plan, dev, st, allow_alloc);
  return run_all(P, w, g, m, sc, workspace, st, dev, side);
}

// ---- The allocation-free step (muon_step_noalloc) --------------------------
// Its workspace is this file-scope device array, one copy per device, held
// until the process ends.  In host code `scratch` only names the symbol: its
// device address is taken once per device with hipGetSymbolAddress and kept
// in DevState::scratch, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += size_t(gridDim.x) * blockDim.x)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

// Device address of the current device's scratch array, set up on the first
// call on that device: the address is looked up, the array is cleared by a
// fill kernel on `st` and the host waits for it (first call only, so it must
// not be recorded into a graph).
muon_status scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MUON_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(MUON_ERR_HIP, "device index beyond the library's table");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevState& d = g_dev[dev];
  if (!d.scratch) {
    if (capturing(st))
      return fail(MUON_ERR_INVALID_ARG, "the first muon_step_noalloc call on a device sets up its scratch "
                                        "array and must not be recorded into a graph");
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return fail(MUON_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
    hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, st, (uint4*)p, kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
      return fail(MUON_ERR_HIP, "clearing the scratch array failed");
    d.scratch = p;
  }
  *out = d.scratch;
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
  std::string d;
  bool nothing = false;
  muon_status s = muon::validate_shard_update(w_shard, dt, o_full, offset, len, lr, wd, scale, &nothing, &d);
  if (s != MUON_OK) return fail(s, d);
  if (nothing) return MUON_OK;
  hipError_t e = muon::run_shard_update(w_shard, dt == MUON_BF16, o_full + offset, len, lr, wd, scale,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return MUON_OK;
}

muon_status muon_adamw_step(void* const* params, const void* const* grads, float* const* exp_avg,
                            float* const* exp_avg_sq, const int64_t* numels, int32_t n, muon_dtype dt,
                            float lr, float b1, float b2, float eps, float wd, int64_t step, void* stream) {
  std::string d;
  muon_status vs = muon::validate_adamw(params, grads, exp_avg, exp_avg_sq, numels, n, dt, lr, b1, b2, eps, wd, step, &d);
  if (vs != MUON_OK) return fail(vs, d);
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
  std::string d;
  muon_status s = muon::check_workspace(P, workspace, workspace_bytes, &d);
  if (s != MUON_OK) return fail(s, d);
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

void muon_set_side_stream(int32_t enable) { g_side_enabled.store(enable != 0); }

muon_status muon_poll_timeout(int32_t* timed_out) {
  if (!timed_out) return fail(MUON_ERR_INVALID_ARG, "null output pointer");
  *timed_out = 0;
  DevState dev;
  if (muon_status s = device_state(false, &dev); s != MUON_OK) return s;
  *timed_out = take_timeout(dev) ? 1 : 0;
  return MUON_OK;
}

muon_status muon_step(muon_plan plan, void* const* param_ptrs, const void* const* grad_ptrs,
                      void* const* mom_ptrs, const muon_shape* shapes, int32_t n_params, float lr,
                      float mu, int32_t nesterov, float wd, float a, float b, float c, int32_t ns_steps,
                      float scale, void* workspace, size_t workspace_bytes, void* stream) {
  std::string d;
  const muon::Plan* P = plan ? &plan->p : nullptr;
  muon_status s = muon::validate_step(P, param_ptrs, grad_ptrs, mom_ptrs, shapes, n_params, lr, mu, nesterov, wd,
                                      a, b, c, ns_steps, scale, workspace, workspace_bytes, &d);
  if (s != MUON_OK) return fail(s, d);
  muon::StepScalars sc{lr, mu, wd, scale, a, b, c, nesterov, ns_steps, 0};
  return enqueue(plan, *P, param_ptrs, grad_ptrs, mom_ptrs, sc, workspace, (hipStream_t)stream);
}

muon_status muon_step_noalloc(muon_plan plan, void* const* param_ptrs, const void* const* grad_ptrs,
                              void* const* mom_ptrs, const muon_shape* shapes, int32_t n_params, float lr,
                              float mu, int32_t nesterov, float wd, float a, float b, float c,
                              int32_t ns_steps, float scale, void* stream) {
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "null plan");
  if (plan->p.ws_bytes > kScratchBytes)
    return fail(MUON_ERR_WORKSPACE, "the plan needs " + std::to_string(plan->p.ws_bytes) +
                                        " bytes of workspace; the static scratch array holds " +
                                        std::to_string(kScratchBytes) + " (use muon_step with a workspace)");
  std::string d;
  // every argument but the workspace, checked before any device work
  muon_status s = muon::validate_step(&plan->p, param_ptrs, grad_ptrs, mom_ptrs, shapes, n_params, lr, mu, nesterov,
                                      wd, a, b, c, ns_steps, scale, (const void*)uintptr_t(256), kScratchBytes, &d);
  if (s != MUON_OK) return fail(s, d);
  const hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  if ((s = scratch_address(st, &ws)) != MUON_OK) return s;
  muon::StepScalars sc{lr, mu, wd, scale, a, b, c, nesterov, ns_steps, 0};
  // no side stream: this entry point makes nothing, and its launches stay on `st`
  return enqueue(nullptr, plan->p, param_ptrs, grad_ptrs, mom_ptrs, sc, ws, st, false);
}

muon_status muon_ns(muon_plan plan, const void* const* in_ptrs, float* const* out_ptrs,
                    const muon_shape* shapes, int32_t n_params, float a, float b, float c,
                    int32_t ns_steps, void* workspace, size_t workspace_bytes, void* stream) {
  std::string d;
  const muon::Plan* P = plan ? &plan->p : nullptr;
  muon_status s = muon::validate_ns(P, in_ptrs, out_ptrs, shapes, n_params, a, b, c, ns_steps, workspace,
                                    workspace_bytes, &d);
  if (s != MUON_OK) return fail(s, d);
  muon::StepScalars sc{0.f, 0.f, 0.f, 1.f, a, b, c, 0, ns_steps, 1};
  return enqueue(plan, *P, (void* const*)out_ptrs, in_ptrs, nullptr, sc, workspace, (hipStream_t)stream);
}

muon_status muon_kernel_timing(int32_t enable) {
  if (hipError_t e = muon::timer_enable(enable != 0); e != hipSuccess)
    return fail(MUON_ERR_HIP, std::string("creating timing events failed: ") + hipGetErrorString(e));
  return MUON_OK;
}

muon_status muon_kernel_timing_read(double* ms, int64_t* launches, double* alg_flops, double* exec_flops) {
  if (!ms || !launches || !alg_flops || !exec_flops) return fail(MUON_ERR_INVALID_ARG, "null output pointer");
  if (hipError_t e = muon::timer_read(ms, launches, alg_flops, exec_flops); e != hipSuccess)
    return fail(MUON_ERR_HIP, std::string("reading timing events failed: ") + hipGetErrorString(e));
  return MUON_OK;
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
    case MUON_ERR_TIMEOUT: return "MUON_ERR_TIMEOUT";
  }
  return "MUON_ERR_UNKNOWN";
}

const char* muon_last_error_detail(void) { return g_detail.c_str(); }

int32_t muon_version(void) { return 200; }

}  // extern "C"
