// Persistent kernel for skinny matrices (bf16, m <= 32 rows in the wide
// orientation), e.g. the 74 x [24, 10240] batch named in item 3 of the
// HyperParallel FSDP Muon optimizer RFC.
//
// Every matrix is split into S column slabs, one workgroup per slab.  A
// workgroup keeps its slab of the NS iterate X in registers for the whole
// step, so HBM sees only the compulsory traffic: G and M read, M written,
// W read and written.  Per NS step the only data exchanged between the
// workgroups of one matrix is their partial Gram matrix X_slab X_slab^T
// (m x m fp32), published to the workspace and combined after a per-matrix
// barrier.  Each workgroup then forms the same A and P = aI + bA + cA^2
// (all fp32, fixed summation order) and applies P to its own columns.
//
// Arithmetic: X is held in bf16 between steps; the Gram uses bf16 MFMA with
// fp32 accumulation (exact products); P is split into bf16 hi + lo parts so
// the apply X' = P X is accurate to about 16 mantissa bits of P; the last
// step's result O stays fp32 up to the weight update.
//
// Register layout (wave64, MFMA 32x32x16): a "block" is 32 columns of the
// slab.  Lane l (h = l / 32, c = l % 32) holds column c of the block at the
// 16 rows  row(r) = 8*(r/4) + 4*h + (r%4), r = 0..15.  This is the output
// layout of the 32x32 MFMA, so the apply X' = P X maps it onto itself when
// the contraction index is permuted the same way in P's operand: no data
// movement between NS steps.  The Gram contracts over columns instead, so
// each block is restaged through LDS once per step.
#include "common.hpp"
#include "launch.hpp"

namespace muon {

namespace {

constexpr int kNB = 10;        // 32-column blocks per wave (slab <= 4 * 10 * 32 = 1280 columns)
constexpr int kLdr = 36;       // LDS column stride (bf16) of the transpose staging
constexpr int kPart = 1024 + 64;  // floats per published slab partial
constexpr int kErrSlot = 2040;    // u32 index of the timeout flag in the sync region

__device__ __forceinline__ int row_of(int r, int h) { return ((r >> 2) << 3) + (h << 2) + (r & 3); }
// X row that k-slot q (0..7) of k-step t holds in lane half h
__device__ __forceinline__ int krow(int t, int h, int q) { return 16 * t + ((q >> 2) << 3) + (h << 2) + (q & 3); }

// Per-matrix sense-reversing barrier among the S workgroups of matrix z.
// sync[2z] counts arrivals, sync[2z+1] is the generation.  The wait is
// bounded: on timeout a flag is raised and the workgroup carries on, so the
// grid always drains.
__device__ void matrix_barrier(uint32_t* sync, int z, int S, unsigned spin_limit) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = sync + 2 * z;
    uint32_t* gen = sync + 2 * z + 1;
    const uint32_t g0 = __hip_atomic_load(gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == uint32_t(S - 1)) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      unsigned it = 0;
      while (__hip_atomic_load(gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == g0) {
        __builtin_amdgcn_s_sleep(2);
        if (++it > spin_limit) {
          __hip_atomic_store(sync + kErrSlot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
  __threadfence();
}

struct SkShared {
  uint16_t stage[4][32 * kLdr];   // per-wave transpose staging, column-major [col][row]
  float red[4][1024];             // per-wave Gram partials
  float A[32][33];                // combined Gram (fp32)
  uint16_t Phi[32][34], Plo[32][34];
  float ss[4];
};

}  // namespace

// MODE 0: muon_step (momentum in, weight update out); MODE 1: muon_ns (O out)
template <typename PT, int MODE>
__global__ __launch_bounds__(256, 3) void skinny_kernel(MatTable tab, StepScalars sc, int m, int64_t n,
                                                        int S, int64_t slab_w, float* __restrict__ part,
                                                        uint32_t* __restrict__ sync, unsigned spin_limit) {
  static_assert(sizeof(PT) == 2, "skinny path is bf16");
  constexpr bool step_mode = MODE == 0;
  __shared__ SkShared sh;
  const int z = blockIdx.x / S, s = blockIdx.x % S;
  // copy this matrix's descriptor out of the argument block
  const bool tr = tab.tr[z] != 0;
  const PT* G = (const PT*)tab.e[z].g;
  float* Mm = tab.e[z].m;
  void* Wout = tab.e[z].w;
  // 32-bit element offsets: the plan keeps m * n below 2^31 on this path
  const int c0 = int(int64_t(s) * slab_w);
  const int c1 = int((int64_t(c0) + slab_w < n) ? int64_t(c0) + slab_w : n);
  const int nn = int(n);
  // element offset of (row, col) in the stored matrix: row * rs + col * cs
  const int rs = tr ? 1 : nn, cs = tr ? m : 1;
  const uint32_t elems = uint32_t(m) * uint32_t(nn);
  const rsrc_t rG = make_rsrc(G, elems * 2);
  const rsrc_t rM = make_rsrc(Mm, step_mode ? elems * 4 : 0);
  const rsrc_t rW = make_rsrc(Wout, elems * (MODE == 1 ? 4 : 2));
  const int v = threadIdx.x >> 6;  // wave index (uniform within the wave)
  float* part_z = part + int64_t(z) * 2 * S * kPart;

  // Thread-index-derived values are re-derived through opaque() at the top of
  // each phase: otherwise the compiler hoists every address it can out of
  // the NS loop and keeps them all live, which costs more registers than
  // the slab of X itself.
  //
  // Padding elements (rows >= m, columns >= c1) use an out-of-range buffer
  // offset: their loads return 0 and their stores are dropped.
  auto eoff = [=](int row, int col) -> uint32_t {
    return (row < m && col < c1) ? uint32_t(row * rs + col * cs) : kOob;
  };

  // the slab of X held by this lane: 16 bf16 per block, packed in pairs
  // (dword d holds rows row_of(2d, h) and row_of(2d+1, h))
  uint32_t xw[kNB][8];
  float ss = 0.f;

  // ---- momentum, Nesterov, NS input --------------------------------------
#pragma unroll
  for (int q = 0; q < kNB; ++q) {
    const int lane = opaque(int(threadIdx.x)) & 63, h = lane >> 5;
    const int col = c0 + (v * kNB + q) * 32 + (lane & 31);
    // all loads of the block first (stores to M below could alias later
    // loads as far as the compiler knows), then the arithmetic and stores
    uint32_t e[16];
    float gv[16], mv[16], uu[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = eoff(row_of(r, h), col);
      gv[r] = bf2f(buf_ld_u16(rG, e[r] * 2));
      if (step_mode) mv[r] = buf_ld_f32(rM, e[r] * 4);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float u = gv[r];
      if (step_mode) {
        const float mn = fmaf(sc.mu, mv[r], gv[r]);
        buf_st_f32(rM, e[r] * 4, mn);
        u = sc.nesterov ? fmaf(sc.mu, mn, gv[r]) : mn;
      }
      ss = fmaf(u, u, ss);  // padding reads 0, adds nothing
      uu[r] = u;
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) xw[q][d] = f2bf2(uu[2 * d], uu[2 * d + 1]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- helpers ---------------------------------------------------------------
  // Gram contribution of one block: stage the block column-major in this
  // wave's LDS area, read it back row-per-lane, one MFMA per 16 columns.
  auto gram_block = [&](const uint32_t* x, f32x16& gacc, int lane) {
    const int h = lane >> 5, cl = lane & 31;
    uint16_t* stg = sh.stage[v];
#pragma unroll
    for (int g = 0; g < 4; ++g) *(u32x2*)(stg + cl * kLdr + 8 * g + 4 * h) = u32x2{x[2 * g], x[2 * g + 1]};
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = stg[(16 * tt + 8 * h + e) * kLdr + cl];
      const bf16x8 fb = as_bf16x8(f);
      gacc = mfma32x32x16(fb, fb, gacc);
    }
  };

  // combine the 4 wave partials and publish this slab's partial
  auto publish = [&](const f32x16& gacc, int par, bool with_ss) {
    const int t = opaque(int(threadIdx.x)), lane = t & 63, h = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) sh.red[v][row_of(r, h) * 32 + cl] = gacc[r];
    float tot = 0.f;
    if (with_ss) tot = block_sum_256(ss, sh.ss);  // contains __syncthreads
    __syncthreads();
    float* dst = part_z + (int64_t(par) * S + s) * kPart;
    for (int e = t; e < m * m; e += 256) {
      const int i = e / m, j = e - i * m;
      const int o = i * 32 + j;
      dst[e] = (sh.red[0][o] + sh.red[1][o]) + (sh.red[2][o] + sh.red[3][o]);
    }
    if (with_ss && t == 0) dst[1024] = tot;
  };

  // after the barrier: combine all slab partials (fixed order) into A and
  // form P = ps * (aI + bA + cA^2) with its hi/lo split; on the first step
  // also the normalisation (A = s^2 * sum, ps = s)
  auto form_p = [&](int par, bool first, float& s_out) {
    const int t = opaque(int(threadIdx.x));
    const float* src = part_z + int64_t(par) * S * kPart;
    float s2 = 1.f, ps = 1.f;
    if (first) {
      float tot = 0.f;
      for (int q = 0; q < S; ++q) tot += src[int64_t(q) * kPart + 1024];
      const float sn = 1.0f / (sqrtf(tot) + kNsEps);
      s2 = sn * sn;
      ps = sn;
      s_out = sn;
    }
    for (int e = t; e < 1024; e += 256) {
      const int i = e >> 5, j = e & 31;
      float a = 0.f;
      if (i < m && j < m) {
        for (int q = 0; q < S; ++q) a += src[int64_t(q) * kPart + i * m + j];
        a *= s2;
      }
      sh.A[i][j] = a;
    }
    __syncthreads();
    for (int e = t; e < 1024; e += 256) {
      const int i = e >> 5, j = e & 31;
      float p = 0.f;
      if (i < m && j < m) {
        float a2 = 0.f;
        for (int k = 0; k < m; ++k) a2 = fmaf(sh.A[i][k], sh.A[k][j], a2);
        p = fmaf(sc.c, a2, sc.b * sh.A[i][j]);
        if (i == j) p += sc.a;
        p *= ps;
      }
      const uint16_t ph = f2bf(p);
      sh.Phi[i][j] = ph;
      sh.Plo[i][j] = f2bf(p - bf2f(ph));
    }
    __syncthreads();
  };

  // this lane's operand registers of P (hi, lo) for the two k-steps: the
  // contraction index is permuted to match the row layout of X
  u16x8 ph[2], pl[2];
  auto load_p = [&]() {
    const int lane = opaque(int(threadIdx.x)) & 63, h = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kr = krow(tt, h, q);
        ph[tt][q] = sh.Phi[cl][kr];
        pl[tt][q] = sh.Plo[cl][kr];
      }
  };
  auto apply = [&](const uint32_t* x) {
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], x[2], x[3]});
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, u32x4{x[4], x[5], x[6], x[7]});
    f32x16 acc = f32x16{};
    acc = mfma32x32x16(as_bf16x8(ph[0]), x0, acc);
    acc = mfma32x32x16(as_bf16x8(pl[0]), x0, acc);
    acc = mfma32x32x16(as_bf16x8(ph[1]), x1, acc);
    acc = mfma32x32x16(as_bf16x8(pl[1]), x1, acc);
    return acc;
  };

  // O for one block (16 values per lane) -> fp32 store or weight update;
  // all W loads are issued before the stores
  const float keep = 1.0f - sc.lr * sc.wd, stepc = -sc.lr * sc.scale;
  auto emit_block = [&](const f32x16& o, int q) {
    const int lane = opaque(int(threadIdx.x)) & 63, h = lane >> 5;
    const int col = c0 + (v * kNB + q) * 32 + (lane & 31);
    uint32_t e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = eoff(row_of(r, h), col);
    if (!step_mode) {
#pragma unroll
      for (int r = 0; r < 16; ++r) buf_st_f32(rW, e[r] * 4, o[r]);
    } else {
      float w[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) w[r] = bf2f(buf_ld_u16(rW, e[r] * 2));
#pragma unroll
      for (int r = 0; r < 16; ++r) buf_st_u16(rW, e[r] * 2, f2bf(fmaf(stepc, o[r], w[r] * keep)));
    }
  };

  // ---- Gram of X0 -----------------------------------------------------------
  f32x16 gacc = f32x16{};
  {
    const int lane = opaque(int(threadIdx.x)) & 63;
#pragma unroll
    for (int q = 0; q < kNB; ++q) gram_block(xw[q], gacc, lane);
  }

  const int steps = sc.ns_steps;
  float snorm = 1.f;

  if (steps == 0) {
    publish(gacc, 0, true);
    matrix_barrier(sync, z, S, spin_limit);
    form_p(0, true, snorm);
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      f32x16 o;
#pragma unroll
      for (int r = 0; r < 16; ++r) o[r] = snorm * bf2f(uint16_t(xw[q][r >> 1] >> (16 * (r & 1))));
      emit_block(o, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }

  for (int k = 0; k < steps - 1; ++k) {
    const int par = k & 1;
    publish(gacc, par, k == 0);
    matrix_barrier(sync, z, S, spin_limit);
    form_p(par, k == 0, snorm);
    load_p();
    gacc = f32x16{};
    const int lane = opaque(int(threadIdx.x)) & 63;
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      const f32x16 acc = apply(xw[q]);
#pragma unroll
      for (int d = 0; d < 8; ++d) xw[q][d] = f2bf2(acc[2 * d], acc[2 * d + 1]);
      gram_block(xw[q], gacc, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // last NS step: O = P X in fp32, then the update
  {
    const int k = steps - 1;
    publish(gacc, k & 1, k == 0);
    matrix_barrier(sync, z, S, spin_limit);
    form_p(k & 1, k == 0, snorm);
    load_p();
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      const f32x16 acc = apply(xw[q]);
      emit_block(acc, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

hipError_t run_skinny(const SkinnyArgs& g, hipStream_t st) {
  const unsigned grid = unsigned(g.count * g.slabs);
  if (g.sc.mode == 0)
    hipLaunchKernelGGL((skinny_kernel<uint16_t, 0>), dim3(grid), dim3(256), 0, st, g.tab, g.sc, g.m, g.n,
                       g.slabs, g.slab_w, g.part, g.sync, g.spin_limit);
  else
    hipLaunchKernelGGL((skinny_kernel<uint16_t, 1>), dim3(grid), dim3(256), 0, st, g.tab, g.sc, g.m, g.n,
                       g.slabs, g.slab_w, g.part, g.sync, g.spin_limit);
  return hipGetLastError();
}

int skinny_max_blocks_per_cu() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, skinny_kernel<uint16_t, 0>, 256, 0) != hipSuccess)
    return 0;
  return nb;
}

}  // namespace muon
