// Elementwise kernels around the Muon step.
//
// shard_update_kernel: one rank's flat shard of a parameter takes the
// decoupled update from the full O, as in item 1(1) of the HyperParallel FSDP
// Muon optimizer RFC (after NS on the gathered momentum, each rank updates
// the slice at its own offset), with the weight decay of its item 6.  The
// arithmetic is that of the last NS epilogue of the step kernels:
// W (1 - lr wd) + (-lr scale) O as one fused multiply-add in fp32, rounded
// once to the parameter type.
//
// adamw_kernel: the companion step for 1-D parameters (norm gains, biases),
// which the Muon sharding optimizer of PaddlePaddle/Paddle pull request 79428
// keeps in buffers apart from the 2-D ones that go through NS.  AdamW
// with decoupled weight decay, one workgroup per chunk of kAdamChunk
// elements of one tensor; the tensor of a workgroup is found by a binary
// search of the chunk prefix sums in the argument block.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace muon {

namespace {

constexpr int kElemThreads = 256;
constexpr int kElemPerThread = 4;
constexpr int64_t kElemPerBlock = int64_t(kElemThreads) * kElemPerThread;

// Vector path: both pointers 16-byte aligned; each thread moves runs of VEC
// consecutive elements (8 bf16 / 4 fp32 of W = 16 bytes), lanes adjacent, so
// every wave access is one contiguous run.  The tail (len % VEC) and
// misaligned shards take the element path.
template <typename PT>
__device__ __forceinline__ void shard_elem(PT* w, const float* o, int64_t e, float keep, float stepc) {
  Elem<PT>::store(w + e, fmaf(stepc, o[e], Elem<PT>::load(w + e) * keep));
}

template <typename PT>
__global__ __launch_bounds__(kElemThreads) void shard_update_kernel(PT* __restrict__ w, const float* __restrict__ o,
                                                                    int64_t len, float lr, float wd, float scale,
                                                                    int vec) {
  const float keep = 1.0f - lr * wd, stepc = -lr * scale;
  constexpr int VEC = 16 / int(sizeof(PT));
  const int64_t tid = int64_t(blockIdx.x) * kElemThreads + threadIdx.x;
  const int64_t nth = int64_t(gridDim.x) * kElemThreads;
  int64_t done = 0;
  if (vec) {
    const int64_t nv = len / VEC;
    for (int64_t i = tid; i < nv; i += nth) {
      const int64_t e = i * VEC;
      u32x4 wv = *(const u32x4*)(w + e);
      float ov[VEC];
#pragma unroll
      for (int q = 0; q < VEC / 4; ++q) {
        const f32x4 x = *(const f32x4*)(o + e + 4 * q);
        ov[4 * q] = x[0]; ov[4 * q + 1] = x[1]; ov[4 * q + 2] = x[2]; ov[4 * q + 3] = x[3];
      }
      if constexpr (sizeof(PT) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = fmaf(stepc, ov[2 * j], bf2f(uint16_t(wv[j] & 0xffffu)) * keep);
          const float hi = fmaf(stepc, ov[2 * j + 1], bf2f(uint16_t(wv[j] >> 16)) * keep);
          wv[j] = f2bf2(lo, hi);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[j] = __float_as_uint(fmaf(stepc, ov[j], __uint_as_float(wv[j]) * keep));
      }
      *(u32x4*)(w + e) = wv;
    }
    done = nv * VEC;
  }
  for (int64_t e = done + tid; e < len; e += nth) shard_elem(w, o, e, keep, stepc);
}

// AdamW on one element (fp32 arithmetic; the order of the operations is the
// same on the vector and element paths, so both give identical bits).
__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v, const AdamScalars& sc,
                                          float keep) {
  p *= keep;
  m = fmaf(sc.b1, m, (1.0f - sc.b1) * g);
  v = fmaf(sc.b2, v, (1.0f - sc.b2) * g * g);
  const float denom = sqrtf(v) / sc.bc2_sqrt + sc.eps;
  p = p - sc.step_size * (m / denom);
}

template <typename PT>
__global__ __launch_bounds__(kElemThreads) void adamw_kernel(AdamTable tab, AdamScalars sc) {
  const int b = blockIdx.x;
  int lo = 0, hi = tab.n - 1;  // last tensor with first_block <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.first_block[mid] <= b) lo = mid; else hi = mid - 1;
  }
  const int t = lo;
  const int64_t n = tab.numel[t];
  const int64_t base = int64_t(b - tab.first_block[t]) * kAdamChunk;
  PT* __restrict__ p = (PT*)tab.p[t];
  const PT* __restrict__ g = (const PT*)tab.g[t];
  float* __restrict__ m = tab.m[t];
  float* __restrict__ v = tab.v[t];
  const float keep = 1.0f - sc.lr * sc.wd;
  constexpr int VEC = 4;  // elements per thread and pass
  const bool vec = ((uintptr_t)p | (uintptr_t)g | (uintptr_t)m | (uintptr_t)v) % (VEC * sizeof(PT)) == 0 &&
                   ((uintptr_t)m | (uintptr_t)v) % 16 == 0 && base + kAdamChunk <= n;
  if (vec) {
    constexpr int NI = int(kAdamChunk / (kElemThreads * VEC));
    // every pass's loads are issued before the first store
    typedef std::conditional_t<sizeof(PT) == 2, u32x2, f32x4> PW;
    PW pwq[NI], gwq[NI];
    f32x4 mvq[NI], vvq[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t e = base + (int64_t(i) * kElemThreads + threadIdx.x) * VEC;
      mvq[i] = *(const f32x4*)(m + e);
      vvq[i] = *(const f32x4*)(v + e);
      pwq[i] = *(const PW*)(p + e);
      gwq[i] = *(const PW*)(g + e);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t e = base + (int64_t(i) * kElemThreads + threadIdx.x) * VEC;
      float pv[VEC], gv[VEC];
      f32x4 mv = mvq[i], vv = vvq[i];
      if constexpr (sizeof(PT) == 2) {
        const u32x2 pw = pwq[i], gw = gwq[i];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          pv[2 * j] = bf2f(uint16_t(pw[j] & 0xffffu)); pv[2 * j + 1] = bf2f(uint16_t(pw[j] >> 16));
          gv[2 * j] = bf2f(uint16_t(gw[j] & 0xffffu)); gv[2 * j + 1] = bf2f(uint16_t(gw[j] >> 16));
        }
      } else {
        const f32x4 pw = pwq[i], gw = gwq[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) { pv[j] = pw[j]; gv[j] = gw[j]; }
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        float mj = mv[j], vj = vv[j];
        adam_elem(pv[j], gv[j], mj, vj, sc, keep);
        mv[j] = mj; vv[j] = vj;
      }
      *(f32x4*)(m + e) = mv;
      *(f32x4*)(v + e) = vv;
      if constexpr (sizeof(PT) == 2) {
        *(u32x2*)(p + e) = u32x2{f2bf2(pv[0], pv[1]), f2bf2(pv[2], pv[3])};
      } else {
        *(f32x4*)(p + e) = f32x4{pv[0], pv[1], pv[2], pv[3]};
      }
    }
    return;
  }
  for (int i = 0; i < int(kAdamChunk / kElemThreads); ++i) {
    const int64_t e = base + i * kElemThreads + threadIdx.x;
    if (e < n) {
      float pv = Elem<PT>::load(p + e), mv = m[e], vv = v[e];
      adam_elem(pv, Elem<PT>::load(g + e), mv, vv, sc, keep);
      m[e] = mv;
      v[e] = vv;
      Elem<PT>::store(p + e, pv);
    }
  }
}

}  // namespace

hipError_t run_adamw(const AdamTable& t, const AdamScalars& s, bool bf16, hipStream_t st) {
  const int blocks = t.first_block[t.n];
  if (blocks == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(adamw_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(kElemThreads), 0, st, t, s);
  else
    hipLaunchKernelGGL(adamw_kernel<float>, dim3(unsigned(blocks)), dim3(kElemThreads), 0, st, t, s);
  return hipGetLastError();
}

hipError_t run_shard_update(void* w, bool bf16, const float* o, int64_t len, float lr, float wd, float scale,
                            hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((len + kElemPerBlock - 1) / kElemPerBlock, 8192);
  const int vec = ((uintptr_t)w % 16 == 0) && ((uintptr_t)o % 16 == 0);
  if (bf16)
    hipLaunchKernelGGL(shard_update_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(kElemThreads), 0, st,
                       (uint16_t*)w, o, len, lr, wd, scale, vec);
  else
    hipLaunchKernelGGL(shard_update_kernel<float>, dim3(unsigned(blocks)), dim3(kElemThreads), 0, st, (float*)w, o,
                       len, lr, wd, scale, vec);
  return hipGetLastError();
}

}  // namespace muon
