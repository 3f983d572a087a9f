// Device-side helpers shared by the gfx950 kernels: bf16 rounding, MFMA
// operand types, wave reductions, and the per-matrix descriptor table that
// every launch receives by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNsEps = 1e-7f;   // added to ||U||_F before dividing

// Largest number of matrices one launch handles.  The per-matrix pointers
// travel in the kernel argument block (24 bytes each), so no host-to-device
// copy or device allocation is needed per call.
constexpr int kMaxChunk = 80;

struct MatRef {
  void* w;          // parameter (muon_step) or fp32 output O (muon_ns)
  const void* g;    // gradient (muon_step) or NS input (muon_ns)
  float* m;         // momentum (muon_step), unused by muon_ns
};

struct MatTable {
  MatRef e[kMaxChunk];
  uint8_t tr[kMaxChunk];  // 1 if the matrix is stored tall ([n][m]) and handled as its transpose
};

// Per-call scalars, identical for every matrix of the call.
struct StepScalars {
  float lr, mu, wd, scale;
  float a, b, c;
  int nesterov;
  int ns_steps;
  int mode;         // 0 = muon_step, 1 = muon_ns
};

// ---- bf16 <-> fp32 ---------------------------------------------------------
// fp32 -> bf16 uses the gfx950 hardware conversion (round to nearest even,
// NaN stays NaN): branch-free, one instruction per pair.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f2bf(v); }
};

// ---- wave / block reductions in a fixed order -----------------------------
__device__ __forceinline__ float wave_sum(float v) {
  // butterfly over 64 lanes; every lane ends with the same value and the
  // order of additions is fixed by the lane pattern
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over a 256-thread block in a fixed order; result valid in every thread.
__device__ __forceinline__ float block_sum_256(float v, float* lds4) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds4[wid] = v;
  __syncthreads();
  float r = (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
  return r;
}

// ---- raw buffer access ----------------------------------------------------
// A buffer resource bounds every access by its byte size: loads outside it
// return 0 and stores outside it are dropped.  An element index of kOob
// (times an element size of 2 or 4 bytes: 1 or 2 GiB) masks a lane without a
// branch for any buffer smaller than 1 GiB; kOobByte is the same mask as a
// byte offset (2 GiB), for accesses indexed in bytes whatever their width.
constexpr uint32_t kOob = 0x20000000u;
constexpr uint32_t kOobByte = 0x80000000u;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float buf_ld_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint16_t buf_ld_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st_f32(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st_u16(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_ld_b128(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st_b128(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// Hides a value from the optimiser so that an expression computed from it is
// not merged with an identical one far away (which would keep the result
// live, and spilled, in between).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u16x8& v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace muon
