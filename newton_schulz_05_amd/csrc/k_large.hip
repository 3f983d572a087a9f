// Kernels of the multi-launch path (bf16 MFMA for m > 32, and the fp32 path).
//
// Per chunk of matrices that share a wide shape (m <= n), with the workspace
// buffers X [mp][np] (row-major NS iterate), Xt [np][mp] (its transpose, two
// copies for ping-pong), A [mp][mp] fp32, and P:
//   momentum_kernel   M <- mu*M + G; U = G + mu*M (or M); writes U into X and
//                     Xt in the NS storage type and per-tile sums of U^2
//   norm_kernel       s = 1 / (||U||_F + eps) per matrix, fixed-order sum
//   gram (MFMA)       A = sc * X X^T on upper tiles (fp32, upper tiles only);
//                     H = bf16(A) and L = bf16(A - H) for the split A^2,
//                     mirrored to full matrices (they are GEMM operands)
//   poly (MFMA)       S = H H + H L + L H  (A^2 to ~16 mantissa bits), or
//                     S = H H in the first steps when m >= 512 (split_a2);
//                     P = ps * (a I + b A + c S); stores the off-diagonal part
//                     in bf16 and the diagonal in fp32
//   apply (MFMA)      X' = Poff Xt^T + diag(Pd) X; stores X' and X'^T in bf16,
//                     or on the last step O (fp32) or the weight update
// Wide bf16 groups (m >= 512, n >= 2 m) take several steps per Gram and
// apply (ns_group_bf16): between them, m x m products form T = P A and
// A' = P T (EpiSymMul) and R = P' R (EpiPairR), and the apply uses R.
// The fp32 path runs the same sequence with fp32 FMA tiles and a full fp32 P.
//
// The NS step itself (A = X X^T; X <- aX + (bA + cA^2)X) is Newton-Schulz on
// the momentum as in item 1(1) of the HyperParallel FSDP Muon optimizer RFC;
// batching matrices of one trailing shape in one launch is its item 3; the
// decoupled decay in the last epilogue is its item 6.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace muon {

// ============================================================================
// momentum + Nesterov + per-tile sum of squares + NS input in both layouts
// ============================================================================
// One 64x64 tile of the matrix in its stored orientation [rows][cols] per
// block; the grid covers the padded extent so that the padding of X and Xt is
// written with zeros.  The sum of squares of a tile that holds matrix
// elements goes to slot (r0 / 64) * ceil(cols / 64) + c0 / 64: the slots, and
// with them the order in which norm_kernel adds them, depend on the stored
// shape alone and not on the padding (which follows the GEMM tile, and so
// the group the matrix is in).  Tiles of padding only write no slot.
// With Xl and Xtl (bf16 muon_step), U is also split into hi + lo bf16
// planes, U ~ hi + lo to about 16 mantissa bits: X and Xt get hi, Xl and Xtl
// get lo = bf16(U - hi).
template <typename PT, typename XT>
__global__ __launch_bounds__(256) void momentum_kernel(MatTable tab, StepScalars sc, int tilesR,
                                                       int tilesC, XT* __restrict__ X,
                                                       XT* __restrict__ Xt0, XT* __restrict__ Xl,
                                                       XT* __restrict__ Xtl, int64_t xstride,
                                                       int64_t mp, int64_t np, int64_t m,
                                                       int64_t n, float* __restrict__ normpart,
                                                       int64_t tiles) {
  __shared__ float tileT[64][65];
  __shared__ float red[4];
  const int z = blockIdx.y;
  const bool tr = tab.tr[z] != 0;
  const int64_t rows = tr ? n : m, cols = tr ? m : n;        // stored shape
  const int64_t rowsP = tr ? np : mp, colsP = tr ? mp : np;  // padded stored shape
  const int tile = blockIdx.x;
  const int tC = tr ? tilesR : tilesC;                       // tiles per stored row
  const int64_t r0 = int64_t(tile / tC) * 64, c0 = int64_t(tile % tC) * 64;
  // norm slot of this tile, or -1 for a tile of padding only
  const int64_t slot = (r0 < rows && c0 < cols) ? (r0 / 64) * ((cols + 63) / 64) + c0 / 64 : -1;
  const int t = threadIdx.x;
  const int cg = t & 15, rg = t >> 4;
  const PT* G = (const PT*)tab.e[z].g;
  float* M = tab.e[z].m;
  XT* nat = (tr ? Xt0 : X) + int64_t(z) * xstride;  // same orientation as the stored matrix
  XT* trn = (tr ? X : Xt0) + int64_t(z) * xstride;  // transposed
  const bool lo = Xl != nullptr;
  XT* natl = lo ? (tr ? Xtl : Xl) + int64_t(z) * xstride : nullptr;
  XT* trnl = lo ? (tr ? Xl : Xtl) + int64_t(z) * xstride : nullptr;
  const int64_t ldn = colsP, ldt = rowsP;
  float ss = 0.f;
  // Vector path (bf16, tile inside the matrix, 16-byte aligned rows): thread
  // t moves 8 consecutive columns of rows t/8 and t/8 + 32 with 16-byte
  // accesses, and 8 consecutive rows of two transposed columns.
  if constexpr (sizeof(PT) == 2 && sizeof(XT) == 2) {
    if (sc.mode == 0 && cols % 8 == 0 && r0 + 64 <= rows && c0 + 64 <= cols) {
      const int cgrp = t & 7, rr = t >> 3;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int lr = rr + 32 * q;
        const int64_t idx = (r0 + lr) * cols + c0 + 8 * cgrp;
        const u32x4 gw = *(const u32x4*)(G + idx);
        f32x4 m0 = *(const f32x4*)(M + idx), m1 = *(const f32x4*)(M + idx + 4);
        float u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float g = bf2f(uint16_t((k & 1) ? (gw[k >> 1] >> 16) : (gw[k >> 1] & 0xffffu)));
          const float mo = (k < 4) ? m0[k] : m1[k - 4];
          const float mn = fmaf(sc.mu, mo, g);
          if (k < 4) m0[k] = mn; else m1[k - 4] = mn;
          u[k] = sc.nesterov ? fmaf(sc.mu, mn, g) : mn;
          ss = fmaf(u[k], u[k], ss);
        }
        *(f32x4*)(M + idx) = m0;
        *(f32x4*)(M + idx + 4) = m1;
        u32x4 xw;
#pragma unroll
        for (int d = 0; d < 4; ++d) xw[d] = f2bf2(u[2 * d], u[2 * d + 1]);
        *(u32x4*)(nat + (r0 + lr) * ldn + c0 + 8 * cgrp) = xw;
        if (lo) {
          u32x4 lw;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            lw[d] = f2bf2(u[2 * d] - bf2f(uint16_t(xw[d] & 0xffffu)), u[2 * d + 1] - bf2f(uint16_t(xw[d] >> 16)));
          *(u32x4*)(natl + (r0 + lr) * ldn + c0 + 8 * cgrp) = lw;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) tileT[lr][8 * cgrp + k] = u[k];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int lc = rr + 32 * q;
        float uv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) uv[k] = tileT[8 * cgrp + k][lc];
        u32x4 tw;
#pragma unroll
        for (int d = 0; d < 4; ++d) tw[d] = f2bf2(uv[2 * d], uv[2 * d + 1]);
        *(u32x4*)(trn + (c0 + lc) * ldt + r0 + 8 * cgrp) = tw;
        if (lo) {
          u32x4 lw;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            lw[d] = f2bf2(uv[2 * d] - bf2f(uint16_t(tw[d] & 0xffffu)), uv[2 * d + 1] - bf2f(uint16_t(tw[d] >> 16)));
          *(u32x4*)(trnl + (c0 + lc) * ldt + r0 + 8 * cgrp) = lw;
        }
      }
      const float tot = block_sum_256(ss, red);
      if (t == 0) normpart[int64_t(z) * tiles + slot] = tot;
      return;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lr = rg + 16 * q;
    const int64_t r = r0 + lr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lc = cg * 4 + j;
      const int64_t c = c0 + lc;
      float u = 0.f;
      if (r < rows && c < cols) {
        const int64_t idx = r * cols + c;
        const float g = Elem<PT>::load(G + idx);
        if (sc.mode == 0) {
          const float mn = fmaf(sc.mu, M[idx], g);
          M[idx] = mn;
          u = sc.nesterov ? fmaf(sc.mu, mn, g) : mn;
        } else {
          u = g;
        }
        ss = fmaf(u, u, ss);
      }
      // the value stored is what NS consumes (rounded to the storage type)
      XT xv;
      Elem<XT>::store(&xv, u);
      if (r < rowsP && c < colsP) {
        nat[r * ldn + c] = xv;
        if (lo) Elem<XT>::store(natl + r * ldn + c, u - Elem<XT>::load(&xv));
      }
      tileT[lr][lc] = u;
    }
  }
  __syncthreads();
  // transposed copy: row (c0 + lc) of trn, columns r0 .. r0+63
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int lc = rg + 16 * q;
    const int64_t c = c0 + lc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lr = cg * 4 + j;
      const int64_t r = r0 + lr;
      if (c < colsP && r < rowsP) {
        XT xv;
        const float u = tileT[lr][lc];
        Elem<XT>::store(&xv, u);
        trn[c * ldt + r] = xv;
        if (lo) Elem<XT>::store(trnl + c * ldt + r, u - Elem<XT>::load(&xv));
      }
    }
  }
  const float tot = block_sum_256(ss, red);
  if (t == 0 && slot >= 0) normpart[int64_t(z) * tiles + slot] = tot;
}

// s = 1 / (sqrt(sum of squares) + eps); scal[z] = {s, s^2, sumsq, 0}.
// `tiles` = ceil(m / 64) * ceil(n / 64) slots per matrix, added per thread in
// index order and then across threads in a fixed tree.
__global__ __launch_bounds__(256) void norm_kernel(const float* __restrict__ normpart, int64_t tiles,
                                                   float* __restrict__ scal) {
  __shared__ float red[4];
  const int z = blockIdx.x;
  const float* p = normpart + int64_t(z) * tiles;
  float v = 0.f;
  for (int64_t i = threadIdx.x; i < tiles; i += 256) v += p[i];
  const float tot = block_sum_256(v, red);
  if (threadIdx.x == 0) {
    const float s = 1.0f / (sqrtf(tot) + kNsEps);
    scal[z * 4 + 0] = s;
    scal[z * 4 + 1] = s * s;
    scal[z * 4 + 2] = tot;
    scal[z * 4 + 3] = 0.f;
  }
}

// ============================================================================
// Epilogues.
//
// bf16 MFMA path: the GEMM stages each 32 x 32 MFMA tile of the output
// through LDS and hands the epilogue runs of kRun = 8 consecutive elements,
// four lanes to a 32-element row of the tile and 16 rows per wave
// instruction:
//   row(z, i, j0, v[8], diag): C[i][j0 .. j0+7], which it may replace by
//       the final values (the column pass sees them), and
//   col(z, j, i0, v[8], diag): the final values C[i0 .. i0+7][j], for the
//       mirrored (symmetric outputs) or transposed (X^T, tall W) stores.
// So a bf16 store instruction writes 64 contiguous bytes of each of 16 rows.
// Measured on this GPU with a few workgroups writing 256 x 256 tiles (so
// that no shared bandwidth limits them), a CU stores 100-110 GB/s in that
// pattern against 58-65 GB/s with two lanes to a row (16 elements a lane,
// two 16-byte pieces 32 bytes apart per instruction), and fp32 runs of 16
// written that way only 31-35 GB/s.  `diag` is true on tiles on the diagonal of a symmetric
// output, where only i <= j is owned by the row pass and i < j is mirrored.
// Memory reads happen outside row() and col(), so that no read waits behind
// the stores of an earlier sub-tile (the vector memory counter retires loads
// and stores in issue order, so a wait for a load is a wait for every older
// store):
//   uni(z)                        the matrix's values (scale factors, the
//                                 stored orientation), once per tile before
//                                 any store;
//   fetch(u, z, i, j0, j, i0, in) the sub-tile's inputs (runs of the
//                                 operands, per-row values), issued one
//                                 sub-tile ahead.  Full runs are loaded even
//                                 on diagonal tiles; the entries below the
//                                 diagonal are not used.
// fp32 path: the GEMM hands a run of 4 consecutive rows (i0 .. i0+3) of one
// column j.
// ============================================================================

// elements per epilogue run
constexpr int kRun = 8;

// kRun consecutive elements; elements [k0, k1) are loaded / stored (the
// others of v are left alone), with 16-byte vectors when the run is whole
// and aligned.
template <typename T> struct Seg;
template <> struct Seg<float> {
  __device__ static __forceinline__ void load(const float* p, int k0, int k1, float* v) {
    if (k0 == 0 && k1 == kRun && ((uintptr_t)p & 15) == 0) {
#pragma unroll
      for (int q = 0; q < kRun / 4; ++q) {
        const f32x4 x = ((const f32x4*)p)[q];
        v[4 * q] = x[0]; v[4 * q + 1] = x[1]; v[4 * q + 2] = x[2]; v[4 * q + 3] = x[3];
      }
      return;
    }
    for (int k = k0; k < k1; ++k) v[k] = p[k];
  }
  __device__ static __forceinline__ void store(float* p, int k0, int k1, const float* v) {
    if (k0 == 0 && k1 == kRun && ((uintptr_t)p & 15) == 0) {
#pragma unroll
      for (int q = 0; q < kRun / 4; ++q) ((f32x4*)p)[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      return;
    }
    for (int k = k0; k < k1; ++k) p[k] = v[k];
  }
};
template <> struct Seg<uint16_t> {
  __device__ static __forceinline__ void load(const uint16_t* p, int k0, int k1, float* v) {
    if (k0 == 0 && k1 == kRun && ((uintptr_t)p & 15) == 0) {
#pragma unroll
      for (int q = 0; q < kRun / 8; ++q) {
        const u32x4 x = ((const u32x4*)p)[q];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          v[8 * q + 2 * d] = bf2f(uint16_t(x[d] & 0xffffu));
          v[8 * q + 2 * d + 1] = bf2f(uint16_t(x[d] >> 16));
        }
      }
      return;
    }
    for (int k = k0; k < k1; ++k) v[k] = bf2f(p[k]);
  }
  __device__ static __forceinline__ void store(uint16_t* p, int k0, int k1, const float* v) {
    if (k0 == 0 && k1 == kRun && ((uintptr_t)p & 15) == 0) {
#pragma unroll
      for (int q = 0; q < kRun / 8; ++q)
        ((u32x4*)p)[q] = u32x4{f2bf2(v[8 * q], v[8 * q + 1]), f2bf2(v[8 * q + 2], v[8 * q + 3]),
                               f2bf2(v[8 * q + 4], v[8 * q + 5]), f2bf2(v[8 * q + 6], v[8 * q + 7])};
      return;
    }
    for (int k = k0; k < k1; ++k) p[k] = f2bf(v[k]);
  }
};

__device__ __forceinline__ int clamp_run(int64_t x) { return x <= 0 ? 0 : (x >= kRun ? kRun : int(x)); }

// kRun consecutive elements held as loaded (16-byte vectors, not yet
// converted), so that an epilogue issues the loads of a sub-tile before the
// stores of the previous one and waits for them only where it uses them.
// The address must be 16-byte aligned.
template <typename T> struct Run;
template <> struct Run<float> {
  f32x4 q[kRun / 4];
  __device__ __forceinline__ void fetch(const float* p) {
#pragma unroll
    for (int k = 0; k < kRun / 4; ++k) q[k] = ((const f32x4*)p)[k];
  }
  __device__ __forceinline__ float operator[](int k) const { return q[k >> 2][k & 3]; }
};
template <> struct Run<uint16_t> {
  u32x4 q[kRun / 8];
  __device__ __forceinline__ void fetch(const uint16_t* p) {
#pragma unroll
    for (int k = 0; k < kRun / 8; ++k) q[k] = ((const u32x4*)p)[k];
  }
  __device__ __forceinline__ float operator[](int k) const {
    const uint32_t w = q[k >> 3][(k >> 1) & 3];
    return bf2f(uint16_t((k & 1) ? (w >> 16) : (w & 0xffffu)));
  }
};

struct NatStore {
  // store O (fp32) or apply the weight update at the matrix's stored position
  template <typename PT>
  __device__ static __forceinline__ void put(const MatRef& r, const StepScalars& sc, bool tr,
                                             int64_t m, int64_t n, int64_t i, int64_t j, float o) {
    if (i >= m || j >= n) return;
    const int64_t idx = tr ? (j * m + i) : (i * n + j);
    if (sc.mode == 1) {
      ((float*)r.w)[idx] = o;
    } else {
      PT* W = (PT*)r.w;
      const float w = Elem<PT>::load(W + idx);
      const float keep = 1.0f - sc.lr * sc.wd;
      Elem<PT>::store(W + idx, fmaf(-sc.lr * sc.scale, o, w * keep));
    }
  }
  // the same for `cnt` consecutive stored elements starting at idx0; `pre`,
  // when given, holds the kRun W values already loaded (cnt == kRun)
  template <typename PT>
  __device__ static __forceinline__ void put_seg(const MatRef& r, const StepScalars& sc, int64_t idx0, int cnt,
                                                 const float* o, const Run<PT>* pre = nullptr) {
    if (cnt <= 0) return;
    if (sc.mode == 1) {
      Seg<float>::store((float*)r.w + idx0, 0, cnt, o);
      return;
    }
    PT* W = (PT*)r.w + idx0;
    float w[kRun] = {};
    if (pre) {
#pragma unroll
      for (int k = 0; k < kRun; ++k) w[k] = (*pre)[k];
    } else {
      Seg<PT>::load(W, 0, cnt, w);
    }
    const float keep = 1.0f - sc.lr * sc.wd;
#pragma unroll
    for (int k = 0; k < kRun; ++k) w[k] = fmaf(-sc.lr * sc.scale, o[k], w[k] * keep);
    Seg<PT>::store(W, 0, cnt, w);
  }
};

// Gram (bf16 path): A = sc2 * acc as its bf16 hi/lo split H, L: H is a GEMM
// operand and so mirrored, L is written on the upper tiles and mirrored when
// A^2 takes the split products (with_lo).  The epilogues that read A at the
// same positions (the poly's b A, the d A of T = P A) take H + L, which
// holds A to about 16 mantissa bits.  Against an fp32 copy of A (and of T),
// in an emulation of the GPU's rounding points, the error of O was the same
// to two digits (lean recipe at 4096^2, precise at 1536 x 2048; rank m/8
// and log-spaced spectra), and the planes move a third fewer bytes.
struct EpiGramBf16 {
  uint16_t* H; uint16_t* L; const float* scal; int use_scale; int with_lo; int64_t mp;
  static constexpr bool kCol = true;
  struct Uni { float s2; };
  struct In {};
  __device__ __forceinline__ Uni uni(int z) const { return Uni{use_scale ? scal[z * 4 + 1] : 1.0f}; }
  __device__ __forceinline__ void fetch(const Uni&, int, int64_t, int64_t, int64_t, int64_t, In&) const {}
  __device__ __forceinline__ void row(const Uni& un, int z, int64_t i, int64_t j0, float* v, bool diag,
                                      const In&) const {
    const float s2 = un.s2;
    float lo[kRun];
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      v[k] *= s2;
      lo[k] = v[k] - bf2f(f2bf(v[k]));
    }
    const int k0 = diag ? clamp_run(i - j0) : 0;  // diagonal tiles: j >= i
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    Seg<uint16_t>::store(H + o, k0, kRun, v);
    Seg<uint16_t>::store(L + o, k0, kRun, lo);
  }
  __device__ __forceinline__ void col(const Uni&, int z, int64_t j, int64_t i0, const float* v, bool diag,
                                      const In&) const {
    float lo[kRun];
#pragma unroll
    for (int k = 0; k < kRun; ++k) lo[k] = v[k] - bf2f(f2bf(v[k]));
    const int k1 = diag ? clamp_run(j - i0) : kRun;  // diagonal tiles: mirror i < j only
    const int64_t o = int64_t(z) * mp * mp + j * mp + i0;
    Seg<uint16_t>::store(H + o, 0, k1, v);
    if (with_lo) Seg<uint16_t>::store(L + o, 0, k1, lo);
  }
};

// Poly (bf16 path): P = ps*(a I + b A + c S), A read as its planes AH + AL;
// off-diagonal bf16 (mirrored), with its lo part bf16(P - hi) in PoffL when
// given, diagonal fp32 in Pd
struct EpiPolyBf16 {
  const uint16_t* AH; const uint16_t* AL; uint16_t* Poff; uint16_t* PoffL; float* Pd;
  const float* scal; int use_scale; float a, b, c; int64_t mp, m;
  static constexpr bool kCol = true;
  struct Uni { float ps; };
  struct In { Run<uint16_t> h, l; };
  __device__ __forceinline__ Uni uni(int z) const { return Uni{use_scale ? scal[z * 4 + 0] : 1.0f}; }
  __device__ __forceinline__ void fetch(const Uni&, int z, int64_t i, int64_t j0, int64_t, int64_t, In& in) const {
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    in.h.fetch(AH + o);
    in.l.fetch(AL + o);
  }
  __device__ __forceinline__ void row(const Uni& un, int z, int64_t i, int64_t j0, float* v, bool diag,
                                      const In& in) const {
    const float ps = un.ps;
    const int k0 = diag ? clamp_run(i - j0) : 0;
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    float pv[kRun];
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      float p = fmaf(c, v[k], b * (in.h[k] + in.l[k]));
      if (i == j0 + k) {
        p = ps * (p + a);
        Pd[int64_t(z) * mp + i] = (i < m) ? p : 0.f;
        pv[k] = 0.f;
      } else {
        p = ps * p;
        pv[k] = p;
      }
      v[k] = p;
    }
    Seg<uint16_t>::store(Poff + o, k0, kRun, pv);
    if (PoffL) {
      float lo[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) lo[k] = pv[k] - bf2f(f2bf(pv[k]));
      Seg<uint16_t>::store(PoffL + o, k0, kRun, lo);
    }
  }
  __device__ __forceinline__ void col(const Uni&, int z, int64_t j, int64_t i0, const float* v, bool diag,
                                      const In&) const {
    const int k1 = diag ? clamp_run(j - i0) : kRun;
    const int64_t o = int64_t(z) * mp * mp + j * mp + i0;
    Seg<uint16_t>::store(Poff + o, 0, k1, v);
    if (PoffL) {
      float lo[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) lo[k] = v[k] - bf2f(f2bf(v[k]));
      Seg<uint16_t>::store(PoffL + o, 0, k1, lo);
    }
  }
};

// Grouped steps, m x m products of commuting symmetric matrices (bf16 path):
// C = acc + d[i] * S[i][j], with acc = Poff B^T from the GEMM, d the fp32
// diagonal of the left factor and S the right factor, read as its planes
// SH + SL (upper tiles).  Gives T = P_j A_j and A_{j+1} = P_j T.  C is
// stored as bf16 hi H, mirrored to a full matrix since it is a GEMM operand,
// and lo L on the upper tiles (mirrored when with_lo).
struct EpiSymMul {
  const uint16_t* SH; const uint16_t* SL; const float* d; uint16_t* H; uint16_t* L; int with_lo; int64_t mp;
  static constexpr bool kCol = true;
  struct Uni {};
  struct In { Run<uint16_t> h, l; float d; };
  __device__ __forceinline__ Uni uni(int) const { return Uni{}; }
  __device__ __forceinline__ void fetch(const Uni&, int z, int64_t i, int64_t j0, int64_t, int64_t, In& in) const {
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    in.h.fetch(SH + o);
    in.l.fetch(SL + o);
    in.d = d[int64_t(z) * mp + i];
  }
  __device__ __forceinline__ void row(const Uni&, int z, int64_t i, int64_t j0, float* v, bool diag,
                                      const In& in) const {
    const int k0 = diag ? clamp_run(i - j0) : 0;  // diagonal tiles: j >= i
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    float lo[kRun];
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      v[k] = fmaf(in.d, in.h[k] + in.l[k], v[k]);
      lo[k] = v[k] - bf2f(f2bf(v[k]));
    }
    Seg<uint16_t>::store(H + o, k0, kRun, v);
    Seg<uint16_t>::store(L + o, k0, kRun, lo);
  }
  __device__ __forceinline__ void col(const Uni&, int z, int64_t j, int64_t i0, const float* v, bool diag,
                                      const In&) const {
    const int k1 = diag ? clamp_run(j - i0) : kRun;  // diagonal tiles: mirror i < j only
    const int64_t o = int64_t(z) * mp * mp + j * mp + i0;
    Seg<uint16_t>::store(H + o, 0, k1, v);
    if (with_lo) {
      float lo[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) lo[k] = v[k] - bf2f(f2bf(v[k]));
      Seg<uint16_t>::store(L + o, 0, k1, lo);
    }
  }
};

// Grouped steps: R = ps * F1 F0 for two commuting symmetric factors stored as
// off-diagonal bf16 plus fp32 diagonal (F0 = Poff0 + diag(Pd0), the same for
// F1; with lo planes Poff0L / Poff1L the off-diagonals are hi + lo):
// acc = Poff1 Poff0^T from the GEMM, plus Pd1[i] Poff0[i][j] +
// Poff1[i][j] Pd0[j] + [i == j] Pd1[i] Pd0[i].  Off-diagonal R in bf16
// (mirrored; its lo part in RoffL when given), diagonal in fp32, the layout
// the apply and the next R take.  Lo: the factors may carry lo planes (the
// precise recipe), which the lean recipe's epilogue holds no registers for.
template <bool Lo>
struct EpiPairR {
  const uint16_t* Poff0; const uint16_t* Poff0L; const float* Pd0;
  const uint16_t* Poff1; const uint16_t* Poff1L; const float* Pd1;
  uint16_t* Roff; uint16_t* RoffL; float* Rd; const float* scal; int use_scale; int64_t mp;
  static constexpr bool kCol = true;
  // its inputs are too many registers to hold for two sub-tiles at once:
  // they are fetched just before their sub-tile
  static constexpr bool kAhead = false;
  struct Uni { float ps; };
  struct InH { Run<uint16_t> p0, p1; Run<float> d0; float d1; };
  struct InL : InH { Run<uint16_t> p0l, p1l; };
  using In = std::conditional_t<Lo, InL, InH>;
  __device__ __forceinline__ Uni uni(int z) const { return Uni{use_scale ? scal[z * 4 + 0] : 1.0f}; }
  __device__ __forceinline__ void fetch(const Uni&, int z, int64_t i, int64_t j0, int64_t, int64_t, In& in) const {
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    in.p0.fetch(Poff0 + o);
    in.p1.fetch(Poff1 + o);
    if constexpr (Lo) {
      if (Poff0L) in.p0l.fetch(Poff0L + o);
      if (Poff1L) in.p1l.fetch(Poff1L + o);
    }
    in.d0.fetch(Pd0 + int64_t(z) * mp + j0);
    in.d1 = Pd1[int64_t(z) * mp + i];
  }
  __device__ __forceinline__ void row(const Uni& un, int z, int64_t i, int64_t j0, float* v, bool diag,
                                      const In& in) const {
    const float ps = un.ps;
    const int k0 = diag ? clamp_run(i - j0) : 0;
    const int64_t o = int64_t(z) * mp * mp + i * mp + j0;
    float rv[kRun];
    const float d1 = in.d1;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      float p0 = in.p0[k], p1 = in.p1[k];
      if constexpr (Lo) {
        if (Poff0L) p0 += in.p0l[k];
        if (Poff1L) p1 += in.p1l[k];
      }
      const float d0 = in.d0[k];
      float r = fmaf(d1, p0, fmaf(p1, d0, v[k]));
      if (i == j0 + k) {
        r = ps * fmaf(d1, d0, r);
        Rd[int64_t(z) * mp + i] = r;
        rv[k] = 0.f;
      } else {
        r = ps * r;
        rv[k] = r;
      }
      v[k] = r;
    }
    Seg<uint16_t>::store(Roff + o, k0, kRun, rv);
    if (RoffL) {
      float lo[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) lo[k] = rv[k] - bf2f(f2bf(rv[k]));
      Seg<uint16_t>::store(RoffL + o, k0, kRun, lo);
    }
  }
  __device__ __forceinline__ void col(const Uni&, int z, int64_t j, int64_t i0, const float* v, bool diag,
                                      const In&) const {
    const int k1 = diag ? clamp_run(j - i0) : kRun;
    const int64_t o = int64_t(z) * mp * mp + j * mp + i0;
    Seg<uint16_t>::store(Roff + o, 0, k1, v);
    if (RoffL) {
      float lo[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) lo[k] = v[k] - bf2f(f2bf(v[k]));
      Seg<uint16_t>::store(RoffL + o, 0, k1, lo);
    }
  }
};

// Apply (bf16 path): X' = acc + Pd[i] * X[i][j] (X = hi + lo when Xl is
// given); X' and X'^T in bf16, or on the last step (Last) the weight update
// (O) at the stored position
template <typename PT, bool Last>
struct EpiApplyBf16 {
  MatTable tab; StepScalars sc; uint16_t* X; const uint16_t* Xl; uint16_t* XtN; const float* Pd;
  int64_t mp, np, m, n;
  static constexpr bool kCol = true;
  // the matrix's stored orientation and W; per run X's run (hi and lo
  // planes), Pd[i], and on the last step the W run the update reads (the row
  // run for a member stored as is, the column run for a transposed one) when
  // it is whole and 16-byte aligned (otherwise the update loads W itself)
  struct Uni { MatRef e; int tr; };
  struct InX { Run<uint16_t> x, xl; float d; };
  struct InW : InX { Run<PT> w; int64_t widx; int wcnt; bool wpre; };
  using In = std::conditional_t<Last, InW, InX>;
  __device__ __forceinline__ Uni uni(int z) const { return Uni{tab.e[z], tab.tr[z] != 0}; }
  __device__ __forceinline__ void fetch(const Uni& un, int z, int64_t i, int64_t j0, int64_t jc, int64_t ic,
                                        In& in) const {
    const int64_t o = int64_t(z) * mp * np + i * np + j0;
    in.x.fetch(X + o);
    if (Xl) in.xl.fetch(Xl + o);
    in.d = Pd[int64_t(z) * mp + i];
    if constexpr (Last) {
      if (!un.tr) {
        in.widx = i * n + j0;
        in.wcnt = (i < m) ? clamp_run(n - j0) : 0;
      } else {
        in.widx = jc * m + ic;
        in.wcnt = (jc < n) ? clamp_run(m - ic) : 0;
      }
      const PT* W = (const PT*)un.e.w + in.widx;
      in.wpre = sc.mode != 1 && in.wcnt == kRun && ((uintptr_t)W & 15) == 0;
      if (in.wpre) in.w.fetch(W);
    }
  }
  __device__ __forceinline__ void row(const Uni& un, int z, int64_t i, int64_t j0, float* v, bool,
                                      const In& in) const {
#pragma unroll
    for (int k = 0; k < kRun; ++k) v[k] = fmaf(in.d, Xl ? in.x[k] + in.xl[k] : in.x[k], v[k]);
    if constexpr (!Last) {
      Seg<uint16_t>::store(X + int64_t(z) * mp * np + i * np + j0, 0, kRun, v);
    } else {
      if (!un.tr) NatStore::put_seg<PT>(un.e, sc, in.widx, in.wcnt, v, in.wpre ? &in.w : nullptr);
    }
  }
  __device__ __forceinline__ void col(const Uni& un, int z, int64_t j, int64_t i0, const float* v, bool,
                                      const In& in) const {
    if constexpr (!Last) {
      Seg<uint16_t>::store(XtN + int64_t(z) * mp * np + j * mp + i0, 0, kRun, v);
    } else {
      if (un.tr) NatStore::put_seg<PT>(un.e, sc, in.widx, in.wcnt, v, in.wpre ? &in.w : nullptr);
    }
  }
};

// fp32 path epilogues
struct EpiGramF32 {
  float* A; const float* scal; int use_scale; int64_t mp;
  __device__ __forceinline__ void operator()(int z, int64_t i0, int64_t j, const float* v, bool diag) const {
    const float s2 = use_scale ? scal[z * 4 + 1] : 1.0f;
    const int64_t base = int64_t(z) * mp * mp;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + q;
      if (diag && i > j) continue;
      const float a = v[q] * s2;
      A[base + i * mp + j] = a;
      if (i != j) A[base + j * mp + i] = a;
    }
  }
};

struct EpiPolyF32 {
  const float* A; float* P; const float* scal; int use_scale; float a, b, c; int64_t mp, m;
  __device__ __forceinline__ void operator()(int z, int64_t i0, int64_t j, const float* v, bool diag) const {
    const float ps = use_scale ? scal[z * 4 + 0] : 1.0f;
    const int64_t base = int64_t(z) * mp * mp;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + q;
      if (diag && i > j) continue;
      float p = fmaf(c, v[q], b * A[base + i * mp + j]);
      if (i == j) p = (i < m) ? ps * (p + a) : 0.f; else p = ps * p;
      P[base + i * mp + j] = p;
      if (i != j) P[base + j * mp + i] = p;
    }
  }
};

template <typename PT>
struct EpiApplyF32 {
  MatTable tab; StepScalars sc; float* X; float* XtN;
  int64_t mp, np, m, n; int last;
  __device__ __forceinline__ void operator()(int z, int64_t i0, int64_t j, const float* v, bool) const {
    if (!last) {
      float* Xz = X + int64_t(z) * mp * np;
#pragma unroll
      for (int q = 0; q < 4; ++q) Xz[(i0 + q) * np + j] = v[q];
      *(f32x4*)(XtN + int64_t(z) * mp * np + j * mp + i0) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
      const bool tr = tab.tr[z] != 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) NatStore::put<PT>(tab.e[z], sc, tr, m, n, i0 + q, j, v[q]);
    }
  }
};

// ============================================================================
// Tile scheduling: full grid or upper triangle (symmetric outputs)
// ============================================================================
__device__ __forceinline__ void tile_coords(int t, int T, bool upper, int& ti, int& tj) {
  if (!upper) { ti = t / T; tj = t % T; return; }
  int r = 0, len = T;
  while (t >= len) { t -= len; ++r; --len; }
  ti = r; tj = r + t;
}

// Workgroup b of a launch of N runs on XCD b mod 8, and each XCD takes its
// workgroups in order.  Work item of b: each XCD gets a contiguous range of
// the items (the last N mod 8 workgroups take the items left over), so the
// items an XCD runs together are neighbours and share operand blocks in its
// L2.  With the grouped tile orders below, the 8192 x 28672 pair's step
// went from 53.5 to 52.2 ms and the MoE experts' from 3.37 to 2.96 ms.
__device__ __forceinline__ int xcd_item(int b, int N) {
  const int nx = N >> 3;
  return (b < 8 * nx) ? (b & 7) * nx + (b >> 3) : b;
}
// Tile (ti, tj) of item t of a Tm x Tn grid in column-major groups of kGM
// tile rows: the tiles that run together share kGM row blocks of A and a
// few column blocks of B.
constexpr int kGM = 4;
__device__ __forceinline__ void grouped_coords(int t, int Tm, int Tn, int& ti, int& tj) {
  const int g = t / (kGM * Tn), w = t - g * (kGM * Tn);
  const int gm = (Tm - g * kGM < kGM) ? Tm - g * kGM : kGM;
  ti = g * kGM + w % gm;
  tj = w / gm;
}
// The same for the upper triangle (i <= j) of a T x T grid: groups of kGM
// tile rows r0 .. r0+gm-1, each taken column by column from j = r0 (the
// first gm - 1 columns hold 1, 2, .. gm - 1 tiles of the group).
__device__ __forceinline__ void grouped_upper_coords(int t, int T, int& ti, int& tj) {
  int r0 = 0;
  for (;;) {
    const int gm = (T - r0 < kGM) ? T - r0 : kGM;
    const int size = gm * (T - r0) - gm * (gm - 1) / 2;
    if (t < size) {
      const int tri = gm * (gm - 1) / 2;
      if (t < tri) {
        int jj = 0;
        while ((jj + 1) * (jj + 2) / 2 <= t) ++jj;
        ti = r0 + (t - jj * (jj + 1) / 2);
        tj = r0 + jj;
      } else {
        const int w = t - tri;
        ti = r0 + w % gm;
        tj = r0 + gm - 1 + w / gm;
      }
      return;
    }
    t -= size;
    r0 += gm;
  }
}

// ============================================================================
// bf16 MFMA GEMM, "NT": C[i][j] = sum_k A[i][k] * B[j][k] (+ split products)
// A, B row-major with k contiguous; all dims padded to the tile size.
//
// TILE x TILE output tile per block: 256 -> 8 waves (2 x 4) of 128 x 64,
// 128 -> 4 waves (2 x 2) of 64 x 64, 64 -> 4 waves of 32 x 32 (only for the
// partial last round of a 128-tile grid); 32x32x16 MFMAs.  Operand tiles go from
// global memory straight into LDS (buffer loads with the LDS destination, 16
// bytes a lane), two stages, so no VGPRs are spent on staging; each lane's
// address is one 32-bit offset per operand plane, the row and k of a load
// in its scalar offset (with 64-bit addresses per load the compiler kept 16
// pointers per lane live and strength-reduced them every k-tile).  Against
// global_load_lds with per-load 64-bit addresses and a loop with a branch per
// k-tile: the 8192 x 28672 pair 53.5 -> 50.9 ms, the mixed 32-layer set
// 635 -> 615 ms, the MoE slab 3.00 -> 2.66 ms (same box, bitwise identical).  Each 16-byte chunk of a row
// sits at chunk index (c ^ g(row)) so that the fragment reads (32 rows x 2
// chunks per instruction) hit distinct banks:
//   BK = 64 (8 chunks a row): g(r) = (r & 7) ^ ((r >> 3) & 3)
//   BK = 32 (4 chunks a row): g(r) = ((r >> 1) ^ (r >> 3)) & 3
// PR selects the products (operands given as bf16 hi planes Ah, Bh and, for
// the split products, lo planes Al, Bl with A ~ Ah + Al, B ~ Bh + Bl):
//   kHH = 1: Ah Bh^T       kHL = 2: Ah Bl^T       kLH = 4: Al Bh^T
// always with kHH; per k slice the products are taken in the order HH, HL,
// LH.  One plane per side (PR = kHH) uses BK = 64; with a lo plane on either
// side BK = 32, so the LDS footprint of the three or four planes stays within
// that of two at BK = 64.
constexpr int kHH = 1, kHL = 2, kLH = 4;

// whether an epilogue's inputs are fetched one sub-tile ahead (the default)
// or just before their run (Epi::kAhead = false: inputs used by the row
// pass only)
template <typename Epi, typename = void> struct EpiAhead { static constexpr bool value = true; };
template <typename Epi> struct EpiAhead<Epi, decltype(void(Epi::kAhead))> { static constexpr bool value = Epi::kAhead; };

template <int TILE>
struct GemmGeom {
  static constexpr int NT = (TILE == 256) ? 512 : 256;
  static constexpr int WN = (TILE == 256) ? 4 : 2;
  static constexpr int WM = 2;
  static constexpr int TMW = TILE / WM, TNW = TILE / WN;
  static constexpr int FM = TMW / 32, FN = TNW / 32;
  // co-resident workgroups per CU (LDS: 128 KB, 64 KB, 32 KB per workgroup)
  static constexpr int PER_CU = (TILE == 256) ? 1 : (TILE == 128) ? 2 : 4;
};

// 16 bytes per lane from a buffer resource into LDS: lane l reads
// voff + soff and writes lds_base + 16 l
__device__ __forceinline__ void dma16_buf(rsrc_t r, u16x8* lds_base, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, int(voff), soff, 0, 0);
}

template <int CPR>
__device__ __forceinline__ int chunk_swz(int row) {
  if constexpr (CPR == 8) return (row & 7) ^ ((row >> 3) & 3);
  else return ((row >> 1) ^ (row >> 3)) & 3;
}

template <int TILE, int PR, typename Epi>
__global__ __launch_bounds__(GemmGeom<TILE>::NT, GemmGeom<TILE>::PER_CU) void gemm_bf16_kernel(
    const uint16_t* __restrict__ Ah, const uint16_t* __restrict__ Al, int64_t lda, int64_t sA,
    const uint16_t* __restrict__ Bh, const uint16_t* __restrict__ Bl, int64_t ldb, int64_t sB,
    int64_t K, int tilesN, int upper, int per, int base, int split, int nwork, Epi epi) {
  using G = GemmGeom<TILE>;
  constexpr int NA = (PR & kLH) ? 2 : 1;        // A planes
  constexpr int NB = (PR & kHL) ? 2 : 1;        // B planes
  constexpr int NPL = NA + NB;
  constexpr int BK = (NPL > 2) ? 32 : 64;
  constexpr int CPR = BK / 8;                   // 16-byte chunks per row
  constexpr int PLANE = TILE * CPR;             // chunks per operand plane
  constexpr int NW = G::NT / 64;
  constexpr int LP = PLANE / G::NT;             // loads per thread per plane
  constexpr int KS = BK / 16;
  // three planes at BK = 32 (the applies with a lo plane on one side) take a
  // ring of three stages, 144 KB; two or four planes two stages, 128 KB
  constexpr int NST = (NPL == 3 && TILE == 256) ? 3 : 2;
  __shared__ u16x8 lds[NST][NPL][PLANE];        // [stage][Ah, (Al), Bh, (Bl)]
  // Work items w = blockIdx.x, blockIdx.x + gridDim.x, ... < nwork: a full
  // grid stays resident (one round of workgroups) and each workgroup takes
  // its next tile after its epilogue, so the rounds of the CUs drift apart
  // instead of each waiting for the slowest CU (the mixed 32-layer set
  // 601 -> 592 ms, same box).  A split launch has one item per workgroup.
  for (int w = int(blockIdx.x); w < nwork; w += int(gridDim.x)) {
  // Work item f = matrix * per + tile, in units of the tiles that tilesN
  // counts, tiles in the grouped order (which only decides which workgroup
  // computes a tile, never how).  With split, each such tile (twice TILE on a
  // side) is done by four workgroups, one per TILE-quarter; a symmetric
  // output skips the quarter below the diagonal.
  const int f = base + (split ? (w >> 2) : xcd_item(w, nwork));
  const int z = __builtin_amdgcn_readfirstlane(f / per);
  int ti, tj;
  if (upper) grouped_upper_coords(f - z * per, tilesN, ti, tj);
  else grouped_coords(f - z * per, per / tilesN, tilesN, ti, tj);
  if (split) {
    const int q = int(blockIdx.x & 3);
    ti = 2 * ti + (q >> 1);
    tj = 2 * tj + (q & 1);
    if (upper && ti > tj) continue;
  }
  const int64_t row0 = int64_t(ti) * TILE, col0 = int64_t(tj) * TILE;
  // the thread's lane terms are recomputed per tile (an opaque copy of the
  // thread index), so no per-lane value is held across the epilogue
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  const int lane = t & 63, wv = t >> 6;
  const int wr = (wv / G::WN) * G::TMW, wc = (wv % G::WN) * G::TNW;

  const uint16_t* gsrc[NPL];
  gsrc[0] = Ah + int64_t(z) * sA + row0 * lda;
  gsrc[NA] = Bh + int64_t(z) * sB + col0 * ldb;
  if constexpr (NA == 2) gsrc[1] = Al + int64_t(z) * sA + row0 * lda;
  if constexpr (NB == 2) gsrc[NA + 1] = Bl + int64_t(z) * sB + col0 * ldb;

  f32x16 acc[G::FM][G::FN];
#pragma unroll
  for (int a = 0; a < G::FM; ++a)
#pragma unroll
    for (int b = 0; b < G::FN; ++b) acc[a][b] = f32x16{};

  // wave w's p-th load of a plane fills chunks [(p*NW + w)*64, +64): lane l
  // takes chunk c = (p*NW + w)*64 + l, i.e. row c / CPR, stored position
  // c % CPR, which holds logical chunk (c % CPR) ^ g(row)
  // Lane l of wave w's p-th load of a plane moves row RL (p NW + w) + l / CPR
  // (RL = 64 / CPR rows per load) and stored chunk l % CPR, which holds
  // logical chunk (l % CPR) ^ g(row); g(row) does not depend on p (NW is a
  // multiple of 4), so a lane's byte offset within the load's rows is the
  // same for all its loads of a plane.  The loads go through buffer
  // resources over the tile's rows: one 32-bit lane offset per plane, the
  // load's row and k in the scalar offset.
  constexpr int RL = 64 / CPR;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  rsrc_t rs[NPL];
#pragma unroll
  for (int s = 0; s < NPL; ++s) rs[s] = make_rsrc(gsrc[s], uint32_t(TILE * ((s < NA) ? lda : ldb) * 2));
  uint32_t voff[2];
  {
    const int r0 = wvu * RL + lane / CPR;  // row of load 0
    const int ch = (lane % CPR) ^ chunk_swz<CPR>(r0);
    voff[0] = uint32_t(((lane / CPR) * lda + ch * 8) * 2);
    voff[1] = uint32_t(((lane / CPR) * ldb + ch * 8) * 2);
  }
  auto gload = [&](int64_t k0, int st) {
#pragma unroll
    for (int s = 0; s < NPL; ++s) {
      const int64_t ld = (s < NA) ? lda : ldb;
#pragma unroll
      for (int p = 0; p < LP; ++p) {
        const int soff = int((int64_t((p * NW + wvu) * RL) * ld + k0) * 2);
        dma16_buf(rs[s], &lds[st][s][(p * NW + wvu) * 64], voff[s < NA ? 0 : 1], soff);
      }
    }
  };
  bf16x8 fa[2][NA][G::FM], fb[2][NB][G::FN];
  auto lread = [&](int st, int ks, int buf) {
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int s = 0; s < NA; ++s) {
#pragma unroll
      for (int x = 0; x < G::FM; ++x) {
        const int r = wr + x * 32 + (lane & 31);
        fa[buf][s][x] = as_bf16x8(lds[st][s][r * CPR + (ch ^ chunk_swz<CPR>(r))]);
      }
    }
#pragma unroll
    for (int s = 0; s < NB; ++s) {
#pragma unroll
      for (int x = 0; x < G::FN; ++x) {
        const int r = wc + x * 32 + (lane & 31);
        fb[buf][s][x] = as_bf16x8(lds[st][NA + s][r * CPR + (ch ^ chunk_swz<CPR>(r))]);
      }
    }
  };
  auto mfma_slice = [&](int q, int a0, int a1) {
#pragma unroll
    for (int a = a0; a < a1; ++a)
#pragma unroll
      for (int b = 0; b < G::FN; ++b) {
        acc[a][b] = mfma32x32x16(fa[q][0][a], fb[q][0][b], acc[a][b]);
        if constexpr ((PR & kHL) != 0) acc[a][b] = mfma32x32x16(fa[q][0][a], fb[q][NB - 1][b], acc[a][b]);
        if constexpr ((PR & kLH) != 0) acc[a][b] = mfma32x32x16(fa[q][NA - 1][a], fb[q][0][b], acc[a][b]);
      }
  };
  // a k-tile in stage st: all its fragment reads and three quarters of its
  // MFMAs (head), then the last quarter from registers (tail): the last k
  // slice when there are 4, the second half of the last slice's rows of
  // MFMA tiles when there are 2
  constexpr int TA = (KS >= 4) ? 0 : G::FM / 2;
  auto head = [&](int st) {
    lread(st, 0, 0);
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      lread(st, ks + 1, (ks + 1) & 1);
      mfma_slice(ks & 1, 0, G::FM);
    }
    mfma_slice((KS - 1) & 1, 0, TA);
  };
  auto tail = [&]() { mfma_slice((KS - 1) & 1, TA, G::FM); };
  // stage st's loads have landed and every wave has read the other stage
  auto stage_sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Two stages: the loads of k-tile t+1 fly while k-tile t is multiplied.
  // A quarter of each k-tile's MFMAs is issued after the barrier that frees
  // its stage, once the next loads into that stage are issued, so the waves
  // have MFMAs to issue while those loads start (the order of the products
  // into each accumulator is unchanged).  The scheduling barriers fix this
  // order: left to itself the compiler moved a varying share of a stage's
  // MFMAs below the wait, up to all of them in one build of the three-plane
  // apply (10% slower); none (every MFMA before the wait) was 1-2% slower
  // than its own choice, a quarter 3-10% faster on the single-product
  // launches and the same on the three-product ones.  KT is even (K is a multiple of 128): the loop body
  // is straight-line code over a pair of k-tiles, the last pair peeled.
  const int KT = int(K / BK);
  if constexpr (NST == 3) {
    // Three stages: the loads of k-tiles t+1 and t+2 fly while k-tile t is
    // multiplied, so a load has two k-tiles' MFMAs (~2 us) to arrive instead
    // of one (the three-plane apply of the 8192 x 28672 pair 13.2 -> 12.5 ms,
    // bitwise identical).  The loads are written as inline asm (M0 = the
    // LDS destination, then the buffer load with the lds modifier; no
    // register is written, so nothing of the asm's stays live) and waited
    // for with explicit vmcnt counts: issued through the builtin, the
    // compiler would wait for every load in flight before each barrier and
    // before every fragment read of another stage, which undoes the ring.
    // No other vector memory access is issued in this loop, and the last
    // wait is vmcnt(0), so the compiler's own counts stay valid after it.
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    i32x4_t rv[NPL];
#pragma unroll
    for (int s = 0; s < NPL; ++s) {
      const uint64_t ga = (uint64_t)(uintptr_t)gsrc[s];
      rv[s] = i32x4_t{int(__builtin_amdgcn_readfirstlane(uint32_t(ga))),
                      int(__builtin_amdgcn_readfirstlane(uint32_t(ga >> 32) & 0xffffu)),
                      int(uint32_t(TILE * ((s < NA) ? lda : ldb) * 2)), 0x00020000};
    }
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(
        uint32_t((uintptr_t)(__attribute__((address_space(3))) u16x8*)(&lds[0][0][0])));
    constexpr int NL = NPL * LP;  // loads per k-tile and thread
    auto gload3 = [&](int64_t k0, int st) {
#pragma unroll
      for (int s = 0; s < NPL; ++s) {
        const int64_t ld = (s < NA) ? lda : ldb;
#pragma unroll
        for (int p = 0; p < LP; ++p) {
          const int soff = __builtin_amdgcn_readfirstlane(int((int64_t((p * NW + wvu) * RL) * ld + k0) * 2));
          const uint32_t m0v = lbase + uint32_t(((st * NPL + s) * PLANE + (p * NW + wvu) * 64) * 16);
          // M0 is declared clobbered; these kernels use it nowhere else (the
          // compiler warns that a reserved register is not preserved)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                       :: "s"(m0v), "v"(voff[s < NA ? 0 : 1]), "s"(rv[s]), "s"(soff) : "memory", "m0");
#pragma clang diagnostic pop
        }
      }
    };
    auto bar3 = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    gload3(0, 0);
    gload3(BK, 1);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NL) : "memory");  // k-tile 0 in stage 0
    bar3();
    gload3(2 * BK, 2);
    head(0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NL) : "memory");  // k-tile 1 in stage 1
    bar3();
    int sr = 1, sd = 0;
    for (int kt = 1; kt + 2 < KT; ++kt) {
      gload3(int64_t(kt + 2) * BK, sd);   // into the stage k-tile kt - 1 used
      tail();                             // k-tile kt - 1
      head(sr);                           // k-tile kt
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NL) : "memory");  // k-tile kt + 1 landed
      bar3();
      sr = (sr == 2) ? 0 : sr + 1;
      sd = (sd == 2) ? 0 : sd + 1;
    }
    tail();                               // k-tile KT - 3
    head(sr);                             // k-tile KT - 2
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bar3();
    sr = (sr == 2) ? 0 : sr + 1;
    tail();
    head(sr);                             // k-tile KT - 1
    tail();
  } else {
  gload(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  gload(BK, 1);
  head(0);
  for (int kt = 0; kt + 2 < KT; kt += 2) {
    stage_sync();                     // k-tile kt + 1 in stage 1
    gload(int64_t(kt + 2) * BK, 0);
    tail();                           // k-tile kt
    head(1);                          // k-tile kt + 1
    stage_sync();                     // k-tile kt + 2 in stage 0
    gload(int64_t(kt + 3) * BK, 1);
    tail();                           // k-tile kt + 1
    head(0);                          // k-tile kt + 2
  }
  stage_sync();                       // k-tile KT - 1 in stage 1
  tail();                             // k-tile KT - 2
  head(1);                            // k-tile KT - 1
  tail();
  }

  // Epilogue: each wave stages one 32 x 32 MFMA tile at a time in its own LDS
  // slot (the operand stages are free now) and reads it back as row runs and
  // column runs of kRun elements: lane l takes rows (l / 4) and (l / 4) + 16,
  // columns kRun (l % 4) .. (the column pass the same with rows and columns
  // exchanged).
  __syncthreads();
  constexpr int kLd = 36;  // slot row stride in floats
  constexpr int kLpr = 32 / kRun;        // lanes per row of the sub-tile
  constexpr int kRH = 64 / kLpr;         // rows per wave instruction (16)
  float* slot = reinterpret_cast<float*>(&lds[0][0][0]) + wv * (32 * kLd);
  const bool diag = upper && (ti == tj);
  const int er = lane / kLpr, ec = (lane % kLpr) * kRun;
  // the matrix's values once, then the wave's MFMA tiles in order, each
  // one's inputs (two runs a lane) fetched one tile ahead
  const typename Epi::Uni un = epi.uni(z);
  constexpr int NTL = G::FM * G::FN;
  typename Epi::In in[2][2];
  auto fetch = [&](int u, typename Epi::In* dst) {
    const int64_t ti0 = row0 + wr + (u / G::FN) * 32, tj0 = col0 + wc + (u % G::FN) * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      epi.fetch(un, z, ti0 + er + h * kRH, tj0 + ec, tj0 + er + h * kRH, ti0 + ec, dst[h]);
  };
  constexpr bool ahead = EpiAhead<Epi>::value;
  if (ahead) fetch(0, in[0]);
#pragma unroll
  for (int u = 0; u < NTL; ++u) {
    if (ahead && u + 1 < NTL) fetch(u + 1, in[(u + 1) & 1]);
    const int a = u / G::FN, b = u % G::FN;
    const int64_t ti0 = row0 + wr + a * 32, tj0 = col0 + wc + b * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) slot[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * kLd + (lane & 31)] = acc[a][b][r];
    float v[2][kRun];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // inputs fetched just before their run (the row pass is their only user)
      if (!ahead) epi.fetch(un, z, ti0 + er + h * kRH, tj0 + ec, tj0 + er + h * kRH, ti0 + ec, in[u & 1][h]);
#pragma unroll
      for (int k = 0; k < kRun; ++k) v[h][k] = slot[(er + h * kRH) * kLd + ec + k];
      epi.row(un, z, ti0 + er + h * kRH, tj0 + ec, v[h], diag, in[u & 1][h]);
    }
    if constexpr (Epi::kCol) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kRun; ++k) slot[(er + h * kRH) * kLd + ec + k] = v[h][k];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int k = 0; k < kRun; ++k) v[h][k] = slot[(ec + k) * kLd + er + h * kRH];
        epi.col(un, z, tj0 + er + h * kRH, ti0 + ec, v[h], diag, in[u & 1][h]);
      }
    }
  }
  __syncthreads();  // the staging slots overlap the next tile's first stage
  }
}

// ============================================================================
// fp32 FMA GEMM, NT, 64x64 tile, BK = 16, 256 threads with 4x4 outputs each
// ============================================================================
constexpr int GF_M = 64, GF_K = 16;

template <typename Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       int64_t sA, const float* __restrict__ B,
                                                       int64_t ldb, int64_t sB, int64_t K,
                                                       int tilesN, int upper, Epi epi) {
  __shared__ float As[GF_K][GF_M + 4];
  __shared__ float Bs[GF_K][GF_M + 4];
  const int z = blockIdx.y;
  int ti, tj;
  tile_coords(blockIdx.x, tilesN, upper != 0, ti, tj);
  const int64_t row0 = int64_t(ti) * GF_M, col0 = int64_t(tj) * GF_M;
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const float* gA = A + int64_t(z) * sA + row0 * lda;
  const float* gB = B + int64_t(z) * sB + col0 * ldb;
  float acc[4][4] = {};
  const int lr = t >> 2, lk = (t & 3) * 4;
  for (int64_t k0 = 0; k0 < K; k0 += GF_K) {
    const f32x4 va = *(const f32x4*)(gA + int64_t(lr) * lda + k0 + lk);
    const f32x4 vb = *(const f32x4*)(gB + int64_t(lr) * ldb + k0 + lk);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) { As[lk + q][lr] = va[q]; Bs[lk + q][lr] = vb[q]; }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < GF_K; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) { a[q] = As[k][ty * 4 + q]; b[q] = Bs[k][tx * 4 + q]; }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(a[x], b[y], acc[x][y]);
    }
  }
  const bool diag = upper && (ti == tj);
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    float v[4] = {acc[0][y], acc[1][y], acc[2][y], acc[3][y]};
    epi(z, row0 + ty * 4, col0 + tx * 4 + y, v, diag);
  }
}

// ============================================================================
// ns_steps == 0: O = s * U taken from X, then the store / update
// ============================================================================
template <typename PT, typename XT>
__global__ __launch_bounds__(256) void ns0_kernel(MatTable tab, StepScalars sc, const XT* __restrict__ X,
                                                  const XT* __restrict__ Xl, int64_t mp, int64_t np, int64_t m,
                                                  int64_t n, const float* __restrict__ scal) {
  const int z = blockIdx.y;
  const bool tr = tab.tr[z] != 0;
  const float s = scal[z * 4 + 0];
  const XT* Xz = X + int64_t(z) * mp * np;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < m * n; e += int64_t(gridDim.x) * 256) {
    const int64_t i = e / n, j = e % n;
    float u = Elem<XT>::load(Xz + i * np + j);
    if (Xl) u += Elem<XT>::load(Xl + int64_t(z) * mp * np + i * np + j);
    NatStore::put<PT>(tab.e[z], sc, tr, m, n, i, j, s * u);
  }
}

// ============================================================================
// Host launchers
// ============================================================================
static hipError_t last_launch() { return hipGetLastError(); }

// One batched bf16 GEMM launch over `per` tiles of each of `count` matrices.
// A grid runs in rounds of PER_CU workgroups per CU: the main launch is one
// resident round of workgroups that take the full rounds' tiles in turn.
// When the last round is partial, its tiles run in a second launch at half
// the tile size, four workgroups per tile (three on the diagonal of a
// symmetric output), so that round costs a fraction of a full one on an
// otherwise idle chip.  Tile size changes no bit of the result.
template <int TILE, int PR, typename Epi>
static hipError_t gemm_launch(const uint16_t* Ah, const uint16_t* Al, int64_t lda, int64_t sA, const uint16_t* Bh,
                              const uint16_t* Bl, int64_t ldb, int64_t sB, int64_t K, int tilesN, int upper, int per,
                              int count, int cus, const Epi& epi, hipStream_t st) {
  if (K % 128 != 0) return hipErrorInvalidValue;  // the main loop takes k-tiles in pairs
  const int total = per * count;
  const int round = cus * GemmGeom<TILE>::PER_CU;
  const int main = (cus > 0 && total > round) ? total - total % round : total;
  const int grid = (cus > 0 && main > round) ? round : main;
  hipLaunchKernelGGL((gemm_bf16_kernel<TILE, PR, Epi>), dim3(unsigned(grid)), dim3(GemmGeom<TILE>::NT), 0, st,
                     Ah, Al, lda, sA, Bh, Bl, ldb, sB, K, tilesN, upper, per, 0, 0, main, epi);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (main == total) return hipSuccess;
  constexpr int SUB = TILE / 2;
  hipLaunchKernelGGL((gemm_bf16_kernel<SUB, PR, Epi>), dim3(unsigned(4 * (total - main))),
                     dim3(GemmGeom<SUB>::NT), 0, st, Ah, Al, lda, sA, Bh, Bl, ldb, sB, K, tilesN, upper, per, main, 1,
                     4 * (total - main), epi);
  return hipGetLastError();
}

// A^2 takes the single product H H in the first NS steps and the split-bf16
// products (H H + H L + L H, about 16 mantissa bits of A) after them: the
// single product is taken in steps k < min(kPlainSteps, ns_steps - 2) for
// m >= kPlain3FromM, in steps k < min(kPlainStepsMid, ns_steps - 2) for
// kPlainMinM <= m < kPlain3FromM, and never for smaller m.  NS pulls every singular value towards
// its fixed band and damps a perturbation of P on the way there; once the
// bulk of the normalised singular values (about 1/sqrt(m) at the start, times
// up to a = 3.4445 per step) has reached the band, the rounding of A shows in
// O.  In an emulation of this recipe on Gaussian inputs with the quintic
// coefficients, the single product in steps 0-2 moved the relative Frobenius
// error of O by under 3% of itself at 512^2, 1024^2, 512 x 1024 and
// 1024 x 3584 for 4 to 7 steps (6.89e-3 -> 6.92e-3 at 512^2 and 5 steps;
// inputs with singular values spread over 1e-1 .. 1e-4 the same), while a
// single product in step 3 (of 5 or 6) or in the last step raised it by
// 15-240%; at m = 33 .. 130 step 2 already counts (5.6e-3 -> 8.4e-3 at
// 130 x 200).  Inputs of low rank or with spectra over three decades, in
// the grouped precise recipe, need step 2 split below m = 1536: emulated
// (and on the GPU to three digits) for 5 steps, rank m/8 gave 3.4e-2 with
// a single product in step 2 against 6.5e-3 split at 512 x 1024, 1.5e-2
// against 6.0e-3 at 768 x 1024, 9.5e-3 against 6.4e-3 at 1024^2, 7.4e-3
// against 6.0e-3 at 1280 x 2048, 6.5e-3 against 5.8e-3 at 1536 x 2048; and
// singular values log-spaced over [1e-3, 1] 1.0e-2 against 3.5e-3 at
// 512 x 1024.
constexpr int kPlainSteps = 3;
constexpr int kPlainStepsMid = 2;
constexpr int64_t kPlainMinM = 512;
constexpr int64_t kPlain3FromM = 1536;

static inline bool split_a2(int64_t m, int k, int steps) {
  if (m < kPlainMinM) return true;
  return k >= std::min(m >= kPlain3FromM ? kPlainSteps : kPlainStepsMid, steps - 2);
}

// A group of G >= 1 consecutive NS steps k .. k+G-1 of the bf16 path, with
// one Gram and one apply.  Every P_j, A_j and product below is a polynomial
// in A_k, so they commute and the products are symmetric (upper tiles,
// mirrored).  For j = 0 .. G-1:
//   j = 0   Gram  A_0 = sc X X^T                  -> H, L
//           poly  P_0 = a I + b A_0 + c A_0^2     -> Pb[0] (scaled by s only
//                 when G = 1 and k = 0)
//   j >= 1  T     T = P_{j-1} A_{j-1}             -> Th, Tl
//           A'    A_j = P_{j-1} T                 -> H, L
//           poly  P_j from A_j                    -> Pb[j % 2]
//           R     R_j = P_j R_{j-1}, R_0 = s P_0  -> Rb[j % 2] (off-diagonal
//                 bf16, diagonal fp32; s only when k = 0)
//   apply   X_{k+G} = Roff Xt^T + diag(Rd) X with R = R_{G-1} (P_0 when G = 1)
// A_j = X_{k+j} X_{k+j}^T in exact arithmetic, so this is the oracle's
// iteration with one m x n product pair per group.
//
// Precision.  An error made in an early NS step in the direction of a small
// singular value is multiplied by up to a = 3.4445 in every later step, so
// ill-conditioned inputs (such as momenta, whose spectra spread over
// decades) need the early iterates to more than bf16 precision.  Hence:
//   - in muon_step, X_0 = U carries its lo plane (U ~ hi + lo to about 16
//     mantissa bits), used by the first apply (products kHH + kHL and the
//     diagonal term) and, in the precise recipe, by the first Gram;
//   - the first group spans the first min(4, N - 1) steps (all N when the
//     recipe takes them whole), so X is rounded to bf16 only after the
//     steps whose errors would be multiplied most;
//   - the precise recipe (m < kLeanFromM, or more than kLeanMaxSteps steps)
//     also splits the m x m chain: P, T and R carry lo planes and T, A' and
//     R take the split products (R the single one from kRSingleFromM up, with
//     at most kLeanMaxSteps steps), and the apply uses the lo plane of R.
// See ns_recipe (plan.cpp) for which shapes take which recipe.
template <int TILE, typename PT>
static hipError_t ns_group_bf16(const LargeArgs& g, hipStream_t st, int k, int G, int cur, int last) {
  const LargeLayout& L = g.L;
  uint8_t* ws = (uint8_t*)g.ws;
  uint16_t* X = (uint16_t*)(ws + L.x);
  uint16_t* Xt[2] = {(uint16_t*)(ws + L.xt0), (uint16_t*)(ws + L.xt1)};
  uint16_t* Xl = (uint16_t*)(ws + L.xl);
  uint16_t* Xtl = (uint16_t*)(ws + L.xtl);
  float* scal = (float*)(ws + L.scal);
  uint16_t* H = (uint16_t*)(ws + L.h);
  uint16_t* Lo = (uint16_t*)(ws + L.l);
  uint16_t* Th = (uint16_t*)(ws + L.th);
  // the lean recipe holds up to kLeanMaxSteps steps; beyond, the precise chain
  const bool cs = g.precise || g.sc.ns_steps > kLeanMaxSteps;
  uint16_t* Tl = (uint16_t*)(ws + L.tl);
  uint16_t* Pb[2] = {(uint16_t*)(ws + L.poff), (uint16_t*)(ws + L.poff2)};
  uint16_t* PbL[2] = {cs ? (uint16_t*)(ws + L.poffl0) : nullptr, cs ? (uint16_t*)(ws + L.poffl1) : nullptr};
  float* Pdb[2] = {(float*)(ws + L.pdiag), (float*)(ws + L.pdiag2)};
  uint16_t* Rb[2] = {(uint16_t*)(ws + L.roff0), (uint16_t*)(ws + L.roff1)};
  uint16_t* RbL[2] = {cs ? (uint16_t*)(ws + L.roffl0) : nullptr, cs ? (uint16_t*)(ws + L.roffl1) : nullptr};
  float* Rdb[2] = {(float*)(ws + L.rdiag0), (float*)(ws + L.rdiag1)};
  const int64_t mp = g.mp, np = g.np;
  if (mp % TILE != 0 || np % TILE != 0 || G < 1) return hipErrorInvalidValue;
  const int Tm = int(mp / TILE), Tn = int(np / TILE);
  const int up = Tm * (Tm + 1) / 2;
  const int steps = g.sc.ns_steps;
  const bool xlo = (k == 0) && g.x0_lo;       // X_0 = U carries its lo plane
  const int64_t as = L.a_stride, xs = L.x_stride;
  hipError_t e;
  // symmetric m x m product launches: C = Ah Bh^T (+ split products)
  auto sym1 = [&](const uint16_t* a, const uint16_t* b, const auto& epi) {
    return gemm_launch<TILE, kHH>(a, nullptr, mp, as, b, nullptr, mp, as, mp, Tm, 1, up, g.count, g.cus, epi, st);
  };
  auto sym3 = [&](const uint16_t* ah, const uint16_t* al, const uint16_t* bh, const uint16_t* bl, const auto& epi) {
    return gemm_launch<TILE, kHH | kHL | kLH>(ah, al, mp, as, bh, bl, mp, as, mp, Tm, 1, up, g.count, g.cus, epi, st);
  };
  auto poly = [&](int j) {
    const bool sp = split_a2(g.m, k + j, steps);
    uint16_t* pl = (cs || G == 1) ? PbL[j & 1] : nullptr;
    EpiPolyBf16 ep{H, Lo, Pb[j & 1], pl, Pdb[j & 1], scal, (G == 1 && k == 0) ? 1 : 0, g.sc.a, g.sc.b, g.sc.c, mp, g.m};
    return sp ? sym3(H, Lo, H, Lo, ep) : sym1(H, H, ep);
  };
  // Gram: with X_0's lo plane in the precise recipe, X X^T ~ Xh Xh^T + Xh Xl^T + Xl Xh^T
  EpiGramBf16 eg{H, Lo, scal, k == 0, (split_a2(g.m, k, steps) || cs) ? 1 : 0, mp};
  e = (xlo && cs) ? gemm_launch<TILE, kHH | kHL | kLH>(X, Xl, np, xs, X, Xl, np, xs, np, Tm, 1, up, g.count, g.cus,
                                                       eg, st)
                  : gemm_launch<TILE, kHH>(X, nullptr, np, xs, X, nullptr, np, xs, np, Tm, 1, up, g.count, g.cus, eg, st);
  if (e != hipSuccess) return e;
  if ((e = poly(0)) != hipSuccess) return e;
  // R_j = P_j R_{j-1} is needed only by R_{j+1} and the apply, so when the
  // symmetric launches are a partial round (CUs left idle), it runs on the
  // side stream beside T_{j+1}, A'_{j+1} and the poly of step j+1 (the MoE
  // experts 8 x [1536, 2048]: 2.30 -> 2.18 ms per step, bitwise identical).
  // It reads P_j and R_{j-1} and writes the other R buffer; the one buffer a
  // later main-stream launch overwrites is P_0 (R_0 of R_1), by the poly of
  // step 2, which therefore waits for R_1.  The apply waits for the last R.
  const bool ovl = g.side && g.ev_fork && g.ev_join && up * g.count < g.cus * GemmGeom<TILE>::PER_CU;
  // Work enqueued on the side stream that the launch stream has not waited
  // for.  Every return after a fork joins first, errors included, so no R
  // launch can still run beside what the caller enqueues next.
  bool pend = false;
  auto join = [&]() -> hipError_t {
    if (!pend) return hipSuccess;
    pend = false;
    const hipError_t e1 = hipEventRecord(g.ev_join, g.side);
    const hipError_t e2 = hipStreamWaitEvent(st, g.ev_join, 0);
    return e1 != hipSuccess ? e1 : e2;
  };
  auto bail = [&](hipError_t err) {
    (void)join();
    return err;
  };
  for (int j = 1; j < G; ++j) {
    const int pp = (j - 1) & 1;  // P_{j-1}
    // T = P A from A's planes into T's, A' = P T from T's planes into A's
    EpiSymMul et{H, Lo, Pdb[pp], Th, Tl, cs ? 1 : 0, mp};
    if ((e = cs ? sym3(Pb[pp], PbL[pp], H, Lo, et) : sym1(Pb[pp], H, et)) != hipSuccess) return bail(e);
    EpiSymMul ea{Th, Tl, Pdb[pp], H, Lo, (split_a2(g.m, k + j, steps) || cs) ? 1 : 0, mp};
    if ((e = cs ? sym3(Pb[pp], PbL[pp], Th, Tl, ea) : sym1(Pb[pp], Th, ea)) != hipSuccess) return bail(e);
    if (j == 2 && (e = join()) != hipSuccess) return e;  // R_1 has read P_0
    if ((e = poly(j)) != hipSuccess) return bail(e);
    hipStream_t rs = st;
    if (ovl) {
      if ((e = hipEventRecord(g.ev_fork, st)) != hipSuccess) return bail(e);
      if ((e = hipStreamWaitEvent(g.side, g.ev_fork, 0)) != hipSuccess) return bail(e);
      pend = true;
      rs = g.side;
    }
    auto sym1r = [&](const uint16_t* a, const uint16_t* b, const auto& epi) {
      return gemm_launch<TILE, kHH>(a, nullptr, mp, as, b, nullptr, mp, as, mp, Tm, 1, up, g.count, g.cus, epi, rs);
    };
    auto sym3r = [&](const uint16_t* ah, const uint16_t* al, const uint16_t* bh, const uint16_t* bl,
                     const auto& epi) {
      return gemm_launch<TILE, kHH | kHL | kLH>(ah, al, mp, as, bh, bl, mp, as, mp, Tm, 1, up, g.count, g.cus, epi,
                                                rs);
    };
    // R_j = P_j R_{j-1}; R_0 = s P_0 is P_0 itself with the scale applied here
    const uint16_t* r0 = (j == 1) ? Pb[0] : Rb[(j - 1) & 1];
    const uint16_t* r0l = (j == 1) ? PbL[0] : RbL[(j - 1) & 1];
    const float* rd0 = (j == 1) ? Pdb[0] : Rdb[(j - 1) & 1];
    const bool r3 = cs && !(g.m >= kRSingleFromM && steps <= kLeanMaxSteps);
    if (cs) {
      EpiPairR<true> er{r0, r0l, rd0, Pb[j & 1], PbL[j & 1], Pdb[j & 1], Rb[j & 1], RbL[j & 1], Rdb[j & 1], scal,
                        (k == 0 && j == 1) ? 1 : 0, mp};
      e = r3 ? sym3r(Pb[j & 1], PbL[j & 1], r0, r0l, er) : sym1r(Pb[j & 1], r0, er);
    } else {
      EpiPairR<false> er{r0, nullptr, rd0, Pb[j & 1], nullptr, Pdb[j & 1], Rb[j & 1], nullptr, Rdb[j & 1], scal,
                         (k == 0 && j == 1) ? 1 : 0, mp};
      e = sym1r(Pb[j & 1], r0, er);
    }
    if (e != hipSuccess) return bail(e);
  }
  if ((e = join()) != hipSuccess) return e;
  // apply with R (P_0 for a single step): A = R (+ its lo plane, precise),
  // B = Xt (+ X_0's lo plane)
  const uint16_t* ra = (G == 1) ? Pb[0] : Rb[(G - 1) & 1];
  const uint16_t* ral = (G == 1) ? PbL[0] : RbL[(G - 1) & 1];
  const float* rd = (G == 1) ? Pdb[0] : Rdb[(G - 1) & 1];
  const uint16_t* bl = xlo ? Xtl : nullptr;
  // algorithmic work of this apply (one m x m by m x n product per matrix)
  // and the MFMA work it executes (one such product per operand-plane pair)
  const double alg = 2.0 * double(g.m) * double(g.m) * double(g.n) * g.count;
  const int prods = 1 + (xlo ? 1 : 0) + (cs ? 1 : 0);
  auto apply = [&](const auto& eap) {
    if (cs && xlo)
      return gemm_launch<TILE, kHH | kHL | kLH>(ra, ral, mp, as, Xt[cur], bl, mp, xs, mp, Tn, 0, Tm * Tn, g.count,
                                                g.cus, eap, st);
    if (cs)
      return gemm_launch<TILE, kHH | kLH>(ra, ral, mp, as, Xt[cur], nullptr, mp, xs, mp, Tn, 0, Tm * Tn, g.count,
                                          g.cus, eap, st);
    if (xlo)
      return gemm_launch<TILE, kHH | kHL>(ra, nullptr, mp, as, Xt[cur], bl, mp, xs, mp, Tn, 0, Tm * Tn, g.count,
                                          g.cus, eap, st);
    return gemm_launch<TILE, kHH>(ra, nullptr, mp, as, Xt[cur], nullptr, mp, xs, mp, Tn, 0, Tm * Tn, g.count, g.cus,
                                  eap, st);
  };
  timer_begin(st);
  if (last)
    e = apply(EpiApplyBf16<PT, true>{g.tab, g.sc, X, xlo ? Xl : nullptr, Xt[cur ^ 1], rd, mp, np, g.m, g.n});
  else
    e = apply(EpiApplyBf16<PT, false>{g.tab, g.sc, X, xlo ? Xl : nullptr, Xt[cur ^ 1], rd, mp, np, g.m, g.n});
  if (e != hipSuccess) return e;
  timer_end(st, alg, alg * prods);
  return hipSuccess;
}

// Steps taken together from step k of `steps`: the first min(steps, 5) when
// the recipe takes them whole, otherwise the first min(4, steps - 1) (all of
// them when steps <= 2); then pairs, then a single step when the count left
// is odd.  A longer chain A_{j+1} = P_j A_j P_j is unstable: a rounding
// error that leaves A a slightly negative eigenvalue (A is X X^T, so none
// exists in exact arithmetic) is multiplied by P^2, about a^2 = 11.9, in
// every step and never brought back, which overflowed a 10-step chain of a
// square Gaussian 300 x 300 input on the GPU.
// In an emulation of these roundings (quintic coefficients) this order was
// the most accurate of those tried for m >= 512: early steps, whose
// normalised singular values are small and whose P is near a I, lose nothing
// in the m x m space, while the last steps need A from a fresh Gram of X.
// At 1024 x 3584 with 5 steps and no lo planes, the relative Frobenius error
// of O was 4.2e-3 for single steps and 3.2e-3 grouped on Gaussian inputs,
// 1.9e-2 and 6.4e-3 with singular values spread over [1e-2, 1], 3.0e-2 and
// 8.1e-3 over [1e-3, 1]; one group of all 5 steps gave 2.7e-3, 3.0e-2 and
// 4.7e-2 with a bf16 chain, and below 2e-3 with the split chain of the
// precise recipe.
constexpr int kWholeMaxSteps = 5;

static inline int group_len(int k, int steps, bool whole) {
  if (k == 0) return whole ? std::min(steps, kWholeMaxSteps) : (steps <= 2 ? steps : std::min(4, steps - 1));
  return (steps - k >= 2) ? 2 : 1;
}

template <typename PT, typename XT>
static hipError_t run_large_t(const LargeArgs& g, hipStream_t st) {
  const LargeLayout& L = g.L;
  uint8_t* ws = (uint8_t*)g.ws;
  XT* X = (XT*)(ws + L.x);
  XT* Xt[2] = {(XT*)(ws + L.xt0), (XT*)(ws + L.xt1)};
  float* A = (float*)(ws + L.a);
  float* normpart = (float*)(ws + L.normpart);
  float* scal = (float*)(ws + L.scal);
  const int64_t mp = g.mp, np = g.np, m = g.m, n = g.n;
  const int count = g.count;

  // momentum: 64x64 tiles over the padded matrix (64 divides mp and np); in
  // muon_step the bf16 NS input also gets its lo planes
  XT* Xl = (g.x0_lo) ? (XT*)(ws + L.xl) : nullptr;
  XT* Xtl = (g.x0_lo) ? (XT*)(ws + L.xtl) : nullptr;
  {
    const int tilesM = int(mp / 64), tilesN = int(np / 64);
    dim3 grid(unsigned(tilesM * tilesN), unsigned(count));
    hipLaunchKernelGGL((momentum_kernel<PT, XT>), grid, dim3(256), 0, st, g.tab, g.sc, tilesM,
                       tilesN, X, Xt[0], Xl, Xtl, L.x_stride, mp, np, m, n, normpart, L.tiles);
    if (hipError_t e = last_launch(); e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(norm_kernel, dim3(count), dim3(256), 0, st, normpart, L.tiles, scal);
  if (hipError_t e = last_launch(); e != hipSuccess) return e;

  const int steps = g.sc.ns_steps;
  if (steps == 0) {
    hipLaunchKernelGGL((ns0_kernel<PT, XT>), dim3(unsigned(std::min<int64_t>(4096, (m * n + 255) / 256)), count),
                       dim3(256), 0, st, g.tab, g.sc, X, Xl, mp, np, m, n, scal);
    return last_launch();
  }
  int cur = 0;
  for (int k = 0; k < steps; ++k) {
    const int last = (k == steps - 1);
    if constexpr (sizeof(XT) == 2) {
      const int G = group_len(k, steps, g.whole);
      const int lastG = (k + G == steps);
      const hipError_t e = (g.tile == 256) ? ns_group_bf16<256, PT>(g, st, k, G, cur, lastG)
                                           : ns_group_bf16<128, PT>(g, st, k, G, cur, lastG);
      if (e != hipSuccess) return e;
      k += G - 1;  // the group took steps k .. k + G - 1
    } else {
      float* Pf = (float*)(ws + L.poff);
      const int Tm = int(mp / GF_M), Tn = int(np / GF_M);
      EpiGramF32 eg{A, scal, k == 0, mp};
      hipLaunchKernelGGL((gemm_f32_kernel<EpiGramF32>), dim3(unsigned(Tm * (Tm + 1) / 2), count), dim3(256),
                         0, st, (const float*)X, np, L.x_stride, (const float*)X, np, L.x_stride, np, Tm, 1, eg);
      if (hipError_t e = last_launch(); e != hipSuccess) return e;
      EpiPolyF32 ep{A, Pf, scal, k == 0, g.sc.a, g.sc.b, g.sc.c, mp, m};
      hipLaunchKernelGGL((gemm_f32_kernel<EpiPolyF32>), dim3(unsigned(Tm * (Tm + 1) / 2), count), dim3(256),
                         0, st, (const float*)A, mp, L.a_stride, (const float*)A, mp, L.a_stride, mp, Tm, 1, ep);
      if (hipError_t e = last_launch(); e != hipSuccess) return e;
      EpiApplyF32<PT> ea{g.tab, g.sc, (float*)X, (float*)Xt[cur ^ 1], mp, np, m, n, last};
      hipLaunchKernelGGL((gemm_f32_kernel<EpiApplyF32<PT>>), dim3(unsigned(Tm * Tn), count), dim3(256), 0,
                         st, (const float*)Pf, mp, L.a_stride, (const float*)Xt[cur], mp, L.x_stride, mp, Tn, 0, ea);
      if (hipError_t e = last_launch(); e != hipSuccess) return e;
    }
    cur ^= 1;
  }
  return hipSuccess;
}

hipError_t run_large(const LargeArgs& g, hipStream_t st) {
  if (g.bf16) return run_large_t<uint16_t, uint16_t>(g, st);
  return run_large_t<float, float>(g, st);
}

}  // namespace muon
