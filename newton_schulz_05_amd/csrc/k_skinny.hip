// Persistent kernel for skinny matrices (bf16, m <= 32 rows in the wide
// orientation), e.g. the 74 x [24, 10240] batch named in item 3 of the
// HyperParallel FSDP Muon optimizer RFC.
//
// Every matrix is split into S column slabs, one workgroup per slab.  A
// workgroup keeps its slab of X0 = U (the NS input, before normalisation) in
// registers for the whole step, so HBM sees only the compulsory traffic:
// G and M read, M written, W read and written.
//
// NS runs in Gram space.  Every iterate is X_k = Q_k X0 with Q_k a
// polynomial in A0 = X0 X0^T, so all the matrices below commute and
//   A_k = X_k X_k^T = Q_k A0 Q_k,   P_k = a I + b A_k + c A_k^2,
//   Q_{k+1} = P_k Q_k,              A_{k+1} = P_k A_k P_k,
// with Q_0 = s I and A_0 = s^2 X0 X0^T (s = 1 / (||U||_F + eps)).  In exact
// arithmetic O = Q_K X0 is the NS result of the oracle.  For m <= 32 the m x m
// recurrences cost nothing next to the m x n products, so a step needs ONE
// Gram of X0 (a single exchange of slab partials between the workgroups of a
// matrix) and ONE apply O = Q_K X0, instead of one Gram, one exchange and one
// apply per NS iteration.  The m x m arithmetic is fp32 throughout (no bf16
// rounding of an iterate), which is also more accurate than iterating on a
// bf16 X.
//
// Arithmetic: X0 is held in bf16 (in muon_step as U's hi part, with its lo
// part as 8-bit codes); the Gram uses bf16 MFMA with fp32 accumulation
// (exact products), of hi + lo in muon_step; Q_K is split into bf16 hi + lo
// parts so the apply is accurate to about 16 mantissa bits of Q_K, and adds
// Q_hi times X0's lo part; O stays fp32 up to the weight update.
//
// Register layout (wave64, MFMA 32x32x16): a "block" is 32 columns of the
// slab.  Lane l (h = l / 32, c = l % 32) holds column c of the block at the
// 16 rows  row(r) = 8*(r/4) + 4*h + (r%4), r = 0..15, which is the output
// layout of the 32x32 MFMA; the apply O = Q X0 takes X0 in this layout when
// the contraction index of Q's operand is permuted to match.  The Gram
// contracts over columns instead, so each block is restaged through LDS.
#include "common.hpp"
#include "launch.hpp"

namespace muon {

namespace {

constexpr int kNB = 8;            // 32-column blocks per wave (slab <= 4 * 8 * 32 = 1024 columns)
constexpr int kLdr = 36;          // LDS column stride (bf16) of the Gram's restaging
constexpr int kPartW = 544;       // 8-byte words per published slab partial (upper triangle <= 528, + sum of squares)
constexpr int kCoherent = 16;     // buffer cache policy: device-coherent access (sc1)
constexpr int kGather = 12;       // partial words each thread has in flight while gathering

__device__ __forceinline__ int row_of(int r, int h) { return ((r >> 2) << 3) + (h << 2) + (r & 3); }

// In muon_step the NS input U (fp32) is held as hi = bf16(U) in registers
// and its remainder lo = U - hi as an 8-bit code.  The code is the
// difference of the fp32 bit patterns of U and of hi (hi's pattern is its
// bf16 bits times 2^16), an integer d with |d| <= 2^15 since U rounds to the
// nearest hi (the patterns of same-signed floats are monotonic, across
// binades too), rounded to a multiple of 2^8: code = floor((d + 128) / 2^8),
// clamped to 127.  The decoded value is the float whose pattern is hi's plus
// code * 2^8, i.e. U with its 8 lowest mantissa bits rounded away, and
// lo = that - hi is exact and exactly a bf16 value (at most 8 significant
// bits).  hi + lo holds U to about 2^-16 relative.  A zero, subnormal or
// non-finite hi decodes to lo = 0 whatever the code (the codes of padding
// rows are not written).
__device__ __forceinline__ uint32_t lo_code(float u, uint32_t hi) {
  const int d = int(__float_as_uint(u) - (hi << 16));
  const int c = (d + 128) >> 8;  // >= -128
  return uint32_t(c < 127 ? c : 127) & 0xffu;
}
// lo (as bf16 bits) of the value whose hi is `hi` and whose code is the
// byte `code` (bits 0-7)
__device__ __forceinline__ uint32_t lo_decode(uint32_t hi, uint32_t code) {
  const uint32_t h = hi << 16;
  // code * 2^8, sign-extended from the byte by a shift pair
  const uint32_t dd = uint32_t(int(code << 24) >> 16);
  const float v = __uint_as_float(h + dd) - __uint_as_float(h);
  const uint32_t ef = (h >> 23) & 0xffu;
  return (ef - 1u < 254u) ? uint32_t(f2bf(v)) : 0u;
}
// codes of the 16 values of a lane's block (U in u, hi in the bf16 pairs
// x), value r in byte r % 4 of word r / 4
__device__ __forceinline__ void lo_codes(const float* u, const uint32_t* x, uint32_t* code) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t c = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = 4 * w + b;
      c |= lo_code(u[r], (x[r >> 1] >> (16 * (r & 1))) & 0xffffu) << (8 * b);
    }
    code[w] = c;
  }
}
// lo as bf16 pairs in the register layout of x (hi pairs)
__device__ __forceinline__ void lo_words(const uint32_t* x, const uint32_t* code, uint32_t* xl) {
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t c = code[d >> 1] >> (16 * (d & 1));
    xl[d] = lo_decode(x[d] & 0xffffu, c & 0xffu) | (lo_decode(x[d] >> 16, (c >> 8) & 0xffu) << 16);
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt 0) but not for its global memory accesses, so the momentum stores
// and the W prefetch keep draining across it.  The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Fixed-order sum over the 256 threads (result in every thread).
__device__ __forceinline__ float sum_256(float v, float* lds4) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) lds4[wid] = v;
  lds_barrier();
  return (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
}

// Cross-workgroup exchange.  Every workgroup publishes its slab's partial
// Gram (upper triangle, plus the sum of squares on the first step) as 8-byte
// words that pair each value with a tag naming the call and the NS step.
// The words are written and read with device-coherent accesses (they bypass
// the per-XCD L2 write-back path), and an 8-byte word is written as a unit,
// so a reader that sees the expected tag also sees the value: the tags are
// the barrier, and no counter, fence or cache flush is needed.  Two parity
// buffers suffice: a workgroup can only publish step k+2 after every
// workgroup of its matrix has published step k+1, i.e. finished reading k.
// Waits are bounded: on timeout a flag is raised and the workgroup carries
// on, so the grid always drains.
__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
  return uint64_t(__float_as_uint(v)) | (uint64_t(tag) << 32);
}

// i-th entry of the row-major upper triangle of an m x m matrix
__device__ __forceinline__ void tri_ij(int e, int m, int& i, int& j) {
  int r = 0, len = m;
  while (e >= len) { e -= len; ++r; --len; }
  i = r;
  j = r + e;
}

// every partial buffer (at most kSkinnyCapacity slabs of two parities) lies
// below the byte offset that masks a lane
static_assert(uint64_t(kSkinnyCapacity) * 2 * kPartW * 8 < kOobByte, "partial buffer reaches the lane mask");

// LDS of one workgroup.  The momentum phase stages blocks through `stage`;
// the Gram-space recurrence keeps Q and its successor (fp32) there, and the
// apply finds the Q operand table (`pop`) there.  `red` (wave partials,
// gathered slab partials, a copy of Q, the O staging of the apply) shares
// its bytes with the Gram-space matrices, which live between the gather and
// the end of the recurrence.  For m <= 24 (KS = 6) the lo codes of U stay
// in LDS from the momentum phase to the apply: 12 bytes per lane, block and
// wave (24 KB), which keeps 3 workgroups per CU.
template <int KS>
struct SkShared {
  alignas(16) uint16_t stage[4][32 * kLdr];
  union {
    float red[4][32 * 33];
    struct {
      float A[32][33];
      float mat[2][32][33];
    } gs;
  } u;
  alignas(16) uint8_t codes[KS == 6 ? 4 * kNB * 64 * 12 : 16];
  float ss[4];
  int fail;                       // set when a wait of this workgroup timed out
};

// One 16 x 16 quadrant of A B for 32 x 32 fp32 matrices in LDS (stride 33):
// wave w takes quadrant (w / 2, w % 2) over the whole contraction with the
// fp32 MFMA (16x16x4), even and odd k-steps in two chains added at the end.
// The order is fixed, so every workgroup computes bitwise the same product.
// Lane (l16, l4) ends with rows r0 + 4 l4 + r, column c0 + l16 (r = 0..3).
// Only the first KS k-steps of 4 are taken: rows and columns at and beyond
// m are zero, so KS >= ceil(m / 4) loses nothing.  Every operand is read
// from LDS before the first MFMA, and the products alternate between two
// accumulators (even and odd k-steps), added at the end.
template <int KS>
__device__ __forceinline__ f32x4 quad32(const float (*A)[33], const float (*B)[33], int t) {
  const int lane = t & 63, w = t >> 6;
  const int r0 = (w >> 1) * 16, c0 = (w & 1) * 16, l16 = lane & 15, l4 = lane >> 4;
  float a[KS], b[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    a[s] = A[r0 + l16][4 * s + l4];
    b[s] = B[4 * s + l4][c0 + l16];
  }
  f32x4 e = f32x4{0.f, 0.f, 0.f, 0.f}, o = e;
#pragma unroll
  for (int s = 0; s < KS; s += 2) {
    e = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], e, 0, 0, 0);
    if (s + 1 < KS) o = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s + 1], b[s + 1], o, 0, 0, 0);
  }
  return e + o;
}

// C[i][j] = epi(i, j, (A B)[i][j]), then a barrier.  C must not alias A or B
// (no barrier separates this round's reads from its writes).
template <int KS, typename Epi>
__device__ __forceinline__ void mm32(float (*C)[33], const float (*A)[33], const float (*B)[33], int t, Epi epi) {
  const f32x4 acc = quad32<KS>(A, B, t);
  const int lane = t & 63, w = t >> 6;
  const int r0 = (w >> 1) * 16, c0 = (w & 1) * 16, l16 = lane & 15, l4 = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = r0 + 4 * l4 + r, j = c0 + l16;
    C[i][j] = epi(i, j, acc[r]);
  }
  lds_barrier();
}

// C1 = A1 B1 and C2 = A2 B2 in one round (the two chains overlap).
template <int KS>
__device__ __forceinline__ void mm32x2(float (*C1)[33], const float (*A1)[33], const float (*B1)[33],
                                       float (*C2)[33], const float (*A2)[33], const float (*B2)[33], int t) {
  const f32x4 p = quad32<KS>(A1, B1, t);
  const f32x4 q = quad32<KS>(A2, B2, t);
  const int lane = t & 63, w = t >> 6;
  const int r0 = (w >> 1) * 16, c0 = (w & 1) * 16, l16 = lane & 15, l4 = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = r0 + 4 * l4 + r, j = c0 + l16;
    C1[i][j] = p[r];
    C2[i][j] = q[r];
  }
  lds_barrier();
}

}  // namespace

// MODE 0: muon_step (momentum in, weight update out); MODE 1: muon_ns (O out).
// KS: k-steps of 4 in the m x m products of the Gram-space recurrence,
// 6 when m <= 24, else 8.
template <typename PT, int MODE, int KS>
__global__ __launch_bounds__(256, 3) void skinny_kernel(MatTable tab, StepScalars sc, int m, int64_t n,
                                                        int S, int64_t slab_w, float* __restrict__ part,
                                                        uint32_t* __restrict__ sync, unsigned spin_limit,
                                                        uint32_t epoch_host, const uint32_t* __restrict__ epoch_dev,
                                                        uint32_t* __restrict__ host_flag, uint8_t* __restrict__ lobuf) {
  static_assert(sizeof(PT) == 2, "skinny path is bf16");
  // launches recorded into a graph read their number from the counter that
  // the one-thread kernel before them advanced; others get it from the host
  const uint32_t epoch = epoch_dev ? (kDeviceEpochBit | (*epoch_dev & (kDeviceEpochBit - 1))) : epoch_host;
  constexpr bool step_mode = MODE == 0;
  __shared__ SkShared<KS> sh;
  // the Q operand registers of the apply, per lane: [k-step][hi, lo][lane]
  u16x8 (*pop)[2][64] = reinterpret_cast<u16x8 (*)[2][64]>(&sh.stage[0][0]);
  if (threadIdx.x == 0) sh.fail = 0;  // read only after several barriers
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
  // this chunk's partial buffer: [matrix][parity][slab][kPartW] 8-byte words
  const rsrc_t rP = make_rsrc(part, uint32_t(gridDim.x) * 2u * uint32_t(kPartW) * 8u);
  const uint32_t part_z = uint32_t(z) * 2u * uint32_t(S) * uint32_t(kPartW);  // word index
  const int v = threadIdx.x >> 6;  // wave index (uniform within the wave)
  const int ntri = m * (m + 1) / 2;  // published Gram entries
  // lo codes of U (muon_step), in the register layout: kLoB bytes per lane,
  // wave and block of each workgroup (12 when m <= 24: a lane's last 4 values
  // are then padding rows)
  constexpr uint32_t kLoB = (KS == 6) ? 12u : 16u;
  const rsrc_t rL = make_rsrc(lobuf, step_mode ? uint32_t(gridDim.x) * 4u * kNB * 64u * 16u : 0u);
  auto lo_off = [&](int q, int lane) -> uint32_t {
    return ((uint32_t(blockIdx.x) * 4u + uint32_t(v)) * kNB + uint32_t(q)) * 64u * kLoB + uint32_t(lane) * kLoB;
  };
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  auto lo_store = [&](int q, int lane, const uint32_t* code) {
    if constexpr (kLoB == 12u)
      __builtin_amdgcn_raw_buffer_store_b96(u32x3{code[0], code[1], code[2]}, rL, int(lo_off(q, lane)), 0, 0);
    else
      buf_st_b128(rL, lo_off(q, lane), u32x4{code[0], code[1], code[2], code[3]});
  };
  auto lo_load = [&](int q, int lane) -> u32x4 {
    if constexpr (kLoB == 12u) {
      const u32x3 c = __builtin_amdgcn_raw_buffer_load_b96(rL, int(lo_off(q, lane)), 0, 0);
      return u32x4{c[0], c[1], c[2], 0u};
    } else {
      return buf_ld_b128(rL, lo_off(q, lane));
    }
  };

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
  // Wide matrices with 16-byte aligned rows take the vector path: lane
  // (r = lane / 2, half = lane % 2) moves 16 consecutive columns of row r with
  // 16-byte accesses, and the block is transposed to the register layout
  // through this wave's LDS staging.  The next block's loads are issued once
  // the current block's hi Gram (m <= 24) or all its Gram products (m > 24)
  // are issued: earlier, the prefetch registers live across the block's
  // arithmetic made the kernel spill (m <= 24: 16 -> 0 bytes, C2 1% faster;
  // m > 24: 76 -> 40 bytes, 74 x [32, 10240] 10% faster).  Other blocks use
  // element accesses.
  const bool vec = !tr && (nn % 8) == 0;
  uint16_t* stg = sh.stage[v];
  auto full = [&](int q) { return vec && c0 + (v * kNB + q) * 32 + 32 <= c1; };
  auto row_off = [&](int q, int lane) -> uint32_t {
    const int r = lane >> 1, hc = lane & 1;
    return (r < m) ? uint32_t(r * nn + c0 + (v * kNB + q) * 32 + 16 * hc) : kOob;
  };
  u32x4 pg[2][2], pm[2][4];  // prefetched G and M of a block (ping-pong by block parity)
  // The Gram of X0, block by block inside the momentum loop while the next
  // block's loads are in flight: with the block staged column-major in this
  // wave's LDS area ([column][row], bf16), a lane reads row (lane % 32),
  // 8 columns per 16-column half, which is both the A and the B fragment of
  // the block's MFMA (one per 16 columns).
  // In muon_step U's lo part enters too, X0 X0^T = (Xh + Xl)(Xh + Xl)^T =
  // Xh Xh^T + Xh Xl^T + Xl Xh^T + Xl Xl^T: per block Xh Xh^T over its 32
  // columns, then the lo products per 16 columns in that order, with
  // lo = bf16(U - hi) staged over hi (U to about 2^-16, like the codes the
  // apply decodes) and one lo fragment held at a time (register pressure).
  // On rank-3 inputs [24, 10240] the relative Frobenius error of the step's
  // O was 1.06e-2 to 1.20e-2 with Xh Xh^T alone (GPU, two seeds) and about
  // 2.6e-3 with the lo products.  Xl Xl^T, though of relative size 2^-18, keeps A0 a Gram
  // matrix: without it A0 lacks a positive semidefinite term and has
  // negative eigenvalues of about that size where U has none (low rank),
  // which the NS recurrence multiplies by about a^2 per step (a rank-3
  // input went to NaN in 10 steps).
  auto gram_frag = [&](int tt, int lane) {
    const int h = lane >> 5, cl = lane & 31;
    u16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = stg[(16 * tt + 8 * h + e) * kLdr + cl];
    return as_bf16x8(f);
  };
  auto gram_frags = [&](bf16x8* f2, int lane) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) f2[tt] = gram_frag(tt, lane);
  };
  // stage a block held in the register layout (x: bf16 pairs) column-major
  auto stage_reg = [&](const uint32_t* x, int lane) {
    const int h = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int g = 0; g < 4; ++g) *(u32x2*)(stg + cl * kLdr + 8 * g + 4 * h) = u32x2{x[2 * g], x[2 * g + 1]};
  };

  f32x16 gacc = f32x16{};
  auto issue = [&](int q) {
    const uint32_t e0 = row_off(q, opaque(int(threadIdx.x)) & 63);
    pg[q & 1][0] = buf_ld_b128(rG, e0 * 2);
    pg[q & 1][1] = buf_ld_b128(rG, e0 * 2 + 16);
    if (step_mode) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pm[q & 1][i] = buf_ld_b128(rM, e0 * 4 + 16 * i);
    }
  };
  // Wave priorities order the phases that share a SIMD: the latency-bound
  // exchange and Gram-space recurrence (3) before the momentum streaming (2)
  // before the weight update (0).
  __builtin_amdgcn_s_setprio(2);
  if (full(0)) issue(0);
#pragma unroll
  for (int q = 0; q < kNB; ++q) {
    const int lane = opaque(int(threadIdx.x)) & 63, h = lane >> 5, cl = lane & 31;
    if (full(q)) {
      const int r = lane >> 1, hc = lane & 1;
      const uint32_t e0 = row_off(q, lane);
      float gv[16], u[16];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w = pg[q & 1][j >> 2][j & 3];
        gv[2 * j] = bf2f(uint16_t(w & 0xffffu));
        gv[2 * j + 1] = bf2f(uint16_t(w >> 16));
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        u[j] = gv[j];
        if (step_mode) {
          const float mn = fmaf(sc.mu, __uint_as_float(pm[q & 1][j >> 2][j & 3]), gv[j]);
          pm[q & 1][j >> 2][j & 3] = __float_as_uint(mn);
          u[j] = sc.nesterov ? fmaf(sc.mu, mn, gv[j]) : mn;
        }
        ss = fmaf(u[j], u[j], ss);  // padding rows read 0 and add nothing
      }
      if (step_mode) {
#pragma unroll
        for (int i = 0; i < 4; ++i) buf_st_b128(rM, e0 * 4 + 16 * i, pm[q & 1][i]);
      }
      // stage column-major [col][row] (bf16), then read the register layout
      // and the Gram's fragments
#pragma unroll
      for (int j = 0; j < 16; ++j) stg[(16 * hc + j) * kLdr + r] = f2bf(u[j]);
      __builtin_amdgcn_wave_barrier();
      // with m <= 24 (KS 6) dwords 6 and 7 hold rows 24-31, padding: zeros
      // known to the compiler, so they hold no registers
#pragma unroll
      for (int d = 0; d < 8; ++d)
        xw[q][d] = (KS == 6 && d >= 6) ? 0u : *(const uint32_t*)(stg + cl * kLdr + row_of(2 * d, h));
      bf16x8 fb[2];
      gram_frags(fb, lane);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) gacc = mfma32x32x16(fb[tt], fb[tt], gacc);
      if (KS == 6 && q + 1 < kNB && full(q + 1)) issue(q + 1);
      if constexpr (step_mode) {
        // lo staged over hi; one lo fragment at a time (register pressure)
#pragma unroll
        for (int j = 0; j < 16; ++j) stg[(16 * hc + j) * kLdr + r] = f2bf(u[j] - bf2f(f2bf(u[j])));
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 fl = gram_frag(tt, lane);
          gacc = mfma32x32x16(fb[tt], fl, gacc);
          gacc = mfma32x32x16(fl, fb[tt], gacc);
          gacc = mfma32x32x16(fl, fl, gacc);
        }
        __builtin_amdgcn_wave_barrier();
      }
      if (KS != 6 && q + 1 < kNB && full(q + 1)) issue(q + 1);
      if (step_mode) {
        // each code goes straight to its place in the register layout:
        // row r is value 4 (r / 8) + r % 4 of lane 32 ((r / 4) % 2) + column
        const int dl = ((r >> 2) & 1) * 32 + 16 * hc, dv = 4 * (r >> 3) + (r & 3);
        if constexpr (KS == 6) {
          uint8_t* cb = sh.codes + (v * kNB + q) * 64 * 12;
          if (r < m) {
#pragma unroll
            for (int j = 0; j < 16; ++j) cb[(dl + j) * 12 + dv] = uint8_t(lo_code(u[j], f2bf(u[j])));
          }
        } else {
          // through this wave's staging area (free until the Gram restages
          // the block), then one 16-byte store per lane
          uint8_t* st8 = reinterpret_cast<uint8_t*>(stg);
#pragma unroll
          for (int j = 0; j < 16; ++j) st8[(dl + j) * 16 + dv] = uint8_t(lo_code(u[j], f2bf(u[j])));
          __builtin_amdgcn_wave_barrier();
          const u32x4 cw = *(const u32x4*)(st8 + lane * 16);
          __builtin_amdgcn_wave_barrier();
          const uint32_t code[4] = {cw[0], cw[1], cw[2], cw[3]};
          lo_store(q, lane, code);
        }
      }
    } else {
      const int col = c0 + (v * kNB + q) * 32 + cl;
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
        ss = fmaf(u, u, ss);
        uu[r] = u;
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) xw[q][d] = (KS == 6 && d >= 6) ? 0u : f2bf2(uu[2 * d], uu[2 * d + 1]);
      bf16x8 fb[2];
      stage_reg(xw[q], lane);
      __builtin_amdgcn_wave_barrier();
      gram_frags(fb, lane);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) gacc = mfma32x32x16(fb[tt], fb[tt], gacc);
      if constexpr (step_mode) {
        uint32_t xl[8];
#pragma unroll
        for (int d = 0; d < 8; ++d)
          xl[d] = (KS == 6 && d >= 6) ? 0u
                                      : f2bf2(uu[2 * d] - bf2f(uint16_t(xw[q][d] & 0xffffu)),
                                              uu[2 * d + 1] - bf2f(uint16_t(xw[q][d] >> 16)));
        stage_reg(xl, lane);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 fl = gram_frag(tt, lane);
          gacc = mfma32x32x16(fb[tt], fl, gacc);
          gacc = mfma32x32x16(fl, fb[tt], gacc);
          gacc = mfma32x32x16(fl, fl, gacc);
        }
        __builtin_amdgcn_wave_barrier();
      }
      if (step_mode) {
        uint32_t code[4];
        lo_codes(uu, xw[q], code);
        if constexpr (KS == 6) {
          uint32_t* cw = reinterpret_cast<uint32_t*>(sh.codes + ((v * kNB + q) * 64 + lane) * 12);
          cw[0] = code[0]; cw[1] = code[1]; cw[2] = code[2];
        } else {
          lo_store(q, lane, code);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- helpers ---------------------------------------------------------------
  // combine the 4 wave partials and publish this slab's partial for NS step
  // k: upper triangle of the Gram, then (first step) the sum of squares
  auto publish = [&](const f32x16& gacc, int k, bool with_ss) {
    const int t = opaque(int(threadIdx.x)), lane = t & 63, h = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) sh.u.red[v][row_of(r, h) * 32 + cl] = gacc[r];
    float tot = 0.f;
    if (with_ss) tot = sum_256(ss, sh.ss);  // contains a barrier
    lds_barrier();
    const uint32_t tag = (epoch << 5) | uint32_t(k + 1);
    const uint32_t dst = part_z + (uint32_t(k & 1) * S + s) * kPartW;
    for (int e = t; e < ntri; e += 256) {
      int i, j;
      tri_ij(e, m, i, j);
      const int o = i * 32 + j;
      const float val = (sh.u.red[0][o] + sh.u.red[1][o]) + (sh.u.red[2][o] + sh.u.red[3][o]);
      const uint64_t w = tagged(val, tag);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), rP, int((dst + e) * 8), 0, kCoherent);
    }
    if (with_ss && t == 0) {
      const uint64_t w = tagged(tot, tag);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), rP, int((dst + 528) * 8), 0, kCoherent);
    }
  };

  // Gather the slab partials once their tags show up and combine them in
  // slab order (identical in every workgroup): A = s^2 * X0 X0^T (padded
  // with zeros to 32 x 32) and s_out = s.
  auto gather_a = [&](int k, bool first, float& s_out) {
    const int t = opaque(int(threadIdx.x));
    const uint32_t tag = (epoch << 5) | uint32_t(k + 1);
    const uint32_t src = part_z + uint32_t(k & 1) * S * kPartW;
    lds_barrier();  // every thread has read red for its publish before gbuf (= red) is written
    // words per slab: the triangle, plus the sum of squares on the first step
    const int nw = ntri + (first ? 1 : 0);
    // The per-wave staging area (free between publish and the last apply)
    // holds `per` slabs of words at a time.  Each thread has up to kGather
    // loads in flight, then waits for their tags and parks the values in LDS.
    float* gbuf = &sh.u.red[0][0];
    const int per = min(S, min(4 * 32 * 33, 256 * kGather) / nw);
    float acc[3] = {0.f, 0.f, 0.f};  // this thread's entries t, t+256, t+512
    for (int q0 = 0; q0 < S; q0 += per) {
      const int nq = min(per, S - q0);
      const int tot = nq * nw;
      auto woff = [&](int j) -> uint32_t {
        const int idx = t + 256 * j;
        const int q = idx / nw, e = idx - q * nw;
        return (idx < tot) ? (src + (q0 + q) * kPartW + (e < ntri ? e : 528)) * 8 : kOobByte;
      };
      u32x2 w[kGather];
#pragma unroll
      for (int j = 0; j < kGather; ++j) w[j] = __builtin_amdgcn_raw_buffer_load_b64(rP, int(woff(j)), 0, kCoherent);
      unsigned it = 0;
      for (;;) {
        bool ready = true;
#pragma unroll
        for (int j = 0; j < kGather; ++j) ready &= (t + 256 * j >= tot) || (w[j][1] == tag);
        if (ready) break;
        if (++it > spin_limit) {
          // give up: flag the workspace (and the host-visible word, if any),
          // and leave W (or O) of this slab unwritten
          sh.fail = 1;
          __hip_atomic_store(sync + kSyncErrWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (host_flag) __hip_atomic_store(host_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int j = 0; j < kGather; ++j)
          if (t + 256 * j < tot && w[j][1] != tag) w[j] = __builtin_amdgcn_raw_buffer_load_b64(rP, int(woff(j)), 0, kCoherent);
      }
#pragma unroll
      for (int j = 0; j < kGather; ++j)
        if (t + 256 * j < tot) gbuf[t + 256 * j] = __uint_as_float(w[j][0]);
      lds_barrier();
      // fixed slab order within and across rounds
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int e = t + 256 * r;
        if (e < nw)
          for (int q = 0; q < nq; ++q) acc[r] += gbuf[q * nw + e];
      }
      lds_barrier();
    }
    float s2 = 1.f;
    if (first) {
      // word ntri (the sum of squares) is entry ntri: broadcast it via LDS
      if (t == ntri % 256) sh.ss[0] = (ntri < 256) ? acc[0] : (ntri < 512) ? acc[1] : acc[2];
      lds_barrier();
      const float sn = 1.0f / (sqrtf(sh.ss[0]) + kNsEps);
      s2 = sn * sn;
      s_out = sn;
    }
    // zero the padded A, then fill both triangles
    for (int e = t; e < 32 * 33; e += 256) (&sh.u.gs.A[0][0])[e] = 0.f;
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int e = t + 256 * r;
      if (e < ntri) {
        int i, j;
        tri_ij(e, m, i, j);
        sh.u.gs.A[i][j] = acc[r] * s2;
        sh.u.gs.A[j][i] = acc[r] * s2;
      }
    }
    lds_barrier();
  };

  // Gram-space NS: from A = A0 and s, run the recurrence and leave Q_K
  // (hi/lo bf16) in the per-lane MFMA operand layout `pop`.
  auto gram_space_ns = [&](float snorm) {
    const int t = opaque(int(threadIdx.x));
    float (*A)[33] = sh.u.gs.A;
    float (*P)[33] = sh.u.gs.mat[0];
    float (*T)[33] = sh.u.gs.mat[1];
    // Q and its successor live in the (now idle) transpose staging area
    float (*Q)[33] = (float (*)[33])(void*)&sh.stage[0][0];
    float (*Qn)[33] = Q + 32;
    for (int e = t; e < 32 * 33; e += 256) {
      const int i = e / 33, j = e - i * 33;
      (&Q[0][0])[e] = (i == j && i < m) ? snorm : 0.f;
    }
    lds_barrier();
    const float ca = sc.a, cb = sc.b, cc = sc.c;
    const int mm = m;
    const int steps = sc.ns_steps;
    // P, Q and A are polynomials in A0, so they commute: A <- P A P = P (P A).
    // Per step: P = a I + b A + c A^2;  then Q <- P Q and T = P A together;
    // then A <- P T (skipped after the last step).
    for (int k = 0; k < steps; ++k) {
      mm32<KS>(P, A, A, t, [=](int i, int j, float a2) {
        float p = fmaf(cc, a2, cb * A[i][j]);
        return (i == j && i < mm) ? p + ca : p;
      });
      if (k + 1 < steps) {
        mm32x2<KS>(Qn, P, Q, T, P, A, t);
        mm32<KS>(A, P, T, t, [](int, int, float v) { return v; });
      } else {
        mm32<KS>(Qn, P, Q, t, [](int, int, float v) { return v; });
      }
      { float (*tq)[33] = Q; Q = Qn; Qn = tq; }
    }
    // Q lives in the staging area, where its operand table goes: copy it to
    // `red` (free again: the Gram-space matrices are dead) first
    float (*Qc)[33] = reinterpret_cast<float (*)[33]>(&sh.u.red[0][0]);
    for (int e = t; e < 32 * 32; e += 256) Qc[e >> 5][e & 31] = Q[e >> 5][e & 31];
    lds_barrier();
    // Q (fp32) -> hi/lo bf16 operand registers: Q[i][kr] is k-slot q of lane
    // (h, i) in k-step tt, where X0 row kr sits at k-slot q of lane half h
    for (int e = t; e < 32 * 32; e += 256) {
      const int i = e >> 5, kr = e & 31;
      const float qv = Qc[i][kr];
      const uint16_t hi = f2bf(qv);
      const int tt = kr >> 4, hh = (kr >> 2) & 1, q = ((kr >> 3) & 1) * 4 + (kr & 3);
      pop[tt][0][hh * 32 + i][q] = hi;
      pop[tt][1][hh * 32 + i][q] = f2bf(qv - bf2f(hi));
    }
    lds_barrier();
  };

  // O = (Qh + Ql) X0 for one block, with X0 = Xh + Xl in muon_step: per 16
  // rows Qh Xh, Ql Xh, then Qh Xl
  auto apply = [&](const uint32_t* x, const uint32_t* xl, int lane) {
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], x[2], x[3]});
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, u32x4{x[4], x[5], x[6], x[7]});
    f32x16 acc = f32x16{};
    acc = mfma32x32x16(as_bf16x8(pop[0][0][lane]), x0, acc);
    acc = mfma32x32x16(as_bf16x8(pop[0][1][lane]), x0, acc);
    if (step_mode)
      acc = mfma32x32x16(as_bf16x8(pop[0][0][lane]), __builtin_bit_cast(bf16x8, u32x4{xl[0], xl[1], xl[2], xl[3]}), acc);
    acc = mfma32x32x16(as_bf16x8(pop[1][0][lane]), x1, acc);
    acc = mfma32x32x16(as_bf16x8(pop[1][1][lane]), x1, acc);
    if (step_mode)
      acc = mfma32x32x16(as_bf16x8(pop[1][0][lane]), __builtin_bit_cast(bf16x8, u32x4{xl[4], xl[5], xl[6], xl[7]}), acc);
    return acc;
  };

  // O for one block (16 values per lane) -> fp32 store or weight update
  const float keep = 1.0f - sc.lr * sc.wd, stepc = -sc.lr * sc.scale;
  auto emit_block = [&](const f32x16& o, int q, bool failed) {
    if (failed) return;  // a wait timed out: W (or O) keeps its contents
    const int lane = opaque(int(threadIdx.x)) & 63, h = lane >> 5, cl = lane & 31;
    if (full(q)) {
      // O through LDS (fp32, column-major, stride 33) to row-major vectors
      float* fst = sh.u.red[v];
#pragma unroll
      for (int r = 0; r < 16; ++r) fst[cl * 33 + row_of(r, h)] = o[r];
      __builtin_amdgcn_wave_barrier();
      const int r = lane >> 1, hc = lane & 1;
      float ov[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) ov[j] = fst[(16 * hc + j) * 33 + r];
      __builtin_amdgcn_wave_barrier();
      const uint32_t e0 = row_off(q, lane);
      if (!step_mode) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          buf_st_b128(rW, e0 * 4 + 16 * i, u32x4{__float_as_uint(ov[4 * i]), __float_as_uint(ov[4 * i + 1]),
                                                 __float_as_uint(ov[4 * i + 2]), __float_as_uint(ov[4 * i + 3])});
      } else {
        const u32x4 wa = buf_ld_b128(rW, e0 * 2), wb = buf_ld_b128(rW, e0 * 2 + 16);
        u32x4 na, nb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w = (j < 4) ? wa[j] : wb[j - 4];
          const float lo = fmaf(stepc, ov[2 * j], bf2f(uint16_t(w & 0xffffu)) * keep);
          const float hi = fmaf(stepc, ov[2 * j + 1], bf2f(uint16_t(w >> 16)) * keep);
          if (j < 4) na[j] = f2bf2(lo, hi); else nb[j - 4] = f2bf2(lo, hi);
        }
        buf_st_b128(rW, e0 * 2, na);
        buf_st_b128(rW, e0 * 2 + 16, nb);
      }
      return;
    }
    const int col = c0 + (v * kNB + q) * 32 + cl;
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

  // ---- Gram of X0, one exchange, Gram-space NS, apply and update ------------
  __builtin_amdgcn_s_setprio(3);
  publish(gacc, 0, true);
  float snorm = 1.f;
  gather_a(0, true, snorm);
  gram_space_ns(snorm);
  __builtin_amdgcn_s_setprio(0);
  {
    const int lane = opaque(int(threadIdx.x)) & 63;
    const bool failed = sh.fail != 0;
    // every block's lo codes are requested at once, so that their latency is
    // paid once
    // (m > 24: from the workspace; m <= 24: kept in LDS)
    u32x4 cw[KS == 6 ? 1 : kNB];
    if constexpr (step_mode && KS != 6) {
#pragma unroll
      for (int q = 0; q < kNB; ++q) cw[q] = lo_load(q, lane);
    }
#pragma unroll
    for (int q = 0; q < kNB; ++q) {
      uint32_t xl[8];
      if (step_mode) {
        uint32_t code[4];
        if constexpr (KS == 6) {
          const uint32_t* cp = reinterpret_cast<const uint32_t*>(sh.codes + ((v * kNB + q) * 64 + lane) * 12);
          code[0] = cp[0]; code[1] = cp[1]; code[2] = cp[2]; code[3] = 0u;
        } else {
          code[0] = cw[q][0]; code[1] = cw[q][1]; code[2] = cw[q][2]; code[3] = cw[q][3];
        }
        lo_words(xw[q], code, xl);
      }
      const f32x16 acc = apply(xw[q], xl, lane);
      emit_block(acc, q, failed);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int MODE, int KS>
static void launch_skinny(const SkinnyArgs& g, hipStream_t st) {
  const unsigned grid = unsigned(g.count * g.slabs);
  hipLaunchKernelGGL((skinny_kernel<uint16_t, MODE, KS>), dim3(grid), dim3(256), 0, st, g.tab, g.sc, g.m, g.n,
                     g.slabs, g.slab_w, g.part, g.sync, g.spin_limit, g.epoch, g.epoch_dev, g.host_flag, g.lobuf);
}

hipError_t run_skinny(const SkinnyArgs& g, hipStream_t st) {
  const bool small = g.m <= 24;
  if (g.sc.mode == 0) {
    if (small) launch_skinny<0, 6>(g, st); else launch_skinny<0, 8>(g, st);
  } else {
    if (small) launch_skinny<1, 6>(g, st); else launch_skinny<1, 8>(g, st);
  }
  return hipGetLastError();
}

__global__ void epoch_bump_kernel(uint32_t* c) { *c = *c + 1u; }

hipError_t run_epoch_bump(uint32_t* counter, hipStream_t st) {
  hipLaunchKernelGGL(epoch_bump_kernel, dim3(1), dim3(1), 0, st, counter);
  return hipGetLastError();
}

int skinny_max_blocks_per_cu() {
  int nb = 0;
  // the capacity the persistent launch relies on: the least of the variants
  int lo = 1 << 30;
  const void* ks[4] = {(const void*)skinny_kernel<uint16_t, 0, 6>, (const void*)skinny_kernel<uint16_t, 0, 8>,
                       (const void*)skinny_kernel<uint16_t, 1, 6>, (const void*)skinny_kernel<uint16_t, 1, 8>};
  for (const void* k : ks) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, 256, 0) != hipSuccess) return 0;
    lo = std::min(lo, nb);
  }
  return lo;
}

}  // namespace muon
