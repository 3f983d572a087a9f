// Host-side plan: validation, grouping by trailing shape, chunking and the
// workspace layout.  Pure C++ (no HIP calls), so it also builds with g++ for
// host-only tests.
//
// Grouping follows item 3 of the HyperParallel FSDP Muon optimizer RFC
// (parameters with the same trailing two dimensions form one batch), with one
// addition: a tall matrix [M, N] (M > N) is orthogonalised as its transpose,
// so it joins the group of the wide shape [N, M].
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/muon.h"

namespace muon {

enum Path : int32_t {
  PATH_SKINNY = 0,  // bf16, m <= 32: one persistent kernel per chunk
  PATH_MFMA = 1,    // bf16, m > 32: momentum kernel + (Gram, poly, apply) per NS step
  PATH_F32 = 2      // fp32 params: the same pipeline in fp32 arithmetic
};

// Geometry constants the kernels are compiled for.
constexpr int64_t kSkinnyMaxM = 32;          // rows of the padded MFMA tile
constexpr int64_t kSkinnyBlocksPerWave = 8;  // 32-column blocks each wave keeps in registers
constexpr int64_t kSkinnyWaves = 4;
constexpr int64_t kSkinnyMaxSlab = 32 * kSkinnyBlocksPerWave * kSkinnyWaves;  // 1024 columns
constexpr int64_t kSkinnyCapacity = 768;     // co-resident workgroups assumed (3 per CU x 256 CUs)
constexpr int64_t kSkinnyPartStride = 1024 + 64;  // floats per slab partial (32x32 Gram + sum of squares)
constexpr int64_t kMfmaTile = 128;           // MFMA path: default GEMM tile and padding
constexpr int64_t kMfmaTileBig = 256;        // MFMA path: tile for groups with work for the whole chip
constexpr int64_t kF32Tile = 64;             // row/column padding of the fp32 path
constexpr int64_t kMomTile = 64;             // momentum kernel tile (rows and columns)
constexpr size_t kSyncBytes = 8192;          // barrier counters (skinny path)
constexpr size_t kChunkBytesCap = size_t(24) << 30;  // workspace bytes one chunk may use
constexpr int kMaxChunkMats = 80;            // must equal kMaxChunk in common.hpp

struct MatEntry {
  int32_t param;   // index into the parameter list
  int64_t e;       // slice within an expert slab (0 for a 2-D parameter)
  int64_t rows, cols;
  bool tr;         // rows > cols: handled as the transpose
};

struct Chunk {
  int32_t first;   // first index into Group::mats
  int32_t count;
};

// Byte offsets (relative to the workspace base) of one chunk's buffers on the
// MFMA and fp32 paths.  Per-matrix strides are in elements of the buffer type.
struct LargeLayout {
  size_t x, xt0, xt1, a, h, l, poff, pdiag, normpart, scal;
  size_t th, poff2, pdiag2, roff0, roff1, rdiag0, rdiag1;  // grouped steps only, else 0
  int64_t x_stride, a_stride, tiles;  // elements per matrix (X / A) and momentum tiles per matrix
  size_t bytes;                       // total bytes of the chunk region
};

struct Group {
  int64_t m, n;                // canonical wide shape (m <= n)
  Path path;
  std::vector<int32_t> mats;   // indices into Plan::mats, plan order
  int64_t n_tr = 0;
  std::vector<Chunk> chunks;
  int64_t mp = 0, np = 0;      // padded dims (MFMA / fp32 paths)
  int32_t tile = 0;            // MFMA path: GEMM output tile (128 or 256)
  bool grouped = false;        // MFMA path: NS steps taken in groups (mfma_grouped)
  int32_t slabs = 0;           // skinny: column slabs per matrix
  int64_t slab_w = 0;          // skinny: columns per slab (multiple of 32)
  int32_t max_chunk = 0;       // largest chunk of this group
};

struct Plan {
  std::vector<muon_shape> shapes;
  muon_dtype param_dt, grad_dt, mom_dt;
  std::vector<MatEntry> mats;
  std::vector<Group> groups;
  size_t ws_sync_off = 0;
  size_t ws_dyn_off = 0;       // start of the per-chunk region
  size_t ws_bytes = 0;
};

// Builds the plan; returns MUON_OK or an error with `detail` filled.
muon_status build_plan(const muon_shape* shapes, int32_t n_params, muon_dtype param_dt,
                       muon_dtype grad_dt, muon_dtype mom_dt, Plan* out, std::string* detail);

// Layout of one chunk of `count` matrices of group g (MFMA / fp32 paths).
LargeLayout large_layout(const Group& g, int32_t count, muon_dtype param_dt);

// Bytes of the skinny partial-sum buffer for one chunk.
size_t skinny_bytes(const Group& g, int32_t count);

// NS cost 3 m^2 n + m^3 of one matrix (m = min, n = max of its dimensions).
double ns_cost(int64_t rows, int64_t cols);

// Greedy whole-matrix assignment of the plan's matrices to n_ranks ranks
// (largest cost first, each to the least loaded rank; ties in plan order and
// to the lowest rank).  owner[j] is the rank of matrix j; cost[r] the total
// of rank r.
void assign_greedy(const Plan& P, int32_t n_ranks, std::vector<int32_t>* owner, std::vector<double>* cost);

// GEMM tile of an MFMA-path group of `count` matrices of wide shape [m, n].
int32_t mfma_tile(int64_t m, int64_t n, int64_t count);

// Whether an MFMA-path group of wide shape [m, n] takes its NS steps in
// groups: steps k .. k+G-1 with one Gram of X_k and one apply of
// R = P_{k+G-1} ... P_k, the A_j in between formed in the m x m space
// (A_{j+1} = P_j A_j P_j).  A group of G steps costs 3 m^2 n + (4 G - 3) m^3
// flops (single-product A^2) instead of G (3 m^2 n + m^3), a saving once
// n > m; taken for m >= 512 and n >= 2 m.
bool mfma_grouped(int64_t m, int64_t n);

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }

}  // namespace muon
