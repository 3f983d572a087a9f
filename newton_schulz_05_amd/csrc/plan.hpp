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
// Largest n of a bf16 MFMA-path group: a 256-row operand tile of the padded
// row length (< 2^22 elements) spans less than 2^31 bytes, the range of the
// 32-bit buffer offsets its loads use.
constexpr int64_t kMfmaMaxN = (int64_t(1) << 22) - 256;
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
constexpr size_t kChunkBytesCap = size_t(32) << 30;  // workspace bytes one chunk may use
constexpr int64_t kRoundTiles = 256;         // MFMA path: tiles of one round (one per CU)
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
  size_t th, poff2, pdiag2, roff0, roff1, rdiag0, rdiag1;  // bf16 path (grouped steps), else 0
  size_t xl, xtl;                                          // bf16 path: lo planes of X_0 and its transpose
  size_t tl, poffl0, poffl1, roffl0, roffl1;               // bf16 path: lo planes of T, P, R (precise chain)
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
  bool whole = false;          // MFMA path: all NS steps in one group (ns_recipe)
  bool precise = false;        // MFMA path: split m x m chain and lo planes (ns_recipe)
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

// Bytes of the skinny path's region for one chunk: the slab partials, then
// (from skinny_lo_offset) the lo codes of U.
size_t skinny_bytes(const Group& g, int32_t count);
size_t skinny_lo_offset(const Group& g, int32_t count);

// NS cost 3 m^2 n + m^3 of one matrix (m = min, n = max of its dimensions).
double ns_cost(int64_t rows, int64_t cols);

// Greedy whole-matrix assignment of the plan's matrices to n_ranks ranks
// (largest cost first, each to the least loaded rank; ties in plan order and
// to the lowest rank).  owner[j] is the rank of matrix j; cost[r] the total
// of rank r.
void assign_greedy(const Plan& P, int32_t n_ranks, std::vector<int32_t>* owner, std::vector<double>* cost);

// GEMM tile of an MFMA-path group of `count` matrices of wide shape [m, n].
int32_t mfma_tile(int64_t m, int64_t n, int64_t count);

// How an MFMA-path group of wide shape [m, n] takes its NS steps.  Every
// group of steps k .. k+G-1 has one Gram of X_k and one apply of
// R = P_{k+G-1} ... P_k, the A_j in between formed in the m x m space
// (A_{j+1} = P_j A_j P_j); a group of G steps costs 3 m^2 n + (4 G - 3) m^3
// flops with single products.
//   whole   : all steps in one group (m < kWholeBelowM), else the first
//             min(4, N - 1) steps, then pairs, then a single step;
//   precise : the m x m chain takes split-bf16 products with lo planes of
//             P, T and R, the first Gram uses X_0's lo plane and the applies
//             R's (m < kLeanFromM).  The lean recipe (m >= kLeanFromM) keeps
//             the chain in single products and only the first apply uses
//             X_0's lo plane.
// The thresholds come from an emulation of these roundings on inputs with
// singular values spread over [1e-2, 1] and [1e-3, 1] and rank-m/8 inputs:
// the lean recipe keeps the relative Frobenius error of O under 1e-2 at
// m = 4096 (at most 7.5e-3) but not at m = 1536 (1.5e-2 on rank-m/8), and
// below m = 512 grouping with a bf16 chain loses accuracy (4.5e-2 at
// 64 x 200) where one whole group with the split chain stays under 2e-3.
// The lean recipe also holds only up to kLeanMaxSteps NS steps (at 8 steps
// [4096, 4096] reached 1.4e-2 on the GPU, the precise recipe 3.5e-3 at
// [1024, 1024]); a call with more steps takes the precise chain, whose lo
// planes every bf16 workspace therefore holds.
// Within the precise recipe, R = P_j R_{j-1} takes the single product of
// the hi planes (its epilogue still adds the diagonal terms with the lo
// planes and writes R's lo plane) when m >= kRSingleFromM and the call has
// at most kLeanMaxSteps steps: emulated on the same inputs, the rank-m/8
// error rose from 5.7e-3 to 6.6e-3 at [1024, 2048] and from 5.0e-3 to
// 5.8e-3 at [1536, 2048], but to 8.7e-3 at [512, 1024] and 2.5e-2 at
// [64, 200] in a whole group, so smaller m keeps the split R.
constexpr int64_t kWholeBelowM = 512;
constexpr int64_t kLeanFromM = 4096;
constexpr int kLeanMaxSteps = 5;
constexpr int64_t kRSingleFromM = 1024;
struct NsRecipe {
  bool whole, precise;
};
NsRecipe ns_recipe(int64_t m, int64_t n);

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }

}  // namespace muon
