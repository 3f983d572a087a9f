// Host-side plan construction (see plan.hpp).
#include "plan.hpp"

#include <algorithm>
#include <map>
#include <numeric>
#include <queue>
#include <utility>

namespace muon {

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Split `count` matrices into the fewest chunks of at most `cap` each, with
// sizes as even as possible (the split never changes any result: every matrix
// is computed the same way in any chunk).
std::vector<Chunk> split_n(int32_t count, int32_t n) {
  std::vector<Chunk> out;
  int32_t base = count / n, extra = count % n, first = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t c = base + (i < extra ? 1 : 0);
    out.push_back(Chunk{first, c});
    first += c;
  }
  return out;
}

std::vector<Chunk> split_even(int32_t count, int32_t cap) {
  if (cap < 1) cap = 1;
  return split_n(count, (count + cap - 1) / cap);
}

// The MFMA path's chunks: the fewest of at most `cap` matrices, unless up to
// three more leave fewer symmetric tiles (sym per matrix) in partial last
// rounds of kRoundTiles, which run as a second launch at half the tile size
// and a lower rate; ties go to fewer chunks.  The 32-layer set's wide group
// (96 x [4096, 14336], 136 tiles a matrix) takes 3 chunks of 32, 17 whole
// rounds each, instead of 4 of 24 with 192 tiles left over in each.
std::vector<Chunk> split_rounds(int32_t count, int32_t cap, int64_t sym) {
  if (cap < 1) cap = 1;
  const int32_t n0 = (count + cap - 1) / cap;
  int32_t best = n0;
  int64_t best_left = -1;
  for (int32_t n = n0; n <= std::min(count, n0 + 3); ++n) {
    int64_t left = 0;
    for (const Chunk& c : split_n(count, n)) left += (int64_t(c.count) * sym) % kRoundTiles;
    if (best_left < 0 || left < best_left) { best = n; best_left = left; }
  }
  return split_n(count, best);
}

}  // namespace

LargeLayout large_layout(const Group& g, int32_t count, muon_dtype param_dt) {
  LargeLayout L{};
  const size_t es = (param_dt == MUON_BF16) ? 2 : 4;  // X element size
  const int64_t mp = g.mp, np = g.np;
  L.x_stride = mp * np;
  L.a_stride = mp * mp;
  // norm slots: one per 64x64 momentum tile that holds matrix elements, so
  // their number and order depend on (m, n) alone, not on the padding
  L.tiles = ceil_div(g.m, kMomTile) * ceil_div(g.n, kMomTile);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  const size_t xb = size_t(count) * size_t(mp) * size_t(np) * es;
  L.x = take(xb);
  L.xt0 = take(xb);
  L.xt1 = take(xb);
  // fp32 A (the fp32 path; the bf16 path holds A as its planes H + L)
  L.a = (param_dt == MUON_BF16) ? 0 : take(size_t(count) * size_t(mp) * size_t(mp) * 4);
  if (param_dt == MUON_BF16) {
    L.h = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    L.l = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    L.poff = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
  } else {
    L.h = L.l = 0;
    L.poff = take(size_t(count) * size_t(mp) * size_t(mp) * 4);  // full fp32 P
  }
  L.pdiag = take(size_t(count) * size_t(mp) * 4);
  if (param_dt == MUON_BF16) {
    L.xl = take(xb);
    L.xtl = take(xb);
    L.th = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    L.poff2 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    L.pdiag2 = take(size_t(count) * size_t(mp) * 4);
    L.roff0 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    L.roff1 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    L.rdiag0 = take(size_t(count) * size_t(mp) * 4);
    L.rdiag1 = take(size_t(count) * size_t(mp) * 4);
    {  // the precise chain's lo planes (also taken by the lean recipe beyond kLeanMaxSteps steps)
      L.tl = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
      L.poffl0 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
      L.poffl1 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
      L.roffl0 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
      L.roffl1 = take(size_t(count) * size_t(mp) * size_t(mp) * 2);
    }
  }
  L.normpart = take(size_t(count) * size_t(L.tiles) * 4);
  L.scal = take(size_t(count) * 4 * 4);
  L.bytes = off;
  return L;
}

NsRecipe ns_recipe(int64_t m, int64_t n) {
  (void)n;
  return NsRecipe{m < kWholeBelowM, m < kLeanFromM};
}

double ns_cost(int64_t rows, int64_t cols) {
  const double m = double(std::min(rows, cols)), n = double(std::max(rows, cols));
  return 3.0 * m * m * n + m * m * m;
}

void assign_greedy(const Plan& P, int32_t n_ranks, std::vector<int32_t>* owner, std::vector<double>* cost) {
  const size_t nm = P.mats.size();
  std::vector<double> c(nm);
  for (size_t j = 0; j < nm; ++j) c[j] = ns_cost(P.mats[j].rows, P.mats[j].cols);
  std::vector<size_t> order(nm);
  std::iota(order.begin(), order.end(), size_t(0));
  std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return c[x] > c[y]; });
  // min-heap of (total, rank): the least loaded rank, lowest rank on ties
  using Slot = std::pair<double, int32_t>;
  std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
  for (int32_t r = 0; r < n_ranks; ++r) heap.push(Slot{0.0, r});
  owner->assign(nm, 0);
  cost->assign(size_t(n_ranks), 0.0);
  for (size_t j : order) {
    Slot s = heap.top();
    heap.pop();
    (*owner)[j] = s.second;
    s.first += c[j];
    (*cost)[size_t(s.second)] = s.first;
    heap.push(s);
  }
}

int32_t mfma_tile(int64_t m, int64_t n, int64_t count) {
  // The 256 tile (one 8-wave block per CU) runs the large products faster,
  // enough so that half a round of it (128 symmetric blocks, 256 apply
  // blocks) beats the 128 tile (two blocks per CU): the MoE experts
  // 8 x [1536, 2048] (168 symmetric blocks at 256) went from 2.94 to 2.77 ms
  // per step with it.  It must not pad more than 10% beyond the 128 tile
  // (m^2 n work).
  const int64_t t = ceil_div(m, kMfmaTileBig), u = ceil_div(n, kMfmaTileBig);
  const int64_t sym = count * t * (t + 1) / 2, full = count * t * u;
  const double big = double(t * kMfmaTileBig) * double(t * kMfmaTileBig) * double(u * kMfmaTileBig);
  const double small = double(round_up(m, kMfmaTile)) * double(round_up(m, kMfmaTile)) *
                       double(round_up(n, kMfmaTile));
  return (sym >= 128 && full >= 256 && big <= 1.10 * small) ? int32_t(kMfmaTileBig) : int32_t(kMfmaTile);
}

size_t skinny_lo_offset(const Group& g, int32_t count) {
  return align256(size_t(count) * 2 * size_t(g.slabs) * size_t(kSkinnyPartStride) * 4);
}

size_t skinny_bytes(const Group& g, int32_t count) {
  // slab partials, then (m > 24; smaller m keeps them in LDS) the lo codes
  // of U: 16 bytes per lane, block and wave
  return skinny_lo_offset(g, count) +
         (g.m > 24 ? size_t(count) * size_t(g.slabs) * size_t(kSkinnyWaves * kSkinnyBlocksPerWave * 64 * 16) : 0);
}

muon_status build_plan(const muon_shape* shapes, int32_t n_params, muon_dtype param_dt,
                       muon_dtype grad_dt, muon_dtype mom_dt, Plan* out, std::string* detail) {
  if (!shapes || !out) { *detail = "null shapes or output pointer"; return MUON_ERR_INVALID_ARG; }
  if (n_params < 1) { *detail = "n_params must be >= 1"; return MUON_ERR_INVALID_ARG; }
  if (param_dt != MUON_F32 && param_dt != MUON_BF16) {
    *detail = "param dtype must be MUON_F32 or MUON_BF16"; return MUON_ERR_DTYPE;
  }
  if (grad_dt != param_dt) { *detail = "grad dtype must equal param dtype"; return MUON_ERR_DTYPE; }
  if (mom_dt != MUON_F32) { *detail = "momentum dtype must be MUON_F32"; return MUON_ERR_DTYPE; }

  Plan P;
  P.param_dt = param_dt;
  P.grad_dt = grad_dt;
  P.mom_dt = mom_dt;
  P.shapes.assign(shapes, shapes + n_params);

  // key (m, n) -> group index, groups in order of first appearance
  std::map<std::pair<int64_t, int64_t>, int32_t> key2g;
  for (int32_t i = 0; i < n_params; ++i) {
    const muon_shape& s = shapes[i];
    if (s.batch < 1 || s.rows < 1 || s.cols < 1) {
      *detail = "parameter " + std::to_string(i) + ": every dimension must be >= 1 "
                "(1-D parameters belong to another optimizer)";
      return MUON_ERR_SHAPE;
    }
    if (s.rows > (int64_t(1) << 31) || s.cols > (int64_t(1) << 31) ||
        s.rows * s.cols > (int64_t(1) << 40)) {
      *detail = "parameter " + std::to_string(i) + ": matrix too large";
      return MUON_ERR_SHAPE;
    }
    const int64_t m = std::min(s.rows, s.cols), n = std::max(s.rows, s.cols);
    auto key = std::make_pair(m, n);
    auto it = key2g.find(key);
    int32_t gi;
    if (it == key2g.end()) {
      gi = (int32_t)P.groups.size();
      key2g[key] = gi;
      Group g;
      g.m = m;
      g.n = n;
      P.groups.push_back(g);
    } else {
      gi = it->second;
    }
    for (int64_t e = 0; e < s.batch; ++e) {
      MatEntry me{i, e, s.rows, s.cols, s.rows > s.cols};
      P.groups[gi].mats.push_back((int32_t)P.mats.size());
      if (me.tr) P.groups[gi].n_tr++;
      P.mats.push_back(me);
    }
  }

  size_t dyn = 0;
  for (Group& g : P.groups) {
    const int32_t count = (int32_t)g.mats.size();
    if (param_dt == MUON_F32) {
      g.path = PATH_F32;
    } else if (g.m <= kSkinnyMaxM && ceil_div(g.n, kSkinnyMaxSlab) <= kSkinnyCapacity) {
      g.path = PATH_SKINNY;
    } else {
      g.path = PATH_MFMA;
      if (g.n > kMfmaMaxN) {
        *detail = "bf16 matrices with min(rows, cols) > 32 (or too wide for the skinny path) are limited to "
                  "max(rows, cols) <= " + std::to_string(kMfmaMaxN);
        return MUON_ERR_SHAPE;
      }
    }
    if (g.path == PATH_SKINNY) {
      g.slabs = (int32_t)ceil_div(g.n, kSkinnyMaxSlab);
      g.slab_w = round_up(ceil_div(g.n, g.slabs), 32);
      int32_t cap = (int32_t)std::min<int64_t>(kMaxChunkMats, kSkinnyCapacity / g.slabs);
      g.chunks = split_even(count, cap);
    } else {
      g.tile = (g.path == PATH_MFMA) ? mfma_tile(g.m, g.n, count) : int32_t(kF32Tile);
      if (g.path == PATH_MFMA) {
        const NsRecipe r = ns_recipe(g.m, g.n);
        g.whole = r.whole;
        g.precise = r.precise;
      }
      const int64_t t = g.tile;
      g.mp = round_up(g.m, t);
      g.np = round_up(g.n, t);
      LargeLayout one = large_layout(g, 1, param_dt);
      int32_t cap = (int32_t)std::max<size_t>(1, kChunkBytesCap / std::max<size_t>(one.bytes, 1));
      cap = std::min(cap, kMaxChunkMats);
      if (g.path == PATH_MFMA) {
        const int64_t tm = g.mp / g.tile;
        g.chunks = split_rounds(count, cap, tm * (tm + 1) / 2);
      } else {
        g.chunks = split_even(count, cap);
      }
    }
    for (const Chunk& c : g.chunks) g.max_chunk = std::max(g.max_chunk, c.count);
    size_t need = (g.path == PATH_SKINNY) ? skinny_bytes(g, g.max_chunk)
                                          : large_layout(g, g.max_chunk, param_dt).bytes;
    dyn = std::max(dyn, need);
  }
  P.ws_sync_off = 0;
  P.ws_dyn_off = kSyncBytes;
  P.ws_bytes = kSyncBytes + align256(dyn);
  *out = std::move(P);
  return MUON_OK;
}

}  // namespace muon
