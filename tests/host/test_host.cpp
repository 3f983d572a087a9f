// Host-only checks of the plan builder and the argument validation of the
// C ABI, built with g++ and AddressSanitizer / UndefinedBehaviorSanitizer by
// tests/test_host_native.py.  No HIP: plan.cpp and validate.cpp make no HIP
// call.  Prints "ALL OK" and exits 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <set>
#include <string>
#include <vector>

#include "../../newton_schulz_05_amd/csrc/plan.hpp"
#include "../../newton_schulz_05_amd/csrc/validate.hpp"

using namespace muon;

static int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static Plan make(const std::vector<muon_shape>& s, muon_dtype dt = MUON_BF16, muon_status want = MUON_OK) {
  Plan P;
  std::string d;
  const muon_status st = build_plan(s.data(), int32_t(s.size()), dt, dt, MUON_F32, &P, &d);
  CHECK(st == want);
  if (st != MUON_OK) CHECK(!d.empty());
  return P;
}

// Structural invariants of a plan: every matrix in exactly one group and one
// chunk, chunk limits, workspace regions inside the workspace and disjoint.
static void check_plan(const Plan& P) {
  std::set<int32_t> seen;
  size_t need = 0;
  for (const Group& g : P.groups) {
    CHECK(g.m <= g.n && g.m >= 1);
    int32_t covered = 0, first = 0;
    for (const Chunk& c : g.chunks) {
      CHECK(c.first == first);
      CHECK(c.count >= 1 && c.count <= kMaxChunkMats);
      CHECK(c.count <= g.max_chunk);
      first += c.count;
      covered += c.count;
    }
    CHECK(covered == int32_t(g.mats.size()));
    for (int32_t j : g.mats) {
      CHECK(seen.insert(j).second);
      const MatEntry& me = P.mats[size_t(j)];
      CHECK(std::min(me.rows, me.cols) == g.m && std::max(me.rows, me.cols) == g.n);
      CHECK(me.tr == (me.rows > me.cols));
    }
    if (g.path == PATH_SKINNY) {
      CHECK(g.m <= kSkinnyMaxM);
      CHECK(int64_t(g.max_chunk) * g.slabs <= kSkinnyCapacity);
      CHECK(g.slab_w % 32 == 0 && g.slab_w <= kSkinnyMaxSlab && g.slab_w * g.slabs >= g.n);
      need = std::max(need, skinny_bytes(g, g.max_chunk));
    } else {
      CHECK(g.mp % g.tile == 0 && g.np % g.tile == 0 && g.mp >= g.m && g.np >= g.n);
      CHECK(g.mp - g.m < g.tile && g.np - g.n < g.tile);
      const LargeLayout L = large_layout(g, g.max_chunk, P.param_dt);
      // the norm slots follow the matrix's own 64 x 64 tiles, not the padding
      CHECK(L.tiles == ceil_div(g.m, kMomTile) * ceil_div(g.n, kMomTile));
      const size_t offs[] = {L.x, L.xt0, L.xt1, L.a, L.poff, L.pdiag, L.normpart, L.scal};
      for (size_t o : offs) CHECK(o % 256 == 0 && o < L.bytes);
      if (P.param_dt == MUON_BF16) {
        const size_t lo[] = {L.xl, L.xtl, L.th, L.poff2, L.roff0, L.roff1, L.rdiag0, L.rdiag1};
        for (size_t o : lo) CHECK(o != 0 && o % 256 == 0 && o < L.bytes);
        const size_t pl[] = {L.tl, L.poffl0, L.poffl1, L.roffl0, L.roffl1};
        for (size_t o : pl) CHECK(o != 0 && o % 256 == 0 && o < L.bytes);
      }
      CHECK(L.xt0 >= L.x + size_t(g.max_chunk) * size_t(L.x_stride) * (P.param_dt == MUON_BF16 ? 2 : 4));
      CHECK(L.scal + size_t(g.max_chunk) * 16 <= L.bytes);
      need = std::max(need, L.bytes);
    }
  }
  CHECK(seen.size() == P.mats.size());
  CHECK(P.ws_dyn_off >= kSyncBytes && P.ws_bytes >= P.ws_dyn_off + need);
}

static void test_workload_plans() {
  // the five workloads
  check_plan(make({{1, 64, 128}, {1, 64, 128}, {1, 64, 128}, {1, 64, 128}}, MUON_F32));
  std::vector<muon_shape> c2(74, muon_shape{1, 24, 10240});
  Plan p2 = make(c2);
  check_plan(p2);
  CHECK(p2.groups.size() == 1 && p2.groups[0].path == PATH_SKINNY && p2.groups[0].slabs == 10);
  Plan p3 = make({{8, 2048, 1536}, {32, 24, 10240}});
  check_plan(p3);
  CHECK(p3.groups.size() == 2 && p3.groups[0].n_tr == 8 && p3.groups[0].tile == 256);
  std::vector<muon_shape> c4;
  for (int l = 0; l < 32; ++l) {
    for (int q = 0; q < 4; ++q) c4.push_back({1, 4096, 4096});
    c4.push_back({1, 14336, 4096});
    c4.push_back({1, 14336, 4096});
    c4.push_back({1, 4096, 14336});
  }
  Plan p4 = make(c4);
  check_plan(p4);
  CHECK(p4.groups.size() == 2 && p4.groups[1].mats.size() == 96 && p4.groups[1].n_tr == 64);
  CHECK(p4.groups[0].tile == 256 && !p4.groups[0].whole && !p4.groups[0].precise && !p4.groups[1].precise);
  CHECK(p3.groups[0].precise && !p3.groups[0].whole);
  Plan p5 = make({{1, 8192, 28672}, {1, 8192, 28672}});
  check_plan(p5);
  CHECK(p5.groups[0].tile == 256 && !p5.groups[0].precise);
  Plan ps = make({{1, 100, 300}});
  CHECK(ps.groups[0].whole && ps.groups[0].precise);
}

static void test_edge_plans() {
  check_plan(make({{1, 1, 1}}));
  check_plan(make({{1, 1, 5000}, {1, 5000, 1}, {3, 32, 33}, {1, 33, 32}, {2, 33, 34}}));
  check_plan(make({{1, 32, 786432}}));       // the widest skinny matrix: 768 slabs
  check_plan(make({{1, 32, 786433}}));       // one column more: MFMA path
  CHECK(make({{1, 32, 786433}}).groups[0].path == PATH_MFMA);
  std::vector<muon_shape> many(300, muon_shape{1, 24, 1024});
  Plan pm = make(many);
  check_plan(pm);
  CHECK(pm.groups[0].chunks.size() == 4);
  std::vector<muon_shape> mfma(90, muon_shape{1, 64, 200});
  Plan pf = make(mfma);
  check_plan(pf);
  CHECK(pf.groups[0].chunks.size() == 2 && pf.groups[0].chunks[0].count == 45);
  // errors
  make({{0, 4, 4}}, MUON_BF16, MUON_ERR_SHAPE);
  make({{1, 0, 4}}, MUON_BF16, MUON_ERR_SHAPE);
  make({{1, 4, -1}}, MUON_BF16, MUON_ERR_SHAPE);
  make({{1, int64_t(1) << 32, 4}}, MUON_BF16, MUON_ERR_SHAPE);
  make({{1, 4, 4}}, muon_dtype(7), MUON_ERR_DTYPE);
  Plan P;
  std::string d;
  muon_shape s{1, 4, 4};
  CHECK(build_plan(&s, 1, MUON_BF16, MUON_F32, MUON_F32, &P, &d) == MUON_ERR_DTYPE);
  CHECK(build_plan(&s, 1, MUON_BF16, MUON_BF16, MUON_BF16, &P, &d) == MUON_ERR_DTYPE);
  CHECK(build_plan(&s, 0, MUON_BF16, MUON_BF16, MUON_F32, &P, &d) == MUON_ERR_INVALID_ARG);
  CHECK(build_plan(nullptr, 1, MUON_BF16, MUON_BF16, MUON_F32, &P, &d) == MUON_ERR_INVALID_ARG);
}

static void test_tile_padding_independence() {
  // nine [2000, 2900] take 256-tiles (padded [2048, 3072]); one alone takes
  // 128-tiles ([2048, 2944]); the norm slots are the same either way
  CHECK(mfma_tile(2000, 2900, 9) == 256);
  CHECK(mfma_tile(2000, 2900, 1) == 128);
  Plan a = make(std::vector<muon_shape>(9, muon_shape{1, 2000, 2900}));
  Plan b = make({{1, 2000, 2900}});
  CHECK(a.groups[0].np != b.groups[0].np);
  CHECK(large_layout(a.groups[0], 1, MUON_BF16).tiles == large_layout(b.groups[0], 1, MUON_BF16).tiles);
}

static void test_assign() {
  std::vector<muon_shape> s = {{4, 96, 160}, {1, 24, 3000}, {1, 24, 3000}, {1, 200, 96}, {1, 96, 200}, {2, 24, 1000}};
  Plan P = make(s);
  for (int32_t R = 1; R <= 12; ++R) {
    std::vector<int32_t> own;
    std::vector<double> cost;
    assign_greedy(P, R, &own, &cost);
    CHECK(own.size() == P.mats.size() && cost.size() == size_t(R));
    std::vector<double> sum(size_t(R), 0.0);
    for (size_t j = 0; j < own.size(); ++j) {
      CHECK(own[j] >= 0 && own[j] < R);
      sum[size_t(own[j])] += ns_cost(P.mats[j].rows, P.mats[j].cols);
    }
    for (int32_t r = 0; r < R; ++r) CHECK(std::fabs(sum[size_t(r)] - cost[size_t(r)]) <= 1e-9 * (1.0 + cost[size_t(r)]));
  }
}

static void test_validation() {
  std::vector<muon_shape> s = {{1, 24, 1000}, {2, 64, 96}};
  Plan P = make(s);
  const int n = 2;
  alignas(256) static unsigned char fake[1024];
  void* p[2] = {fake + 16, fake + 32};
  const void* g[2] = {fake + 48, fake + 64};
  void* m[2] = {fake + 80, fake + 96};
  void* ws = fake + 256;
  const size_t wsb = P.ws_bytes;
  std::string d;
  auto step = [&](void* const* pp, const void* const* gg, void* const* mm, const muon_shape* sh, int32_t nn, float lr,
                  int32_t nest, int32_t steps, const void* w, size_t wb) {
    d.clear();
    const muon_status st = validate_step(&P, pp, gg, mm, sh, nn, lr, 0.95f, nest, 0.1f, 3.4445f, -4.775f, 2.0315f,
                                         steps, 1.0f, w, wb, &d);
    if (st != MUON_OK) CHECK(!d.empty());
    return st;
  };
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, 5, ws, wsb) == MUON_OK);
  CHECK(validate_step(nullptr, p, g, m, s.data(), n, 0.02f, 0.95f, 1, 0.1f, 1, 1, 1, 5, 1, ws, wsb, &d) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), 1, 0.02f, 1, 5, ws, wsb) == MUON_ERR_PLAN_MISMATCH);
  std::vector<muon_shape> s2 = s;
  s2[1].batch = 3;
  CHECK(step(p, g, m, s2.data(), n, 0.02f, 1, 5, ws, wsb) == MUON_ERR_PLAN_MISMATCH);
  CHECK(step(p, g, m, nullptr, n, 0.02f, 1, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  void* pnull[2] = {fake + 16, nullptr};
  CHECK(step(pnull, g, m, s.data(), n, 0.02f, 1, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  void* pmis[2] = {fake + 16, fake + 40};
  CHECK(step(pmis, g, m, s.data(), n, 0.02f, 1, 5, ws, wsb) == MUON_ERR_ALIGNMENT);
  CHECK(step(p, nullptr, m, s.data(), n, 0.02f, 1, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, nullptr, s.data(), n, 0.02f, 1, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), n, std::numeric_limits<float>::infinity(), 1, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), n, std::nanf(""), 1, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 2, 5, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, -1, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, kMaxNsSteps + 1, ws, wsb) == MUON_ERR_INVALID_ARG);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, kMaxNsSteps, ws, wsb) == MUON_OK);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, 0, ws, wsb) == MUON_OK);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, 5, nullptr, wsb) == MUON_ERR_WORKSPACE);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, 5, fake + 16, wsb) == MUON_ERR_WORKSPACE);
  CHECK(step(p, g, m, s.data(), n, 0.02f, 1, 5, ws, wsb - 1) == MUON_ERR_WORKSPACE);
  // muon_ns
  float* o[2] = {(float*)(fake + 16), (float*)(fake + 32)};
  CHECK(validate_ns(&P, g, o, s.data(), n, 1, 1, 1, 5, ws, wsb, &d) == MUON_OK);
  CHECK(validate_ns(&P, g, o, s.data(), n, std::nanf(""), 1, 1, 5, ws, wsb, &d) == MUON_ERR_INVALID_ARG);
  float* omis[2] = {(float*)(fake + 16), (float*)(fake + 36)};
  CHECK(validate_ns(&P, g, omis, s.data(), n, 1, 1, 1, 5, ws, wsb, &d) == MUON_ERR_ALIGNMENT);
  // shard update
  bool nothing = false;
  float* of = (float*)(fake + 512);
  CHECK(validate_shard_update(fake, MUON_BF16, of, 0, 0, 0.1f, 0.1f, 1, &nothing, &d) == MUON_OK && nothing);
  CHECK(validate_shard_update(fake, MUON_BF16, of, 0, 16, 0.1f, 0.1f, 1, &nothing, &d) == MUON_OK && !nothing);
  CHECK(validate_shard_update(of + 4, MUON_F32, of, 0, 16, 0.1f, 0.1f, 1, &nothing, &d) == MUON_ERR_INVALID_ARG);
  CHECK(validate_shard_update(fake, MUON_BF16, of, -1, 16, 0.1f, 0.1f, 1, &nothing, &d) == MUON_ERR_INVALID_ARG);
  CHECK(validate_shard_update(fake, muon_dtype(5), of, 0, 16, 0.1f, 0.1f, 1, &nothing, &d) == MUON_ERR_DTYPE);
  CHECK(validate_shard_update(nullptr, MUON_BF16, of, 0, 16, 0.1f, 0.1f, 1, &nothing, &d) == MUON_ERR_INVALID_ARG);
  // AdamW
  int64_t numels[2] = {8, 0};
  float* mv[2] = {(float*)(fake + 128), nullptr};
  CHECK(validate_adamw(p, g, mv, mv, numels, 2, MUON_BF16, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &d) == MUON_OK);
  CHECK(validate_adamw(p, g, mv, mv, numels, 2, MUON_BF16, 1e-3f, 1.0f, 0.95f, 1e-8f, 0.1f, 1, &d) == MUON_ERR_INVALID_ARG);
  CHECK(validate_adamw(p, g, mv, mv, numels, 2, MUON_BF16, 1e-3f, 0.9f, 0.95f, 0.0f, 0.1f, 1, &d) == MUON_ERR_INVALID_ARG);
  CHECK(validate_adamw(p, g, mv, mv, numels, 2, MUON_BF16, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 0, &d) == MUON_ERR_INVALID_ARG);
  int64_t neg[2] = {8, -1};
  CHECK(validate_adamw(p, g, mv, mv, neg, 2, MUON_BF16, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &d) == MUON_ERR_SHAPE);
  float* mvmis[2] = {(float*)(fake + 130), nullptr};
  CHECK(validate_adamw(p, g, mvmis, mv, numels, 2, MUON_BF16, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &d) == MUON_ERR_ALIGNMENT);
  CHECK(validate_adamw(nullptr, g, mv, mv, numels, 2, MUON_BF16, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &d) == MUON_ERR_INVALID_ARG);
  CHECK(validate_adamw(nullptr, nullptr, nullptr, nullptr, nullptr, 0, MUON_F32, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1, &d) == MUON_OK);
}

int main() {
  test_workload_plans();
  test_edge_plans();
  test_tile_padding_independence();
  test_assign();
  test_validation();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
