// Host check of the planner's grouped-GEMM tile lists (no device).  The
// planner's internals live in an anonymous namespace of muonh.cpp, so this
// translation unit includes that file; kernel launches come from the stubs.
//
// For every matrix set, both Newton-Schulz element types and both settings
// of `symmetric`, the plan built by build_plan must satisfy:
//  - coverage: every output tile of every product appears exactly once
//    (X X^T and A A: the upper tiles tm <= tn when symmetric, all tiles
//    otherwise; B'X: all tiles), padding slots aside, and nothing else;
//  - XCD placement: list entry i runs on XCD i mod 8 (the hardware's
//    round-robin), and all tiles of one unit (a matrix's group of up to 8
//    row panels) sit on the same XCD;
//  - order: within an XCD's share, the contraction length never increases
//    (longest first);
//  - the executed-FLOP count of the plan equals the sum over listed tiles;
//  - the small-problem path lists each 64 x 64 tile of the valid dims once;
//  - the momentum-unit, chunk and partial-slot tables (check_tables).
// Prints "all checks passed" and exits 0, or exits 1 at the first failure.
#include "../../pretraining_optimizer_amd/csrc/muonh.cpp"

#include <cstdio>
#include <map>
#include <set>
#include <string>

namespace {

#define CHECK(cond, what)                                                                  \
  do {                                                                                     \
    if (!(cond)) {                                                                         \
      std::fprintf(stderr, "CHECK failed (%s) at line %d: %s\n", (what), __LINE__, #cond); \
      return 1;                                                                            \
    }                                                                                      \
  } while (0)

muonh_matrix_desc md(int64_t r, int64_t c) {
  muonh_matrix_desc d;
  std::memset(&d, 0, sizeof(d));
  d.rows = r;
  d.cols = c;
  d.g_dtype = MUONH_BF16;
  return d;
}

std::vector<muonh_matrix_desc> qwen3(int64_t dm, int64_t dff, int64_t q, int64_t kv, bool fused) {
  std::vector<muonh_matrix_desc> v;
  for (int l = 0; l < 28; ++l) {
    if (fused) {
      v.push_back(md(q + 2 * kv, dm));
    } else {
      v.push_back(md(q, dm));
      v.push_back(md(kv, dm));
      v.push_back(md(kv, dm));
    }
    v.push_back(md(dm, q));
    if (fused) {
      v.push_back(md(2 * dff, dm));
    } else {
      v.push_back(md(dff, dm));
      v.push_back(md(dff, dm));
    }
    v.push_back(md(dm, dff));
  }
  return v;
}

// Ragged shapes from a fixed linear congruential sequence: sides in [1, 4096].
std::vector<muonh_matrix_desc> ragged(int count, uint64_t seed) {
  std::vector<muonh_matrix_desc> v;
  uint64_t s = seed;
  auto next = [&]() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (int64_t)(s >> 33);
  };
  for (int i = 0; i < count; ++i) v.push_back(md(1 + next() % 4096, 1 + next() % 4096));
  return v;
}

int check_big(const Plan& P, const std::string& name) {
  const char* what = name.c_str();
  double exec = 0.0;
  for (int k = 0; k < 3; ++k) {
    const auto& list = P.tiles[k];
    const bool sym = (k != kApply) && P.opt.symmetric != 0;
    std::map<std::tuple<int, int, int>, int> seen;
    std::map<std::pair<int, int>, int> unit_xcd;   // (prob, tm / 8) -> XCD
    std::vector<int64_t> last_k(kMaxXcd, INT64_MAX);
    for (size_t i = 0; i < list.size(); ++i) {
      const GemmTile& t = list[i];
      if (t.prob < 0) continue;
      CHECK(t.prob < P.n, what);
      const auto& m = P.mats[t.prob];
      const int mt = (int)(m.m_pad / kGemmTile), nt = (int)(m.n_pad / kGemmTile);
      const int cols = (k == kApply) ? nt : mt;
      CHECK(t.tm >= 0 && t.tm < mt && t.tn >= 0 && t.tn < cols, what);
      if (sym) CHECK(t.tm <= t.tn, what);
      CHECK(++seen[std::make_tuple((int)t.prob, (int)t.tm, (int)t.tn)] == 1, what);
      const int x = (int)(i % kMaxXcd);
      auto u = unit_xcd.emplace(std::make_pair((int)t.prob, t.tm / 8), x);
      CHECK(u.first->second == x, what);
      const int64_t K = (k == kGram) ? m.n_pad : m.m_pad;
      CHECK(K <= last_k[x], what);
      last_k[x] = K;
      exec += P.opt.ns_steps * 2.0 * kGemmTile * kGemmTile * (double)K;
    }
    size_t expected = 0;
    for (const auto& m : P.mats) {
      const int64_t mt = m.m_pad / kGemmTile, nt = m.n_pad / kGemmTile;
      expected += (k == kApply) ? (size_t)(mt * nt) : (size_t)(sym ? mt * (mt + 1) / 2 : mt * mt);
    }
    CHECK(seen.size() == expected, what);
    CHECK(list.empty() || list.back().prob >= 0, what);   // trailing padding trimmed
  }
  CHECK(std::fabs(exec - P.ns_exec) <= 1e-9 * P.ns_exec, what);
  return 0;
}

int check_small(const Plan& P, const std::string& name) {
  const char* what = name.c_str();
  for (int k = 0; k < 3; ++k) {
    std::set<std::tuple<int, int, int>> seen;
    for (const auto& t : P.tiles[k]) {
      CHECK(t.prob >= 0 && t.prob < P.n, what);
      const auto& m = P.mats[t.prob];
      const int mt = (int)((m.m + kSmallGemmTile - 1) / kSmallGemmTile);
      const int nt = (int)((m.n + kSmallGemmTile - 1) / kSmallGemmTile);
      CHECK(t.tm >= 0 && t.tm < mt && t.tn >= 0 && t.tn < (k == kApply ? nt : mt), what);
      CHECK(seen.insert(std::make_tuple((int)t.prob, (int)t.tm, (int)t.tn)).second, what);
    }
    size_t expected = 0;
    for (const auto& m : P.mats) {
      const int64_t mt = (m.m + kSmallGemmTile - 1) / kSmallGemmTile;
      const int64_t nt = (m.n + kSmallGemmTile - 1) / kSmallGemmTile;
      expected += (size_t)((k == kApply) ? mt * nt : mt * mt);
    }
    CHECK(seen.size() == expected, what);
  }
  return 0;
}

// The per-matrix tables the elementwise kernels and the finalisers index:
// momentum units (row segments of the padded grid when X_0 keeps M's
// orientation in the bf16 plan, 64 x 128 tiles otherwise) contiguous from the
// matrix's first unit and covering its padded grid once, row units before
// tile units; flat chunks covering its elements in order; and the partial
// slots of the last B'X launch laid out back to back.
int check_tables(const Plan& P, const std::string& name) {
  const char* what = name.c_str();
  int64_t part = 0;
  for (int32_t i = 0; i < P.n; ++i) {
    const auto& m = P.mats[i];
    const int64_t r_pad = m.tall ? m.n_pad : m.m_pad, c_pad = m.tall ? m.m_pad : m.n_pad;
    const bool rows = P.bf16 && !m.tall;
    const int64_t nseg = (c_pad + kMomRowSeg - 1) / kMomRowSeg;
    const int64_t want = rows ? r_pad * nseg : (r_pad / kMomTileR) * (c_pad / kMomTileC);
    CHECK(m.mom_ntiles == want, what);
    CHECK(m.mom_tile0 >= 0 && m.mom_tile0 + m.mom_ntiles <= (int64_t)P.mom_tiles.size(), what);
    CHECK(rows ? m.mom_tile0 + m.mom_ntiles <= P.mom_rows : m.mom_tile0 >= P.mom_rows, what);
    std::set<std::pair<int, int>> seen;
    for (int64_t j = m.mom_tile0; j < m.mom_tile0 + m.mom_ntiles; ++j) {
      const MomTile& u = P.mom_tiles[j];
      CHECK(u.mat == i && u.kind == (rows ? 1 : 0), what);
      CHECK(u.tr >= 0 && u.tc >= 0, what);
      CHECK(rows ? (u.tr < r_pad && u.tc < nseg) : (u.tr < r_pad / kMomTileR && u.tc < c_pad / kMomTileC), what);
      CHECK(seen.insert({u.tr, u.tc}).second, what);
    }
    const int64_t elems = m.rows * m.cols;
    CHECK(m.nchunks == (elems + kChunk - 1) / kChunk, what);
    for (int64_t j = 0; j < m.nchunks; ++j) {
      const Chunk& c = P.chunks[m.chunk0 + j];
      CHECK(c.mat == i && c.start == j * kChunk && c.len == std::min<int64_t>(kChunk, elems - c.start), what);
    }
    CHECK(m.part0 == part, what);
    part += m.nparts;
  }
  CHECK(part == P.nparts, what);
  int64_t units = 0, chunks = 0;
  for (const auto& m : P.mats) units += m.mom_ntiles, chunks += m.nchunks;
  CHECK(units == (int64_t)P.mom_tiles.size() && chunks == (int64_t)P.chunks.size(), what);
  return 0;
}

}  // namespace

int main() {
  std::vector<std::pair<std::string, std::vector<muonh_matrix_desc>>> sets = {
      {"qwen3_1.7b", qwen3(2048, 6144, 2048, 1024, false)},
      {"qwen3_1.7b_fused", qwen3(2048, 6144, 2048, 1024, true)},
      {"qwen3_0.6b", qwen3(1024, 3072, 2048, 1024, false)},
      {"ragged_64", ragged(64, 7)},
      {"ragged_5", ragged(5, 11)},
      {"single", {md(256, 128)}},
      {"vectors", {md(1, 37), md(37, 1), md(1, 1)}},
  };
  std::vector<muonh_matrix_desc> m170;
  for (int l = 0; l < 12; ++l) {
    for (int q = 0; q < 4; ++q) m170.push_back(md(768, 768));
    m170.push_back(md(2048, 768));
    m170.push_back(md(2048, 768));
    m170.push_back(md(768, 2048));
  }
  sets.push_back({"diag170m", m170});
  int plans = 0, small = 0;
  for (const auto& [name, mats] : sets) {
    for (int ns : {MUONH_BF16, MUONH_F32})
      for (int sym : {1, 0}) {
        muonh_options opt;
        muonh_default_options(&opt);
        opt.ns_dtype = ns;
        opt.symmetric = sym;
        Plan P;
        const int rc = build_plan(mats.data(), (int32_t)mats.size(), opt, P);
        const std::string tag = name + (ns == MUONH_BF16 ? " bf16" : " f32") + (sym ? " sym" : " full");
        if (rc != MUONH_OK) {
          std::fprintf(stderr, "build_plan failed for %s: %s\n", tag.c_str(), muonh_last_error());
          return 1;
        }
        if ((P.small_gemm ? check_small(P, tag) : check_big(P, tag)) != 0) return 1;
        if (check_tables(P, tag) != 0) return 1;
        ++plans;
        small += P.small_gemm;
      }
  }
  std::printf("%d plans (%d on the small-problem path): all checks passed\n", plans, small);
  return 0;
}
