// Host side of the MuonH library: argument validation, the plan (Newton-Schulz
// orientation, padding, shape buckets, XCD-aware tile lists, workspace
// layout), the launch sequence of one step and the C ABI of include/muonh.h.
//
// The step computed is the Hyperball update of Eq. (1) in "Puro-2B: Poor
// Lab's Qwen2-1.5B Trained on RTX 5090 within $5090" (arXiv HTML §3.3) on
// top of momentum and Newton-Schulz (the Muon update named there), with the
// ordinary-Muon (Eq. (3)) and ELR-aligned (Eq. (5)) updates of §3.3.1 as
// alternative modes.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"

using namespace muonh;

namespace {
thread_local std::string g_last_error;
}  // namespace

int muonh::set_last_error(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

namespace {

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(MUONH_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));       \
  } while (0)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kMaxDim = 1 << 16;   // padded Newton-Schulz dims fit int32 tile math
constexpr size_t kAlign = 256;
constexpr size_t kNoBuffer = ~(size_t)0;   // workspace offset of a buffer the plan does not have

struct MatPlan {
  int64_t rows, cols;
  int tall, g_bf16;
  int64_t m, n, m_pad, n_pad;
  float radius_in;
  size_t off_X[2], off_XT[2], off_A, off_B, off_U;
  int64_t mom_tile0, mom_ntiles, chunk0, nchunks;
  int64_t part0, nparts;   // update-statistics partial slots (tile x wavefront of the last B'X)
};

struct Plan {
  muonh_options opt;
  int32_t n = 0;
  bool bf16 = true;
  size_t tsize = 2;
  std::vector<MatPlan> mats;
  std::vector<MomTile> mom_tiles;   // row units (the first mom_rows), then tile units
  int64_t mom_rows = 0;
  bool small_gemm = false;          // the small-problem GEMM path (64 x 64 tiles)
  std::vector<Chunk> chunks;
  std::vector<GemmTile> tiles[3];
  int n_buckets = 0;
  double ns_dense = 0, ns_exec = 0, elem_bytes = 0;
  // workspace layout (byte offsets)
  size_t off_geo, off_ptrs, off_scal, off_stats, off_need, off_elr, off_eta;
  size_t off_mom_tiles, off_chunks, off_tiles[3];
  size_t off_probs_gram[2], off_probs_poly, off_probs_apply[2];
  size_t off_part_mom, off_part_radius, off_part_upd;
  int64_t nparts = 0;
  size_t total = 0;
};

int check_options(const muonh_options& o) {
  if (!(o.ns_steps >= 1 && o.ns_steps <= 16))
    return fail(MUONH_EINVAL, "ns_steps must be in [1, 16]");
  if (o.ns_dtype != MUONH_BF16 && o.ns_dtype != MUONH_F32)
    return fail(MUONH_EINVAL, "ns_dtype must be MUONH_BF16 or MUONH_F32");
  if (o.mode < MUONH_MODE_HYPERBALL || o.mode > MUONH_MODE_ELR_ALIGNED)
    return fail(MUONH_EINVAL, "unknown mode");
  if (!std::isfinite(o.beta) || !std::isfinite(o.ns_a) || !std::isfinite(o.ns_b) ||
      !std::isfinite(o.ns_c) || !std::isfinite(o.ns_eps) || o.ns_eps < 0.0f ||
      !std::isfinite(o.weight_decay))
    return fail(MUONH_EINVAL, "non-finite or negative option value");
  if (o.nesterov != 0 && o.nesterov != 1) return fail(MUONH_EINVAL, "nesterov must be 0 or 1");
  if (o.deterministic != 0 && o.deterministic != 1)
    return fail(MUONH_EINVAL, "deterministic must be 0 or 1");
  return MUONH_OK;
}

int check_shapes(const muonh_matrix_desc* mats, int32_t n) {
  if (n <= 0) return fail(MUONH_EINVAL, "matrix count must be >= 1");
  if (!mats) return fail(MUONH_EINVAL, "null matrix list");
  for (int32_t i = 0; i < n; ++i) {
    const auto& d = mats[i];
    if (d.rows < 1 || d.cols < 1)
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": dims must be >= 1");
    if (std::min(d.rows, d.cols) > kMaxDim || std::max(d.rows, d.cols) > kMaxDim)
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": dims above 65536");
    if (d.g_dtype != MUONH_F32 && d.g_dtype != MUONH_BF16)
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": g_dtype must be F32 or BF16");
    if (!std::isfinite(d.radius))
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": non-finite radius");
  }
  return MUONH_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_pointers(const muonh_matrix_desc* mats, int32_t n, bool need_gm) {
  for (int32_t i = 0; i < n; ++i) {
    const auto& d = mats[i];
    if (!d.w || !aligned16(d.w))
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": w is null or not 16-byte aligned");
    if (need_gm) {
      if (!d.g || !aligned16(d.g))
        return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": g is null or not 16-byte aligned");
      if (!d.m || !aligned16(d.m))
        return fail(MUONH_EINVAL, "matrix " + std::to_string(i) + ": m is null or not 16-byte aligned");
    }
  }
  return MUONH_OK;
}

// XCD-aware tile list for one grouped GEMM launch.
//   dims[p] = (M tiles, N tiles, K), upper = list only tm <= tn.
// Units are (problem, group of up to 8 row panels); units are placed on the
// 8 XCDs by longest-processing-time first, each XCD's units are ordered by
// contraction length (longest first), then problem and group, tiles inside a
// unit run column-major (a column of 8 row tiles shares its Q panel,
// consecutive columns share the P panels), and the per-XCD lists are
// interleaved so workgroup 8j + x runs XCD x's j-th tile.
std::vector<GemmTile> build_tile_list(const std::vector<std::tuple<int, int, int64_t>>& dims,
                                      bool upper) {
  struct Unit {
    int prob, g0, g1;
    double cost;
  };
  constexpr int kGroup = 8;
  std::vector<Unit> units;
  for (size_t p = 0; p < dims.size(); ++p) {
    const int mt = std::get<0>(dims[p]), nt = std::get<1>(dims[p]);
    const int64_t K = std::get<2>(dims[p]);
    for (int g0 = 0; g0 < mt; g0 += kGroup) {
      const int g1 = std::min(mt, g0 + kGroup);
      int64_t cnt = 0;
      for (int tm = g0; tm < g1; ++tm) cnt += upper ? (nt - tm) : nt;
      units.push_back({(int)p, g0, g1, (double)cnt * (double)K});
    }
  }
  std::vector<int> order(units.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return units[a].cost > units[b].cost; });
  std::vector<std::vector<int>> bins(kMaxXcd);
  std::vector<double> load(kMaxXcd, 0.0);
  for (int u : order) {
    const int b = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    bins[b].push_back(u);
    load[b] += units[u].cost;
  }
  std::vector<std::vector<GemmTile>> lists(kMaxXcd);
  size_t longest = 0;
  for (int x = 0; x < kMaxXcd; ++x) {
    // Longest contraction first (then by problem and group): the XCD's CUs
    // take tiles in list order as they free up, so short tiles fill the end
    // of the launch instead of a long one starting last.
    std::sort(bins[x].begin(), bins[x].end(), [&](int a, int b) {
      const int64_t ka = std::get<2>(dims[units[a].prob]), kb = std::get<2>(dims[units[b].prob]);
      if (ka != kb) return ka > kb;
      return std::make_pair(units[a].prob, units[a].g0) < std::make_pair(units[b].prob, units[b].g0);
    });
    for (int u : bins[x]) {
      const Unit& un = units[u];
      const int nt = std::get<1>(dims[un.prob]);
      for (int tn = 0; tn < nt; ++tn)
        for (int tm = un.g0; tm < un.g1; ++tm)
          if (!upper || tm <= tn) lists[x].push_back({un.prob, (int16_t)tm, (int16_t)tn});
    }
    longest = std::max(longest, lists[x].size());
  }
  std::vector<GemmTile> out(longest * kMaxXcd, GemmTile{-1, 0, 0});
  for (int x = 0; x < kMaxXcd; ++x)
    for (size_t j = 0; j < lists[x].size(); ++j) out[j * kMaxXcd + x] = lists[x][j];
  // Trim trailing empty slots.
  while (!out.empty() && out.back().prob < 0) out.pop_back();
  return out;
}

int build_plan(const muonh_matrix_desc* mats, int32_t n, const muonh_options& opt, Plan& P) {
  int rc = check_options(opt);
  if (rc) return rc;
  rc = check_shapes(mats, n);
  if (rc) return rc;
  P.opt = opt;
  P.n = n;
  P.bf16 = opt.ns_dtype == MUONH_BF16;
  P.tsize = P.bf16 ? 2 : 4;
  P.mats.resize(n);
  std::map<std::pair<int64_t, int64_t>, int> buckets;
  int64_t nchunks = 0;
  std::vector<MomTile> row_units, tile_units;
  for (int32_t i = 0; i < n; ++i) {
    MatPlan& m = P.mats[i];
    m.rows = mats[i].rows;
    m.cols = mats[i].cols;
    m.tall = m.rows > m.cols;
    m.g_bf16 = mats[i].g_dtype == MUONH_BF16;
    m.m = std::min(m.rows, m.cols);
    m.n = std::max(m.rows, m.cols);
    m.m_pad = round_up(m.m, kPad);
    m.n_pad = round_up(m.n, kPad);
    m.radius_in = mats[i].radius;
    buckets[{m.m_pad, m.n_pad}]++;
    const int64_t r_pad = m.tall ? m.n_pad : m.m_pad, c_pad = m.tall ? m.m_pad : m.n_pad;
    // Momentum units: row segments where X_0 keeps M's orientation and has
    // no transposed copy, 64 x 128 tiles otherwise.  All row units come first
    // (one launch each kind); mom_tile0 is made global after the loop.
    if (P.bf16 && !m.tall) {
      const int64_t nseg = (c_pad + kMomRowSeg - 1) / kMomRowSeg;
      m.mom_tile0 = (int64_t)row_units.size();
      m.mom_ntiles = r_pad * nseg;
      for (int64_t r = 0; r < r_pad; ++r)
        for (int64_t sg = 0; sg < nseg; ++sg)
          row_units.push_back({i, (int32_t)r, (int32_t)sg, 1});
    } else {
      m.mom_tile0 = -1 - (int64_t)tile_units.size();   // made global below
      m.mom_ntiles = (r_pad / kMomTileR) * (c_pad / kMomTileC);
      for (int64_t tr = 0; tr < r_pad / kMomTileR; ++tr)
        for (int64_t tc = 0; tc < c_pad / kMomTileC; ++tc)
          tile_units.push_back({i, (int32_t)tr, (int32_t)tc, 0});
    }
    const int64_t elems = m.rows * m.cols;
    m.chunk0 = nchunks;
    m.nchunks = (elems + kChunk - 1) / kChunk;
    for (int64_t s = 0; s < elems; s += kChunk)
      P.chunks.push_back({i, (int32_t)std::min<int64_t>(kChunk, elems - s), s});
    nchunks += m.nchunks;
    const double mm = (double)m.m, nn = (double)m.n;
    P.ns_dense += opt.ns_steps * (4.0 * mm * mm * nn + 2.0 * mm * mm * mm);
    P.elem_bytes += (double)elems * ((m.g_bf16 ? 2.0 : 4.0) + 8.0 + 8.0);
  }
  P.n_buckets = (int)buckets.size();
  P.mom_rows = (int64_t)row_units.size();
  P.mom_tiles = std::move(row_units);
  P.mom_tiles.insert(P.mom_tiles.end(), tile_units.begin(), tile_units.end());
  for (auto& m : P.mats)
    if (m.mom_tile0 < 0) m.mom_tile0 = P.mom_rows + (-1 - m.mom_tile0);
  // GEMM path: 256 x 256 tiles, or, when the largest product (B'X) has too
  // few of them to occupy the GPU, the small-problem path (64 x 64 tiles over
  // the valid dims).  MUONH_GEMM_TILE=64 or 256 forces one of the two.
  int64_t big_tiles = 0;
  for (const auto& m : P.mats) big_tiles += (m.m_pad / kGemmTile) * (m.n_pad / kGemmTile);
  P.small_gemm = big_tiles < kSmallPlanTiles;
  if (const char* f = std::getenv("MUONH_GEMM_TILE")) {
    if (std::strcmp(f, "64") == 0) P.small_gemm = true;
    if (std::strcmp(f, "256") == 0) P.small_gemm = false;
  }
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  // Partial slots of the last B'X launch: one per output tile and wavefront.
  for (auto& m : P.mats) {
    m.part0 = P.nparts;
    m.nparts = P.small_gemm
                   ? cdiv(m.m, kSmallGemmTile) * cdiv(m.n, kSmallGemmTile) * (kGemmThreads / 64)
                   : (m.m_pad / kGemmTile) * (m.n_pad / kGemmTile) * (kGemmThreads / 64);
    P.nparts += m.nparts;
  }

  // GEMM tile lists.
  if (P.small_gemm) {
    const int64_t kks = 64 / (int64_t)P.tsize;   // K elements per stage of the small kernel
    for (int32_t p = 0; p < n; ++p) {
      const auto& m = P.mats[p];
      const int mt = (int)cdiv(m.m, kSmallGemmTile), nt = (int)cdiv(m.n, kSmallGemmTile);
      for (int tm = 0; tm < mt; ++tm)
        for (int tn = 0; tn < mt; ++tn) {
          P.tiles[kGram].push_back({p, (int16_t)tm, (int16_t)tn});
          P.tiles[kPoly].push_back({p, (int16_t)tm, (int16_t)tn});
        }
      for (int tm = 0; tm < mt; ++tm)
        for (int tn = 0; tn < nt; ++tn) P.tiles[kApply].push_back({p, (int16_t)tm, (int16_t)tn});
      const double t2 = 2.0 * kSmallGemmTile * kSmallGemmTile;
      const double kn = (double)(cdiv(m.n, kks) * kks), km = (double)(cdiv(m.m, kks) * kks);
      P.ns_exec += opt.ns_steps * t2 * ((double)mt * mt * kn + (double)mt * mt * km + (double)mt * nt * km);
    }
  } else {
    std::vector<std::tuple<int, int, int64_t>> d_gram, d_poly, d_apply;
    for (const auto& m : P.mats) {
      const int mt = (int)(m.m_pad / kGemmTile), nt = (int)(m.n_pad / kGemmTile);
      d_gram.emplace_back(mt, mt, m.n_pad);
      d_poly.emplace_back(mt, mt, m.m_pad);
      d_apply.emplace_back(mt, nt, m.m_pad);
    }
    const bool sym = opt.symmetric != 0;
    P.tiles[kGram] = build_tile_list(d_gram, sym);
    P.tiles[kPoly] = build_tile_list(d_poly, sym);
    P.tiles[kApply] = build_tile_list(d_apply, false);
    for (int k = 0; k < 3; ++k)
      for (const auto& t : P.tiles[k])
        if (t.prob >= 0) {
          const auto& m = P.mats[t.prob];
          const double K = (k == kGram) ? (double)m.n_pad : (double)m.m_pad;
          P.ns_exec += opt.ns_steps * 2.0 * kGemmTile * kGemmTile * K;
        }
  }

  // Workspace layout: tables first, then the large per-matrix buffers.
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  P.off_geo = take(sizeof(MatGeom) * n);
  P.off_ptrs = take(sizeof(MatPtrs) * n);
  P.off_scal = take(sizeof(MatScalars) * n);
  P.off_stats = take(sizeof(muonh_stats) * n);
  P.off_need = take(sizeof(int32_t) * n);
  P.off_elr = take(sizeof(float) * n);
  P.off_eta = take(sizeof(double) * n);
  P.off_mom_tiles = take(sizeof(MomTile) * P.mom_tiles.size());
  P.off_chunks = take(sizeof(Chunk) * P.chunks.size());
  for (int k = 0; k < 3; ++k) P.off_tiles[k] = take(sizeof(GemmTile) * std::max<size_t>(1, P.tiles[k].size()));
  for (int k = 0; k < 2; ++k) P.off_probs_gram[k] = take(sizeof(GemmProb) * n);
  P.off_probs_poly = take(sizeof(GemmProb) * n);
  for (int k = 0; k < 2; ++k) P.off_probs_apply[k] = take(sizeof(GemmProb) * n);
  P.off_part_mom = take(sizeof(double) * kMomParts * P.mom_tiles.size());
  P.off_part_radius = take(sizeof(double) * P.chunks.size());   // one ||W_0||^2 partial per chunk
  P.off_part_upd = take(sizeof(double) * 3 * (size_t)std::max<int64_t>(1, P.nparts));
  // Every Newton-Schulz buffer row is kRowSkewBytes longer than the padded
  // dim: with power-of-two pitches the 256 rows a tile streams at one K
  // offset would all land in the same L2 channel.
  // The bf16 path keeps the iterate in one layout (the GEMM reads X^T out of
  // X through transposing LDS reads); the fp32 path also stores X^T.
  const int64_t skew = kRowSkewBytes / (int64_t)P.tsize;
  const bool dual = P.tsize == 4;
  for (auto& m : P.mats) {
    const size_t ldn = (size_t)(m.n_pad + skew), ldm = (size_t)(m.m_pad + skew);
    for (int k = 0; k < 2; ++k) {
      m.off_X[k] = take((size_t)m.m_pad * ldn * P.tsize);
      m.off_XT[k] = dual ? take((size_t)m.n_pad * ldm * P.tsize) : kNoBuffer;
    }
    m.off_A = take((size_t)m.m_pad * ldm * P.tsize);
    m.off_B = take((size_t)m.m_pad * ldm * P.tsize);
    m.off_U = take((size_t)m.rows * m.cols * P.tsize);
  }
  P.total = off;
  return MUONH_OK;
}

// Host image of the workspace's table region [0, pl.off_part_mom) for a
// workspace at device address `ws`: geometry, radii (R where given, else 0
// with need = 1), zeroed statistics and step-size slots, the momentum units,
// chunk and tile lists, the GEMM problem descriptors and, when `mats` carries
// pointers (any w non-null), the pointer table.  The partial-sum slots that
// follow are rewritten by every step before they are read.
void build_table_image(const Plan& pl, uint8_t* ws, const muonh_matrix_desc* mats,
                       std::vector<uint8_t>& img, std::vector<int32_t>& need) {
  const int32_t n = pl.n;
  img.assign(pl.off_part_mom, 0);
  need.assign(n, 0);
  auto put = [&](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(img.data() + off, src, bytes);
  };
  std::vector<MatGeom> geo(n);
  std::vector<MatScalars> scal(n);
  std::vector<GemmProb> gram[2], poly(n), apply[2];
  for (int k = 0; k < 2; ++k) {
    gram[k].resize(n);
    apply[k].resize(n);
  }
  for (int32_t i = 0; i < n; ++i) {
    const MatPlan& m = pl.mats[i];
    MatGeom& g = geo[i];
    g.rows = m.rows;
    g.cols = m.cols;
    g.tall = m.tall;
    g.g_bf16 = m.g_bf16;
    g.m_pad = (int32_t)m.m_pad;
    g.n_pad = (int32_t)m.n_pad;
    g.r_pad = (int32_t)(m.tall ? m.n_pad : m.m_pad);
    g.c_pad = (int32_t)(m.tall ? m.m_pad : m.n_pad);
    g.ld_skew = (int32_t)(kRowSkewBytes / pl.tsize);
    for (int k = 0; k < 2; ++k) {
      g.X[k] = ws + m.off_X[k];
      g.XT[k] = m.off_XT[k] == kNoBuffer ? nullptr : ws + m.off_XT[k];
    }
    g.U = ws + m.off_U;
    g.mom_tile0 = m.mom_tile0;
    g.mom_ntiles = m.mom_ntiles;
    g.chunk0 = m.chunk0;
    g.nchunks = m.nchunks;
    g.part0 = m.part0;
    g.nparts = m.nparts;
    scal[i] = MatScalars{m.radius_in > 0.0f ? (double)m.radius_in : 0.0, 0.0, 1.0f, 1.0f, 0.0f, 0.0f};
    need[i] = m.radius_in > 0.0f ? 0 : 1;
    const int32_t M = (int32_t)m.m_pad, N = (int32_t)m.n_pad;
    const int32_t LM = M + g.ld_skew, LN = N + g.ld_skew;   // row pitches
    for (int k = 0; k < 2; ++k) {
      GemmProb& a = gram[k][i];
      std::memset(&a, 0, sizeof(a));
      a.P = a.Q = g.X[k];
      a.O = ws + m.off_A;
      a.M = a.N = M;
      a.K = N;
      a.ldp = a.ldq = LN;
      a.ldo = LM;
      a.um = a.un = (int32_t)m.m;
      a.uk = (int32_t)m.n;
      a.mat = i;
      GemmProb& c = apply[k][i];
      std::memset(&c, 0, sizeof(c));
      c.P = ws + m.off_B;
      c.Q = g.XT[k] ? g.XT[k] : g.X[k];   // bf16: X itself, read K-major
      c.E = nullptr;
      c.O = g.X[k ^ 1];
      c.OT = g.XT[k ^ 1];
      c.U = g.U;
      c.M = M;
      c.N = N;
      c.K = M;
      c.ldp = LM;
      c.ldq = g.XT[k] ? LM : LN;
      c.lde = LM;
      c.ldo = LN;
      c.ldot = LM;
      c.um = (int32_t)m.m;
      c.un = (int32_t)m.n;
      c.uk = (int32_t)m.m;
      c.u_tall = m.tall;
      c.mat = i;
      c.part0 = (int32_t)m.part0;
    }
    GemmProb& b = poly[i];
    std::memset(&b, 0, sizeof(b));
    b.P = b.Q = b.E = ws + m.off_A;
    b.O = ws + m.off_B;
    b.M = b.N = b.K = M;
    b.ldp = b.ldq = b.lde = b.ldo = LM;
    b.um = b.un = b.uk = (int32_t)m.m;
    b.mat = i;
  }
  put(pl.off_geo, geo.data(), sizeof(MatGeom) * n);
  put(pl.off_scal, scal.data(), sizeof(MatScalars) * n);
  put(pl.off_need, need.data(), sizeof(int32_t) * n);
  put(pl.off_mom_tiles, pl.mom_tiles.data(), sizeof(MomTile) * pl.mom_tiles.size());
  put(pl.off_chunks, pl.chunks.data(), sizeof(Chunk) * pl.chunks.size());
  put(pl.off_probs_poly, poly.data(), sizeof(GemmProb) * n);
  for (int k = 0; k < 3; ++k)
    put(pl.off_tiles[k], pl.tiles[k].data(), sizeof(GemmTile) * pl.tiles[k].size());
  for (int k = 0; k < 2; ++k) {
    put(pl.off_probs_gram[k], gram[k].data(), sizeof(GemmProb) * n);
    put(pl.off_probs_apply[k], apply[k].data(), sizeof(GemmProb) * n);
  }
  bool have_ptrs = false;
  for (int32_t i = 0; i < n; ++i) have_ptrs |= mats[i].w != nullptr;
  if (have_ptrs) {
    std::vector<MatPtrs> ptrs(n);
    for (int32_t i = 0; i < n; ++i)
      ptrs[i] = MatPtrs{reinterpret_cast<float*>(mats[i].w), mats[i].g,
                        reinterpret_cast<float*>(mats[i].m)};
    put(pl.off_ptrs, ptrs.data(), sizeof(MatPtrs) * n);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// handle

struct muonh_handle {
  Plan plan;
  int device = -1;
  uint8_t* ws = nullptr;
  bool owns_ws = false;
  // Pinned staging for per-step uploads (pointer table, per-matrix LR factors).
  uint8_t* staging = nullptr;
  size_t staging_bytes = 0;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  std::vector<MatPtrs> cur_ptrs;   // what the device pointer table holds
  bool ptrs_valid = false;
  // The stream of the handle's last enqueued work (init, a step, a copy of
  // u).  Work enqueued on another stream first waits for it (order_ev), so
  // the handle's workspace is only ever used in call order.
  hipStream_t last_stream = nullptr;
  hipEvent_t order_ev = nullptr;
  int64_t steps_done = 0;
  // timing: a ring of per-step event sets, folded into totals lazily
  static constexpr int kRing = 4;
  bool timing = false;
  std::vector<hipEvent_t> ev[kRing];
  bool ev_pending[kRing] = {false, false, false, false};
  int ev_next = 0;
  int ev_cur = 0;
  double phase_total[7] = {0, 0, 0, 0, 0, 0, 0};
  int32_t timed_steps = 0;
  // MUONH_DEBUG_SYNC=1: synchronise after every launch and report which
  // kernel failed (slow; for attributing device faults).
  bool debug_sync = false;
  // Recorded step for muonh_step_graph (made on its first call).
  hipStream_t cap_stream = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;

  template <typename T> T* at(size_t off) { return reinterpret_cast<T*>(ws + off); }
};

namespace {

// Orders work about to be enqueued on `st` after everything the handle
// enqueued before (on h->last_stream), then makes `st` the last stream.
// Every entry point that enqueues device work calls this first.
int order_after_last(muonh_handle* h, hipStream_t st) {
  if (st != h->last_stream) {
    HIP_TRY(hipEventRecord(h->order_ev, h->last_stream));
    HIP_TRY(hipStreamWaitEvent(st, h->order_ev, 0));
    h->last_stream = st;
  }
  return MUONH_OK;
}

int upload_async(muonh_handle* h, void* dst, const void* src, size_t bytes, size_t staging_off,
                 hipStream_t st) {
  // The staging buffer is reused: wait until the previous upload has been
  // consumed by the device before overwriting it.
  if (h->upload_pending) {
    HIP_TRY(hipEventSynchronize(h->upload_done));
    h->upload_pending = false;
  }
  std::memcpy(h->staging + staging_off, src, bytes);
  HIP_TRY(hipMemcpyAsync(dst, h->staging + staging_off, bytes, hipMemcpyHostToDevice, st));
  return MUONH_OK;
}

int check_same_list(const muonh_handle* h, const muonh_matrix_desc* mats, int32_t n) {
  if (n != h->plan.n) return fail(MUONH_EMISMATCH, "matrix count differs from init");
  if (!mats) return fail(MUONH_EINVAL, "null matrix list");
  for (int32_t i = 0; i < n; ++i) {
    const auto& m = h->plan.mats[i];
    if (mats[i].rows != m.rows || mats[i].cols != m.cols ||
        (mats[i].g_dtype == MUONH_BF16) != (m.g_bf16 != 0))
      return fail(MUONH_EMISMATCH, "matrix " + std::to_string(i) + ": shape or dtype differs from init");
  }
  return MUONH_OK;
}

int record(muonh_handle* h, size_t idx, hipStream_t st) {
  if (!h->timing) return MUONH_OK;
  HIP_TRY(hipEventRecord(h->ev[h->ev_cur][idx], st));
  return MUONH_OK;
}

// Wait for event set k, add its phase durations to the totals.
int fold_events(muonh_handle* h, int k) {
  if (!h->ev_pending[k]) return MUONH_OK;
  const auto& ev = h->ev[k];
  const int S = h->plan.opt.ns_steps;
  HIP_TRY(hipEventSynchronize(ev[3 * (size_t)S + 3]));
  auto el = [&](size_t a, size_t b, double* acc) -> int {
    float ms = 0.0f;
    HIP_TRY(hipEventElapsedTime(&ms, ev[a], ev[b]));
    *acc += ms;
    return MUONH_OK;
  };
  int rc;
  if ((rc = el(0, 1, &h->phase_total[0]))) return rc;
  size_t e = 1;
  for (int it = 0; it < S; ++it)
    for (int k3 = 0; k3 < 3; ++k3, ++e) {
      const int ph = (k3 == 2 && it == S - 1) ? 4 : 1 + k3;   // last B X launch apart
      if ((rc = el(e, e + 1, &h->phase_total[ph]))) return rc;
    }
  if ((rc = el(e, e + 1, &h->phase_total[5]))) return rc;
  if ((rc = el(e + 1, e + 2, &h->phase_total[6]))) return rc;
  h->ev_pending[k] = false;
  h->timed_steps++;
  return MUONH_OK;
}

}  // namespace

extern "C" {

void muonh_default_options(muonh_options* opt) {
  if (!opt) return;
  std::memset(opt, 0, sizeof(*opt));
  opt->beta = 0.95f;
  opt->ns_steps = 5;
  opt->ns_a = 3.4445f;
  opt->ns_b = -4.7750f;
  opt->ns_c = 2.0315f;
  opt->ns_eps = 1e-7f;
  opt->ns_dtype = MUONH_BF16;
  opt->nesterov = 0;
  opt->mode = MUONH_MODE_HYPERBALL;
  opt->weight_decay = 0.0f;
  opt->symmetric = 1;
  opt->deterministic = 1;
  opt->workspace = nullptr;
  opt->workspace_bytes = 0;
}

int muonh_workspace_size(const muonh_matrix_desc* mats, int32_t n, const muonh_options* opt,
                         size_t* bytes) {
  if (!opt || !bytes) return fail(MUONH_EINVAL, "null argument");
  Plan P;
  const int rc = build_plan(mats, n, *opt, P);
  if (rc) return rc;
  *bytes = P.total;
  return MUONH_OK;
}

int muonh_plan_query(const muonh_matrix_desc* mats, int32_t n, const muonh_options* opt,
                     muonh_plan_info* info) {
  if (!opt || !info) return fail(MUONH_EINVAL, "null argument");
  Plan P;
  const int rc = build_plan(mats, n, *opt, P);
  if (rc) return rc;
  std::memset(info, 0, sizeof(*info));
  info->n_matrices = n;
  info->n_buckets = P.n_buckets;
  for (int k = 0; k < 3; ++k) {
    int64_t c = 0;
    for (const auto& t : P.tiles[k]) c += t.prob >= 0;
    info->gemm_tiles[k] = c;
  }
  info->mom_tiles = (int64_t)P.mom_tiles.size();
  info->flat_chunks = (int64_t)P.chunks.size();
  info->ns_dense_flops = P.ns_dense;
  info->ns_exec_flops = P.ns_exec;
  info->elem_bytes = P.elem_bytes;
  info->workspace_bytes = P.total;
  return MUONH_OK;
}

int muonh_init(muonh_handle** out, const muonh_matrix_desc* mats, int32_t n,
               const muonh_options* opt, void* stream) {
  if (!out) return fail(MUONH_EINVAL, "null handle pointer");
  *out = nullptr;
  if (!opt) return fail(MUONH_EINVAL, "null options");
  Plan P;
  int rc = build_plan(mats, n, *opt, P);
  if (rc) return rc;
  for (int32_t i = 0; i < n; ++i)
    if (mats[i].radius <= 0.0f && (!mats[i].w || !aligned16(mats[i].w)))
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) +
                                    ": radius <= 0 needs a 16-byte aligned w to measure ||W_0||");
  if (opt->workspace && opt->workspace_bytes < P.total)
    return fail(MUONH_ENOMEM, "workspace too small: need " + std::to_string(P.total) + " bytes");
  if (opt->workspace && (reinterpret_cast<uintptr_t>(opt->workspace) & (kAlign - 1)) != 0)
    return fail(MUONH_EINVAL, "workspace must be 256-byte aligned");

  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MUONH_ENODEV, std::string("device is ") + prop.gcnArchName + ", library is built for gfx950");

  auto* h = new muonh_handle();
  h->plan = std::move(P);
  h->device = dev;
  const Plan& pl = h->plan;
  if (const char* e = std::getenv("MUONH_DEBUG_SYNC")) h->debug_sync = std::atoi(e) != 0;
  if (const char* e = std::getenv("MUONH_LOG"); e && std::atoi(e) != 0) {
    // MUONH_LOG=1: the plan on stderr.
    size_t gt[3] = {0, 0, 0};
    for (int k = 0; k < 3; ++k)
      for (const auto& t : pl.tiles[k]) gt[k] += t.prob >= 0;
    std::fprintf(stderr,
                 "muonh: %d matrices in %d shape buckets, ns %s x%d; GEMM tiles (%dx%d) gram %zu "
                 "poly %zu apply %zu; %zu momentum tiles, %zu chunks; workspace %.3f GB; NS %.3e "
                 "dense / %.3e executed FLOP per step\n",
                 n, pl.n_buckets, pl.bf16 ? "bf16" : "fp32", pl.opt.ns_steps,
                 pl.small_gemm ? kSmallGemmTile : kGemmTile, pl.small_gemm ? kSmallGemmTile : kGemmTile,
                 gt[0], gt[1], gt[2],
                 pl.mom_tiles.size(), pl.chunks.size(), pl.total / 1e9, pl.ns_dense, pl.ns_exec);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  auto bail = [&](int code) {
    muonh_destroy(h);
    return code;
  };

  h->last_stream = st;
  if (opt->workspace) {
    h->ws = reinterpret_cast<uint8_t*>(opt->workspace);
  } else {
    void* p = nullptr;
    if (hipMalloc(&p, pl.total) != hipSuccess)
      return bail(fail(MUONH_ENOMEM, "hipMalloc of " + std::to_string(pl.total) + " bytes failed"));
    h->ws = reinterpret_cast<uint8_t*>(p);
    h->owns_ws = true;
  }
  h->staging_bytes = align_up(sizeof(MatPtrs) * n, kAlign) + sizeof(float) * n;
  if (hipHostMalloc(reinterpret_cast<void**>(&h->staging), h->staging_bytes, hipHostMallocDefault) !=
      hipSuccess)
    return bail(fail(MUONH_ENOMEM, "hipHostMalloc of the staging buffer failed"));
  if (hipEventCreateWithFlags(&h->upload_done, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->order_ev, hipEventDisableTiming) != hipSuccess)
    return bail(fail(MUONH_EHIP, "hipEventCreate failed"));

  // The tables (geometry, radii, tile lists, problem descriptors, chunk
  // tables, pointers when given) as one host image, uploaded in one copy.
  std::vector<uint8_t> img;
  std::vector<int32_t> need;
  build_table_image(pl, h->ws, mats, img, need);
  if (hipMemcpy(h->ws, img.data(), img.size(), hipMemcpyHostToDevice) != hipSuccess)
    return bail(fail(MUONH_EHIP, "hipMemcpy of the plan tables failed"));
  // Zero the iterate / Gram buffers once so their padding starts at zero.
  const size_t big0 = pl.mats.empty() ? pl.total : pl.mats[0].off_X[0];
  if (hipMemsetAsync(h->ws + big0, 0, pl.total - big0, st) != hipSuccess)
    return bail(fail(MUONH_EHIP, "hipMemsetAsync of the workspace failed"));

  // Radius R = ||W_0||_F where not given (the image carries the pointers).
  bool any_need = false;
  for (int32_t i = 0; i < n; ++i) any_need |= need[i] != 0;
  if (any_need) {
    h->cur_ptrs.resize(n);
    for (int32_t i = 0; i < n; ++i)
      h->cur_ptrs[i] = MatPtrs{reinterpret_cast<float*>(mats[i].w), mats[i].g,
                               reinterpret_cast<float*>(mats[i].m)};
    h->ptrs_valid = true;
    hipError_t e = launch_radius(h->at<Chunk>(pl.off_chunks), (int64_t)pl.chunks.size(),
                                 h->at<MatPtrs>(pl.off_ptrs), h->at<double>(pl.off_part_radius), st);
    if (e == hipSuccess)
      e = launch_finalize_radius(n, h->at<MatGeom>(pl.off_geo), h->at<double>(pl.off_part_radius),
                                 h->at<int32_t>(pl.off_need), h->at<MatScalars>(pl.off_scal), st);
    if (e != hipSuccess)
      return bail(fail(MUONH_EHIP, std::string("radius kernels: ") + hipGetErrorString(e)));
  }
  h->last_stream = st;
  *out = h;
  return MUONH_OK;
}

namespace {

// Checks shared by both step entry points, then the uploads the step reads
// from device memory: the pointer table (only when the caller's pointers
// changed) and the per-matrix LR factors.  *scale_dev receives the device
// copy of elr_scale, or NULL.
int prepare_step(muonh_handle* h, const muonh_matrix_desc* mats, int32_t n,
                 const muonh_step_args* args, hipStream_t st, const float** scale_dev) {
  if (!h || !args) return fail(MUONH_EINVAL, "null argument");
  int rc = check_same_list(h, mats, n);
  if (rc) return rc;
  if ((rc = check_pointers(mats, n, true))) return rc;
  if (!std::isfinite(args->elr)) return fail(MUONH_EINVAL, "elr is not finite");
  const Plan& pl = h->plan;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != h->device) return fail(MUONH_EINVAL, "current device differs from the one at init");
  // The workspace was last used (or initialised) on h->last_stream.
  if ((rc = order_after_last(h, st))) return rc;

  // Pointer table (uploaded only when the caller's pointers change).
  std::vector<MatPtrs> ptrs(n);
  for (int32_t i = 0; i < n; ++i)
    ptrs[i] = MatPtrs{reinterpret_cast<float*>(mats[i].w), mats[i].g,
                      reinterpret_cast<float*>(mats[i].m)};
  bool uploaded = false;
  if (!h->ptrs_valid || std::memcmp(ptrs.data(), h->cur_ptrs.data(), sizeof(MatPtrs) * n) != 0) {
    if ((rc = upload_async(h, h->ws + pl.off_ptrs, ptrs.data(), sizeof(MatPtrs) * n, 0, st)))
      return rc;
    h->cur_ptrs = ptrs;
    h->ptrs_valid = true;
    uploaded = true;
  }
  *scale_dev = nullptr;
  if (args->elr_scale) {
    for (int32_t i = 0; i < n; ++i)
      if (!std::isfinite(args->elr_scale[i])) return fail(MUONH_EINVAL, "elr_scale has a non-finite entry");
    if ((rc = upload_async(h, h->ws + pl.off_elr, args->elr_scale, sizeof(float) * n,
                           align_up(sizeof(MatPtrs) * n, kAlign), st)))
      return rc;
    *scale_dev = h->at<float>(pl.off_elr);
    uploaded = true;
  }
  if (uploaded) {
    HIP_TRY(hipEventRecord(h->upload_done, st));
    h->upload_pending = true;
  }
  return MUONH_OK;
}

// Enqueues the launches of one step on `st`.  The step size is prm.elr times
// scale_dev[i], or, when eta_dev is given, eta_dev[i] from device memory.
int enqueue_step(muonh_handle* h, hipStream_t st, const ElemParams& prm, const float* scale_dev,
                 const double* eta_dev) {
  const Plan& pl = h->plan;
  const int32_t n = pl.n;
  const int S = pl.opt.ns_steps;
  int rc;
  if (h->timing) {
    const int k = h->ev_next;
    if ((rc = fold_events(h, k))) return rc;   // the set about to be reused
    const size_t need_ev = 2 + 3 * (size_t)S + 2;
    while (h->ev[k].size() < need_ev) {
      hipEvent_t e;
      HIP_TRY(hipEventCreate(&e));
      h->ev[k].push_back(e);
    }
    h->ev_cur = k;
    h->ev_next = (k + 1) % muonh_handle::kRing;
  }
  const int bf = pl.bf16 ? 1 : 0;
  auto* geo = h->at<MatGeom>(pl.off_geo);
  auto* dptrs = h->at<MatPtrs>(pl.off_ptrs);
  auto* scal = h->at<MatScalars>(pl.off_scal);
  auto* part_upd = h->at<double>(pl.off_part_upd);
  size_t evi = 0;
#define LAUNCH(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ == hipSuccess && h->debug_sync) e_ = hipStreamSynchronize(st);                   \
    if (e_ != hipSuccess) return fail(MUONH_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

  if ((rc = record(h, evi++, st))) return rc;
  LAUNCH(launch_momentum(bf, h->at<MomTile>(pl.off_mom_tiles), pl.mom_rows,
                         (int64_t)pl.mom_tiles.size() - pl.mom_rows, geo,
                         dptrs, h->at<double>(pl.off_part_mom), prm, st));
  LAUNCH(launch_finalize_norm(n, geo, h->at<double>(pl.off_part_mom), scal, pl.opt.ns_eps, st));
  if ((rc = record(h, evi++, st))) return rc;
  // One grouped launch per product, on the plan's GEMM path.
  auto gemm = [&](int mode, size_t probs_off, int first, int last) -> hipError_t {
    const GemmProb* probs = h->at<GemmProb>(probs_off);
    const int tk = mode == kGram ? kGram : (mode == kPoly ? kPoly : kApply);
    const GemmTile* tiles = h->at<GemmTile>(pl.off_tiles[tk]);
    const int64_t nt = (int64_t)pl.tiles[tk].size();
    if (pl.small_gemm)
      return launch_gemm_small(bf, mode, probs, tiles, nt, scal, first, last, pl.opt.ns_a,
                               pl.opt.ns_b, pl.opt.ns_c, dptrs, part_upd, st);
    return launch_gemm(bf, mode, probs, tiles, nt, scal, first, last, pl.opt.symmetric, pl.opt.ns_a,
                       pl.opt.ns_b, pl.opt.ns_c, dptrs, part_upd, st);
  };
  for (int it = 0; it < S; ++it) {
    const int par = it & 1;
    const int first = it == 0, last = it == S - 1;
    LAUNCH(gemm(kGram, pl.off_probs_gram[par], first, 0));
    if ((rc = record(h, evi++, st))) return rc;
    LAUNCH(gemm(kPoly, pl.off_probs_poly, 0, 0));
    if ((rc = record(h, evi++, st))) return rc;
    LAUNCH(gemm(kApply, pl.off_probs_apply[par], first, last));
    if ((rc = record(h, evi++, st))) return rc;
  }
  // <W,u>, ||u||^2 and ||W||^2 were reduced per tile by the last B'X launch.
  LAUNCH(launch_finalize_update(n, geo, part_upd, scal, h->at<muonh_stats>(pl.off_stats),
                                scale_dev, eta_dev, prm, st));
  if ((rc = record(h, evi++, st))) return rc;
  LAUNCH(launch_update(bf, h->at<Chunk>(pl.off_chunks), (int64_t)pl.chunks.size(), geo, dptrs,
                       scal, st));
  if ((rc = record(h, evi++, st))) return rc;
#undef LAUNCH
  if (h->timing) h->ev_pending[h->ev_cur] = true;
  return MUONH_OK;
}

ElemParams step_params(const Plan& pl, float elr) {
  return ElemParams{pl.opt.beta, pl.opt.nesterov, pl.opt.ns_eps, pl.opt.mode, pl.opt.weight_decay,
                    elr};
}

void drop_graph(muonh_handle* h) {
  if (h->graph_exec) (void)hipGraphExecDestroy(h->graph_exec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  h->graph_exec = nullptr;
  h->graph = nullptr;
}

}  // namespace

int muonh_step(muonh_handle* h, const muonh_matrix_desc* mats, int32_t n,
               const muonh_step_args* args, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float* scale_dev = nullptr;
  int rc = prepare_step(h, mats, n, args, st, &scale_dev);
  if (rc) return rc;
  if ((rc = enqueue_step(h, st, step_params(h->plan, args->elr), scale_dev, nullptr))) return rc;
  h->last_stream = st;
  h->steps_done++;
  return MUONH_OK;
}

int muonh_step_graph(muonh_handle* h, const muonh_matrix_desc* mats, int32_t n,
                     const muonh_step_args* args, void* stream) {
  if (h && h->timing) return fail(MUONH_ESTATE, "per-phase timing is on: use muonh_step");
  if (h && h->debug_sync) return fail(MUONH_ESTATE, "MUONH_DEBUG_SYNC is set: use muonh_step");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const float* scale_dev = nullptr;
  int rc = prepare_step(h, mats, n, args, st, &scale_dev);
  if (rc) return rc;
  const Plan& pl = h->plan;
  double* eta = h->at<double>(pl.off_eta);
  {
    const hipError_t e = launch_set_eta(n, scale_dev, args->elr, eta, st);
    if (e != hipSuccess) return fail(MUONH_EHIP, std::string("launch_set_eta: ") + hipGetErrorString(e));
  }
  if (!h->graph_exec) {
    // Record the launches once on a private stream; every argument they take
    // is fixed by the plan (tables, workspace addresses, the pointer table's
    // address), and the step size comes from `eta`.
    if (!h->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
    HIP_TRY(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
    rc = enqueue_step(h, h->cap_stream, step_params(pl, 0.0f), nullptr, eta);
    hipGraph_t g = nullptr;
    const hipError_t e_end = hipStreamEndCapture(h->cap_stream, &g);
    if (rc) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (e_end != hipSuccess || !g) {
      if (g) (void)hipGraphDestroy(g);
      return fail(MUONH_EHIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e_end));
    }
    h->graph = g;
    const hipError_t e_inst = hipGraphInstantiate(&h->graph_exec, g, nullptr, nullptr, 0);
    if (e_inst != hipSuccess) {
      h->graph_exec = nullptr;
      drop_graph(h);
      return fail(MUONH_EHIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e_inst));
    }
  }
  HIP_TRY(hipGraphLaunch(h->graph_exec, st));
  h->last_stream = st;
  h->steps_done++;
  return MUONH_OK;
}

}  // extern "C"

int muonh::run_step_in_workspace(const muonh_matrix_desc* mats, int32_t n, const muonh_options& opt,
                                 const muonh_step_args& args, hipStream_t st, uint8_t* ws,
                                 size_t ws_bytes, InWorkspaceHost& host) {
  Plan P;
  int rc = build_plan(mats, n, opt, P);
  if (rc) return rc;
  if (opt.workspace)
    return fail(MUONH_EINVAL, "options.workspace must be NULL: this step uses the library's static buffer");
  for (int32_t i = 0; i < n; ++i)
    if (!(mats[i].radius > 0.0f))
      return fail(MUONH_EINVAL, "matrix " + std::to_string(i) +
                                    ": the allocation-free step needs the radius R (> 0) in the descriptor");
  if ((rc = check_pointers(mats, n, true))) return rc;
  if (!std::isfinite(args.elr)) return fail(MUONH_EINVAL, "elr is not finite");
  if (args.elr_scale)
    for (int32_t i = 0; i < n; ++i)
      if (!std::isfinite(args.elr_scale[i])) return fail(MUONH_EINVAL, "elr_scale has a non-finite entry");
  if (P.total > ws_bytes)
    return fail(MUONH_ENOMEM, "the plan needs " + std::to_string(P.total) +
                                  " bytes of workspace; the static buffer holds " +
                                  std::to_string(ws_bytes));
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));

  // The tables, pointers and per-matrix LR factors as one host image.  The
  // buffer is reused across calls: wait until the device has read the
  // previous upload from it before it is rewritten.
  std::vector<int32_t> need;
  std::vector<uint8_t> img;
  build_table_image(P, ws, mats, img, need);
  const float* scale_dev = nullptr;
  if (args.elr_scale) {
    std::memcpy(img.data() + P.off_elr, args.elr_scale, sizeof(float) * n);
    scale_dev = reinterpret_cast<const float*>(ws + P.off_elr);
  }
  if (host.pending) {
    HIP_TRY(hipEventSynchronize(host.uploaded));
    host.pending = false;
  }
  host.img.swap(img);
  HIP_TRY(hipMemcpyAsync(ws, host.img.data(), host.img.size(), hipMemcpyHostToDevice, st));
  HIP_TRY(hipEventRecord(host.uploaded, st));
  host.pending = true;
  // The buffer keeps the previous call's contents: the Newton-Schulz
  // buffers (whose padding must read as zero) are cleared.
  const size_t big0 = P.mats[0].off_X[0];
  {
    const hipError_t e = launch_fill_zero(ws + big0, P.total - big0, st);
    if (e != hipSuccess) return fail(MUONH_EHIP, std::string("launch_fill_zero: ") + hipGetErrorString(e));
  }
  // A transient handle over the region (it owns nothing).
  muonh_handle h;
  h.plan = std::move(P);
  h.device = dev;
  h.ws = ws;
  h.last_stream = st;
  if (const char* e = std::getenv("MUONH_DEBUG_SYNC")) h.debug_sync = std::atoi(e) != 0;
  return enqueue_step(&h, st, step_params(h.plan, args.elr), scale_dev, nullptr);
}

extern "C" {

int muonh_get_radii(muonh_handle* h, float* out, int32_t n) {
  if (!h || !out) return fail(MUONH_EINVAL, "null argument");
  if (n != h->plan.n) return fail(MUONH_EMISMATCH, "count differs from init");
  HIP_TRY(hipStreamSynchronize(h->last_stream));
  std::vector<MatScalars> s(n);
  HIP_TRY(hipMemcpy(s.data(), h->ws + h->plan.off_scal, sizeof(MatScalars) * n, hipMemcpyDeviceToHost));
  for (int32_t i = 0; i < n; ++i) out[i] = (float)s[i].R;
  return MUONH_OK;
}

int muonh_get_stats(muonh_handle* h, muonh_stats* out, int32_t n) {
  if (!h || !out) return fail(MUONH_EINVAL, "null argument");
  if (n != h->plan.n) return fail(MUONH_EMISMATCH, "count differs from init");
  if (h->steps_done == 0) return fail(MUONH_ESTATE, "no step has run yet");
  HIP_TRY(hipStreamSynchronize(h->last_stream));
  HIP_TRY(hipMemcpy(out, h->ws + h->plan.off_stats, sizeof(muonh_stats) * n, hipMemcpyDeviceToHost));
  return MUONH_OK;
}

int muonh_copy_update(muonh_handle* h, int32_t idx, void* dst_device, void* stream) {
  if (!h || !dst_device) return fail(MUONH_EINVAL, "null argument");
  if (idx < 0 || idx >= h->plan.n) return fail(MUONH_EINVAL, "matrix index out of range");
  if (h->steps_done == 0) return fail(MUONH_ESTATE, "no step has run yet");
  const MatPlan& m = h->plan.mats[idx];
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // after the step that wrote u, and before any later step overwrites it
  const int rc = order_after_last(h, st);
  if (rc) return rc;
  const hipError_t e = launch_copy_update(h->plan.bf16 ? 1 : 0, h->ws + m.off_U, m.rows * m.cols,
                                          reinterpret_cast<float*>(dst_device), st);
  if (e != hipSuccess) return fail(MUONH_EHIP, std::string("copy_update: ") + hipGetErrorString(e));
  return MUONH_OK;
}

int muonh_set_timing(muonh_handle* h, int32_t enable) {
  if (!h) return fail(MUONH_EINVAL, "null handle");
  if (h->ws) HIP_TRY(hipStreamSynchronize(h->last_stream));
  h->timing = enable != 0;
  for (int k = 0; k < muonh_handle::kRing; ++k) h->ev_pending[k] = false;
  for (double& t : h->phase_total) t = 0.0;
  h->timed_steps = 0;
  return MUONH_OK;
}

int muonh_get_timing(muonh_handle* h, float* phases_ms, int32_t n_phases, int32_t* n_steps) {
  if (!h || !phases_ms || !n_steps) return fail(MUONH_EINVAL, "null argument");
  if (n_phases < 7) return fail(MUONH_EINVAL, "need room for 7 phases");
  // Fold the pending sets oldest first.
  for (int j = 0; j < muonh_handle::kRing; ++j) {
    const int k = (h->ev_next + j) % muonh_handle::kRing;
    const int rc = fold_events(h, k);
    if (rc) return rc;
  }
  for (int k = 0; k < n_phases; ++k) phases_ms[k] = k < 7 ? (float)h->phase_total[k] : 0.0f;
  *n_steps = h->timed_steps;
  for (double& t : h->phase_total) t = 0.0;
  h->timed_steps = 0;
  return MUONH_OK;
}

int muonh_destroy(muonh_handle* h) {
  if (!h) return MUONH_OK;
  if (h->ws) (void)hipStreamSynchronize(h->last_stream);
  if (h->owns_ws && h->ws) (void)hipFree(h->ws);
  if (h->staging) (void)hipHostFree(h->staging);
  if (h->upload_done) (void)hipEventDestroy(h->upload_done);
  if (h->order_ev) (void)hipEventDestroy(h->order_ev);
  drop_graph(h);
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  for (auto& set : h->ev)
    for (auto e : set) (void)hipEventDestroy(e);
  delete h;
  return MUONH_OK;
}

const char* muonh_status_str(int status) {
  switch (status) {
    case MUONH_OK: return "ok";
    case MUONH_EINVAL: return "invalid argument";
    case MUONH_EMISMATCH: return "matrix list differs from init";
    case MUONH_ENOMEM: return "out of memory / workspace too small";
    case MUONH_EHIP: return "HIP runtime error";
    case MUONH_ESTATE: return "call out of order";
    case MUONH_ENODEV: return "no usable gfx950 device";
    default: return "unknown status";
  }
}

const char* muonh_last_error(void) { return g_last_error.c_str(); }

double muonh_lr_linear(double eta0, double eta_min, double s, double S) {
  if (!(S > 0.0)) return eta_min;
  s = std::min(std::max(s, 0.0), S);
  return eta0 + (eta_min - eta0) * s / S;
}

double muonh_lr_power(double k, double peak, double floor_, double warmup, double tau, double p) {
  if (k <= warmup) return warmup > 0.0 ? peak * k / warmup : peak;
  return floor_ + (peak - floor_) * std::pow(1.0 + (k - warmup) / tau, -p);
}

double muonh_lr_wsd(double k, double peak, double total, double decay_ratio, double warmup,
                    double eta_min) {
  if (warmup > 0.0 && k < warmup) return peak * k / warmup;
  const double d0 = total * (1.0 - decay_ratio);
  if (k <= d0) return peak;
  return muonh_lr_linear(peak, eta_min, k - d0, total - d0);
}

double muonh_lr_linear_hold(double eta0, double eta_min, double s, double S, double s_hold) {
  return muonh_lr_linear(eta0, eta_min, std::min(s, s_hold), S);
}

double muonh_lr_cosine(double k, double total, double eta_max, double eta_min, double warmup) {
  if (warmup > 0.0 && k < warmup) return eta_max * k / warmup;
  const double span = std::max(total - warmup, 1.0);
  const double t = std::min(std::max((k - warmup) / span, 0.0), 1.0);
  return eta_min + 0.5 * (eta_max - eta_min) * (1.0 + std::cos(M_PI * t));
}

double muonh_elr_from_base(double eta_base, double multiplier) { return multiplier * eta_base; }

}  // extern "C"
