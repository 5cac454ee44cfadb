// Host-only exercise of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: plan building and workspace sizing over the
// benchmark's shape sets, ragged, vector and maximal shapes; argument
// validation and error codes; the learning-rate helpers; the AdamW option
// and argument checks; and init failing cleanly where no device is present.
// Exits non-zero on the first failed check (a sanitizer report also fails).
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "muonh.h"

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "CHECK failed at line %d: %s (last error: %s)\n", __LINE__, #cond, \
                   muonh_last_error());                                          \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

static muonh_matrix_desc desc(int64_t r, int64_t c, int32_t dt = MUONH_BF16) {
  muonh_matrix_desc d;
  std::memset(&d, 0, sizeof(d));
  d.rows = r;
  d.cols = c;
  d.g_dtype = dt;
  return d;
}

static std::vector<muonh_matrix_desc> qwen3(int64_t dm, int64_t dff, bool fused) {
  std::vector<muonh_matrix_desc> v;
  for (int l = 0; l < 28; ++l) {
    if (fused) {
      v.push_back(desc(4096, dm));
    } else {
      v.push_back(desc(2048, dm));
      v.push_back(desc(1024, dm));
      v.push_back(desc(1024, dm));
    }
    v.push_back(desc(dm, 2048));
    if (fused) {
      v.push_back(desc(2 * dff, dm));
    } else {
      v.push_back(desc(dff, dm));
      v.push_back(desc(dff, dm));
    }
    v.push_back(desc(dm, dff));
  }
  return v;
}

static int plan_checks(const std::vector<muonh_matrix_desc>& mats, int32_t ns_dtype) {
  muonh_options opt;
  muonh_default_options(&opt);
  opt.ns_dtype = ns_dtype;
  size_t bytes = 0;
  CHECK(muonh_workspace_size(mats.data(), (int32_t)mats.size(), &opt, &bytes) == MUONH_OK);
  muonh_plan_info info;
  CHECK(muonh_plan_query(mats.data(), (int32_t)mats.size(), &opt, &info) == MUONH_OK);
  CHECK(info.workspace_bytes == bytes && bytes > 0);
  CHECK(info.n_matrices == (int32_t)mats.size());
  CHECK(info.n_buckets >= 1 && info.mom_tiles >= 1 && info.flat_chunks >= 1);
  CHECK(info.gemm_tiles[0] >= 1 && info.gemm_tiles[1] >= 1 && info.gemm_tiles[2] >= 1);
  double dense = 0.0;
  for (const auto& d : mats) {
    const double m = (double)std::min(d.rows, d.cols), n = (double)std::max(d.rows, d.cols);
    dense += opt.ns_steps * (4.0 * m * m * n + 2.0 * m * m * m);
  }
  CHECK(std::fabs(info.ns_dense_flops / dense - 1.0) < 1e-12);
  CHECK(info.ns_exec_flops > 0.0);
  opt.symmetric = 0;
  muonh_plan_info full;
  CHECK(muonh_plan_query(mats.data(), (int32_t)mats.size(), &opt, &full) == MUONH_OK);
  CHECK(full.gemm_tiles[0] >= info.gemm_tiles[0] && full.gemm_tiles[2] == info.gemm_tiles[2]);
  return 0;
}

int main() {
  // ---- plans over the benchmark's sets, both Newton-Schulz types
  for (int32_t dt : {MUONH_BF16, MUONH_F32}) {
    if (plan_checks(qwen3(2048, 6144, false), dt)) return 1;
    if (plan_checks(qwen3(2048, 6144, true), dt)) return 1;
    if (plan_checks(qwen3(1024, 3072, false), dt)) return 1;
  }
  // ragged, vectors, tall/wide, a 64-matrix pseudo-random set and the largest dims
  std::vector<muonh_matrix_desc> odd = {desc(1, 1), desc(1, 37), desc(37, 1), desc(300, 200),
                                        desc(257, 1031), desc(1000, 260), desc(515, 515),
                                        desc(65536, 1, MUONH_F32), desc(1, 65536)};
  uint64_t x = 12345;
  for (int i = 0; i < 64; ++i) {
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    const int64_t r = 1 + (int64_t)((x >> 33) % 4096);
    x = x * 6364136223846793005ull + 1442695040888963407ull;
    const int64_t c = 1 + (int64_t)((x >> 33) % 4096);
    odd.push_back(desc(r, c, i & 1 ? MUONH_F32 : MUONH_BF16));
  }
  for (int32_t dt : {MUONH_BF16, MUONH_F32})
    if (plan_checks(odd, dt)) return 1;
  {
    std::vector<muonh_matrix_desc> big = {desc(65536, 65536), desc(32768, 33024)};
    if (plan_checks(big, MUONH_BF16)) return 1;
  }

  // ---- argument validation
  muonh_options opt;
  muonh_default_options(&opt);
  size_t bytes = 0;
  std::vector<muonh_matrix_desc> one = {desc(64, 64)};
  CHECK(muonh_workspace_size(nullptr, 1, &opt, &bytes) == MUONH_EINVAL);
  CHECK(muonh_workspace_size(one.data(), 0, &opt, &bytes) == MUONH_EINVAL);
  CHECK(muonh_workspace_size(one.data(), 1, &opt, nullptr) == MUONH_EINVAL);
  CHECK(std::strlen(muonh_last_error()) > 0);
  for (auto bad : {desc(0, 4), desc(4, 0), desc(-1, 4), desc(65537, 4), desc(4, 65537)}) {
    CHECK(muonh_workspace_size(&bad, 1, &opt, &bytes) == MUONH_EINVAL);
  }
  {
    auto bad = desc(8, 8, 7);
    CHECK(muonh_workspace_size(&bad, 1, &opt, &bytes) == MUONH_EINVAL);
    bad = desc(8, 8);
    bad.radius = NAN;
    CHECK(muonh_workspace_size(&bad, 1, &opt, &bytes) == MUONH_EINVAL);
  }
  {
    muonh_options o = opt;
    o.ns_steps = 0;
    CHECK(muonh_workspace_size(one.data(), 1, &o, &bytes) == MUONH_EINVAL);
    o = opt;
    o.ns_steps = 17;
    CHECK(muonh_workspace_size(one.data(), 1, &o, &bytes) == MUONH_EINVAL);
    o = opt;
    o.ns_dtype = 9;
    CHECK(muonh_workspace_size(one.data(), 1, &o, &bytes) == MUONH_EINVAL);
    o = opt;
    o.mode = 5;
    CHECK(muonh_workspace_size(one.data(), 1, &o, &bytes) == MUONH_EINVAL);
  }
  // init: null handle pointer, then (no device here) a clean failure with *h == NULL
  CHECK(muonh_init(nullptr, one.data(), 1, &opt, nullptr) == MUONH_EINVAL);
  {
    std::vector<muonh_matrix_desc> ok = {desc(64, 64), desc(100, 30)};
    for (auto& d : ok) {
      d.w = reinterpret_cast<void*>(0x100000);
      d.g = reinterpret_cast<void*>(0x200000);
      d.m = reinterpret_cast<void*>(0x300000);
      d.radius = 2.0f;
    }
    muonh_handle* h = reinterpret_cast<muonh_handle*>(0x1);
    const int rc = muonh_init(&h, ok.data(), 2, &opt, nullptr);
    CHECK(rc != MUONH_OK && h == nullptr);
    // radius <= 0 makes init measure ||W_0||, so w must then be valid first
    ok[0].w = reinterpret_cast<void*>(0x100004);   // misaligned
    ok[0].radius = 0.0f;
    CHECK(muonh_init(&h, ok.data(), 2, &opt, nullptr) == MUONH_EINVAL && h == nullptr);
    ok[0].w = nullptr;
    CHECK(muonh_init(&h, ok.data(), 2, &opt, nullptr) == MUONH_EINVAL && h == nullptr);
    // a caller workspace that is too small or misaligned
    ok[0].w = reinterpret_cast<void*>(0x100000);
    muonh_options o = opt;
    o.workspace = reinterpret_cast<void*>(0x400000);
    o.workspace_bytes = 1024;
    CHECK(muonh_init(&h, ok.data(), 2, &o, nullptr) == MUONH_ENOMEM && h == nullptr);
    size_t need = 0;
    CHECK(muonh_workspace_size(ok.data(), 2, &opt, &need) == MUONH_OK);
    o.workspace = reinterpret_cast<void*>(0x400010);
    o.workspace_bytes = need;
    CHECK(muonh_init(&h, ok.data(), 2, &o, nullptr) == MUONH_EINVAL && h == nullptr);
  }
  CHECK(muonh_destroy(nullptr) == MUONH_OK);
  CHECK(muonh_step(nullptr, one.data(), 1, nullptr, nullptr) == MUONH_EINVAL);
  CHECK(muonh_step_graph(nullptr, one.data(), 1, nullptr, nullptr) == MUONH_EINVAL);
  // The option struct's layout, as the Python binding mirrors it.
  CHECK(sizeof(muonh_options) == 64 && offsetof(muonh_options, workspace) == 48);
  CHECK(offsetof(muonh_options, deterministic) == 44);
  {
    muonh_step_args a;
    std::memset(&a, 0, sizeof(a));
    a.elr = 0.01f;
    CHECK(muonh_step_graph(nullptr, one.data(), 1, &a, nullptr) == MUONH_EINVAL);
  }
  for (int s = -7; s <= 0; ++s) CHECK(muonh_status_str(s) != nullptr);

  // ---- learning-rate helpers (values are pinned against the oracle elsewhere)
  CHECK(muonh_lr_linear(1e-3, 1e-5, 0.0, 100.0) == 1e-3);
  CHECK(std::fabs(muonh_lr_linear(1e-3, 1e-5, 100.0, 100.0) - 1e-5) < 1e-18);
  CHECK(std::fabs(muonh_lr_linear(1e-3, 1e-5, 200.0, 100.0) - 1e-5) < 1e-18);   // clamped
  CHECK(std::isfinite(muonh_lr_power(0.0, 5e-3, 5e-4, 1000.0, 1000.0, 0.5)));
  CHECK(std::isfinite(muonh_lr_power(1e6, 5e-3, 5e-4, 1000.0, 1000.0, 0.5)));
  CHECK(std::isfinite(muonh_lr_wsd(50.0, 0.024, 100.0, 0.2, 0.0, 0.0)));
  CHECK(muonh_lr_linear_hold(1e-3, 1e-5, 90.0, 100.0, 50.0) ==
        muonh_lr_linear(1e-3, 1e-5, 50.0, 100.0));
  CHECK(std::isfinite(muonh_lr_cosine(5.0, 100.0, 1e-5, 1e-6, 10.0)));
  CHECK(muonh_elr_from_base(1e-3, 10.0) == 1e-3 * 10.0);

  // ---- AdamW options and arguments
  muonh_adamw_options ao;
  muonh_adamw_default_options(&ao);
  CHECK(ao.beta1 == 0.9f && ao.beta2 == 0.95f && ao.weight_decay == 0.1f);
  muonh_adamw_tensor t;
  std::memset(&t, 0, sizeof(t));
  t.numel = 10;
  t.g_dtype = MUONH_BF16;
  muonh_adamw_handle* ah = nullptr;
  CHECK(muonh_adamw_init(nullptr, &t, 1, &ao) == MUONH_EINVAL);
  CHECK(muonh_adamw_init(&ah, &t, 0, &ao) == MUONH_EINVAL && ah == nullptr);
  t.numel = 0;
  CHECK(muonh_adamw_init(&ah, &t, 1, &ao) == MUONH_EINVAL && ah == nullptr);
  t.numel = 10;
  t.reserved = 1;
  CHECK(muonh_adamw_init(&ah, &t, 1, &ao) == MUONH_EINVAL && ah == nullptr);
  t.reserved = 0;
  muonh_adamw_options bad = ao;
  bad.beta1 = 1.0f;
  CHECK(muonh_adamw_init(&ah, &t, 1, &bad) == MUONH_EINVAL && ah == nullptr);
  bad = ao;
  bad.eps = 0.0f;
  CHECK(muonh_adamw_init(&ah, &t, 1, &bad) == MUONH_EINVAL && ah == nullptr);
  CHECK(muonh_adamw_step(nullptr, &t, 1, 1e-3f, 1, nullptr) == MUONH_EINVAL);
  CHECK(muonh_adamw_destroy(nullptr) == MUONH_OK);

  std::printf("host driver: all checks passed\n");
  return 0;
}
