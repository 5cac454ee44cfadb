// Host side of the AdamW step for the parameters MuonH does not wrap
// (embeddings, normalisation layers, LM head): validation, the chunk table
// and the launch.  The pages train this group with AdamW at weight decay 0.1
// on the base LR schedule ("Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX
// 5090 within $5090", arXiv HTML §3.3 and App. C, Tab. 8) with Adam betas
// (0.9, 0.95) and epsilon 1e-12 (App. E).  The bias corrections of step t are
// folded into two scalars here, in double precision, so the kernel does one
// fused pass per element.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

using namespace muonh;

struct muonh_adamw_handle {
  int device = -1;
  int32_t n = 0;
  std::vector<int64_t> numel;
  std::vector<int32_t> g_bf16;
  std::vector<Chunk> chunks;
  muonh_adamw_options opt{};
  Chunk* d_chunks = nullptr;
  AdamwPtrs* d_ptrs = nullptr;
  AdamwPtrs* staging = nullptr;       // pinned host copy of the pointer table
  std::vector<AdamwPtrs> cur_ptrs;    // what the device table holds
  bool ptrs_valid = false;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  bool debug_sync = false;            // MUONH_DEBUG_SYNC=1: synchronise after the launch
};

namespace {

int fail(int code, const std::string& msg) { return set_last_error(code, msg.c_str()); }

#define ADAMW_HIP(expr)                                                                 \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(MUONH_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_));       \
  } while (0)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_tensor_list(const muonh_adamw_tensor* t, int32_t n) {
  if (!t) return fail(MUONH_EINVAL, "null tensor list");
  if (n < 1) return fail(MUONH_EINVAL, "tensor count must be >= 1");
  for (int32_t i = 0; i < n; ++i) {
    if (t[i].numel < 1) return fail(MUONH_EINVAL, "tensor " + std::to_string(i) + ": numel < 1");
    if (t[i].g_dtype != MUONH_F32 && t[i].g_dtype != MUONH_BF16)
      return fail(MUONH_EINVAL, "tensor " + std::to_string(i) + ": unknown gradient dtype");
    if (t[i].reserved != 0) return fail(MUONH_EINVAL, "tensor " + std::to_string(i) + ": reserved != 0");
  }
  return MUONH_OK;
}

}  // namespace

extern "C" {

void muonh_adamw_default_options(muonh_adamw_options* opt) {
  if (!opt) return;
  opt->beta1 = 0.9f;
  opt->beta2 = 0.95f;
  opt->eps = 1e-12f;
  opt->weight_decay = 0.1f;
}

int muonh_adamw_destroy(muonh_adamw_handle* h) {
  if (!h) return MUONH_OK;
  if (h->upload_pending) (void)hipEventSynchronize(h->upload_done);
  if (h->upload_done) (void)hipEventDestroy(h->upload_done);
  if (h->d_chunks) (void)hipFree(h->d_chunks);
  if (h->d_ptrs) (void)hipFree(h->d_ptrs);
  if (h->staging) (void)hipHostFree(h->staging);
  delete h;
  return MUONH_OK;
}

int muonh_adamw_init(muonh_adamw_handle** out, const muonh_adamw_tensor* t, int32_t n,
                     const muonh_adamw_options* opt) {
  if (!out) return fail(MUONH_EINVAL, "null handle pointer");
  *out = nullptr;
  int rc = check_tensor_list(t, n);
  if (rc) return rc;
  muonh_adamw_options o;
  if (opt) {
    o = *opt;
  } else {
    muonh_adamw_default_options(&o);
  }
  if (!(o.beta1 >= 0.0f && o.beta1 < 1.0f) || !(o.beta2 >= 0.0f && o.beta2 < 1.0f) ||
      !(o.eps > 0.0f) || !std::isfinite(o.eps) || !(o.weight_decay >= 0.0f) ||
      !std::isfinite(o.weight_decay))
    return fail(MUONH_EINVAL, "options outside 0 <= beta < 1, eps > 0, weight_decay >= 0");

  auto* h = new muonh_adamw_handle();
  h->n = n;
  h->opt = o;
  if (const char* e = std::getenv("MUONH_DEBUG_SYNC")) h->debug_sync = std::atoi(e) != 0;
  for (int32_t i = 0; i < n; ++i) {
    h->numel.push_back(t[i].numel);
    h->g_bf16.push_back(t[i].g_dtype == MUONH_BF16 ? 1 : 0);
    for (int64_t s = 0; s < t[i].numel; s += kChunk)
      h->chunks.push_back(Chunk{i, (int32_t)std::min<int64_t>(kChunk, t[i].numel - s), s});
  }
  auto bail = [&](int code) {
    muonh_adamw_destroy(h);
    return code;
  };
  auto hip = [&](hipError_t e, const char* what) {
    return e == hipSuccess ? MUONH_OK : fail(MUONH_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  };
  if ((rc = hip(hipGetDevice(&h->device), "hipGetDevice")) ||
      (rc = hip(hipMalloc((void**)&h->d_chunks, sizeof(Chunk) * h->chunks.size()), "hipMalloc")) ||
      (rc = hip(hipMalloc((void**)&h->d_ptrs, sizeof(AdamwPtrs) * n), "hipMalloc")) ||
      (rc = hip(hipHostMalloc((void**)&h->staging, sizeof(AdamwPtrs) * n, hipHostMallocDefault),
                "hipHostMalloc")) ||
      (rc = hip(hipEventCreateWithFlags(&h->upload_done, hipEventDisableTiming), "hipEventCreate")) ||
      (rc = hip(hipMemcpy(h->d_chunks, h->chunks.data(), sizeof(Chunk) * h->chunks.size(),
                          hipMemcpyHostToDevice), "hipMemcpy")))
    return bail(rc);
  *out = h;
  return MUONH_OK;
}

int muonh_adamw_step(muonh_adamw_handle* h, const muonh_adamw_tensor* t, int32_t n, float lr,
                     int64_t step, void* stream) {
  if (!h) return fail(MUONH_EINVAL, "null handle");
  if (!t) return fail(MUONH_EINVAL, "null tensor list");
  if (n != h->n) return fail(MUONH_EMISMATCH, "tensor count differs from init");
  if (step < 1) return fail(MUONH_EINVAL, "step count starts at 1");
  if (!std::isfinite(lr)) return fail(MUONH_EINVAL, "lr is not finite");
  std::vector<AdamwPtrs> ptrs(n);
  for (int32_t i = 0; i < n; ++i) {
    if (t[i].numel != h->numel[i] || (t[i].g_dtype == MUONH_BF16 ? 1 : 0) != h->g_bf16[i] ||
        (t[i].g_dtype != MUONH_F32 && t[i].g_dtype != MUONH_BF16))
      return fail(MUONH_EMISMATCH, "tensor " + std::to_string(i) + ": size or dtype differs from init");
    if (!t[i].w || !t[i].g || !t[i].m || !t[i].v)
      return fail(MUONH_EINVAL, "tensor " + std::to_string(i) + ": null pointer");
    if (!aligned(t[i].w, 16) || !aligned(t[i].m, 16) || !aligned(t[i].v, 16) ||
        !aligned(t[i].g, h->g_bf16[i] ? 8 : 16))
      return fail(MUONH_EINVAL, "tensor " + std::to_string(i) + ": misaligned pointer");
    ptrs[i] = AdamwPtrs{static_cast<float*>(t[i].w), t[i].g, static_cast<float*>(t[i].m),
                        static_cast<float*>(t[i].v), h->g_bf16[i], 0};
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool same = h->ptrs_valid && std::memcmp(ptrs.data(), h->cur_ptrs.data(), sizeof(AdamwPtrs) * n) == 0;
  if (!same) {
    // The pinned staging copy is reused: wait until the device consumed the
    // previous upload before overwriting it.
    if (h->upload_pending) {
      ADAMW_HIP(hipEventSynchronize(h->upload_done));
      h->upload_pending = false;
    }
    std::memcpy(h->staging, ptrs.data(), sizeof(AdamwPtrs) * n);
    ADAMW_HIP(hipMemcpyAsync(h->d_ptrs, h->staging, sizeof(AdamwPtrs) * n, hipMemcpyHostToDevice, st));
    ADAMW_HIP(hipEventRecord(h->upload_done, st));
    h->upload_pending = true;
    h->cur_ptrs = ptrs;
    h->ptrs_valid = true;
  }
  const double b1 = h->opt.beta1, b2 = h->opt.beta2;
  const double bc1 = 1.0 - std::pow(b1, (double)step);
  const double bc2 = 1.0 - std::pow(b2, (double)step);
  AdamwParams prm;
  prm.beta1 = h->opt.beta1;
  prm.omb1 = (float)(1.0 - b1);
  prm.beta2 = h->opt.beta2;
  prm.omb2 = (float)(1.0 - b2);
  prm.eps = h->opt.eps;
  prm.decay = (float)(1.0 - (double)lr * h->opt.weight_decay);
  prm.step_size = (float)((double)lr / bc1);
  prm.rbc2 = (float)(1.0 / std::sqrt(bc2));
  ADAMW_HIP(launch_adamw(h->d_chunks, (int64_t)h->chunks.size(), h->d_ptrs, prm, st));
  if (h->debug_sync) ADAMW_HIP(hipStreamSynchronize(st));
  return MUONH_OK;
}

}  // extern "C"
