// Fused, coalesced elementwise / reduction kernels of the MuonH step (gfx950).
//
// The step around the Newton-Schulz products is memory-bound streaming work:
//   momentum_row_kernel / momentum_tile_kernel :
//                     M <- beta M + G, Y = M (or G + beta M), partial ||Y||^2,
//                     Y packed as the first iterate X_0, zero-padded, in the
//                     layouts the grouped GEMM reads (X, and X^T in the fp32
//                     plan): row segments where X_0 keeps M's orientation,
//                     64 x 128 tiles through LDS where it is transposed;
//   (<W,u>, ||u||^2, ||W||^2 are reduced per tile by the last Newton-Schulz
//   product's epilogue, gemm.hip);
//   update_kernel   : W <- k1 W - k2 u  (Hyperball: k1 = R/||W~||,
//                     k2 = k1 eta R / ||u||, from the closed form
//                     ||W~||^2 = ||W||^2 - 2 k <W,u> + k^2 ||u||^2, k = eta R/||u||,
//                     so W~ is never materialised)
// plus one-wavefront-per-matrix finalise kernels.  The Hyperball step is
// Eq. (1) of "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within
// $5090" (arXiv HTML §3.3); the ordinary-Muon and ELR-aligned updates are its
// Eqs. (3) and (5) (§3.3.1).
//
// Reductions are deterministic: per-thread fp32 sums over a fixed set of
// elements, fp64 wavefront shuffles and an fp64 LDS tree in a fixed order,
// per-block partials summed in block order by the finalise kernels.  No
// floating-point atomics.

#include <math.h>

#include <algorithm>

#include "device_util.h"
#include "internal.h"
#include "update_math.h"

namespace muonh {
namespace {

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum of one double per thread over a 256-thread block; result valid in thread 0.
template <int NV>
__device__ __forceinline__ void block_sum(double (&v)[NV], double (*red)[4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const double s = wave_sum(v[k]);
    if (lane == 0) red[k][wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = (red[k][0] + red[k][1]) + (red[k][2] + red[k][3]);
  }
}

template <typename G> struct GradLoad;
template <> struct GradLoad<uint16_t> {
  static __device__ __forceinline__ f32x4_t load4(const void* p, int64_t off) {
    return Vec4<uint16_t>::load_nt(reinterpret_cast<const uint16_t*>(p) + off);
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t off) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[off]);
  }
};
template <> struct GradLoad<float> {
  static __device__ __forceinline__ f32x4_t load4(const void* p, int64_t off) {
    return Vec4<float>::load_nt(reinterpret_cast<const float*>(p) + off);
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t off) {
    return reinterpret_cast<const float*>(p)[off];
  }
};

// ---------------------------------------------------------------------------
// momentum + pack.  One 64 x 128 tile of the padded, original-orientation
// grid per 512-thread block (rows of 512 bytes of M: wider tiles stream
// faster, measured on MI355X); thread (rr, cc) handles rows rr + 16q,
// columns cc..cc+3.  The transposed X_0 is staged through LDS in the
// Newton-Schulz element type.

// ||Y||^2 partial of one momentum unit: one slot per wavefront (a fixed-order
// fp64 shuffle tree inside the wavefront; no block-wide barrier).
__device__ __forceinline__ void write_wave_partial(double* partials, int64_t unit, float ss) {
  const double s = wave_sum((double)ss);
  if ((threadIdx.x & 63) == 0) partials[kMomParts * unit + (threadIdx.x >> 6)] = s;
}

template <typename T> __device__ __forceinline__ T to_elem(float v);
template <> __device__ __forceinline__ float to_elem<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t to_elem<uint16_t>(float v) { return f32_to_bf16(v); }

// 4 consecutive elements already in the element type.
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  st_global<f32x4_t>(p, f32x4_t{a, b, c, d});
}
__device__ __forceinline__ void store4(uint16_t* p, uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
  st_global<u32x2_t>(p, u32x2_t{(uint32_t)a | ((uint32_t)b << 16), (uint32_t)c | ((uint32_t)d << 16)});
}

// LDS image of one momentum tile in the Newton-Schulz element type.
//   fp32: rows of 129 elements (one padding element per row).
//   bf16: rows of 128 elements (256 bytes) whose 8-byte units (4 columns)
//         are XOR-swizzled by row / 4: unit u of row r sits at u ^ ((r/4) & 15).
// With the thread layout below, each half-wavefront of the bf16 writes (one
// 8-byte unit per lane, 32 units of one row) and of the reads (4 rows r =
// 4i + k apart for i = 0..15, one column each) then touches every bank once,
// where a padded linear pitch left both 2-way conflicted (two units or rows
// per bank).
template <typename T> struct MomLds {
  static constexpr int kPitch = kMomTileC + (sizeof(T) == 2 ? 0 : 1);
};
__device__ __forceinline__ int mom_unit_swz(int r) { return (r >> 2) & 15; }

template <typename T, typename G>
__device__ __forceinline__ void momentum_tile(const MomTile& t, int64_t unit, const MatGeom& g,
                                              const MatPtrs& p, double* partials,
                                              const ElemParams& prm,
                                              T (*tile)[MomLds<T>::kPitch]) {
  constexpr int kTpr = kMomTileC / 4;               // threads per row
  constexpr int kRpp = kMomTileThreads / kTpr;      // rows per pass
  constexpr int kPasses = kMomTileR / kRpp;
  const int tid = threadIdx.x;
  const int cc = (tid % kTpr) * 4;
  const int rr = tid / kTpr;
  const int64_t r0 = (int64_t)t.tr * kMomTileR, c0 = (int64_t)t.tc * kMomTileC;
  // X_0 in M's orientation (D) and transposed (Tr); the bf16 plan keeps only
  // X (no X^T), so one of the two is absent.
  T* D = reinterpret_cast<T*>(g.tall ? g.XT[0] : g.X[0]);
  T* Tr = reinterpret_cast<T*>(g.tall ? g.X[0] : g.XT[0]);
  const int64_t ldD = g.c_pad + g.ld_skew, ldT = g.r_pad + g.ld_skew;
  const bool vec_ok = (g.cols & 3) == 0;
  const float beta = prm.beta;
  float ss = 0.0f;

  // All loads of the thread's rows are issued before its first store (M is
  // written in place, so the compiler may not hoist them itself).
  {
    f32x4_t gv[kPasses], mv[kPasses];
    bool full[kPasses];
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const int64_t row = r0 + rr + kRpp * q;
      const int64_t col = c0 + cc;
      full[q] = row < g.rows && vec_ok && col + 3 < g.cols;
      if (full[q]) {
        const int64_t off = row * g.cols + col;
        gv[q] = GradLoad<G>::load4(p.g, off);
        mv[q] = Vec4<float>::load_nt(p.m + off);
      }
    }
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const int tr_ = rr + kRpp * q;   // row inside the tile
      const int64_t row = r0 + tr_;
      const int64_t col = c0 + cc;
      f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
      const int64_t off = row * g.cols + col;
      if (full[q]) {
        const f32x4_t m = beta * mv[q] + gv[q];
        Vec4<float>::store_nt(p.m + off, m);
        y = prm.nesterov ? gv[q] + beta * m : m;
      } else if (row < g.rows) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col + e < g.cols) {
            const float gs = GradLoad<G>::load1(p.g, off + e);
            const float ms = beta * p.m[off + e] + gs;
            p.m[off + e] = ms;
            y[e] = prm.nesterov ? gs + beta * ms : ms;
          }
        }
      }
      ss += y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
      if (Tr) {
        if constexpr (sizeof(T) == 2) {
          u32x2_t o;
          o[0] = pack_bf16x2(y[0], y[1]);
          o[1] = pack_bf16x2(y[2], y[3]);
          *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint8_t*>(&tile[tr_][0]) +
                                      8 * ((cc >> 2) ^ mom_unit_swz(tr_))) = o;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) tile[tr_][cc + e] = to_elem<T>(y[e]);
        }
      }
      if (D) Vec4<T>::store(D + row * ldD + col, y);
    }
  }
  if (Tr) {
    __syncthreads();
    // output row oc (= tile column) holds the tile's 64 rows, 4 per thread
    constexpr int kTpo = kMomTileR / 4;             // threads per output row
    constexpr int kOpp = kMomTileThreads / kTpo;    // output rows per pass
    const int oe = (tid % kTpo) * 4, orow = tid / kTpo;
#pragma unroll
    for (int q = 0; q < kMomTileC / kOpp; ++q) {
      const int oc = orow + kOpp * q;
      if constexpr (sizeof(T) == 2) {
        // rows oe..oe+3 share one swizzle (oe is a multiple of 4)
        const int off = 8 * ((oc >> 2) ^ mom_unit_swz(oe)) + 2 * (oc & 3);
        const uint8_t* b = reinterpret_cast<const uint8_t*>(&tile[oe][0]) + off;
        constexpr int kRow = MomLds<T>::kPitch * (int)sizeof(T);
        store4(Tr + (c0 + oc) * ldT + r0 + oe, *reinterpret_cast<const T*>(b),
               *reinterpret_cast<const T*>(b + kRow), *reinterpret_cast<const T*>(b + 2 * kRow),
               *reinterpret_cast<const T*>(b + 3 * kRow));
      } else {
        store4(Tr + (c0 + oc) * ldT + r0 + oe, tile[oe][oc], tile[oe + 1][oc], tile[oe + 2][oc],
               tile[oe + 3][oc]);
      }
    }
  }
  // Eight wavefronts, kMomParts slots: slot w = wavefront w + wavefront w + 4.
  static_assert(kMomTileThreads / 64 == 2 * kMomParts, "two wavefronts per slot");
  __shared__ double red[kMomTileThreads / 64];
  const double sw = wave_sum((double)ss);
  if ((tid & 63) == 0) red[tid >> 6] = sw;
  __syncthreads();
  if (tid < kMomParts) partials[kMomParts * unit + tid] = red[tid] + red[tid + kMomParts];
}

// momentum + pack for a matrix whose X_0 keeps M's orientation and has no
// transposed copy: columns [tc * kMomRowSeg, +kMomRowSeg) of row tr of the
// padded grid, 4 consecutive columns per thread.  Short blocks over
// consecutive addresses stream faster than 64 x 64 tiles (each of which
// touches 64 rows); pad rows and columns of X_0 are written as zeros.
template <typename T, typename G>
__device__ __forceinline__ void momentum_row(const MomTile& t, int64_t unit, const MatGeom& g,
                                             const MatPtrs& p, double* partials,
                                             const ElemParams& prm) {
  static_assert(kMomRowSeg == kElemThreads * 4, "one 4-column group per thread");
  const int64_t rows = g.rows, cols = g.cols;
  const int64_t c_pad = g.c_pad, ldD = g.c_pad + g.ld_skew;
  T* D = reinterpret_cast<T*>(g.X[0]);
  const int64_t row = t.tr;
  const int64_t col = (int64_t)t.tc * kMomRowSeg + threadIdx.x * 4;
  const float beta = prm.beta;
  float ss = 0.0f;
  if (col < c_pad) {   // c_pad is a multiple of 4
    f32x4_t y = {0.0f, 0.0f, 0.0f, 0.0f};
    if (row < rows) {
      const int64_t off = row * cols + col;
      if ((cols & 3) == 0 && col + 4 <= cols) {
        const f32x4_t gv = GradLoad<G>::load4(p.g, off);
        const f32x4_t m = beta * Vec4<float>::load_nt(p.m + off) + gv;
        Vec4<float>::store_nt(p.m + off, m);
        y = prm.nesterov ? gv + beta * m : m;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col + e < cols) {
            const float gs = GradLoad<G>::load1(p.g, off + e);
            const float ms = beta * p.m[off + e] + gs;
            p.m[off + e] = ms;
            y[e] = prm.nesterov ? gs + beta * ms : ms;
          }
        }
      }
    }
    ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
    Vec4<T>::store(D + row * ldD + col, y);
  }
  write_wave_partial(partials, unit, ss);
}

template <typename T>
__global__ __launch_bounds__(kElemThreads) void momentum_row_kernel(const MomTile* __restrict__ units,
                                                                    const MatGeom* __restrict__ geo,
                                                                    const MatPtrs* __restrict__ ptrs,
                                                                    double* __restrict__ partials,
                                                                    ElemParams prm) {
  const int64_t unit = blockIdx.x;
  const MomTile t = units[unit];
  const MatGeom& g = geo[t.mat];
  const MatPtrs p = ptrs[t.mat];
  if (g.g_bf16)
    momentum_row<T, uint16_t>(t, unit, g, p, partials, prm);
  else
    momentum_row<T, float>(t, unit, g, p, partials, prm);
}

template <typename T>
__global__ __launch_bounds__(kMomTileThreads) void momentum_tile_kernel(const MomTile* __restrict__ units,
                                                                     int64_t first,
                                                                     const MatGeom* __restrict__ geo,
                                                                     const MatPtrs* __restrict__ ptrs,
                                                                     double* __restrict__ partials,
                                                                     ElemParams prm) {
  __shared__ __attribute__((aligned(16))) T tile[kMomTileR][MomLds<T>::kPitch];
  const int64_t unit = first + blockIdx.x;
  const MomTile t = units[unit];
  const MatGeom& g = geo[t.mat];
  const MatPtrs p = ptrs[t.mat];
  if (g.g_bf16)
    momentum_tile<T, uint16_t>(t, unit, g, p, partials, prm, tile);
  else
    momentum_tile<T, float>(t, unit, g, p, partials, prm, tile);
}

// Sum of a matrix's block partials in block order, one wavefront per matrix:
// lane l takes blocks l, l+64, ... then a fixed xor-shuffle tree.
__device__ __forceinline__ double ordered_sum(const double* p, int64_t n, int64_t stride) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (int64_t k = lane; k < n; k += 64) s += p[k * stride];
  return wave_sum(s);
}

// ||Y||^2 of one matrix from its units' partials, one 256-thread block per
// matrix: thread t sums slots t, t + 256, ... in that order, eight loads in
// flight at a time (the row units of a large matrix leave tens of thousands
// of slots), then a fixed tree over the block.
__global__ __launch_bounds__(kElemThreads) void finalize_norm_kernel(const MatGeom* __restrict__ geo,
                                                                     const double* __restrict__ partials,
                                                                     MatScalars* __restrict__ scal,
                                                                     float eps) {
  __shared__ double red[1][4];
  const int mat = blockIdx.x;
  const MatGeom& g = geo[mat];
  const double* p = partials + kMomParts * g.mom_tile0;
  const int64_t n = kMomParts * g.mom_ntiles;
  double s = 0.0;
  int64_t k = threadIdx.x;
  for (; k + 7 * kElemThreads < n; k += 8 * kElemThreads) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[k + u * kElemThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; k < n; k += kElemThreads) s += p[k];
  double v[1] = {s};
  block_sum<1>(v, red);
  if (threadIdx.x == 0) {
    const double yn = sqrt(v[0]);
    scal[mat].y_norm = yn;
    scal[mat].s = (float)(1.0 / (yn + (double)eps));
  }
}

// ---------------------------------------------------------------------------
// flat chunk kernels over W (fp32, dense) and u (compact, ns dtype).

__global__ __launch_bounds__(64) void finalize_update_kernel(
    const MatGeom* __restrict__ geo, const double* __restrict__ partials,
    MatScalars* __restrict__ scal, muonh_stats* __restrict__ stats,
    const float* __restrict__ elr_scale, const double* __restrict__ eta_dev, ElemParams prm) {
  const int mat = blockIdx.x;
  const MatGeom& g = geo[mat];
  // per-(tile, wavefront) partials of the last B'X launch, in slot order
  const double* p = partials + 3 * g.part0;
  const double wu = ordered_sum(p + 0, g.nparts, 3);
  const double uu = ordered_sum(p + 1, g.nparts, 3);
  const double ww = ordered_sum(p + 2, g.nparts, 3);
  if (threadIdx.x != 0) return;
  const double R = scal[mat].R;
  const double eta = eta_dev ? eta_dev[mat]
                             : (double)prm.elr * (elr_scale ? (double)elr_scale[mat] : 1.0);
  const UpdateCoeffs o = update_coeffs(prm.mode, ww, wu, uu, R, eta, (double)prm.weight_decay);
  const double un = sqrt(uu), wn = sqrt(ww);
  const double k1 = o.k1, k2 = o.k2, wt_norm = o.wt_norm, elr = o.elr, inner = o.inner,
               angle = o.angle;
  scal[mat].k1 = (float)k1;
  scal[mat].k2 = (float)k2;
  muonh_stats s;
  s.y_norm = scal[mat].y_norm;
  s.u_norm = un;
  s.w_norm = wn;
  s.inner = inner;
  s.c = inner / R;
  s.wt_norm = wt_norm;
  s.elr = elr;
  s.angle = angle;
  s.nonfinite = !(isfinite(s.y_norm) && isfinite(un) && isfinite(wn) && isfinite(wt_norm) &&
                  isfinite(inner));
  s.reserved = 0;
  stats[mat] = s;
}

// The per-matrix step size eta_i = elr * elr_scale[i] in fp64 (the same
// product the finaliser forms from its arguments), written to device memory
// so that a recorded step reads this call's learning rate.
__global__ __launch_bounds__(256) void set_eta_kernel(int32_t nmat, const float* __restrict__ elr_scale,
                                                      float elr, double* __restrict__ eta) {
  for (int32_t i = threadIdx.x; i < nmat; i += blockDim.x)
    eta[i] = (double)elr * (elr_scale ? (double)elr_scale[i] : 1.0);
}

// The flat streaming kernels (update, AdamW) run one block per slice of
// kSlice elements, kSlicesPerChunk blocks per chunk, each thread one 16-byte
// vector of every stream: many short blocks, dispatched in order, keep the
// addresses in flight within a narrow ascending window, which streams faster
// on HBM3E than long per-block loops (measured on MI355X: 6.5 TB/s against
// 5.3 TB/s for the same read/write mix).
constexpr int kSlice = kElemThreads * 4;
constexpr int kSlicesPerChunk = kChunk / kSlice;
static_assert(kChunk % kSlice == 0, "a chunk is a whole number of slices");

template <typename T>
__global__ __launch_bounds__(kElemThreads) void update_kernel(const Chunk* __restrict__ chunks,
                                                              const MatGeom* __restrict__ geo,
                                                              const MatPtrs* __restrict__ ptrs,
                                                              const MatScalars* __restrict__ scal) {
  const Chunk c = chunks[blockIdx.x / kSlicesPerChunk];
  const int s0 = (int)(blockIdx.x % kSlicesPerChunk) * kSlice;
  if (s0 >= c.len) return;
  const int len = min(kSlice, c.len - s0);
  const MatGeom& g = geo[c.mat];
  float* W = ptrs[c.mat].w + c.start + s0;
  const T* U = reinterpret_cast<const T*>(g.U) + c.start + s0;
  const float k1 = scal[c.mat].k1, k2 = scal[c.mat].k2;
  const int i = threadIdx.x * 4;
  if (i + 4 <= len) {
    const f32x4_t w = Vec4<float>::load_nt(W + i);
    const f32x4_t u = Vec4<T>::load_nt(U + i);
    Vec4<float>::store_nt(W + i, k1 * w - k2 * u);
  } else {
    for (int j = i; j < len; ++j) {
      float u;
      if constexpr (sizeof(T) == 2) u = bf16_to_f32(U[j]); else u = U[j];
      W[j] = k1 * W[j] - k2 * u;
    }
  }
}

// Zero fill of a 16-byte aligned region whose size is a multiple of 16 bytes
// (clears the Newton-Schulz buffers of a workspace that other plans used
// before; a kernel rather than a memset so a captured graph holds no memset
// node).  One 16-byte store per thread and iteration, grid-stride.
__global__ __launch_bounds__(kElemThreads) void fill_zero_kernel(u32x4_t* __restrict__ p, int64_t n16) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kElemThreads)
    p[i] = z;
}

// ||W_0||^2 partials (radius at init).
__global__ __launch_bounds__(kElemThreads) void radius_kernel(const Chunk* __restrict__ chunks,
                                                              const MatPtrs* __restrict__ ptrs,
                                                              double* __restrict__ partials) {
  __shared__ double red[1][4];
  const Chunk c = chunks[blockIdx.x];
  const float* W = ptrs[c.mat].w + c.start;
  const int tid = threadIdx.x;
  float ww = 0.0f;
  const int n4 = c.len & ~3;
  for (int i = tid * 4; i < n4; i += kElemThreads * 4) {
    const f32x4_t w = Vec4<float>::load(W + i);
    ww += w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
  }
  for (int i = n4 + tid; i < c.len; i += kElemThreads) ww += W[i] * W[i];
  double v[1] = {(double)ww};
  block_sum<1>(v, red);
  if (tid == 0) partials[blockIdx.x] = v[0];
}

__global__ __launch_bounds__(64) void finalize_radius_kernel(const MatGeom* __restrict__ geo,
                                                             const double* __restrict__ partials,
                                                             const int32_t* __restrict__ need,
                                                             MatScalars* __restrict__ scal) {
  const int mat = blockIdx.x;
  const MatGeom& g = geo[mat];
  const double ss = ordered_sum(partials + g.chunk0, g.nchunks, 1);
  // R is carried as a float across the interface (descriptor and muonh_get_radii), so the
  // measured value is rounded to float here: the steps then use exactly the R a caller
  // reads back and passes to a new handle, and a resume continues bit for bit.
  if (threadIdx.x == 0 && need[mat]) scal[mat].R = (double)(float)sqrt(ss);
}

template <typename T>
__global__ __launch_bounds__(kElemThreads) void copy_update_kernel(const T* __restrict__ U,
                                                                   int64_t count,
                                                                   float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * kElemThreads + threadIdx.x;
  if (i >= count) return;
  if constexpr (sizeof(T) == 2) dst[i] = bf16_to_f32(U[i]); else dst[i] = U[i];
}

// ---------------------------------------------------------------------------
// AdamW (decoupled weight decay, bias-corrected), one chunk per block, fp32.

__device__ __forceinline__ float adamw_elem(float w, float& m, float& v, float g,
                                            const AdamwParams& p) {
  m = p.beta1 * m + p.omb1 * g;
  v = p.beta2 * v + p.omb2 * (g * g);
  const float denom = sqrtf(v) * p.rbc2 + p.eps;
  return w * p.decay - p.step_size * (m / denom);
}

__device__ __forceinline__ void adamw4(f32x4_t& w, f32x4_t& m, f32x4_t& v, const f32x4_t& g,
                                       const AdamwParams& p) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float me = m[e], ve = v[e];
    w[e] = adamw_elem(w[e], me, ve, g[e], p);
    m[e] = me;
    v[e] = ve;
  }
}

// AdamW streams seven arrays (W, m, v read and written, g read): 128-thread
// blocks over 512-element slices measured faster than the update kernel's
// 256 x 1024 on MI355X.
constexpr int kAdamwThreads = 128;
constexpr int kAdamwSlice = kAdamwThreads * 4;
constexpr int kAdamwSlicesPerChunk = kChunk / kAdamwSlice;
static_assert(kChunk % kAdamwSlice == 0, "a chunk is a whole number of AdamW slices");

template <typename G>
__device__ __forceinline__ void adamw_slice(const Chunk& c, int s0, const AdamwPtrs& q,
                                            const AdamwParams& p) {
  const int len = min(kAdamwSlice, c.len - s0);
  float* W = q.w + c.start + s0;
  float* Mm = q.m + c.start + s0;
  float* V = q.v + c.start + s0;
  const G* Gp = reinterpret_cast<const G*>(q.g) + c.start + s0;
  const int i = threadIdx.x * 4;
  if (i + 4 <= len) {
    f32x4_t w = Vec4<float>::load_nt(W + i), m = Vec4<float>::load_nt(Mm + i);
    f32x4_t v = Vec4<float>::load_nt(V + i);
    const f32x4_t g = Vec4<G>::load_nt(Gp + i);
    adamw4(w, m, v, g, p);
    Vec4<float>::store_nt(W + i, w);
    Vec4<float>::store_nt(Mm + i, m);
    Vec4<float>::store_nt(V + i, v);
  } else {
    for (int j = i; j < len; ++j) {
      float g;
      if constexpr (sizeof(G) == 2) g = bf16_to_f32(Gp[j]); else g = Gp[j];
      float m = Mm[j], v = V[j];
      W[j] = adamw_elem(W[j], m, v, g, p);
      Mm[j] = m;
      V[j] = v;
    }
  }
}

__global__ __launch_bounds__(kAdamwThreads) void adamw_kernel(const Chunk* __restrict__ chunks,
                                                             const AdamwPtrs* __restrict__ ptrs,
                                                             AdamwParams prm) {
  const Chunk c = chunks[blockIdx.x / kAdamwSlicesPerChunk];
  const int s0 = (int)(blockIdx.x % kAdamwSlicesPerChunk) * kAdamwSlice;
  if (s0 >= c.len) return;
  const AdamwPtrs q = ptrs[c.mat];
  if (q.g_bf16)
    adamw_slice<uint16_t>(c, s0, q, prm);
  else
    adamw_slice<float>(c, s0, q, prm);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_momentum(int bf16, const MomTile* units, int64_t nrow, int64_t ntile,
                           const MatGeom* geo, const MatPtrs* ptrs, double* partials,
                           ElemParams prm, hipStream_t st) {
  if (nrow > 0) {
    if (bf16)
      hipLaunchKernelGGL(momentum_row_kernel<uint16_t>, dim3((unsigned)nrow), dim3(kElemThreads), 0,
                         st, units, geo, ptrs, partials, prm);
    else
      hipLaunchKernelGGL(momentum_row_kernel<float>, dim3((unsigned)nrow), dim3(kElemThreads), 0,
                         st, units, geo, ptrs, partials, prm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ntile > 0) {
    if (bf16)
      hipLaunchKernelGGL(momentum_tile_kernel<uint16_t>, dim3((unsigned)ntile), dim3(kMomTileThreads),
                         0, st, units, nrow, geo, ptrs, partials, prm);
    else
      hipLaunchKernelGGL(momentum_tile_kernel<float>, dim3((unsigned)ntile), dim3(kMomTileThreads),
                         0, st, units, nrow, geo, ptrs, partials, prm);
  }
  return hipGetLastError();
}

hipError_t launch_finalize_norm(int32_t nmat, const MatGeom* geo, const double* partials,
                                MatScalars* scal, float eps, hipStream_t st) {
  hipLaunchKernelGGL(finalize_norm_kernel, dim3(nmat), dim3(kElemThreads), 0, st, geo, partials,
                     scal, eps);
  return hipGetLastError();
}

hipError_t launch_finalize_update(int32_t nmat, const MatGeom* geo, const double* partials,
                                  MatScalars* scal, muonh_stats* stats, const float* elr_scale,
                                  const double* eta_dev, ElemParams prm, hipStream_t st) {
  hipLaunchKernelGGL(finalize_update_kernel, dim3(nmat), dim3(64), 0, st, geo, partials, scal,
                     stats, elr_scale, eta_dev, prm);
  return hipGetLastError();
}

hipError_t launch_set_eta(int32_t nmat, const float* elr_scale, float elr, double* eta,
                          hipStream_t st) {
  hipLaunchKernelGGL(set_eta_kernel, dim3(1), dim3(256), 0, st, nmat, elr_scale, elr, eta);
  return hipGetLastError();
}

hipError_t launch_update(int bf16, const Chunk* chunks, int64_t nchunks, const MatGeom* geo,
                         const MatPtrs* ptrs, const MatScalars* scal, hipStream_t st) {
  if (nchunks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(nchunks * kSlicesPerChunk);
  if (bf16)
    hipLaunchKernelGGL(update_kernel<uint16_t>, dim3(grid), dim3(kElemThreads), 0, st, chunks,
                       geo, ptrs, scal);
  else
    hipLaunchKernelGGL(update_kernel<float>, dim3(grid), dim3(kElemThreads), 0, st, chunks, geo,
                       ptrs, scal);
  return hipGetLastError();
}

hipError_t launch_radius(const Chunk* chunks, int64_t nchunks, const MatPtrs* ptrs,
                         double* partials, hipStream_t st) {
  if (nchunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(radius_kernel, dim3((unsigned)nchunks), dim3(kElemThreads), 0, st, chunks,
                     ptrs, partials);
  return hipGetLastError();
}

hipError_t launch_finalize_radius(int32_t nmat, const MatGeom* geo, const double* partials,
                                  const int32_t* need, MatScalars* scal, hipStream_t st) {
  hipLaunchKernelGGL(finalize_radius_kernel, dim3(nmat), dim3(64), 0, st, geo, partials, need,
                     scal);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0 || (bytes & 15u) != 0) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t blocks = std::min<int64_t>((n16 + kElemThreads - 1) / kElemThreads, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kElemThreads), 0, st,
                     reinterpret_cast<u32x4_t*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_copy_update(int bf16, const void* U, int64_t count, float* dst, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((count + kElemThreads - 1) / kElemThreads);
  if (bf16)
    hipLaunchKernelGGL(copy_update_kernel<uint16_t>, dim3(grid), dim3(kElemThreads), 0, st,
                       reinterpret_cast<const uint16_t*>(U), count, dst);
  else
    hipLaunchKernelGGL(copy_update_kernel<float>, dim3(grid), dim3(kElemThreads), 0, st,
                       reinterpret_cast<const float*>(U), count, dst);
  return hipGetLastError();
}

hipError_t launch_adamw(const Chunk* chunks, int64_t nchunks, const AdamwPtrs* ptrs,
                        AdamwParams prm, hipStream_t st) {
  if (nchunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)(nchunks * kAdamwSlicesPerChunk)), dim3(kAdamwThreads),
                     0, st, chunks, ptrs, prm);
  return hipGetLastError();
}

}  // namespace muonh
