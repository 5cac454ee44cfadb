// Grouped MFMA GEMM engine for the Newton-Schulz products (gfx950 / CDNA4).
//
// One launch runs one of the three products of a quintic Newton-Schulz
// iteration for EVERY matrix of the plan, whatever its shape:
//   kGram : A  = alpha X X^T                 (m x m, contraction over n)
//   kPoly : B  = b A + c A A                 (m x m, contraction over m)
//   kApply: X' = alpha (a X + B X)           (m x n, contraction over m)
// (the iteration of the Muon update; the pages name it in "Puro-2B: Poor
// Lab's Qwen2-1.5B Trained on RTX 5090 within $5090", arXiv HTML §3.3).
//
// Every product is written as C = P Q^T with both operands row-major and the
// contraction index contiguous, so both MFMA operands are read the same way:
//   kGram : P = Q = X;   kPoly : P = Q = A (A is symmetric);
//   kApply: P = B, Q = X^T (the iterate is kept in both layouts).
//
// Work decomposition: a 256 x 256 output tile per workgroup of 4 wavefronts
// (2 x 2, each 128 x 128 = 4 x 4 MFMA blocks of 32 x 32).  K advances in
// tiles of 128 bytes per row (64 bf16 / 32 fp32), double-buffered in LDS
// (2 stages x 2 operands x 32 KiB = 128 KiB of the 160 KiB per CU), with the
// next tile's global loads in flight while the current one feeds the MFMAs.
// LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by (row & 7),
// so the 32-row MFMA operand reads and the row-wise stores are free of bank
// conflicts without padding.
//
// The host builds the tile list: for the symmetric products only the upper
// tiles are listed and each off-diagonal tile also writes its mirror, and the
// list is interleaved so that workgroup i (which the hardware places on XCD
// i mod 8) belongs to that XCD's share of whole row panels.

#include "device_util.h"
#include "internal.h"

namespace muonh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRowBytes = 128;                       // one K tile of one row
constexpr int kOperandBytes = kGemmTile * kRowBytes; // 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;       // P and Q
constexpr int kLoadsPerThread = kOperandBytes / 16 / kGemmThreads;  // 8

// One 16-byte LDS operand fragment x one 16-byte fragment -> 32x32 block.
template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {
  // 32x32x16 bf16: lanes 0-31 carry k 0-7, lanes 32-63 carry k 8-15.
  static __device__ __forceinline__ void run(f32x16_t& acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // 32x32x2 fp32, four times: element e of the fragment of lane group g
  // is k = 4g + e of the 8-wide slice; P and Q fragments agree on it.
  static __device__ __forceinline__ void run(f32x16_t& acc, u32x4_t a, u32x4_t b) {
    const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
    const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
  }
};

template <typename T, int MODE>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const GemmProb* __restrict__ probs, const GemmTile* __restrict__ tiles,
    const MatScalars* __restrict__ scal, int first_iter, int last_iter, int symmetric,
    float ca, float cb, float cc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  const GemmTile t = tiles[blockIdx.x];
  if (t.prob < 0) return;
  const GemmProb pr = probs[t.prob];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int row0 = t.tm * kGemmTile;
  const int col0 = t.tn * kGemmTile;

  // Global -> LDS staging: thread owns rows (i*32 + lr), 16-byte chunk lc.
  const int lr = tid >> 3, lc = tid & 7;
  const size_t pstride = (size_t)pr.ldp * sizeof(T);
  const size_t qstride = (size_t)pr.ldq * sizeof(T);
  const uint8_t* pbase = reinterpret_cast<const uint8_t*>(pr.P) + (size_t)(row0 + lr) * pstride + lc * 16;
  const uint8_t* qbase = reinterpret_cast<const uint8_t*>(pr.Q) + (size_t)(col0 + lr) * qstride + lc * 16;
  const int st_off = lr * kRowBytes + ((lc ^ (lr & 7)) << 4);

  u32x4_t ra[kLoadsPerThread], rb[kLoadsPerThread];
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)(((size_t)pr.K * sizeof(T)) / kRowBytes);

  auto gload = [&](int kt) {
    const size_t koff = (size_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      ra[i] = ld_global<u32x4_t>(pbase + (size_t)(i * 32) * pstride + koff);
      rb[i] = ld_global<u32x4_t>(qbase + (size_t)(i * 32) * qstride + koff);
    }
  };
  auto sstore = [&](int stage) {
    uint8_t* s = smem + stage * kStageBytes + st_off;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      *reinterpret_cast<u32x4_t*>(s + i * 32 * kRowBytes) = ra[i];
      *reinterpret_cast<u32x4_t*>(s + kOperandBytes + i * 32 * kRowBytes) = rb[i];
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  // MFMA operand rows: 32 consecutive rows per block; row & 7 == lane & 7.
  const int swz = lane & 7;
  const int a_row = wr * 128 + (lane & 31);
  const int b_row = wc * 128 + (lane & 31);

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* sA = smem + cur * kStageBytes;
    const uint8_t* sB = sA + kOperandBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = ((s * 2 + (lane >> 5)) ^ swz) << 4;
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(sA + (a_row + i * 32) * kRowBytes + ch);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(sB + (b_row + j * 32) * kRowBytes + ch);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mfma<T>::run(acc[i][j], a[i], b[j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------
  // Accumulator register r of block (i, j) holds C[row][col] with
  //   row = 32 i + 8 (r / 4) + 4 (lane / 32) + (r % 4),  col = 32 j + lane % 32
  // (inside the wavefront's 128 x 128 sub-tile): every group of 4 registers
  // is 4 consecutive rows of one column, i.e. 4 contiguous elements of the
  // transposed layout.
  float alpha = 1.0f;
  if (first_iter) {
    const float s = scal[pr.mat].s;
    alpha = (MODE == kGram) ? s * s : s;
  }
  const bool mirror = (MODE == kGram || MODE == kPoly) && symmetric && (t.tm != t.tn);
  T* O = reinterpret_cast<T*>(MODE == kApplyLast ? pr.U : pr.O);
  T* OT = reinterpret_cast<T*>(pr.OT);
  const T* E = reinterpret_cast<const T*>(pr.E);

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = col0 + wc * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = row0 + wr * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
        f32x4_t v;
        v[0] = acc[i][j][4 * g + 0];
        v[1] = acc[i][j][4 * g + 1];
        v[2] = acc[i][j][4 * g + 2];
        v[3] = acc[i][j][4 * g + 3];
        if (MODE == kGram) {
          v *= alpha;
        } else if (MODE == kPoly) {
          const f32x4_t e = Vec4<T>::load(E + (size_t)col * pr.lde + row);
          v = cb * e + cc * v;
        } else {
          const f32x4_t e = Vec4<T>::load(E + (size_t)col * pr.lde + row);
          v = alpha * (ca * e + v);
        }
        if (MODE == kApplyLast) {
          // u in the matrix's own orientation, compact: [um x un] or, for a
          // tall matrix, its transpose [un x um].
          if (col < pr.un && row < pr.um) {
            const size_t base = pr.u_tall ? (size_t)col * pr.um + row : (size_t)row * pr.un + col;
            const size_t step = pr.u_tall ? 1 : (size_t)pr.un;
            Vec4<T>::store1(O + base, v[0]);
            if (row + 1 < pr.um) Vec4<T>::store1(O + base + step, v[1]);
            if (row + 2 < pr.um) Vec4<T>::store1(O + base + 2 * step, v[2]);
            if (row + 3 < pr.um) Vec4<T>::store1(O + base + 3 * step, v[3]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) Vec4<T>::store1(O + (size_t)(row + e) * pr.ldo + col, v[e]);
          if (MODE == kApply) {
            Vec4<T>::store(OT + (size_t)col * pr.ldot + row, v);
          } else if (mirror) {
            Vec4<T>::store(O + (size_t)col * pr.ldo + row, v);
          }
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_t(int mode, const GemmProb* probs, const GemmTile* tiles, int64_t ntiles,
                    const MatScalars* scal, int first_iter, int last_iter, int symmetric,
                    float ca, float cb, float cc, hipStream_t st) {
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)ntiles), block(kGemmThreads);
  switch (mode) {
    case kGram:
      hipLaunchKernelGGL((gemm_kernel<T, kGram>), grid, block, 0, st, probs, tiles, scal,
                         first_iter, last_iter, symmetric, ca, cb, cc);
      break;
    case kPoly:
      hipLaunchKernelGGL((gemm_kernel<T, kPoly>), grid, block, 0, st, probs, tiles, scal,
                         first_iter, last_iter, symmetric, ca, cb, cc);
      break;
    default:
      if (last_iter)
        hipLaunchKernelGGL((gemm_kernel<T, kApplyLast>), grid, block, 0, st, probs, tiles, scal,
                           first_iter, last_iter, symmetric, ca, cb, cc);
      else
        hipLaunchKernelGGL((gemm_kernel<T, kApply>), grid, block, 0, st, probs, tiles, scal,
                           first_iter, last_iter, symmetric, ca, cb, cc);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int bf16, int mode, const GemmProb* probs, const GemmTile* tiles,
                       int64_t ntiles, const MatScalars* scal, int first_iter, int last_iter,
                       int symmetric, float ca, float cb, float cc, hipStream_t st) {
  if (bf16)
    return launch_t<uint16_t>(mode, probs, tiles, ntiles, scal, first_iter, last_iter, symmetric,
                              ca, cb, cc, st);
  return launch_t<float>(mode, probs, tiles, ntiles, scal, first_iter, last_iter, symmetric, ca,
                         cb, cc, st);
}

}  // namespace muonh
