// Grouped MFMA GEMM engine for the Newton-Schulz products (gfx950 / CDNA4).
//
// One launch runs one of the three products of a quintic Newton-Schulz
// iteration for EVERY matrix of the plan, whatever its shape:
//   kGram : A  = alpha X X^T                 (m x m, contraction over n)
//   kPoly : B' = b A + c A A + a I           (m x m, contraction over m)
//   kApply: X' = alpha B' X  (= alpha (a X + B X))   (m x n, contraction over m)
// (the iteration of the Muon update; the pages name it in "Puro-2B: Poor
// Lab's Qwen2-1.5B Trained on RTX 5090 within $5090", arXiv HTML §3.3).
//
// Folding a X into B' = B + a I leaves the update with no epilogue operand.
// Every product is written as C = P Q^T with both operands row-major and the
// contraction index contiguous, so both MFMA operands are read the same way:
//   kGram : P = Q = X;   kPoly : P = Q = A (A is symmetric);
//   kApply: P = B' (symmetric), Q = X^T (fp32: a stored copy; bf16: X read
//           through transposing LDS reads, below).
//
// Work decomposition: a 256 x 256 output tile per workgroup of 4 wavefronts
// (2 x 2, each 128 x 128 = 4 x 4 MFMA blocks of 32 x 32, 256 fp32
// accumulators per lane).  K advances in stages of 128 bytes per operand row
// (64 bf16 / 32 fp32): global loads of whole 128-byte lines into registers
// three stages ahead, LDS writes one stage ahead into a 2-slot ring (2 x 64
// KiB), and one barrier per stage, placed before its last 16-deep sub-step so
// that the next stage's first fragments are read while that sub-step runs.
// Loads, LDS writes and fragment reads are spread between the MFMAs so the
// in-order issue never parks the MFMA pipe behind a memory queue.  LDS rows
// keep their 16-byte chunks XOR-swizzled per row, so the 32-row MFMA operand
// reads are free of bank conflicts without padding.
//
// bf16 B' X reads X in its own row-major layout: a stage of that operand is
// 64 rows (k) x 256 columns (n), and the MFMA B fragments come out of LDS
// through the transposing read ds_read_b64_tr_b16 (one 16-lane group turns
// 4 rows x 16 columns into 16 lanes x 4 k).  The iterate is then stored once
// (no X^T copy) and B' X writes one layout.  The fp32 path keeps X and X^T.
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
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kRowBytes = 128;                       // one K stage of one operand row
constexpr int kStages = 2;                           // LDS ring depth
constexpr int kOperandBytes = kGemmTile * kRowBytes; // 32 KiB
constexpr int kStageBytes = 2 * kOperandBytes;       // P and Q
constexpr int kSubsteps = kRowBytes / 32;            // 16-deep MFMA steps per stage
// K-major Q operand (bf16 B' X): 64 rows of 256 columns per stage.
constexpr int kTrRows = kRowBytes / 2;               // k rows per stage
constexpr int kTrPitch = kGemmTile * 2;              // 512 B per LDS row
static_assert(kTrRows * kTrPitch == kOperandBytes, "both Q layouts fill one operand slot");
// The bf16 epilogue stages each wavefront's 128 x 128 sub-tile in its own
// region of 128 rows x (256 + 16) bytes.
constexpr int kEpiStride = 272;
constexpr int kEpiBytes = 4 * 128 * kEpiStride;
constexpr int kLdsBytes = (kStages * kStageBytes > kEpiBytes) ? kStages * kStageBytes : kEpiBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one CU");

#define MUONH_LDS __attribute__((address_space(3)))

// Chunk c of a 128-byte LDS row r sits at 16-byte slot c ^ swz128(r).  For a
// 16-byte read of one chunk by 32 consecutive rows this is free of bank
// conflicts whether the LDS serves 8 lanes (32 banks) or 16 lanes (64 banks)
// per cycle.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// Chunk c of a 512-byte K-major row k sits at slot c ^ swz_tr(k).  A
// transposing read has each 16-lane group fetch 4 consecutive rows x 32
// bytes, two groups side by side: with these offsets the 16 (row, chunk)
// pairs of two groups fall in distinct banks (64 banks, 32 lanes per cycle)
// and those of one group in distinct banks (32 banks, 16 lanes per cycle).
__device__ __forceinline__ int swz_tr(int k) { return (4 * (k & 1)) ^ (10 * ((k >> 1) & 1)); }

// Workgroup barrier without a memory fence (a fence would also wait for the
// global loads in flight into registers); the empty asm statements keep the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (63 << 8));
  asm volatile("" ::: "memory");
}

// Buffer descriptor word 3 for raw (unformatted, unswizzled) buffer access on
// gfx9-family devices.
constexpr int kBufferConfig = 0x00020000;

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgVmemRead = 0x020, kSgDsRead = 0x100, kSgDsWrite = 0x200;
#define MUONH_SG(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Writes one wavefront's <W,u>, ||u||^2, ||W||^2 partial (fp64 xor-shuffle
// tree over the lanes' fp32 sums, fixed order) to slot `slot`.
__device__ __forceinline__ void write_stats(double* part, int64_t slot, float wu, float uu, float ww) {
  double v[3] = {(double)wu, (double)uu, (double)ww};
#pragma unroll
  for (int k = 0; k < 3; ++k)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[k] += __shfl_xor(v[k], off, 64);
  if ((threadIdx.x & 63) == 0) {
    part[3 * slot + 0] = v[0];
    part[3 * slot + 1] = v[1];
    part[3 * slot + 2] = v[2];
  }
}

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
    float ca, float cb, float cc, const MatPtrs* __restrict__ ptrs, double* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];

  const GemmTile t = tiles[blockIdx.x];
  if (t.prob < 0) return;
  const GemmProb pr = probs[t.prob];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int row0 = t.tm * kGemmTile;
  const int col0 = t.tn * kGemmTile;

  const size_t pstride = (size_t)pr.ldp * sizeof(T);
  const size_t qstride = (size_t)pr.ldq * sizeof(T);
  MUONH_LDS uint8_t* lds = (MUONH_LDS uint8_t*)smem;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // K stages; K is a multiple of 256 elements (the planner pads to it), so
  // nk is even and >= 4.
  const int nk = (int)(((size_t)pr.K * sizeof(T)) / kRowBytes);

  // MFMA operand rows: 32 consecutive rows per block; (row & 15) == (lane & 15).
  // Sub-step s reads 16-byte chunk 2s (lanes 0-31) / 2s+1 (lanes 32-63).
  const int swz = swz128(lane & 15);
  const int a_off = (wr * 128 + (lane & 31)) * kRowBytes;
  // A diagonal tile of a Gram-type product (tm == tn) has P == Q: its B
  // fragments are read from the staged P panel, and its Q loads go through a
  // descriptor with no valid range (they return zeros without a memory
  // access), which takes half of such a tile's operand traffic off the L2.
  const bool diag = (MODE == kGram || MODE == kPoly) && t.tm == t.tn;
  const int b_off = (diag ? 0 : kOperandBytes) + (wc * 128 + (lane & 31)) * kRowBytes;
  // K-major B fragments (kQT): lane l of 16-lane group g = l / 16 fetches the
  // 8 bytes at row 16 s + 4 h + 8 (g / 2) + (l % 16) / 4 of the stage and
  // column 32 j + 16 (g % 2) + 4 (l % 4) of the wavefront's 128 columns; the
  // transposing read then hands lane l the 4 consecutive k of column
  // 32 j + l % 32 (h = 0: the first 4 of the lane's 8 k, h = 1: the last 4).
  constexpr bool kQT = sizeof(T) == 2 && (MODE == kApply || MODE == kApplyLast);
  const int tr_k = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_c = wc * 16 + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
  int tr_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    tr_off[j] = kOperandBytes + tr_k * kTrPitch + (((tr_c + 4 * j) ^ swz_tr(tr_k)) << 4) + (lane & 1) * 8;
  auto load_frag = [&](u32x4_t (&a)[4], u32x4_t (&b)[4], int slot, int s) {
    const uint8_t* st = smem + slot * kStageBytes + (((s * 2 + (lane >> 5)) ^ swz) << 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const u32x4_t*>(st + a_off + i * 32 * kRowBytes);
    if constexpr (kQT) {
      MUONH_LDS uint8_t* sq = lds + slot * kStageBytes + s * 16 * kTrPitch;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2_t lo = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((MUONH_LDS i16x4_t*)(sq + tr_off[j])));
        const u32x2_t hi = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (MUONH_LDS i16x4_t*)(sq + tr_off[j] + 4 * kTrPitch)));
        b[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const u32x4_t*>(st + b_off + j * 32 * kRowBytes);
    }
  };
  // bf16 B'X swaps the MFMA operands: block (i, j) then accumulates the
  // transpose, so each lane holds 4 consecutive COLUMNS of one output row and
  // the row-major epilogue writes 8 bytes per register group instead of 2.
  constexpr bool kSwap = (MODE == kApply) && sizeof(T) == 2;
  auto mma = [&](const u32x4_t (&a)[4], const u32x4_t (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (kSwap)
          Mfma<T>::run(acc[i][j], b[j], a[i]);
        else
          Mfma<T>::run(acc[i][j], a[i], b[j]);
      }
  };
  u32x4_t fa0[4], fb0[4], fa1[4], fb1[4];

  // Thread t owns rows (i*32 + t/8) and 16-byte chunk t%8 of a row-major
  // operand, so one load instruction of a wavefront covers 8 whole 128-byte
  // lines; of a K-major Q operand it owns rows (i*8 + t/32) and chunk t%32
  // (2 whole 512-byte row segments per instruction).  Stage s is loaded into
  // one of two register sets during stage s-3 (P half in sub-step 1, Q half
  // in sub-step 2; for bf16 B'X spread over sub-steps 0-1 and 2-3), written
  // to LDS slot s%2 during stage s-1 (P in sub-step 0, Q in sub-step 1) and
  // published by the barrier that stage s-1 places before its last sub-step.
  static_assert(kSubsteps == 4, "the stage schedule below assumes 4 sub-steps");
  constexpr int kLd = kOperandBytes / 16 / kGemmThreads;   // 8 loads per operand
  const int srow = tid >> 3, schunk = tid & 7;
  const int qrow = tid >> 5, qchunk = tid & 31;
  // Operand loads are buffer loads: a uniform base in the descriptor, a
  // per-thread byte offset fixed for the whole tile and a uniform per-load
  // offset, so no vector address arithmetic is issued between the MFMAs.
  // Offsets stay below 2^31: a row-major operand's base is the tile's panel
  // (256 rows of at most 64 Ki + 32 elements: < 70 MB), and the K-major
  // X of bf16 B'X gets a new base at every stage (64 rows), since the whole
  // of X can exceed 2 GiB.
  const uint8_t* pbase = reinterpret_cast<const uint8_t*>(pr.P) + (size_t)row0 * pstride;
  const uint8_t* qbase = kQT ? reinterpret_cast<const uint8_t*>(pr.Q) + (size_t)col0 * sizeof(T)
                             : reinterpret_cast<const uint8_t*>(pr.Q) + (size_t)col0 * qstride;
  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pbase), (short)0, -1, kBufferConfig);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qbase), (short)0, __builtin_amdgcn_readfirstlane(diag ? 0 : -1),
      kBufferConfig);
  const int pvoff = (int)(srow * pstride) + schunk * 16;
  const int qvoff = kQT ? (int)(qrow * qstride) + qchunk * 16 : (int)(srow * qstride) + schunk * 16;
  const int sst = srow * kRowBytes + ((schunk ^ swz128(srow & 15)) << 4);
  const int sstq = kQT ? qrow * kTrPitch + ((qchunk ^ swz_tr(qrow)) << 4) : sst;
  // s_waitcnt lgkmcnt(0) alone: this wavefront's LDS accesses are done.
  auto wait_lds = [&]() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
  };
  u32x4_t ra0[kLd], rb0[kLd], ra1[kLd], rb1[kLd];
  // Stages past the last one (the pipeline's tail) reload the last stage.
  auto bload = [&](__amdgpu_buffer_rsrc_t rs, int voff, size_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (int)soff, 0));
  };
  // loads i0 .. i1-1 of a register set
  auto gload_p_part = [&](u32x4_t (&r)[kLd], int kt, int i0, int i1) {
    const size_t koff = (size_t)min(kt, nk - 1) * kRowBytes;
#pragma unroll
    for (int i = i0; i < i1; ++i) r[i] = bload(prs, pvoff, (size_t)(i * 32) * pstride + koff);
  };
  auto gload_q_part = [&](u32x4_t (&r)[kLd], int kt, int i0, int i1) {
    if constexpr (kQT) {
      const size_t k0 = (size_t)min(kt, nk - 1) * kTrRows;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(qbase + k0 * qstride), (short)0, -1, kBufferConfig);
#pragma unroll
      for (int i = i0; i < i1; ++i) r[i] = bload(rs, qvoff, (size_t)(i * 8) * qstride);
    } else {
      const size_t koff = (size_t)min(kt, nk - 1) * kRowBytes;
#pragma unroll
      for (int i = i0; i < i1; ++i) r[i] = bload(qrs, qvoff, (size_t)(i * 32) * qstride + koff);
    }
  };
  auto gload_p = [&](u32x4_t (&r)[kLd], int kt) { gload_p_part(r, kt, 0, kLd); };
  auto gload_q = [&](u32x4_t (&r)[kLd], int kt) { gload_q_part(r, kt, 0, kLd); };
  // Where a stage's loads go: all P loads in sub-step 1 and all Q loads in
  // sub-step 2, or (kSpread) half of each one sub-step earlier / later, so
  // every sub-step issues four.  Spreading measured 2% faster for B'X and
  // no better for X X^T or A A.
  constexpr bool kSpread = kQT;
  constexpr int kPSplit = kSpread ? kLd / 2 : 0;     // P loads issued in sub-step 0
  constexpr int kQSplit = kSpread ? kLd / 2 : kLd;   // Q loads issued in sub-step 2
  // Row i of this thread's share sits 4 KiB further in either Q layout.
  // One base register per slot and operand layout, opaque to the compiler,
  // so the operand and row offsets (< 64 KiB) go into the immediate offset
  // field instead of a fresh address computation per write.
  int wbase[2][2];
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    wbase[sl][0] = sl * kStageBytes + sst;
    wbase[sl][1] = sl * kStageBytes + sstq;
    asm volatile("" : "+v"(wbase[sl][0]), "+v"(wbase[sl][1]));
  }
  auto sstore = [&](const u32x4_t (&r)[kLd], int slot, int operand) {
    MUONH_LDS uint8_t* base = lds + wbase[slot][operand];
#pragma unroll
    for (int i = 0; i < kLd; ++i)
      *(MUONH_LDS u32x4_t*)(base + operand * kOperandBytes + i * 4096) = r[i];
  };
  // One K stage read from LDS slot `cur`; register set (ra, rb) holds the
  // next stage, which goes to slot `nxt`, and is then refilled with stage
  // kt_load.  On entry fa0/fb0 hold sub-step 0 of this stage; on exit they
  // hold sub-step 0 of the next stage.  Each sub-step's 16 MFMAs are
  // interleaved with the next sub-step's fragment reads (8, or 12 with
  // K-major B fragments), the LDS writes and the global loads, a few at a
  // time, so no read waits long and the MFMA pipe stays fed.
  auto stage = [&](u32x4_t (&ra)[kLd], u32x4_t (&rb)[kLd], int cur, int nxt, int kt_load) {
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 0: + LDS writes of the P half of the next stage
    load_frag(fa1, fb1, cur, 1);
    mma(fa0, fb0);
    sstore(ra, nxt, 0);
    gload_p_part(ra, kt_load, 0, kPSplit);
    if constexpr (kQT) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 2); MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1);
        MUONH_SG(kSgDsWrite, 1); MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsWrite, 1); MUONH_SG(kSgMfma, 1);
        if constexpr (kSpread) MUONH_SG(kSgVmemRead, 1);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsWrite, 1);
        if (kSpread && (k & 1)) MUONH_SG(kSgVmemRead, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 1: + LDS writes of the Q half, refill of the P half
    load_frag(fa0, fb0, cur, 2);
    mma(fa1, fb1);
    sstore(rb, nxt, 1);
    gload_p_part(ra, kt_load, kPSplit, kLd);
    if constexpr (kQT) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgDsWrite, 1); MUONH_SG(kSgMfma, 1);
        MUONH_SG(kSgVmemRead, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsWrite, 1);
        MUONH_SG(kSgVmemRead, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgMfma, 1);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgDsWrite, 1); MUONH_SG(kSgMfma, 1);
        MUONH_SG(kSgVmemRead, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // sub-step 2: + refill of the Q half
    load_frag(fa1, fb1, cur, 3);
    mma(fa0, fb0);
    gload_q_part(rb, kt_load, 0, kQSplit);
    if constexpr (kQT) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgVmemRead, 1); MUONH_SG(kSgMfma, 1);
        MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgMfma, 1); MUONH_SG(kSgVmemRead, 1); MUONH_SG(kSgDsRead, 1);
        MUONH_SG(kSgMfma, 1);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1); MUONH_SG(kSgMfma, 1); MUONH_SG(kSgVmemRead, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next stage is in LDS; every wavefront has its last fragments of
    // this stage in registers, so slot `cur` may be rewritten after this
    wait_lds();
    lds_barrier();
    // sub-step 3: + fragments of the next stage's sub-step 0, read early
    load_frag(fa0, fb0, nxt, 0);
    mma(fa1, fb1);
    gload_q_part(rb, kt_load, kQSplit, kLd);
    constexpr int kReads = kQT ? 12 : 8;
#pragma unroll
    for (int k = 0; k < kReads; ++k) {
      MUONH_SG(kSgMfma, 1); MUONH_SG(kSgDsRead, 1);
      if (kSpread && k < 4) MUONH_SG(kSgVmemRead, 1);
    }
    MUONH_SG(kSgMfma, 16 - kReads);
    __builtin_amdgcn_sched_barrier(0);
  };
  gload_p(ra0, 0);
  gload_q(rb0, 0);
  gload_p(ra1, 1);
  gload_q(rb1, 1);
  sstore(ra0, 0, 0);    // stage 0 -> slot 0
  sstore(rb0, 0, 1);
  gload_p(ra0, 2);
  gload_q(rb0, 2);
  wait_lds();
  lds_barrier();
  load_frag(fa0, fb0, 0, 0);
  // nk is even: two stages per trip, register sets alternating.
  for (int kt = 0; kt < nk; kt += 2) {
    stage(ra1, rb1, 0, 1, kt + 3);   // stage kt   (slot 0); set 1 = stage kt+1
    stage(ra0, rb0, 1, 0, kt + 4);   // stage kt+1 (slot 1); set 0 = stage kt+2
  }
  wait_vmcnt<0>();   // no load in flight into LDS or registers past this point

  // ---- epilogue --------------------------------------------------------
  // Accumulator register r of block (i, j) holds C[row][col] with
  //   row = 32 i + 8 (r / 4) + 4 (lane / 32) + (r % 4),  col = 32 j + lane % 32
  // (inside the wavefront's 128 x 128 sub-tile): every group of 4 registers
  // is 4 consecutive rows of one column, i.e. 4 contiguous elements of the
  // transposed layout.  With swapped operands (bf16 B'X) row and column trade
  // places.
  float alpha = 1.0f;
  if (first_iter) {
    const float s = scal[pr.mat].s;
    alpha = (MODE == kGram) ? s * s : s;
  }
  const bool mirror = (MODE == kGram || MODE == kPoly) && symmetric && (t.tm != t.tn);

  if constexpr (sizeof(T) == 2) {
    // bf16: the wavefront's 128 x 128 sub-tile is staged through its own
    // LDS region so that every global access is a coalesced 16-byte one: the
    // epilogue operand E is fetched row by row (E is stored at transposed
    // positions, so its rows are columns of the result), and each output
    // layout is written row by row (128 rows of 256 B + 16 B pad).
    lds_barrier();   // every wavefront is done reading the pipeline buffers
    uint8_t* reg = smem + wave * 128 * kEpiStride;
    const int wrow0 = row0 + wr * 128, wcol0 = col0 + wc * 128;
    const int lc = lane & 31, lg = (lane >> 5) * 4;
    if constexpr (MODE == kPoly) {
      // E sub-tile by direct-to-LDS loads into 128 rows of 256 B (no pad),
      // 16-byte chunk q of row c at slot q ^ (c & 15).  Instruction k writes
      // rows 4k..4k+3; lane L lands in row 4k + L/16, slot L%16.
      const uint8_t* eb = reinterpret_cast<const uint8_t*>(pr.E) +
                          ((size_t)wcol0 * pr.lde + wrow0) * sizeof(T);
      const int erow = lane >> 4;
      const int eslot = lane & 15;
      MUONH_LDS uint8_t* ereg = (MUONH_LDS uint8_t*)reg;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int c = 4 * k + erow;
        __builtin_amdgcn_global_load_lds(
            (const MUONH_GLOBAL void*)(eb + (size_t)c * pr.lde * sizeof(T) + ((eslot ^ (c & 15)) << 4)),
            (MUONH_LDS void*)(ereg + k * 1024), 16, 0, 0);
      }
      wait_vmcnt<0>();   // this wavefront's region only: no barrier needed
    }
    // (alpha is 1 except on the first iteration: skip the pass then)
    if (MODE == kPoly || first_iter) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t v;
          v[0] = acc[i][j][4 * g + 0];
          v[1] = acc[i][j][4 * g + 1];
          v[2] = acc[i][j][4 * g + 2];
          v[3] = acc[i][j][4 * g + 3];
          if constexpr (MODE == kPoly) {
            const int ec = j * 32 + lc;
            const u32x2_t eu = *reinterpret_cast<const u32x2_t*>(
                reg + ec * 256 + (((i * 4 + g) ^ (ec & 15)) << 4) + lg * 2);
            f32x4_t e;
            e[0] = __uint_as_float(eu[0] << 16);
            e[1] = __uint_as_float(eu[0] & 0xffff0000u);
            e[2] = __uint_as_float(eu[1] << 16);
            e[3] = __uint_as_float(eu[1] & 0xffff0000u);
            v = cb * e + cc * v;
            // + a on the (valid) diagonal
            const int grow = wrow0 + i * 32 + g * 8 + lg, gcol = wcol0 + j * 32 + lc;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (grow + q == gcol && gcol < pr.um) v[q] += ca;
          } else {
            v *= alpha;
          }
          acc[i][j][4 * g + 0] = v[0];
          acc[i][j][4 * g + 1] = v[1];
          acc[i][j][4 * g + 2] = v[2];
          acc[i][j][4 * g + 3] = v[3];
        }
    }
    // The sub-tile goes to LDS row-major (2-byte writes, 4 per register group)
    // or transposed (one 8-byte write per register group), then leaves as
    // rows of 256 B.  LDS operations of one wavefront complete in issue
    // order, so its reads see all of its writes.
    auto lds_rowmajor = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              *reinterpret_cast<uint16_t*>(reg + (i * 32 + g * 8 + lg + e) * kEpiStride +
                                           (j * 32 + lc) * 2) = f32_to_bf16(acc[i][j][4 * g + e]);
    };
    // Swapped accumulators (bf16 B'X): register group g of block (i, j) is
    // row 32 i + lane % 32, columns 32 j + 8 g + 4 (lane / 32) + 0..3.
    auto lds_rowmajor_swapped = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2_t o;
            o[0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
            o[1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            *reinterpret_cast<u32x2_t*>(reg + (i * 32 + lc) * kEpiStride + (j * 32 + g * 8 + lg) * 2) = o;
          }
    };
    auto lds_transposed = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            u32x2_t o;
            o[0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
            o[1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            *reinterpret_cast<u32x2_t*>(reg + (j * 32 + lc) * kEpiStride + (i * 32 + g * 8 + lg) * 2) = o;
          }
    };
    // LDS row rr -> dst + rr * ld (elements); whole, aligned 256-B rows.
    // Eight LDS reads are in flight before their stores.
    auto store_rows = [&](uint8_t* dst, size_t ld) {
#pragma unroll
      for (int it0 = 0; it0 < 32; it0 += 8) {
        u32x4_t x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int idx = (it0 + k) * 64 + lane, r = idx >> 4, ch = idx & 15;
          x[k] = *reinterpret_cast<const u32x4_t*>(reg + r * kEpiStride + ch * 16);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int idx = (it0 + k) * 64 + lane, r = idx >> 4, ch = idx & 15;
          st_global<u32x4_t>(dst + ((size_t)r * ld) * sizeof(T) + ch * 16, x[k]);
        }
      }
    };
    if constexpr (MODE == kApplyLast) {
      // u, compact, in the matrix's own orientation: [um x un] (row-major
      // pass) or, for a tall matrix, [un x um] (transposed pass); rows and
      // columns past the valid dims are dropped.  The same pass reduces
      // <W,u>, ||u||^2 and ||W||^2 over the stored (bf16) u and the matching
      // W elements (U and W share the layout).  W is read in batches of 8
      // rows of 8 per lane, double-buffered, the first batch issued before
      // the sub-tile goes through LDS; chunks that cannot take 16-byte loads
      // are read element by element in the same batches.
      int rbase, cbase, nrow, ncol, ld;
      if (!pr.u_tall) {
        rbase = wrow0; cbase = wcol0; nrow = pr.um; ncol = pr.un; ld = pr.un;
      } else {
        rbase = wcol0; cbase = wrow0; nrow = pr.un; ncol = pr.um; ld = pr.um;
      }
      uint16_t* U = reinterpret_cast<uint16_t*>(pr.U);
      const float* W = ptrs[pr.mat].w;
      const bool vec_ok = (ld & 7) == 0;
      // chunk `it` of the lane: sub-tile row it*4 + lane/16, columns 8 (lane%16) + 0..7
      auto full = [&](int it) {
        const int gr = rbase + it * 4 + (lane >> 4), gc = cbase + (lane & 15) * 8;
        return vec_ok && gr < nrow && gc + 8 <= ncol;
      };
      auto wptr = [&](int it) {
        return W + (size_t)(rbase + it * 4 + (lane >> 4)) * ld + cbase + (lane & 15) * 8;
      };
      f32x4_t wb[2][8][2];
      auto wload = [&](int buf, int it0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (full(it0 + k)) {
            wb[buf][k][0] = ld_global<f32x4_t>(wptr(it0 + k));
            wb[buf][k][1] = ld_global<f32x4_t>(wptr(it0 + k) + 4);
          } else {
            // Ragged edge, or a leading dimension that is not a multiple of 8:
            // element loads, issued here with the rest of the batch rather than
            // one round trip per chunk in the reduction below.
            const int gr = rbase + (it0 + k) * 4 + (lane >> 4), gc = cbase + (lane & 15) * 8;
            const float* wp = wptr(it0 + k);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              float v = 0.0f;
              if (gr < nrow && gc + q < ncol) v = wp[q];
              wb[buf][k][q >> 2][q & 3] = v;
            }
          }
        }
      };
      wload(0, 0);
      if (!pr.u_tall) lds_rowmajor(); else lds_transposed();
      float swu = 0.0f, suu = 0.0f, sww = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int cur = b & 1;
        if (b + 1 < 4) wload(cur ^ 1, (b + 1) * 8);
        u32x4_t x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int idx = (b * 8 + k) * 64 + lane;
          x[k] = *reinterpret_cast<const u32x4_t*>(reg + (idx >> 4) * kEpiStride + (idx & 15) * 16);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int it = b * 8 + k;
          const int gr = rbase + it * 4 + (lane >> 4), gc = cbase + (lane & 15) * 8;
          if (gr >= nrow || gc >= ncol) continue;
          uint16_t* d = U + (size_t)gr * ld + gc;
          if (full(it)) {
            st_global<u32x4_t>(d, x[k]);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float u = __uint_as_float((x[k][q >> 1] >> (16 * (q & 1))) << 16);
              const float w = wb[cur][k][q >> 2][q & 3];
              swu += w * u;
              suu += u * u;
              sww += w * w;
            }
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (gc + q < ncol) {
                const uint16_t h = (uint16_t)(x[k][q >> 1] >> (16 * (q & 1)));
                st_global<uint16_t>(d + q, h);
                const float u = __uint_as_float((uint32_t)h << 16), w = wb[cur][k][q >> 2][q & 3];
                swu += w * u;
                suu += u * u;
                sww += w * w;
              }
          }
        }
      }
      write_stats(part, (int64_t)pr.part0 + ((int64_t)t.tm * (pr.N / kGemmTile) + t.tn) * 4 + wave,
                  swu, suu, sww);
    } else {
      if constexpr (kSwap)
        lds_rowmajor_swapped();
      else
        lds_rowmajor();
      store_rows(reinterpret_cast<uint8_t*>(pr.O) + ((size_t)wrow0 * pr.ldo + wcol0) * sizeof(T), pr.ldo);
      // The mirrored tile of the symmetric products (B' X keeps one layout).
      if (mirror) {
        lds_transposed();
        store_rows(reinterpret_cast<uint8_t*>(pr.O) + ((size_t)wcol0 * pr.ldo + wrow0) * sizeof(T), pr.ldo);
      }
    }
  } else {
    T* O = reinterpret_cast<T*>(MODE == kApplyLast ? pr.U : pr.O);
    T* OT = reinterpret_cast<T*>(pr.OT);
    const T* E = reinterpret_cast<const T*>(pr.E);
    const float* W = (MODE == kApplyLast) ? ptrs[pr.mat].w : nullptr;
    float swu = 0.0f, suu = 0.0f, sww = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = col0 + wc * 128 + j * 32 + (lane & 31);
        // The block's W elements, loaded before any store to U so that the
        // loads are in flight together (the compiler cannot move a load of W
        // past a store to U on its own).
        float wv[4][4];
        if constexpr (MODE == kApplyLast) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = row0 + wr * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
            const size_t base = pr.u_tall ? (size_t)col * pr.um + row : (size_t)row * pr.un + col;
            const size_t step = pr.u_tall ? 1 : (size_t)pr.un;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              wv[g][e] = 0.0f;
              if (col < pr.un && row + e < pr.um) wv[g][e] = W[base + e * step];
            }
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = row0 + wr * 128 + i * 32 + g * 8 + (lane >> 5) * 4;
          f32x4_t v;
          v[0] = acc[i][j][4 * g + 0];
          v[1] = acc[i][j][4 * g + 1];
          v[2] = acc[i][j][4 * g + 2];
          v[3] = acc[i][j][4 * g + 3];
          if (MODE == kPoly) {
            const f32x4_t e = Vec4<T>::load(E + (size_t)col * pr.lde + row);
            v = cb * e + cc * v;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (row + q == col && col < pr.um) v[q] += ca;   // + a I
          } else {
            v *= alpha;
          }
          if (MODE == kApplyLast) {
            // u in the matrix's own orientation, compact: [um x un] or, for a
            // tall matrix, its transpose [un x um].
            if (col < pr.un && row < pr.um) {
              const size_t base = pr.u_tall ? (size_t)col * pr.um + row : (size_t)row * pr.un + col;
              const size_t step = pr.u_tall ? 1 : (size_t)pr.un;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (row + e < pr.um) {
                  Vec4<T>::store1(O + base + e * step, v[e]);   // + <W,u>, ||u||^2, ||W||^2 over it
                  const float w = wv[g][e];
                  swu += w * v[e];
                  suu += v[e] * v[e];
                  sww += w * w;
                }
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
    if constexpr (MODE == kApplyLast)
      write_stats(part, (int64_t)pr.part0 + ((int64_t)t.tm * (pr.N / kGemmTile) + t.tn) * 4 + wave,
                  swu, suu, sww);
  }
}

// ---------------------------------------------------------------------------
// Small-problem path.  When a plan's products have too few 256 x 256 tiles to
// occupy the GPU (a handful of small matrices), one CU per big tile leaves
// the rest idle and the step is a chain of single-CU launches.  This kernel
// covers the same four products with 64 x 64 output tiles (4 wavefronts, one
// 32 x 32 MFMA block each) and a plain load -> LDS -> MFMA loop over stages
// of 64 bytes of K per operand row.  Only tiles and K stages inside the valid
// (unpadded) dims are visited: the zero padding contributes nothing, and the
// padding of every output stays as initialised (zero).  Every tile is
// computed, so the Gram-type outputs are not mirrored.
constexpr int kSmallTile = kSmallGemmTile;
constexpr int kSmallRowBytes = 64;                  // K bytes per operand row per stage
constexpr int kSmallPitch = kSmallRowBytes + 16;    // LDS row pitch

template <typename T, int MODE>
__global__ __launch_bounds__(kGemmThreads) void gemm_small_kernel(
    const GemmProb* __restrict__ probs, const GemmTile* __restrict__ tiles,
    const MatScalars* __restrict__ scal, int first_iter, float ca, float cb, float cc,
    const MatPtrs* __restrict__ ptrs, double* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t lp[kSmallTile * kSmallPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lq[kSmallTile * kSmallPitch];
  // bf16 B'X reads X itself (K-major Q), as the big path does.
  constexpr bool kQT = (MODE == kApply || MODE == kApplyLast) && sizeof(T) == 2;
  constexpr int kKs = kSmallRowBytes / (int)sizeof(T);   // K elements per stage
  static_assert(!kQT || kKs * kSmallTile * 2 == kGemmThreads * 16, "one K-major chunk per thread");

  const GemmTile t = tiles[blockIdx.x];
  const GemmProb pr = probs[t.prob];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int row0 = t.tm * kSmallTile, col0 = t.tn * kSmallTile;
  const uint8_t* P = reinterpret_cast<const uint8_t*>(pr.P);
  const uint8_t* Q = reinterpret_cast<const uint8_t*>(pr.Q);
  // Row-major operands: thread = (row tid/4, 16-byte chunk tid%4).  K-major
  // Q: thread = (k row tid/8, 8 columns from 8 (tid%8)), scattered into
  // LDS as Q[n][k].
  const int lr = tid >> 2, lc = tid & 3;
  const int qr = tid >> 3, qc = tid & 7;
  const int kend = min(pr.K, (pr.uk + kKs - 1) / kKs * kKs);
  u32x4_t rp = {0u, 0u, 0u, 0u}, rq = {0u, 0u, 0u, 0u};
  auto load = [&](int k0) {
    rp = ld_global<u32x4_t>(P + ((size_t)(row0 + lr) * pr.ldp + k0) * sizeof(T) + lc * 16);
    if constexpr (kQT)
      rq = ld_global<u32x4_t>(Q + ((size_t)(k0 + qr) * pr.ldq + col0) * sizeof(T) + qc * 16);
    else
      rq = ld_global<u32x4_t>(Q + ((size_t)(col0 + lr) * pr.ldq + k0) * sizeof(T) + lc * 16);
  };
  auto stage = [&]() {
    *reinterpret_cast<u32x4_t*>(lp + lr * kSmallPitch + lc * 16) = rp;
    if constexpr (kQT) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(lq + (8 * qc + e) * kSmallPitch + qr * 2) =
            (uint16_t)(rq[e >> 1] >> (16 * (e & 1)));
    } else {
      *reinterpret_cast<u32x4_t*>(lq + lr * kSmallPitch + lc * 16) = rq;
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  if (kend > 0) load(0);
  for (int k0 = 0; k0 < kend; k0 += kKs) {
    __syncthreads();   // the previous stage's fragments have been read
    stage();
    __syncthreads();
    if (k0 + kKs < kend) load(k0 + kKs);
    // Each run consumes 32 bytes of K per row: lanes 0-31 the first 16,
    // lanes 32-63 the second (the fragment contract of Mfma<T>).
#pragma unroll
    for (int s2 = 0; s2 < kSmallRowBytes / 32; ++s2) {
      const int off = s2 * 32 + (lane >> 5) * 16;
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lp + (wr * 32 + (lane & 31)) * kSmallPitch + off);
      const u32x4_t b = *reinterpret_cast<const u32x4_t*>(lq + (wc * 32 + (lane & 31)) * kSmallPitch + off);
      Mfma<T>::run(acc, a, b);
    }
  }

  // Epilogue, element for element as the big path's: register group g of
  // the 32 x 32 block holds rows 8 g + 4 (lane / 32) + 0..3 of column lane % 32.
  float alpha = 1.0f;
  if (first_iter) {
    const float sc = scal[pr.mat].s;
    alpha = (MODE == kGram) ? sc * sc : sc;
  }
  T* O = reinterpret_cast<T*>(MODE == kApplyLast ? pr.U : pr.O);
  T* OT = reinterpret_cast<T*>(pr.OT);
  const T* E = reinterpret_cast<const T*>(pr.E);
  const float* W = (MODE == kApplyLast) ? ptrs[pr.mat].w : nullptr;
  float swu = 0.0f, suu = 0.0f, sww = 0.0f;
  const int col = col0 + wc * 32 + (lane & 31);
  // W elements of the lane, loaded before any store to U (in flight together).
  float wv[4][4];
  if constexpr (MODE == kApplyLast) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int row = row0 + wr * 32 + g * 8 + (lane >> 5) * 4;
      const size_t base = pr.u_tall ? (size_t)col * pr.um + row : (size_t)row * pr.un + col;
      const size_t step = pr.u_tall ? 1 : (size_t)pr.un;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[g][e] = 0.0f;
        if (col < pr.un && row + e < pr.um) wv[g][e] = W[base + e * step];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int row = row0 + wr * 32 + g * 8 + (lane >> 5) * 4;
    f32x4_t v;
    v[0] = acc[4 * g + 0];
    v[1] = acc[4 * g + 1];
    v[2] = acc[4 * g + 2];
    v[3] = acc[4 * g + 3];
    if constexpr (MODE == kPoly) {
      const f32x4_t e = Vec4<T>::load(E + (size_t)col * pr.lde + row);
      v = cb * e + cc * v;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row + q == col && col < pr.um) v[q] += ca;   // + a I
    } else {
      v *= alpha;
    }
    if constexpr (MODE == kApplyLast) {
      if (col < pr.un && row < pr.um) {
        const size_t base = pr.u_tall ? (size_t)col * pr.um + row : (size_t)row * pr.un + col;
        const size_t step = pr.u_tall ? 1 : (size_t)pr.un;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (row + e < pr.um) {
            Vec4<T>::store1(O + base + e * step, v[e]);
            // the statistics use the stored (rounded) u, as the big path does
            const float u = (sizeof(T) == 2) ? bf16_to_f32(f32_to_bf16(v[e])) : v[e];
            const float w = wv[g][e];
            swu += w * u;
            suu += u * u;
            sww += w * w;
          }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) Vec4<T>::store1(O + (size_t)(row + e) * pr.ldo + col, v[e]);
      if (MODE == kApply && OT) Vec4<T>::store(OT + (size_t)col * pr.ldot + row, v);
    }
  }
  if constexpr (MODE == kApplyLast) {
    // compact slots: one per valid tile (ceil(um/64) x ceil(un/64)) and wavefront
    const int ntn = (pr.un + kSmallTile - 1) / kSmallTile;
    write_stats(part, (int64_t)pr.part0 + ((int64_t)t.tm * ntn + t.tn) * 4 + wave, swu, suu, sww);
  }
}

template <typename T>
hipError_t launch_t(int mode, const GemmProb* probs, const GemmTile* tiles, int64_t ntiles,
                    const MatScalars* scal, int first_iter, int last_iter, int symmetric,
                    float ca, float cb, float cc, const MatPtrs* ptrs, double* part,
                    hipStream_t st) {
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)ntiles), block(kGemmThreads);
  switch (mode) {
    case kGram:
      hipLaunchKernelGGL((gemm_kernel<T, kGram>), grid, block, 0, st, probs, tiles, scal,
                         first_iter, last_iter, symmetric, ca, cb, cc, ptrs, part);
      break;
    case kPoly:
      hipLaunchKernelGGL((gemm_kernel<T, kPoly>), grid, block, 0, st, probs, tiles, scal,
                         first_iter, last_iter, symmetric, ca, cb, cc, ptrs, part);
      break;
    default:
      if (last_iter)
        hipLaunchKernelGGL((gemm_kernel<T, kApplyLast>), grid, block, 0, st, probs, tiles, scal,
                           first_iter, last_iter, symmetric, ca, cb, cc, ptrs, part);
      else
        hipLaunchKernelGGL((gemm_kernel<T, kApply>), grid, block, 0, st, probs, tiles, scal,
                           first_iter, last_iter, symmetric, ca, cb, cc, ptrs, part);
      break;
  }
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_small_t(int mode, const GemmProb* probs, const GemmTile* tiles, int64_t ntiles,
                          const MatScalars* scal, int first_iter, int last_iter, float ca, float cb,
                          float cc, const MatPtrs* ptrs, double* part, hipStream_t st) {
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)ntiles), block(kGemmThreads);
  switch (mode) {
    case kGram:
      hipLaunchKernelGGL((gemm_small_kernel<T, kGram>), grid, block, 0, st, probs, tiles, scal,
                         first_iter, ca, cb, cc, ptrs, part);
      break;
    case kPoly:
      hipLaunchKernelGGL((gemm_small_kernel<T, kPoly>), grid, block, 0, st, probs, tiles, scal,
                         first_iter, ca, cb, cc, ptrs, part);
      break;
    default:
      if (last_iter)
        hipLaunchKernelGGL((gemm_small_kernel<T, kApplyLast>), grid, block, 0, st, probs, tiles,
                           scal, first_iter, ca, cb, cc, ptrs, part);
      else
        hipLaunchKernelGGL((gemm_small_kernel<T, kApply>), grid, block, 0, st, probs, tiles, scal,
                           first_iter, ca, cb, cc, ptrs, part);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int bf16, int mode, const GemmProb* probs, const GemmTile* tiles,
                       int64_t ntiles, const MatScalars* scal, int first_iter, int last_iter,
                       int symmetric, float ca, float cb, float cc, const MatPtrs* ptrs,
                       double* part, hipStream_t st) {
  if (bf16)
    return launch_t<uint16_t>(mode, probs, tiles, ntiles, scal, first_iter, last_iter, symmetric,
                              ca, cb, cc, ptrs, part, st);
  return launch_t<float>(mode, probs, tiles, ntiles, scal, first_iter, last_iter, symmetric, ca,
                         cb, cc, ptrs, part, st);
}

hipError_t launch_gemm_small(int bf16, int mode, const GemmProb* probs, const GemmTile* tiles,
                             int64_t ntiles, const MatScalars* scal, int first_iter, int last_iter,
                             float ca, float cb, float cc, const MatPtrs* ptrs, double* part,
                             hipStream_t st) {
  if (bf16)
    return launch_small_t<uint16_t>(mode, probs, tiles, ntiles, scal, first_iter, last_iter, ca, cb,
                                    cc, ptrs, part, st);
  return launch_small_t<float>(mode, probs, tiles, ntiles, scal, first_iter, last_iter, ca, cb, cc,
                               ptrs, part, st);
}

}  // namespace muonh
