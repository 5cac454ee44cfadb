// Internal structures shared by the host planner (muonh.cpp) and the gfx950
// kernels (gemm.hip, elementwise.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/muonh.h"

namespace muonh {

// ---------------------------------------------------------------------------
// Tiling constants.

constexpr int kGemmTile = 256;      // output tile of the grouped GEMM (M and N)
constexpr int kGemmThreads = 256;   // 4 wavefronts of 64, 2 x 2 over the tile
constexpr int kPad = 256;           // Newton-Schulz dims are padded to this multiple
constexpr int kRowSkewBytes = 128;  // extra bytes per row of every Newton-Schulz buffer
constexpr int kMomTileR = 64;       // momentum / pack tile: 64 rows
constexpr int kMomTileC = 128;      //   x 128 columns (512-byte rows of M)
constexpr int kMomTileThreads = 512;  // 8 wavefronts per tile: 4 rows of 4 columns per thread
constexpr int kChunk = 16384;       // elements per chunk of the flat kernels
constexpr int kElemThreads = 256;
constexpr int kMaxXcd = 8;          // MI355X: 8 accelerator complex dies
constexpr int kSmallGemmTile = 64;  // output tile of the small-problem GEMM path
// A plan takes the small-problem path when its largest product has fewer
// 256 x 256 tiles than this (a quarter of the CUs).
constexpr int kSmallPlanTiles = 64;

enum GemmMode : int {
  kGram = 0,   // A = alpha * X X^T                       (alpha = s^2 on the first iteration)
  kPoly = 1,   // B' = b A + c A A + a I
  kApply = 2,  // X' = alpha * B' X = alpha * (a X + B X)   (alpha = s on the first iteration)
  kApplyLast = 3,  // kApply of the last iteration: u written compact, own orientation
};

// One problem of a grouped GEMM launch: C = P Q^T with P [M x K] and Q [N x K]
// both row-major (K contiguous).  All dims are multiples of kGemmTile / the
// K tile; the padding of every operand is zero.
struct GemmProb {
  const void* P;
  const void* Q;
  const void* E;   // epilogue operand read at transposed positions: kPoly: A (symmetric)
  void* O;         // row-major output [M x N] (kApply: X'), ld = ldo
  void* OT;        // transposed output [N x M] (kApply: X'^T), ld = ldot
  void* U;         // kApply, last iteration: compact update in the matrix's own orientation
  int32_t M, N, K;
  int32_t ldp, ldq, lde, ldo, ldot;
  int32_t um, un;  // valid (unpadded) NS dims m x n of the matrix (kPoly: um for the diagonal)
  int32_t uk;      // valid (unpadded) length of the contraction (n for X X^T, m otherwise)
  int32_t u_tall;  // 1: U is [un x um] (the matrix is tall), 0: U is [um x un]
  int32_t mat;     // matrix index
  int32_t part0;   // kApplyLast: first <W,u>/||u||^2/||W||^2 partial slot of the matrix
                   // (one slot per output tile and wavefront)
};

// Tile list entry; prob < 0 marks an empty slot (XCD balancing padding).
struct GemmTile {
  int32_t prob;
  int16_t tm, tn;
};

// One block of the momentum kernel.  kind 0: the 64 x 128 tile (tr, tc) of
// the padded, original-orientation grid (the path that also writes a
// transposed X_0); kind 1: columns [tc * 1024, tc * 1024 + 1024) of row tr
// of that grid (matrices whose X_0 keeps M's orientation and has no
// transposed copy).
struct MomTile {
  int32_t mat;
  int32_t tr, tc;
  int32_t kind;
};
constexpr int kMomRowSeg = 1024;   // columns per kind-1 block
constexpr int kMomParts = 4;       // ||Y||^2 partial slots per unit (one per wavefront)

struct Chunk {
  int32_t mat;
  int32_t len;
  int64_t start;   // element offset inside the matrix
};

// Static per-matrix geometry and workspace addresses (uploaded at init).
struct MatGeom {
  int64_t rows, cols;
  int32_t tall;        // rows > cols: Newton-Schulz runs on the transpose
  int32_t g_bf16;      // gradient dtype
  int32_t m_pad, n_pad;
  int32_t r_pad, c_pad;  // padded dims in the matrix's own orientation
  int32_t ld_skew;     // elements added to every row pitch (kRowSkewBytes / element size)
  void* X[2];          // ping-pong iterate, [m_pad x n_pad]
  void* XT[2];         // its transpose, [n_pad x m_pad]
  void* U;             // compact update u, [rows x cols]
  int64_t mom_tile0;   // first momentum unit; its partials start at kMomParts * mom_tile0
  int64_t mom_ntiles;
  int64_t chunk0;      // first flat chunk
  int64_t nchunks;
  int64_t part0;       // first update-statistics partial slot (last B'X launch)
  int64_t nparts;
};

// Per-step caller pointers (uploaded when they change).
struct MatPtrs {
  float* w;
  const void* g;
  float* m;
};

// Per-matrix device scalars.
struct MatScalars {
  double R;        // hyperball radius
  double y_norm;   // ||Y||_F of this step
  float s;         // 1 / (||Y|| + eps)
  float k1, k2;    // update: W <- k1 W - k2 u
  float pad_;
};

struct ElemParams {
  float beta;
  int32_t nesterov;
  float ns_eps;
  int32_t mode;
  float weight_decay;
  float elr;
};

// ---------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files).  All return hipError_t of
// the launch.

// The last B'X launch also reduces <W,u>, ||u||^2 and ||W||^2 over each
// tile's valid elements into `part` (3 doubles per tile and wavefront);
// `ptrs` gives W.  Other launches ignore both.
hipError_t launch_gemm(int bf16, int mode, const GemmProb* probs, const GemmTile* tiles,
                       int64_t ntiles, const MatScalars* scal, int first_iter, int last_iter,
                       int symmetric, float ca, float cb, float cc, const MatPtrs* ptrs,
                       double* part, hipStream_t st);

// units[0, nrow) are row segments (kind 1), units[nrow, nrow + ntile) tiles
// (kind 0); one launch each.
// The small-problem path (64 x 64 tiles over the valid dims only, every tile
// listed, no mirrored writes); same products and arguments.  Its last B'X
// statistics use ceil(um/64) x ceil(un/64) x 4 slots per matrix.
hipError_t launch_gemm_small(int bf16, int mode, const GemmProb* probs, const GemmTile* tiles,
                             int64_t ntiles, const MatScalars* scal, int first_iter, int last_iter,
                             float ca, float cb, float cc, const MatPtrs* ptrs, double* part,
                             hipStream_t st);

hipError_t launch_momentum(int bf16, const MomTile* units, int64_t nrow, int64_t ntile,
                           const MatGeom* geo, const MatPtrs* ptrs, double* partials,
                           ElemParams prm, hipStream_t st);

hipError_t launch_finalize_norm(int32_t nmat, const MatGeom* geo, const double* partials,
                                MatScalars* scal, float eps, hipStream_t st);


// eta_dev (nullable): per-matrix step sizes in device memory; when given,
// prm.elr and elr_scale are not read.
hipError_t launch_finalize_update(int32_t nmat, const MatGeom* geo, const double* partials,
                                  MatScalars* scal, muonh_stats* stats, const float* elr_scale,
                                  const double* eta_dev, ElemParams prm, hipStream_t st);

// eta[i] = elr * (elr_scale ? elr_scale[i] : 1) in fp64, one workgroup.
hipError_t launch_set_eta(int32_t nmat, const float* elr_scale, float elr, double* eta,
                          hipStream_t st);

hipError_t launch_update(int bf16, const Chunk* chunks, int64_t nchunks, const MatGeom* geo,
                         const MatPtrs* ptrs, const MatScalars* scal, hipStream_t st);

hipError_t launch_radius(const Chunk* chunks, int64_t nchunks, const MatPtrs* ptrs,
                         double* partials, hipStream_t st);

hipError_t launch_finalize_radius(int32_t nmat, const MatGeom* geo, const double* partials,
                                  const int32_t* need, MatScalars* scal, hipStream_t st);

hipError_t launch_copy_update(int bf16, const void* U, int64_t count, float* dst, hipStream_t st);

// Zero fill of a 16-byte aligned region of `bytes` (a multiple of 16).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// AdamW over a list of flat tensors (chunks of kChunk elements).
struct AdamwPtrs {
  float* w;
  const void* g;
  float* m;
  float* v;
  int32_t g_bf16;
  int32_t pad;
};
struct AdamwParams {
  float beta1, omb1;    // beta1, 1 - beta1
  float beta2, omb2;    // beta2, 1 - beta2
  float eps;
  float decay;          // 1 - lr * weight_decay
  float step_size;      // lr / (1 - beta1^t)
  float rbc2;           // 1 / sqrt(1 - beta2^t)
};
hipError_t launch_adamw(const Chunk* chunks, int64_t nchunks, const AdamwPtrs* ptrs,
                        AdamwParams prm, hipStream_t st);

// Records the text of a failure for muonh_last_error() and returns `code`.
int set_last_error(int code, const char* msg);

// Host state one device keeps for the allocation-free step: the host image
// of the plan tables (reused, so an upload's source stays valid until the
// device has read it) and the event recorded after that upload.
struct InWorkspaceHost {
  std::vector<uint8_t> img;    // host image of the tables (C++ heap, grown on demand)
  hipEvent_t uploaded = nullptr;
  bool pending = false;
};

// One MuonH step over `mats` with every buffer the step needs beyond the
// caller's W, G and M inside the device region [ws, ws + ws_bytes): the plan
// is built on the host, its tables uploaded into the region, the
// Newton-Schulz buffers cleared, and the step's launches enqueued on `st`,
// with no device allocation.  Every radius must be given (> 0).  Errors:
// MUONH_EINVAL, MUONH_ENOMEM (the plan needs more than ws_bytes; the text
// names the size), MUONH_EHIP.
int run_step_in_workspace(const muonh_matrix_desc* mats, int32_t n, const muonh_options& opt,
                          const muonh_step_args& args, hipStream_t st, uint8_t* ws, size_t ws_bytes,
                          InWorkspaceHost& host);

}  // namespace muonh
