/*
 * muonh.h -- C ABI of the MI355X (gfx950) MuonH optimizer-step library.
 *
 * What the library computes, per wrapped 2-D fp32 matrix W (r x c), on the
 * caller's HIP stream:
 *
 *   1. momentum         M <- beta*M + G                (heavy-ball, in place)
 *   2. Muon update      u  = NS_5(Y), Y = M (or G + beta*M with Nesterov):
 *                       X_0 = Y / (||Y||_F + eps), then ns_steps times
 *                       A = X X^T, B = b A + c A A, X <- a X + B X
 *   3. Hyperball step   u^ = u/||u||_F, W~ = W - eta R u^, W <- R W~/||W~||_F
 *
 * Step 3 is Eq. (1) of "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090
 * within $5090" (arXiv HTML, §3.3), with the fixed radius R = ||W_0||_F of
 * the same section and the effective LR eta^H = m * eta_base of §3.3.1.
 * The pages name but do not define steps 1-2; the defaults below (beta 0.95,
 * five quintic iterations with (3.4445, -4.7750, 2.0315), eps 1e-7) are the
 * published Muon method's.  Two further modes reuse steps 1-2 with the other
 * updates of §3.3.1: ordinary Muon with decoupled weight decay (Eq. (3)) and
 * effective-LR-aligned Muon (Eq. (5)).
 *
 * Conventions for every entry point:
 *   - Return value: MUONH_OK (0) or a negative MUONH_E* code.  Nothing is
 *     thrown or aborted across the ABI.  muonh_last_error() gives the text of
 *     the last failure on the calling thread.
 *   - Device pointers are HIP device addresses; "stream" is a hipStream_t
 *     passed as void* (NULL = the default stream).
 *   - All matrices are row-major and contiguous (leading dimension = cols).
 *   - Work is enqueued asynchronously; errors from kernels surface at the
 *     next synchronising call (muonh_get_radii / muonh_get_stats).
 *   - A handle is not thread-safe; distinct handles are independent.
 *   - Environment, read at init: MUONH_DEBUG_SYNC=1 synchronises the stream
 *     after every kernel launch so a device fault is reported (MUONH_EHIP) by
 *     the step that caused it, naming the launch (slow; for debugging);
 *     MUONH_LOG=1 prints the plan (buckets, tile and chunk counts, workspace,
 *     FLOP per step) on stderr; MUONH_GEMM_TILE=64 or 256 forces the GEMM
 *     path (by default plans whose B'X product has fewer than 64 tiles of
 *     256 x 256 use 64 x 64 tiles over the unpadded dims; results agree to
 *     rounding, not bitwise).  Also read by muonh_workspace_size and
 *     muonh_plan_query.
 */
#ifndef MUONH_H_
#define MUONH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MUONH_OK         0
#define MUONH_EINVAL    -1   /* bad argument: null pointer, dims <= 0, dtype, alignment */
#define MUONH_EMISMATCH -2   /* step matrix list differs from the one given at init */
#define MUONH_ENOMEM    -3   /* workspace too small or device allocation failed */
#define MUONH_EHIP      -4   /* a HIP runtime call failed (see muonh_last_error) */
#define MUONH_ESTATE    -5   /* call out of order (e.g. copy_update before a step) */
#define MUONH_ENODEV    -6   /* no usable gfx950 device */

/* ---- enumerations ------------------------------------------------------ */
#define MUONH_F32   0        /* IEEE binary32 */
#define MUONH_BF16  1        /* bfloat16 (round-to-nearest-even when produced) */

#define MUONH_MODE_HYPERBALL   0  /* Eq. (1): normalised update + projection to radius R */
#define MUONH_MODE_MUON_WD     1  /* Eq. (3): W <- (1 - wd*eta) W - eta u */
#define MUONH_MODE_ELR_ALIGNED 2  /* Eq. (5): W <- W - eta_t u, eta_t = eta ||W|| / ||u|| */

/* One wrapped matrix.  The same list order, shapes and dtypes are used at
 * init and at every step; the pointers may change between steps.           */
typedef struct muonh_matrix_desc {
  void*       w;         /* fp32 [rows x cols], device, updated in place              */
  const void* g;         /* gradient [rows x cols], device, dtype g_dtype (read only) */
  void*       m;         /* fp32 momentum [rows x cols], device, updated in place     */
  int64_t     rows;      /* r >= 1                                                     */
  int64_t     cols;      /* c >= 1                                                     */
  int32_t     g_dtype;   /* MUONH_F32 or MUONH_BF16                                    */
  float       radius;    /* R; <= 0 means R = ||W||_F measured at init (resume: pass R) */
} muonh_matrix_desc;

typedef struct muonh_options {
  float   beta;          /* momentum coefficient, default 0.95                    */
  int32_t ns_steps;      /* Newton-Schulz iterations, 1..16, default 5             */
  float   ns_a, ns_b, ns_c; /* quintic coefficients, default 3.4445, -4.775, 2.0315 */
  float   ns_eps;        /* X_0 = Y / (||Y|| + eps), default 1e-7                  */
  int32_t ns_dtype;      /* operand type of the NS products: MUONH_BF16 (default) or MUONH_F32;
                            accumulation is always fp32                              */
  int32_t nesterov;      /* 0 (default): Y = M; 1: Y = G + beta*M                   */
  int32_t mode;          /* MUONH_MODE_*, default MUONH_MODE_HYPERBALL              */
  float   weight_decay;  /* lambda of MUONH_MODE_MUON_WD, default 0                  */
  int32_t symmetric;     /* 1 (default): X X^T and A A computed on upper tiles only */
  int32_t deterministic; /* 1 (default): every reduction runs in a fixed order (no
                            floating-point atomics), so repeated steps on the same
                            inputs are bitwise equal; 0 is accepted and behaves the
                            same (there is no faster non-deterministic path)        */
  void*   workspace;     /* optional caller-owned device memory; NULL: library allocates */
  size_t  workspace_bytes;
} muonh_options;

typedef struct muonh_step_args {
  float        elr;        /* eta: effective LR of this step (Hyperball: eta^H = m eta_base) */
  const float* elr_scale;  /* optional host array [n]: per-matrix factor on elr, or NULL     */
  int64_t      step;       /* caller's step counter (recorded, not used in the arithmetic)   */
  int32_t      want_stats; /* reserved: statistics are always produced on the device         */
} muonh_step_args;

/* Per-matrix diagnostics of the last step (cf. the per-group effective LR,
 * weight-norm and update-norm traces of App. D, Fig. 15).                  */
typedef struct muonh_stats {
  double y_norm;    /* ||Y||_F, the Newton-Schulz input                      */
  double u_norm;    /* ||u||_F, raw Newton-Schulz output                     */
  double w_norm;    /* ||W_t||_F before the step                             */
  double inner;     /* <W_t, u^>                                             */
  double c;         /* <W_t, u^> / R                                         */
  double wt_norm;   /* ||W~||_F (Hyperball) / ||W_{t+1}||_F (other modes)    */
  double elr;       /* effective LR: ||W_{t+1}^pre - W_t|| / ||W_t||          */
  double angle;     /* Hyperball: atan2(eta sqrt(1-c^2), 1 - eta c)          */
  int32_t nonfinite;/* 1 if any of the norms above is NaN or Inf             */
  int32_t reserved;
} muonh_stats;

/* Host-side plan summary (pure host computation, no device needed). */
typedef struct muonh_plan_info {
  int32_t n_matrices;
  int32_t n_buckets;        /* distinct padded NS shapes (m_pad x n_pad)            */
  int64_t gemm_tiles[3];    /* 256x256 output tiles per launch: XX^T, AA, BX          */
  int64_t mom_tiles;        /* blocks of the momentum / pack kernel: 64x64 tiles, or
                               1024-column row segments where X_0 is not transposed */
  int64_t flat_chunks;      /* chunks of the reduction and update kernels            */
  double  ns_dense_flops;   /* sum over matrices of steps*(4 m^2 n + 2 m^3)          */
  double  ns_exec_flops;    /* MFMA FLOP issued per step (padding + symmetric tiles) */
  double  elem_bytes;       /* algorithmic HBM bytes of the elementwise kernels/step */
  size_t  workspace_bytes;  /* bytes muonh_workspace_size would return              */
} muonh_plan_info;

typedef struct muonh_handle muonh_handle;

/* Fill *opt with the defaults listed above. */
void muonh_default_options(muonh_options* opt);

/* Bytes of device workspace a plan for these matrices needs (host only). */
int muonh_workspace_size(const muonh_matrix_desc* mats, int32_t n,
                         const muonh_options* opt, size_t* bytes);

/* Host-only plan summary for these matrices (no device work). */
int muonh_plan_query(const muonh_matrix_desc* mats, int32_t n,
                     const muonh_options* opt, muonh_plan_info* info);

/* Build the plan (shape buckets, tile tables, workspace layout) on the
 * current device and, for every matrix with radius <= 0, enqueue
 * R = ||W_0||_F on `stream`.  Keeps shapes and dtypes, not pointers.
 * The library owns only the plan and, when opt->workspace is NULL, its
 * workspace.  On failure *h is NULL.                                        */
int muonh_init(muonh_handle** h, const muonh_matrix_desc* mats, int32_t n,
               const muonh_options* opt, void* stream);

/* One optimizer step over all n matrices (same order / shapes / dtypes as
 * at init), enqueued on `stream`.  W and M are updated in place; G is read.
 * Buffers must stay valid until the stream has passed the step.            */
int muonh_step(muonh_handle* h, const muonh_matrix_desc* mats, int32_t n,
               const muonh_step_args* args, void* stream);

/* The same step as muonh_step (same arguments, same arithmetic: results are
 * bitwise equal), for callers whose steps are bound by launch overhead.  The
 * first call records the step's kernel launches into a HIP graph, on a
 * stream the handle owns; every call then enqueues on `stream` one small
 * kernel that stores this call's per-matrix step sizes
 * elr * elr_scale[i] (fp64) in the workspace, and one launch of the recorded
 * graph.  Pointer changes and elr / elr_scale are taken from each call as in
 * muonh_step; nothing needs recording again.  Returns MUONH_ESTATE when
 * per-phase timing is on or MUONH_DEBUG_SYNC is set (use muonh_step then).
 * Not for use while the caller is itself capturing `stream`.  The graph is
 * released by muonh_destroy.                                                */
int muonh_step_graph(muonh_handle* h, const muonh_matrix_desc* mats, int32_t n,
                     const muonh_step_args* args, void* stream);

/* Allocation-free variant of muonh_step, for callers that cannot allocate
 * device memory: code that must not call hipMalloc or hipFree (tight serving
 * or training loops, harnesses that forbid allocation).  One self-contained
 * step over n matrices with no handle: the plan is built on the host each
 * call, and every buffer the step needs beyond the caller's W, G and M
 * (tables, Newton-Schulz iterates, partial sums) lives in one static device
 * array of the library, MUONH_NOALLOC_MAX_WORKSPACE bytes per GPU, which
 * each GPU the library runs on holds until the process ends.  No device
 * memory is allocated or freed and no pinned host memory is used (the
 * tables are uploaded from a host buffer the library reuses; the host-side
 * plan uses the C++ heap).  The first call on a device looks up that
 * device's address of the array.
 *   mats, n, args, stream: as for muonh_step (pointers, shapes, dtypes);
 *     every desc.radius must be > 0: the caller holds R (||W_0||_F, or the
 *     value muonh_get_radii returns), since nothing persists between calls.
 *   opt: as for muonh_init; opt->workspace must be NULL.
 * Same plan, kernels and launch order as muonh_init + muonh_step with the
 * same options and radii: W and M come out bitwise equal.  Statistics and u
 * are not kept for the caller.
 * Errors: MUONH_EINVAL (as muonh_step, or a radius <= 0, or a workspace
 * given); MUONH_ENOMEM when the list's plan (muonh_workspace_size) exceeds
 * MUONH_NOALLOC_MAX_WORKSPACE, before anything is enqueued; MUONH_ENODEV;
 * MUONH_EHIP.  Every call on a GPU shares that GPU's array, which keeps the
 * last call's contents (each call uploads its own tables and clears the
 * Newton-Schulz buffers): calls that overlap in time on one GPU, on other
 * streams or from other threads, race; calls in order on one stream do
 * not.                                                                     */
#define MUONH_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
int muonh_step_noalloc(const muonh_matrix_desc* mats, int32_t n, const muonh_options* opt,
                       const muonh_step_args* args, void* stream);

/* Synchronise the handle's last stream, then copy the n radii to host.  A
 * radius measured at init is rounded to float when measured, so these are
 * exactly the R the steps use: a new handle given them as the descriptors'
 * radius, with the saved W and M, continues bit for bit.                  */
int muonh_get_radii(muonh_handle* h, float* out, int32_t n);

/* Synchronise, then copy the n per-matrix statistics of the last step. */
int muonh_get_stats(muonh_handle* h, muonh_stats* out, int32_t n);

/* Test/debug: enqueue a copy of the Newton-Schulz output u of matrix idx
 * from the last step, in the matrix's own orientation (rows x cols, fp32,
 * row-major), to dst_device.                                              */
int muonh_copy_update(muonh_handle* h, int32_t idx, void* dst_device, void* stream);

/* Per-kernel timing with HIP events recorded on each step's stream.
 * muonh_set_timing(h, 1) starts recording (and clears the totals); every
 * later step records one event after each launch.  muonh_get_timing
 * synchronises, writes the totals in milliseconds over the *n_steps timed
 * steps since the last read into phases_ms[0..6] = momentum+pack (and its
 * finalise), NS X X^T, NS A A (each summed over the ns_steps launches), NS
 * B X (summed over the first ns_steps-1 launches), the last NS B X launch
 * (it writes u and reduces <W,u>, ||u||^2, ||W||^2 per tile), the finalise
 * of those sums, update; then clears the totals.
 * n_phases must be >= 7.                                                    */
int muonh_set_timing(muonh_handle* h, int32_t enable);
int muonh_get_timing(muonh_handle* h, float* phases_ms, int32_t n_phases, int32_t* n_steps);

/* Release the plan and any library-owned device memory.  NULL is a no-op. */
int muonh_destroy(muonh_handle* h);

const char* muonh_status_str(int status);
const char* muonh_last_error(void);

/* ---- host-only learning-rate helpers ------------------------------------
 * Eq. (11) of App. C: eta0 + (eta_min - eta0) s / S, s clamped to [0, S].   */
double muonh_lr_linear(double eta0, double eta_min, double s, double S);
/* Eq. (10) of App. C: linear warmup to `peak`, then
 * floor + (peak - floor) (1 + (k - warmup)/tau)^(-p).                         */
double muonh_lr_power(double k, double peak, double floor_, double warmup,
                      double tau, double p);
/* Warmup-stable-decay with linear decay over the last decay_ratio*total
 * steps (the §3.3.2 sweeps; plain reading of the pages).                     */
double muonh_lr_wsd(double k, double peak, double total, double decay_ratio,
                    double warmup, double eta_min);
/* Eq. (11) frozen from s_hold on: the constant-LR continuation that feeds
 * checkpoint averaging (§3.4: held from step 218,000 at base LR 4.08e-5).
 * Returns muonh_lr_linear(eta0, eta_min, min(s, s_hold), S).                */
double muonh_lr_linear_hold(double eta0, double eta_min, double s, double S, double s_hold);
/* Cosine decay from eta_max to eta_min over `total` steps after a linear
 * warmup of `warmup` steps (the post-training schedule, App. E); k is
 * clamped to [warmup, total] for the decay part.                            */
double muonh_lr_cosine(double k, double total, double eta_max, double eta_min, double warmup);
/* Effective LR of a Hyperball-wrapped matrix from the base schedule:
 * eta^H = multiplier * eta_base (§3.3.1; multiplier 10 in App. C, Tab. 8).
 * This is the value muonh_step_args.elr takes.                              */
double muonh_elr_from_base(double eta_base, double multiplier);

/* ---- AdamW for the parameters MuonH does not wrap -----------------------
 * The pages train embeddings, normalisation layers, the LM head and every
 * other non-wrapped parameter with AdamW at weight decay 0.1 on the base LR
 * schedule (§3.3; App. C, Tab. 8), and use Adam betas (0.9, 0.95) and
 * epsilon 1e-12 (App. E).  The update rule is the standard decoupled-decay
 * AdamW with bias correction, for step count t = 1, 2, ... and LR lr:
 *     W <- W (1 - lr wd);  m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
 *     W <- W - lr (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps)
 * computed in fp32 per element, one multi-tensor launch per step.
 * Conventions are those listed at the top of this file.                     */
typedef struct muonh_adamw_handle muonh_adamw_handle;

typedef struct muonh_adamw_tensor {
  void* w;          /* fp32 parameter, device, contiguous, updated in place    */
  const void* g;    /* gradient, device, g_dtype                                */
  void* m;          /* fp32 first moment, device, in place (zeros before t = 1) */
  void* v;          /* fp32 second moment, device, in place (zeros before t = 1)*/
  int64_t numel;    /* elements, >= 1                                           */
  int32_t g_dtype;  /* MUONH_F32 or MUONH_BF16                                  */
  int32_t reserved; /* must be 0                                                */
} muonh_adamw_tensor;

typedef struct muonh_adamw_options {
  float beta1;         /* 0.9  */
  float beta2;         /* 0.95 */
  float eps;           /* 1e-12 */
  float weight_decay;  /* 0.1  */
} muonh_adamw_options;

/* Fill *opt with the defaults listed above. */
void muonh_adamw_default_options(muonh_adamw_options* opt);

/* Plan the chunk table for these tensors (sizes and gradient dtypes are kept,
 * pointers are not) and allocate its small device tables on the current
 * device.  Errors: MUONH_EINVAL for n < 1, numel < 1, an unknown dtype, a
 * nonzero reserved field or options outside 0 <= beta < 1, eps > 0,
 * weight_decay >= 0; MUONH_EHIP for a HIP failure.  On failure *h is NULL. */
int muonh_adamw_init(muonh_adamw_handle** h, const muonh_adamw_tensor* t, int32_t n,
                     const muonh_adamw_options* opt);

/* One AdamW step at step count `step` (>= 1) with learning rate `lr` over the
 * same list (order, sizes, dtypes) as init; pointers may change between
 * steps.  w, m, v and an fp32 g must be 16-byte aligned, a bf16 g 8-byte
 * aligned.  Asynchronous on `stream`.  Errors: MUONH_EINVAL (null or
 * misaligned pointer, step < 1, non-finite lr), MUONH_EMISMATCH (list
 * differs from init), MUONH_EHIP.                                            */
int muonh_adamw_step(muonh_adamw_handle* h, const muonh_adamw_tensor* t, int32_t n,
                     float lr, int64_t step, void* stream);

/* Release the handle (waits for its last upload).  NULL is a no-op. */
int muonh_adamw_destroy(muonh_adamw_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* MUONH_H_ */
