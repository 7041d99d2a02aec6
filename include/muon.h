/*
 * muon.h — C ABI of the MI355X (gfx950) Muon optimizer step (and the AdamW
 * step a hybrid Muon optimizer runs on its other parameters, declared below).
 *
 * One Muon call performs one optimizer step on 2-D hidden-layer weight matrices:
 *
 *   M' = mu*M + G;  U = G + mu*M'                 momentum, Nesterov look-ahead
 *   X0 = U scaled by 1 / (||U||_F + eps), eps = 1e-7   (U^T first if rows > cols)
 *   ns_steps times:  X <- a X + b (X X^T) X + c (X X^T)^2 X
 *   O  = X (transposed back if rows > cols)
 *   O~ = O - (<W,O>_F / ||W||_F^2) W              MuonGS only, when ||W|| > 0
 *   W' = (1 - lr*wd) W - lr * 0.2*sqrt(max(rows,cols)) * O~
 *
 * Sources (page title and passage):
 *  - update order: "[Deep Learning] Muon — 행렬 업데이트를 직교화하는 옵티마이저"
 *    (codersblog.github.io), section 3 "Muon의 업데이트 순서", steps 1-5;
 *  - momentum 0.95 / Nesterov / 5 steps / coefficients (3.4445, -4.7750, 2.0315)
 *    / the norm's stabiliser eps: "LLM Pretraining Loss Spike 진단과 처방 ...
 *    Muon 전환 판단" (juhoplayground.github.io), section "Muon head의 실체는
 *    하이브리드 옵티마이저다", its Newton-Schulz snippet and the defaults after it;
 *  - the iteration X_k = aX + b(XX^T)X + c(XX^T)^2 X approximating
 *    (MM^T)^{-1/2}M and the 0.2*sqrt(max(A,B)) scale (eq. 4): "[논문 AI 리뷰]
 *    MUON IS SCALABLE FOR LLM TRAINING TECHNICAL REPORT" (blog.pieroot.xyz),
 *    section 2 "Key Methods and Approach";
 *  - decoupled (AdamW-style) weight decay: the loss-spike page, section
 *    "Moonlight와 MuonClip이 추가한 것";
 *  - MuonGS projection: "MuonGS: Pretraining LLMs with Relaxed Weight-Norm
 *    Control" (onedev.kr), the Gram-Schmidt update in "전제와 한계";
 *  - non-2-D parameters are errors: the codersblog page, section 5.
 *
 * Momentum is the SGD form (M' = mu*M + G), the plainest reading of the
 * pages' "SGD-momentum"; Nesterov is always on (the pages' default).
 * Weight decay uses the unscaled learning rate and applies in every variant.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Memory   W, G and M are DEVICE pointers to row-major rows x cols matrices.
 *           W and G hold `dtype` elements, M is always float32.  G is read
 *           only; W and M are updated in place.  W, G, M and the workspace
 *           must not overlap.  The caller owns every buffer.
 *  Dtype    MUON_DTYPE_F32: W, G float32; the iteration runs in float32.
 *           MUON_DTYPE_BF16: W, G bfloat16; the iteration runs on bf16
 *           matrix cores with float32 accumulation and float32 epilogues;
 *           W' is rounded to bfloat16 (round to nearest even).
 *  Workspace  device memory of at least the size the matching
 *           muon_workspace_bytes* call returns; any alignment; its contents
 *           on entry are ignored and are garbage on exit.
 *  Stats    optional device float array, MUON_STATS_PER_MATRIX floats per
 *           matrix (matrix order: group by group, then index within the
 *           group): ||U||_F, ||W||_F^2, <W,O>_F, ||O||_F^2, ||O~||_F^2 (the
 *           projected O for MuonGS, the equalised O for NorMuon/MeqMuon,
 *           ||O||^2 otherwise), of W and O before the update, returned as
 *           float32: the per-thread partial sums (float32 where the last
 *           Newton-Schulz launch forms them, float64 elsewhere) are added
 *           in float64.
 *           NULL skips them.
 *  Stream   a hipStream_t passed as void*; NULL is the default stream.  The
 *           call only enqueues work: it does not synchronise, allocate device
 *           memory or copy to the host.  Kernel faults surface at the
 *           caller's next synchronisation on that stream.
 *  Errors   every entry point returns a muon_status.  All arguments are
 *           validated before any work is enqueued; on an error nothing is
 *           enqueued and W, M are untouched.  MUON_ERR_HIP means a launch
 *           failed; earlier launches of the same call may have run.
 *           muon_status_string() names a status.
 *  Hyperparameters  lr, momentum, weight_decay, a, b, c must be finite;
 *           ns_steps in [0, MUON_MAX_NS_STEPS]; ns_steps == 0 is legal and
 *           gives O = X0.  variant: see MUON_VARIANT_* below.
 *  Shapes   1 <= rows, cols <= MUON_MAX_DIM.  An empty batch (count == 0 or
 *           ngroups == 0) is a no-op returning MUON_OK.
 *  Concurrency  calls on different streams must use different workspaces.
 *  Environment  MUON_DEBUG=1 synchronises the stream after every launch and
 *           prints the failing phase's name with the HIP error (debugging
 *           only: it breaks the no-synchronisation rule above).
 *           MUON_TRACE=1 opens a roctx range around every Muon and AdamW
 *           call ("muon_step", "muon_adamw_step") and one per launch, named
 *           by its phase (see muon_profile_read), for rocprofv3
 *           --marker-trace; the roctx library is loaded at first use, and
 *           a message on stderr says so if it cannot be.
 */
#ifndef MUON_MI355X_MUON_H
#define MUON_MI355X_MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad count, non-finite or out-of-range scalar */
  MUON_ERR_INVALID_SHAPE = 2,     /* rows or cols outside [1, MUON_MAX_DIM] */
  MUON_ERR_UNSUPPORTED_DTYPE = 3, /* dtype not MUON_DTYPE_F32 / MUON_DTYPE_BF16 */
  MUON_ERR_WORKSPACE_TOO_SMALL = 4,
  MUON_ERR_HIP = 5                /* a HIP runtime call or kernel launch failed */
} muon_status;

enum { MUON_DTYPE_F32 = 0, MUON_DTYPE_BF16 = 1 };
/*
 * variant: one of
 *   MUON_VARIANT_MUON    the step above;
 *   MUON_VARIANT_MUONGS  with the Gram-Schmidt projection O~ (MuonGS page,
 *                        "전제와 한계");
 *   MUON_VARIANT_MUONH   fixed-radius control (the MuonH the MuonGS page
 *                        compares against): W' = ||W||_F * W^ / ||W^||_F with
 *                        W^ = (1 - lr*wd) W - lr*s*O, so ||W||_F never changes;
 *   MUON_VARIANT_NORMUON every row of O (weight orientation) rescaled to the
 *                        mean row norm ||O||_F / sqrt(rows), zero rows kept
 *                        zero ("행과 열을 함께 정규화하는 사전학습 옵티마이저
 *                        MeqMuon 공개" (ailog.hnlab.kr), "핵심 내용": NorMuon
 *                        normalises the update row by row);
 *   MUON_VARIANT_MEQMUON the same along rows or along columns, whichever set
 *                        of norms has the larger std/mean (ties: rows) — the
 *                        same page: MeqMuon chooses the direction by itself;
 *                        the rule is this library's reading;
 * optionally OR-ed with MUON_SCALE_KELLER to use Keller's shape factor
 * s = max(1, rows/cols)^0.5 (last line of the loss-spike page's Newton-Schulz
 * code block) instead of Moonlight's 0.2*sqrt(max(rows, cols)).
 */
enum {
  MUON_VARIANT_MUON = 0,
  MUON_VARIANT_MUONGS = 1,
  MUON_VARIANT_MUONH = 2,
  MUON_VARIANT_NORMUON = 3,
  MUON_VARIANT_MEQMUON = 4
};
#define MUON_SCALE_KELLER 0x100

#define MUON_STATS_PER_MATRIX 5
#define MUON_MAX_DIM 32768
#define MUON_MAX_NS_STEPS 100
/* Groups handled by one launch sequence of muon_step_grouped; more groups are
 * processed as further sequences on the same stream. */
#define MUON_GROUPS_PER_LAUNCH 8

/*
 * A group: `count` matrices of one shape rows x cols.  Give EITHER device
 * pointer tables (W_table, G_table, M_table: device arrays of `count` device
 * pointers each, entries not checked on the host) OR contiguous stacks
 * (W, G, M: device pointers to [count][rows][cols] arrays).  The three
 * pointers of the unused form must be NULL.
 */
typedef struct muon_group {
  int64_t count;
  int64_t rows;
  int64_t cols;
  void* const* W_table;
  const void* const* G_table;
  float* const* M_table;
  void* W;
  const void* G;
  float* M;
} muon_group;

/* Workspace bytes for muon_step / muon_step_batched on count matrices of
 * rows x cols (0 on invalid arguments). */
size_t muon_workspace_bytes(int64_t count, int64_t rows, int64_t cols, int dtype);

/* Workspace bytes for muon_step_grouped over these groups (0 on invalid
 * arguments). */
size_t muon_workspace_bytes_grouped(const muon_group* groups, int ngroups, int dtype);

/* One step on one matrix.  W, G, M: device pointers (see conventions). */
int muon_step(void* W, const void* G, float* M, int64_t rows, int64_t cols, int dtype,
              double lr, double momentum, double weight_decay, int ns_steps,
              double a, double b, double c, int variant,
              void* workspace, size_t workspace_bytes, float* stats, void* stream);

/* One step on `count` same-shape matrices (per-layer stacks, MoE experts).
 * W, G, M: device arrays of `count` device pointers. */
int muon_step_batched(void* const* W, const void* const* G, float* const* M, int64_t count,
                      int64_t rows, int64_t cols, int dtype,
                      double lr, double momentum, double weight_decay, int ns_steps,
                      double a, double b, double c, int variant,
                      void* workspace, size_t workspace_bytes, float* stats, void* stream);

/* One step on several shape groups at once (a whole model): every phase is
 * one launch over the work of all groups.  `groups` is a HOST array. */
int muon_step_grouped(const muon_group* groups, int ngroups, int dtype,
                      double lr, double momentum, double weight_decay, int ns_steps,
                      double a, double b, double c, int variant,
                      void* workspace, size_t workspace_bytes, float* stats, void* stream);

/*
 * muon_step_grouped without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * of MUON_NOALLOC_WORKSPACE_BYTES inside the library (each GPU the library
 * runs on holds its own copy until the process ends); a call whose groups
 * need more (muon_workspace_bytes_grouped) returns
 * MUON_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  The call
 * allocates nothing: on its first call on a device it looks up that device's
 * copy of the array (hipGetSymbolAddress, with the device current).  Every
 * call on one GPU shares that GPU's array and its contents are ignored on
 * entry, so calls that overlap in time on one GPU (different streams, or
 * different host threads) race and must be serialised by the caller.  Other
 * arguments, results and errors are those of muon_step_grouped.
 */
#define MUON_NOALLOC_WORKSPACE_BYTES (((size_t)64) << 20)
int muon_step_grouped_noalloc(const muon_group* groups, int ngroups, int dtype,
                              double lr, double momentum, double weight_decay, int ns_steps,
                              double a, double b, double c, int variant,
                              float* stats, void* stream);

/*
 * AdamW for the parameters a hybrid Muon optimizer keeps off Muon: the input
 * embedding, the output head and the gains and biases ("LLM Pretraining Loss
 * Spike 진단과 처방" (juhoplayground.github.io), section "Muon head의 실체는
 * 하이브리드 옵티마이저다"; "[Deep Learning] Muon" (codersblog.github.io),
 * section 5 hands them to torch.optim.AdamW).  The MuonGS page's experiments
 * paragraph ("전제와 한계") runs it with betas (0.8, 0.95), eps 1e-10, weight
 * decay 1e-3 and peak learning rates 0.7 (embedding), 0.004 (head) and 0.015
 * (1-D parameters).  The pages print no formula; this is textbook decoupled
 * AdamW with bias correction, per element, in float32, at step t >= 1:
 *
 *   m' = beta1 m + (1 - beta1) g
 *   v' = beta2 v + (1 - beta2) g^2
 *   p' = (1 - lr wd) p - lr (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps)
 *
 *  Memory   P, G: DEVICE pointers to n contiguous elements of `dtype` (any
 *           shape, flattened); m, v: DEVICE float32 arrays of n elements
 *           (zero before the first step).  G is read only; P, m and v are
 *           updated in place; P' is rounded to bfloat16 (nearest even) when
 *           dtype is MUON_DTYPE_BF16.  No buffer may overlap another, within
 *           a tensor or across the tensors of one call.  Any alignment works;
 *           tensors whose four pointers are 8-byte (bf16) / 16-byte aligned
 *           take the vector path.
 *  Scalars  0 <= beta1, beta2 < 1; eps finite and >= 0; step >= 1 (it sets
 *           the bias corrections); lr and weight_decay finite (any sign).
 *  Sizes    0 <= n <= MUON_ADAMW_MAX_ELEMENTS; n == 0 skips the tensor.
 *  Stream, errors  as for the Muon entry points: validated before anything
 *           is enqueued, no allocation, no synchronisation.  The grouped call
 *           updates all tensors in one launch per MUON_ADAMW_TENSORS_PER_LAUNCH
 *           tensors (very large tensors are split over several slots).
 */
#define MUON_ADAMW_MAX_ELEMENTS (((int64_t)1) << 40)
#define MUON_ADAMW_TENSORS_PER_LAUNCH 32

typedef struct muon_adamw_tensor {
  void* P;             /* parameters, `dtype` */
  const void* G;       /* gradients, `dtype` */
  float* m;            /* first moment, float32 */
  float* v;            /* second moment, float32 */
  int64_t n;           /* elements */
  double lr;           /* learning rate of this tensor */
  double weight_decay; /* decoupled weight decay of this tensor */
} muon_adamw_tensor;

/* One AdamW step on one tensor. */
int muon_adamw_step(void* P, const void* G, float* m, float* v, int64_t n, int dtype,
                    double lr, double beta1, double beta2, double eps, double weight_decay,
                    int64_t step, void* stream);

/* One AdamW step on `count` tensors with their own lr and weight decay and
 * shared betas, eps and step.  `tensors` is a HOST array. */
int muon_adamw_step_grouped(const muon_adamw_tensor* tensors, int64_t count, int dtype,
                            double beta1, double beta2, double eps, int64_t step, void* stream);

/*
 * Phase timing, for benchmarks and profiling.  While enabled (process-wide),
 * every kernel launch of the step entry points is bracketed by two HIP events
 * recorded on the caller's stream.  muon_profile_read waits for the recorded
 * events, adds each launch's elapsed milliseconds to ms_total[phase] and
 * launches[phase] (arrays of nphases entries, host memory, zeroed by the
 * caller), and forgets the records.  Phases: 0 head, 1 norm_finalize, 2 gram,
 * 3 poly, 4 update, 5 tail_reduce, 6 tail_finalize, 7 tail_apply, 8 adamw
 * (the AdamW entry points), 9 update_tail (the last update launch when it
 * also applies the step, which plain Muon without statistics does on the
 * bf16 path, or writes the per-tile sums of MuonGS, MuonH or statistics:
 * then tail_reduce and tail_apply cover only the matrices it did not).
 * Returns MUON_ERR_INVALID_ARGUMENT for null arrays or nphases < 1, and
 * MUON_ERR_HIP if an event call failed.
 */
#define MUON_NUM_PHASES 10
int muon_profile_enable(int enable);
int muon_profile_read(double* ms_total, int64_t* launches, int nphases);
/* Static name of a phase ("?" when out of range). */
const char* muon_phase_name(int phase);

/* Static string naming a status (never NULL). */
const char* muon_status_string(int status);

/* The HIP error code of the most recent MUON_ERR_HIP on this thread (0 if none). */
int muon_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_MUON_H */
