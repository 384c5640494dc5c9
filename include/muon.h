/*
 * libmuon -- one Muon / MONA optimizer step over a list of weight matrices,
 * on one AMD Instinct MI355X (gfx950).
 *
 * What one call computes, per matrix (rows x cols, row-major):
 *
 *   MONA (only when `accel` is given) -- MONA summary (gist.science paper
 *   2605.26842), section 2 "Methodologie", "Kernalgoritme", steps 1-3:
 *       D  = G - G_prev          (D = 0 on the first step, opts->step == 0)
 *       A  = beta_a * A + (1 - beta_a) * D
 *       G~ = G + alpha * A ;     G_prev = G
 *   MONA-Lite (only when `mona_lite` is given) -- MONA summary, "Efficiëntie
 *   en Implementatie": one bfloat16 state C replaces A and G_prev,
 *       A  = C + (1 - beta_a) * G  (A = 0 on the first step)
 *       G~ = G + alpha * A ;       C = bf16(beta_a * A - (1 - beta_a) * G)
 *   which is MONA's A exactly up to the state's rounding.
 *   Momentum -- same section, step 4:      M = mu * M + G~
 *   Orthogonalisation -- same section, step 4, "O = Newton-Schulz(M)";
 *   polar(X) = U V^T and its Gram form X (X^T X)^{-1/2} with restarts and a
 *   safety divisor d -- Gram Newton-Schulz post (quant_prune_distill 677):
 *       X0 = M / (sqrt(d) * ||M||_F)                (X0 = 0 when M = 0)
 *       K steps of X <- a_k X + (b_k A + c_k A^2) X,   A = X X^T
 *       (restart before step k when r > 0, k > 1, (k-1) % r == 0: the
 *        iterate is divided by sqrt(d); the Gram variant also re-forms its
 *        Gram matrix from the materialised iterate)
 *   Decoupled update -- MONA summary, step 4:
 *       W = W - lr * (gamma * O + lambda * W)
 *
 * The acceleration is applied before orthogonalisation (MONA summary,
 * "Ontwerprichtlijnen").
 *
 * Conventions for every entry point:
 *  - All buffer pointers in muon_param are DEVICE pointers owned by the
 *    caller.  The library never allocates, frees or retains them.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream).  No entry point synchronises the stream or the device.
 *  - Argument errors are reported synchronously, before anything is
 *    enqueued, and leave every buffer untouched.  Launch failures return
 *    MUON_ERR_HIP.  Data is not inspected: NaN/Inf in one matrix propagate
 *    inside that matrix only.
 *  - Calls that share a workspace must be ordered on one stream (or the
 *    caller orders them); the workspace may be reused once stream order
 *    allows.
 */
#ifndef LIBMUON_MUON_H
#define LIBMUON_MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1,        /* NULL pointer, bad size, non-finite scalar, aliasing */
  MUON_ERR_UNSUPPORTED = 2,        /* valid request the library cannot serve */
  MUON_ERR_WORKSPACE_TOO_SMALL = 3,
  MUON_ERR_HIP = 4                 /* a HIP launch or runtime call failed */
} muon_status;

typedef enum muon_dtype {
  MUON_F32 = 0,
  MUON_F16 = 1,
  MUON_BF16 = 2
} muon_dtype;

typedef enum muon_variant {
  MUON_NS_DIRECT = 0,   /* Newton-Schulz on X itself                             */
  MUON_NS_GRAM = 1,     /* Newton-Schulz on the smaller Gram matrix, with restarts */
  MUON_LIMUON = 2       /* randomized SVD of the momentum instead of Newton-Schulz
                           (LiMuon digest, "Метод"; see muon_options.sketch)      */
} muon_variant;

/* One weight matrix and its optimizer state.  Every buffer holds rows*cols
 * elements, row-major, contiguous, on the device; none may overlap another. */
typedef struct muon_param {
  float *weight;        /* fp32, updated in place                                  */
  const void *grad;     /* grad_dtype, read only                                   */
  float *momentum;      /* fp32 state M, updated in place; zero before step 0       */
  float *accel;         /* fp32 MONA state A, updated in place; NULL => plain Muon  */
  void *prev_grad;      /* grad_dtype, previous gradient; NULL iff accel == NULL    */
  int64_t rows, cols;   /* >= 1                                                     */
  float gamma;          /* scale on O in the update (gamma of the MONA update)      */
  float *ortho_out;     /* optional fp32 rows*cols: receives O; NULL => not written */
  void *mona_lite;      /* bfloat16 rows*cols MONA-Lite state, updated in place
                           (contents ignored on step 0); NULL => not Lite.  Not
                           together with accel / prev_grad                      */
} muon_param;

/* Kind of each launch recorded in a muon_trace. */
typedef enum muon_stage {
  MUON_STAGE_E1 = 0,     /* MONA + momentum + Frobenius partials              */
  MUON_STAGE_NORM = 1,   /* per-matrix normalisation scale                     */
  MUON_STAGE_E2 = 2,     /* X0 in the Newton-Schulz dtype, layouts the NS reads */
  MUON_STAGE_GEMM = 3,   /* one grouped Newton-Schulz matrix product           */
  MUON_STAGE_E3 = 4,     /* decoupled weight-decay update                      */
  MUON_STAGE_ADAMW = 5,  /* AdamW over vector parameters (muon_adamw_step)     */
  MUON_STAGE_SMALL = 6   /* LiMuon's (k+p)-wide stages: Gram partials, eigen-
                            decompositions, test-matrix copy                   */
} muon_stage;

/* Optional launch timing.  When muon_options.trace is non-NULL the library
 * records HIP events on the stream around its launches and writes, for each
 * recorded interval i (at most `capacity`), events[2*i] (before) and
 * events[2*i+1] (after), the muon_stage of the interval's launches into
 * stages[i] and their summed algorithmic work into work[i] (FLOPs for GEMM
 * launches, bytes moved for the others).
 *   group == 0: one interval per launch.
 *   group != 0: one interval per run of consecutive launches of the same
 *               stage, with no event between the launches of a run (so the
 *               events do not separate them); launches[i] receives the
 *               number of launches in interval i.
 * The caller creates the events (hipEventCreate, timing enabled) and reads
 * them after synchronising.  `count` returns the number of intervals of the
 * call (which may exceed capacity; the excess is not recorded).  `launches`
 * may be NULL when group == 0. */
typedef struct muon_trace {
  void **events;         /* 2 * capacity hipEvent_t handles                   */
  int32_t *stages;       /* capacity entries, out                             */
  double *work;          /* capacity entries, out                             */
  int32_t capacity;
  int32_t count;         /* out                                               */
  int32_t group;         /* 0: per launch; else per run of one stage          */
  int32_t *launches;     /* capacity entries, out (group != 0)                */
} muon_trace;

/* Settings shared by every matrix of a call.  Pass NULL for the defaults. */
typedef struct muon_options {
  muon_dtype grad_dtype;   /* dtype of grad / prev_grad.              default F32     */
  muon_dtype ns_dtype;     /* dtype of the Newton-Schulz operands.    default F32;
                              F16 / BF16 use the MFMA matrix cores with fp32 accumulate */
  const float *coeffs;     /* HOST array [ns_steps][3] of (a, b, c) per step, or NULL
                              for the quintic (15/8, -5/4, 3/8) at every step            */
  float divisor;           /* safety divisor d >= 1.                  default 1         */
  int32_t restart_every;   /* restart period r >= 0 (0 = never).      default 0         */
  int64_t step;            /* 0-based optimizer step; 0 => MONA's D is zero.  default 0 */
  muon_trace *trace;       /* optional launch timing (see muon_trace).  default NULL */
  /* MUON_LIMUON only (ignored otherwise).  LiMuon digest ("LiMuon: Light and
   * Fast Muon Optimizer for Large Models", section "Метод"): momentum, then a
   * randomized SVD of it in place of Newton-Schulz -- the textbook randomized
   * SVD (Halko, Martinsson & Tropp 2011, Algorithms 4.4 and 5.1).  Per matrix,
   * with X the momentum in its wide orientation (s x l, s <= l; a tall matrix
   * is transposed in and out) and Omega = the first l columns of `sketch`,
   * transposed (l x (rank + oversample)):
   *     Y = X Omega, Q = orth(Y); power_iters times: Q = orth(X orth(X^T Q));
   *     B = Q^T X = U~ S V^T;  O = sum over the `rank` largest S_i that exceed
   *     rcond * S_1 of (Q U~)_i V_i^T
   * O is scale-invariant, so ns_steps, coeffs, divisor and restart_every are
   * ignored.  The products run with fp32 operands: ns_dtype must be F32. */
  const float *sketch;     /* DEVICE fp32 [(rank + oversample) x sketch_ld] Gaussian
                              test matrix, row-major, drawn by the caller (row j =
                              test vector j); read only.        default NULL       */
  int64_t sketch_ld;       /* row stride of sketch, >= every matrix's long side   */
  int32_t rank;            /* k >= 1.                                 default 0 (unset) */
  int32_t oversample;      /* p >= 0, k + p <= 64.                    default 8         */
  int32_t power_iters;     /* q in [0, 16].                           default 1         */
  float rcond;             /* relative singular-value cutoff in [0, 1). default 1e-4    */
} muon_options;

/* Fill `o` with the defaults listed above. */
void muon_options_init(muon_options *o);

/* Device bytes of workspace `muon_step` needs for this exact call (same
 * params shapes, n, ns_steps, variant and options).  Returns 0 when the
 * request is invalid (muon_last_error() says why).  The size depends only on
 * shapes and settings, never on pointer values. */
size_t muon_workspace_size(const muon_param *params, int n, int ns_steps,
                           muon_variant variant, const muon_options *opts);

/* One optimizer step over `n` matrices (n >= 0; n == 0 is a no-op).
 *   params     host array of n muon_param (read during the call only)
 *   lr, mu     learning rate eta and momentum coefficient
 *   beta_a     MONA EMA coefficient, alpha MONA acceleration scale
 *              (ignored for matrices with accel == NULL)
 *   lambda     decoupled weight decay
 *   ns_steps   Newton-Schulz steps K, 0 <= K <= 64 (K = 0 => O = X0)
 *   workspace  device buffer of at least muon_workspace_size(...) bytes,
 *              256-byte aligned, caller-owned; its contents need no
 *              initialisation and are clobbered
 *   stream     hipStream_t (void* here so that C callers need no HIP headers)
 * Errors: MUON_ERR_INVALID_ARG for NULL weight/grad/momentum, accel/prev_grad
 * given without the other, mona_lite together with accel, rows or cols < 1,
 * ns_steps out of range,
 * non-finite scalars, divisor < 1, restart_every < 0, buffers that overlap;
 * for MUON_LIMUON also a NULL sketch, rank < 1, oversample < 0,
 * rank + oversample > 64, power_iters outside [0, 16], rcond outside [0, 1),
 * sketch_ld below a long side, a sketch overlapping another buffer;
 * MUON_ERR_UNSUPPORTED for an unknown dtype (and for MUON_LIMUON with a
 * 16-bit ns_dtype), and for a matrix with rows or cols above 2^20 or more
 * than 2^31 - 1 elements; MUON_ERR_WORKSPACE_TOO_SMALL;
 * MUON_ERR_HIP when a launch fails. */
muon_status muon_step(const muon_param *params, int n,
                      float lr, float mu, float beta_a, float alpha, float lambda,
                      int ns_steps, muon_variant variant, const muon_options *opts,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the static workspace muon_step_static uses on each GPU (64 MiB). */
#define MUON_STATIC_WORKSPACE_BYTES (64u << 20)

/* muon_step without a caller-owned workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, computation and
 * results as muon_step, with the workspace taken from a static device array
 * of MUON_STATIC_WORKSPACE_BYTES that the library holds on every GPU it runs
 * on until the process ends.  The array belongs to the CURRENT device: the
 * stream must belong to it.  The call allocates and frees nothing (the
 * array's device address is looked up once per device, on the first call
 * there).  Every call on one GPU shares that GPU's array and leaves its
 * contents behind, so calls that overlap on one GPU (on two streams, or from
 * two threads without ordering) race; order them on one stream.
 * Errors: as muon_step, plus MUON_ERR_WORKSPACE_TOO_SMALL (before anything is
 * enqueued) when muon_workspace_size(...) of the call exceeds
 * MUON_STATIC_WORKSPACE_BYTES, MUON_ERR_INVALID_ARG when the stream belongs
 * to another device, MUON_ERR_HIP when the array cannot be located. */
muon_status muon_step_static(const muon_param *params, int n,
                             float lr, float mu, float beta_a, float alpha, float lambda,
                             int ns_steps, muon_variant variant, const muon_options *opts,
                             void *stream);

/* One vector-shaped parameter (bias, norm weight, embedding: anything the
 * caller keeps out of Muon) and its AdamW state.  Every buffer holds numel
 * contiguous elements on the device; none may overlap another. */
typedef struct muon_adamw_param {
  float *param;         /* fp32, updated in place                                  */
  const void *grad;     /* grad_dtype, read only                                   */
  float *exp_avg;       /* fp32 first moment m, updated; zero before step 0        */
  float *exp_avg_sq;    /* fp32 second moment v, updated; zero before step 0       */
  int64_t numel;        /* >= 1                                                    */
} muon_adamw_param;

/* One decoupled AdamW step over `n` tensors (n >= 0), the optimizer the MONA
 * summary ("Ontwerprichtlijnen") keeps for vector-shaped parameters.  The
 * pages give no formula; this is the textbook decoupled form (Loshchilov &
 * Hutter 2019, Algorithm 2), with t = step + 1:
 *     m = beta1 m + (1 - beta1) g ;  v = beta2 v + (1 - beta2) g^2
 *     p = p - lr (m / (1 - beta1^t) / (sqrt(v / (1 - beta2^t)) + eps) + weight_decay p)
 * All tensors of a call share grad_dtype and the hyper-parameters, and are
 * updated by one launch per 64 tensors on `stream`.  `trace` (optional) records
 * the launches as MUON_STAGE_ADAMW (see muon_trace).
 * Errors: MUON_ERR_INVALID_ARG for NULL pointers, numel < 1, non-finite
 * scalars, beta1 or beta2 outside [0, 1), eps < 0, step < 0, overlapping
 * buffers; MUON_ERR_UNSUPPORTED for an unknown grad_dtype or numel above
 * 2^31 - 1; MUON_ERR_HIP when a launch fails. */
muon_status muon_adamw_step(const muon_adamw_param *params, int n, muon_dtype grad_dtype,
                            float lr, float beta1, float beta2, float eps, float weight_decay,
                            int64_t step, muon_trace *trace, void *stream);

/* Where one square Newton-Schulz work buffer of param `index` lives in the
 * workspace of the call described by the same (params, n, ns_steps,
 * variant, opts) as muon_workspace_size -- for tests and debugging, e.g.
 * checking that symmetric results (computed on upper-triangular tiles and
 * mirrored: Gram Newton-Schulz post, "half the elements") are stored exactly
 * symmetric.  which: 0..1 for MUON_NS_DIRECT (A = X X^T, B = b A + c A^2),
 * 0..4 for MUON_NS_GRAM (the R, T, P, Q buffers, rotated between steps).
 * After a muon_step the buffer holds the last value the schedule wrote
 * there, stored in ns_dtype (fp16 multiplied by a power-of-two storage
 * scale), side x side, padded to ld x ld with zeros.  Writes *offset
 * (bytes), *ld and *side (elements).  Errors: MUON_ERR_INVALID_ARG for an
 * invalid call, index or which (LiMuon has no square buffers), NULL
 * outputs. */
muon_status muon_debug_square_buffer(const muon_param *params, int n, int ns_steps,
                                     muon_variant variant, const muon_options *opts,
                                     int index, int which,
                                     size_t *offset, int64_t *ld, int64_t *side);

/* Static description of a status code. */
const char *muon_status_string(muon_status s);

/* Thread-local detail about the last non-OK return on this thread ("" if none). */
const char *muon_last_error(void);

/* Library version string, e.g. "libmuon 0.1.0 gfx950". */
const char *muon_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMUON_MUON_H */
