// Kernel argument blocks and launchers of libmuon (internal).
//
// Every kernel takes its per-matrix table by value as a kernel argument
// (at most ~3 KB per launch), in the manner of a multi-tensor apply: a step
// needs no host-to-device table copy, no staging memory and no stream
// synchronisation, and the whole step can be captured in a HIP graph.  Host
// code splits long matrix lists into several launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon.h"

#include <climits>

namespace muon {

enum DType : int32_t { kF32 = 0, kF16 = 1, kBF16 = 2 };

// ------------------------------------------------------------------ E1
// MONA difference + EMA, momentum, per-block partial sums of M^2.
#ifndef MUON_E1_THREADS
#define MUON_E1_THREADS 1024
#endif
constexpr int kE1Threads = MUON_E1_THREADS;
constexpr int kE1ElemsPerThread = 8192 / kE1Threads;       // groups of 4
constexpr int kE1BlockElems = kE1Threads * kE1ElemsPerThread;  // 8192
constexpr int kE1MaxMats = 40;

// E1 modes: plain Muon, MONA (A fp32 + previous gradient), MONA-Lite (one
// bfloat16 state).
enum E1Mode : int32_t { kE1Plain = 0, kE1Mona = 1, kE1Lite = 2 };

struct FinalDesc;
struct E1Mat {
  const void *grad;
  float *mom;
  float *accel;     // MONA: A
  void *prev;       // MONA: previous gradient (grad dtype)
  void *lite;       // MONA-Lite: bfloat16 state
  float *weight;    // for the FinalDesc written by the matrix's block 0
  float *ortho_out;
  int64_t numel;
  int32_t partial_off;   // index of this matrix's first partial in the workspace
  int32_t desc_idx;      // FinalDesc slot, or -1
  int32_t rows, cols;
  float gamma;
  int32_t pad;
};

// begin[i] = first block of matrix i within the launch, ascending; unused
// entries hold INT32_MAX.  A block finds its matrix by counting entries <= its
// index: independent scalar loads, one memory round trip.
struct E1Args {
  int32_t nmat;
  int32_t grad_dtype;
  int32_t first_step;    // MONA / MONA-Lite: D = 0
  int32_t mode;          // E1Mode of every matrix of the launch
  float mu, beta_a, alpha;
  int32_t stream;        // non-temporal loads and stores (state far larger than the caches)
  double *partials;      // workspace
  FinalDesc *desc;       // workspace
  int32_t begin[kE1MaxMats];
  E1Mat mats[kE1MaxMats];
};

// ------------------------------------------------------------------ norm
constexpr int kNormMaxMats = 128;
struct NormMat {
  int32_t partial_off;
  int32_t nparts;
  int32_t scale_idx;
  int32_t pad;
};
struct NormArgs {
  int32_t nmat;
  float inv_sqrt_d;       // 1/sqrt(divisor)
  float store_scale;      // power-of-two storage scale of X0
  int32_t pad;
  const double *partials;
  float *scales;
  NormMat mats[kNormMaxMats];
};

// What the last Newton-Schulz product needs to apply W <- W - lr (gamma O + wd W);
// written by E1 (block 0 of each matrix) into the workspace.
struct FinalDesc {
  float *weight;
  float *ortho_out;     // optional fp32 copy of O
  int32_t rows, cols;
  float gamma;
  int32_t wide;         // rows <= cols: O is the transpose of the tall tile
};

// ------------------------------------------------------------------ E2
// X0 = M * scale, rounded to the NS dtype, written in M's orientation
// ("natural", zero-padded to pr x pc) and transposed (pc x pr).  A matrix
// with at most kE2InlineParts norm partials has its scale reduced inside E2
// (every block of the matrix computes the same fixed-order sum); others read
// the scale written by norm_kernel.
constexpr int kE2Tile = 64;
constexpr int kE2MaxMats = 48;
constexpr int kE2InlineParts = 64;

struct E2Mat {
  const float *mom;
  void *nat;                 // M's own layout, or NULL when not read
  void *trn;                 // its transpose, or NULL when not read
  int32_t rows, cols;        // true M shape
  int32_t ld_nat, ld_trn;    // = padded cols, padded rows
  int32_t tiles_c;           // padded cols / 64
  int32_t scale_idx;
  int32_t partial_off;       // inline norm: first partial
  int32_t nparts;            // inline norm when 0 < nparts <= kE2InlineParts
};
struct E2Args {
  int32_t nmat;
  int32_t ns_dtype;
  float inv_sqrt_d;          // inline norm: 1/sqrt(divisor)
  float store_scale;         // inline norm: storage scale of X0
  int32_t stream;            // non-temporal loads of M (see E1Args::stream)
  int32_t pad;
  const float *scales;
  const double *partials;
  int32_t begin[kE2MaxMats];   // first tile of each matrix (see E1Args)
  E2Mat mats[kE2MaxMats];
};

// ------------------------------------------------------------------ E3
// W = W - lr * (gamma * O + wd * W), O read from the NS workspace.
constexpr int kE3Threads = 256;
constexpr int kE3BlockElems = kE3Threads * 16;
constexpr int kE3MaxMats = 56;
struct E3Mat {
  float *weight;
  const void *o;         // final iterate in W's orientation, leading dim ld_o
  float *ortho_out;      // optional fp32 copy of O
  int64_t numel;
  int32_t cols;
  int32_t ld_o;
  float gamma;
  float inv_o_scale;     // 1 / storage scale of O
  int32_t vec_ok;        // 16-byte aligned and cols % 4 == 0
  int32_t pad;
};
struct E3Args {
  int32_t nmat;
  int32_t ns_dtype;
  float lr, wd;
  int32_t begin[kE3MaxMats];   // first block of each matrix (see E1Args)
  E3Mat mats[kE3MaxMats];
};

// ------------------------------------------------------------------ GEMM
// C = alpha * A B^T + beta * Cin + diag * I   (A: m x k, B: n x k, row-major)
// over a group of same-shaped matrices per class; "half" computes only
// upper-triangular tiles of a symmetric result and mirrors them.
constexpr int kGemmMaxClasses = 8;
struct GemmClass {
  const void *a;
  const void *b;
  void *c;          // may be null (only C2 written)
  void *c2;         // transposed copy of the result, or null
  const void *cin;  // epilogue input (same orientation as C), or null
  int64_t sa, sb, sc, sc2, scin;   // per-matrix element strides
  int32_t lda, ldb, ldc, ldc2, ldcin;
  int32_t K;                       // multiple of the k-stage
  int32_t tiles_m, tiles_n;
  int32_t tiles_per_mat;
  int32_t count;
  int32_t half;
  int32_t diag_limit;              // diag term only where row == col < diag_limit
  float alpha, beta, diag;
  // Final product of the iteration: instead of storing C / C2, apply
  // W <- W - lr (gamma O + wd W) through desc[desc_base + matrix]; the tile
  // is in the tall orientation (rows index the long side).
  int32_t final_mode;
  int32_t desc_base;
  const FinalDesc *desc;
  float lr, wd;
  // Fused polynomial update (launch_poly_update only): b points at the
  // symmetric s x s matrix A, and each block first forms its panel of
  // B = sq_alpha A A + sq_beta A in LDS.  Output tile rows come in groups
  // of m_group tiles (of m_tiles), one group per block: tiles_m counts groups.
  float sq_alpha, sq_beta;
  int32_t m_group, m_tiles;
};
struct GemmArgs {
  int32_t nclass;
  int32_t total_tiles;
  // Workgroup -> tile order over the 8 XCDs: 0 = each XCD walks one
  // contiguous run of the launch's tiles; G > 0 = runs of G tiles dealt to
  // the XCDs in turn (every class of the launch spread over all XCDs);
  // kXcdByClass = each XCD walks a contiguous eighth of every class
  // (xcd_lo / xcd_start, filled by set_xcd_order).
  int32_t xcd_group;
  int32_t tile_begin[kGemmMaxClasses];   // first tile of each class; unused = INT32_MAX
  int32_t xcd_lo[kGemmMaxClasses][9];    // class c's eighth x: tiles [xcd_lo[c][x], xcd_lo[c][x+1]) of the class
  int32_t xcd_start[9];                  // sum over classes of xcd_lo[c][x]
  GemmClass cls[kGemmMaxClasses];
};
constexpr int kXcdByClass = -1;
// Fill xcd_lo / xcd_start from nclass, tile_begin and total_tiles.
inline void set_xcd_order(GemmArgs &a) {
  for (int x = 0; x <= 8; ++x) a.xcd_start[x] = 0;
  for (int c = 0; c < kGemmMaxClasses; ++c) {
    const int64_t t = c < a.nclass ? (int64_t)((c + 1 < a.nclass ? a.tile_begin[c + 1] : a.total_tiles) - a.tile_begin[c]) : 0;
    for (int x = 0; x <= 8; ++x) {
      a.xcd_lo[c][x] = (int32_t)(t * x / 8);
      a.xcd_start[x] += a.xcd_lo[c][x];
    }
  }
}
// Measured choice: runs of 16 for the 256 tile (mixed-K launches stay
// balanced across XCDs, and the large operands are shared through the
// device-wide cache), one run per XCD for the 64 and 128 tiles and the fused
// update (operand reuse in each XCD's L2).
constexpr int kXcdGroup = 16;

// ------------------------------------------------------------------ AdamW
// Decoupled AdamW over a list of fp32 tensors (vector-shaped parameters).
constexpr int kAdamThreads = 256;
constexpr int kAdamBlockElems = kAdamThreads * 16;
constexpr int kAdamMaxTensors = 64;
struct AdamTensor {
  float *param;
  const void *grad;
  float *m;
  float *v;
  int64_t numel;
  int32_t vec_ok;        // 16-byte aligned fp32 buffers, 8-byte aligned 16-bit grad
  int32_t pad;
};
struct AdamArgs {
  int32_t nt;
  int32_t grad_dtype;
  float beta1, beta2;
  float one_minus_beta1, one_minus_beta2;
  float step_size;       // lr / (1 - beta1^t)
  float inv_sqrt_bc2;    // 1 / sqrt(1 - beta2^t)
  float eps;
  float decay;           // lr * weight_decay
  int32_t begin[kAdamMaxTensors];   // first block of each tensor (see E1Args)
  AdamTensor t[kAdamMaxTensors];
};

// ------------------------------------------------------------------ LiMuon
// Small-matrix stages of the randomized-SVD orthogonaliser: the sketch
// width k + p is padded to kLmKP in the panels' storage; panels are fp32
// [rows x kLmKP] row-major.
constexpr int kLmKP = 64;             // panel storage width (k + p <= 64)
constexpr int kLmMaxClasses = 8;
constexpr int kLmSlot = kLmKP * kLmKP;   // floats per small matrix (W, T)

// Thin products C (M x NB) = A (M x K) B^T with B given as NB x K rows (NB =
// 32 or 64 >= k + p; rows of B past k + p are zero), fp32, one block per 64
// rows of one matrix (M is the padded row count, a multiple of 64).  Also
// writes C^T (c2, optional) and, when part_base >= 0, the fp64 Gram matrix
// of the block's 64 rows of C over its first n columns into slot
// part_base + matrix * tiles + tile (n x n doubles per slot).
constexpr int kThinRows = 64;
struct LmThinClass {
  const float *a;
  const float *b;
  float *c;
  float *c2;
  int64_t sa, sb, sc, sc2;   // per-matrix element strides (sb = 0: B shared by the class)
  int32_t lda, ldb, ldc, ldc2;
  int32_t K;                 // multiple of 32
  int32_t tiles;             // M / kThinRows
  int32_t count;
  int32_t part_base;         // first Gram slot, or -1
};
struct LmThinArgs {
  int32_t nclass;
  int32_t n;                 // k + p: columns in the Gram partials
  int32_t begin[kLmMaxClasses];   // first block of each class; unused = INT32_MAX
  double *partials;
  LmThinClass cls[kLmMaxClasses];
};

// Small symmetric factorisations (fp64) of the sum of a matrix's Gram
// partials, one block per matrix, writing a kLmKP x kLmKP fp32 result:
//   kLmOrth:  W^T with P W orthonormal columns spanning the panel P's range:
//             pivoted Cholesky, stopped where the pivot falls to
//             cutoff * max(diag), and the inverse of its triangular factor
//   kLmTrunc: T = V_k D_k^{-1/2} V_k^T (Jacobi eigen-decomposition) over the
//             `rank` largest eigenvalues that exceed cutoff * d_max
enum LmEigMode : int32_t { kLmOrth = 0, kLmTrunc = 1 };
struct LmEigClass {
  float *out;              // first matrix's kLmKP x kLmKP result
  int64_t out_stride;      // elements between matrices' results
  int32_t count;
  int32_t nchunks;         // Gram partials per matrix (n x n doubles each)
  int32_t part_base;
  int32_t pad;
};
struct LmEigArgs {
  int32_t nclass;
  int32_t n;
  int32_t mode;
  int32_t rank;
  double cutoff;                         // relative to the largest diagonal / eigenvalue
  int32_t begin[kLmMaxClasses];          // first block (matrix) of each class
  const double *partials;
  LmEigClass cls[kLmMaxClasses];
};

// Weight update of the LiMuon step: O = P Z^T (P: s-row panel Q T, Z: l-row
// panel X^T Q, both [rows x kLmKP], the first kp columns used) and
// W <- W - lr (gamma O + wd W) in W's own orientation, one block per 64 x 64
// tile of W; per-matrix W, gamma, orientation and the optional O copy come
// from the FinalDesc table E1 wrote.
constexpr int kLmFinalTile = 64;
struct LmFinalClass {
  const float *p;          // first matrix's P panel
  const float *z;          // first matrix's Z panel
  int64_t sp, sz;          // elements between matrices' panels
  int32_t desc_base;       // FinalDesc slot of the class's first matrix
  int32_t count;
  int32_t tiles;           // 64 x 64 tiles of W per matrix
  int32_t pad;
};
struct LmFinalArgs {
  int32_t nclass;
  int32_t kp;
  float lr, wd;
  int32_t begin[kLmMaxClasses];
  const FinalDesc *desc;
  LmFinalClass cls[kLmMaxClasses];
};

// Copy the caller's test matrix (kp rows of the long-side length, row
// stride ld) into each class's zero-padded [kLmKP x lp] buffer.
struct LmPadClass {
  float *dst;
  int32_t l, lp;           // true and padded long side
  int32_t blocks;          // blocks of this class
  int32_t pad;
};
struct LmPadArgs {
  const float *src;
  int64_t ld;
  int32_t kp;
  int32_t nclass;
  int32_t begin[kLmMaxClasses];
  LmPadClass cls[kLmMaxClasses];
};
constexpr int kLmPadElems = 4096;     // padded elements per pad block

hipError_t launch_lm_thin(const LmThinArgs &args, int nb, int blocks, hipStream_t s);
hipError_t launch_lm_eig(const LmEigArgs &args, int blocks, hipStream_t s);
hipError_t launch_lm_pad(const LmPadArgs &args, int blocks, hipStream_t s);
hipError_t launch_lm_final(const LmFinalArgs &args, int blocks, hipStream_t s);

// Record `msg` as the calling thread's muon_last_error() and return `s`.
muon_status record_error(muon_status s, const char *msg);

// Launchers (return the launch status).
hipError_t launch_e1(const E1Args &args, int blocks, hipStream_t s);
hipError_t launch_norm(const NormArgs &args, hipStream_t s);
hipError_t launch_e2(const E2Args &args, int blocks, hipStream_t s);
hipError_t launch_e3(const E3Args &args, int blocks, hipStream_t s);
hipError_t launch_adamw(const AdamArgs &args, int blocks, hipStream_t s);
// tile = 64 or 128 (square block tile); dtype selects the operand type.
hipError_t launch_gemm(const GemmArgs &args, int dtype, int tile, hipStream_t s);
// X'^T = alpha X^T (sq_alpha A A + sq_beta A) + beta X^T for short sides
// padded to sp (64, 128 or 192; every class of the launch has K == sp),
// 16-bit dtypes only.  m_group <= poly_max_group(sp) <= kPolyMaxGroup.
constexpr int kPolyMaxGroup = 4;
int poly_blocks_per_cu(int sp);
int poly_max_group(int sp);
hipError_t launch_poly_update(const GemmArgs &args, int dtype, int sp, hipStream_t s);

}  // namespace muon
