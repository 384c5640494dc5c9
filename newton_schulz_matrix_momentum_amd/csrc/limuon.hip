// Small-matrix stages of the LiMuon orthogonaliser for gfx950.
//
// LiMuon (digest "LiMuon: Light and Fast Muon Optimizer for Large Models",
// section "Метод") replaces Newton-Schulz by a randomized SVD of the
// momentum.  The large products of that SVD (the sketch X Omega, the power
// iterations X^T Q and X Z, the projection X^T Q and the final product) run
// in the grouped MFMA GEMM kernels; what remains are operations on the
// (k + p)-wide panels, implemented here:
//
//   lm_gram_kernel  fp64 partial Gram matrices P^T P of tall fp32 panels,
//                   one block per (matrix, chunk of rows)
//   lm_eig_kernel   one block per matrix: fixed-order sum of its partials,
//                   cyclic Jacobi eigen-decomposition in fp64 (parallel
//                   round-robin pair order), then either the orthonormalising
//                   factor W = V D^{-1/2} (numerical range of the panel) or
//                   the truncated inverse square root V_k D_k^{-1/2} V_k^T
//   lm_pad_kernel   the caller's Gaussian test matrix into zero-padded
//                   per-class buffers
//
// Working from Gram matrices in fp64 (the fp32 panels' products are exact in
// fp64) keeps the orthonormalisation rank-revealing: a direction whose
// eigenvalue falls under the cutoff is dropped instead of amplified.  Every
// reduction has a fixed order, so results are bitwise reproducible.
#include "muon_kernels.h"

#include <math.h>

namespace muon {
namespace {

__device__ __forceinline__ int class_of(const int32_t (&begin)[kLmMaxClasses], int b) {
  int ci = 0;
#pragma unroll
  for (int i = 1; i < kLmMaxClasses; ++i) ci += (begin[i] <= b) ? 1 : 0;
  return ci;
}

// ------------------------------------------------------------------ Gram
constexpr int kGramRows = 64;   // panel rows staged in LDS at a time

__global__ __launch_bounds__(256) void lm_gram_kernel(LmGramArgs args) {
  __shared__ float rows[kGramRows][kLmKP + 1];
  const int b = (int)blockIdx.x;
  const int ci = class_of(args.block_begin, b);
  const LmGramClass &cl = args.cls[ci];
  const int local = b - args.block_begin[ci];
  const int mat = local / cl.nchunks, chunk = local - mat * cl.nchunks;
  const float *P = cl.panel + (int64_t)mat * cl.stride;
  const int n = args.n, nn = n * n;
  const int r0 = chunk * kLmChunk, r1 = min(cl.rows, r0 + kLmChunk);
  constexpr int kPer = kLmSlot / 256;   // entries per thread at n = kLmKP
  double acc[kPer];
  int ei[kPer], ej[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = threadIdx.x + 256 * m;
    acc[m] = 0.0;
    ei[m] = e < nn ? e / n : 0;
    ej[m] = e < nn ? e - (e / n) * n : 0;
  }
  for (int base = r0; base < r1; base += kGramRows) {
    const int cnt = min(kGramRows, r1 - base);
    __syncthreads();
    // stage cnt rows of kLmKP floats: 16-byte loads, 16 per row
    for (int q = threadIdx.x; q < kGramRows * (kLmKP / 4); q += 256) {
      const int r = q / (kLmKP / 4), c4 = q - r * (kLmKP / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < cnt) v = *(const float4 *)(P + (int64_t)(base + r) * kLmKP + 4 * c4);
      rows[r][4 * c4 + 0] = v.x;
      rows[r][4 * c4 + 1] = v.y;
      rows[r][4 * c4 + 2] = v.z;
      rows[r][4 * c4 + 3] = v.w;
    }
    __syncthreads();
    for (int r = 0; r < cnt; ++r) {
#pragma unroll
      for (int m = 0; m < kPer; ++m)
        if (256 * m < nn)   // uniform: skip entry groups past n x n
          acc[m] = fma((double)rows[r][ei[m]], (double)rows[r][ej[m]], acc[m]);
    }
  }
  double *out = args.partials + (int64_t)(cl.part_base + mat * cl.nchunks + chunk) * kLmSlot;
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = threadIdx.x + 256 * m;
    if (e < nn) out[ei[m] * kLmKP + ej[m]] = acc[m];
  }
}

// ------------------------------------------------------------------ eigen
constexpr int kMaxSweeps = 30;

// Pair k of round r of the circle method over N (even) indices: every pair
// of [0, N) meets exactly once in N - 1 rounds, and the N / 2 pairs of a
// round are disjoint.
__device__ __forceinline__ void round_pair(int N, int r, int k, int &p, int &q) {
  const int m = N - 1;
  int a = (r + k) % m;
  int c = (k == 0) ? m : (r - k + m) % m;
  p = min(a, c);
  q = max(a, c);
}

__global__ __launch_bounds__(256) void lm_eig_kernel(LmEigArgs args) {
  __shared__ double a[kLmKP][kLmKP + 1];
  __shared__ double v[kLmKP][kLmKP + 1];
  __shared__ double rot_c[kLmKP / 2], rot_s[kLmKP / 2];
  __shared__ int rot_p[kLmKP / 2], rot_q[kLmKP / 2];
  __shared__ int order[kLmKP];
  __shared__ int rotated;
  const int b = (int)blockIdx.x;
  const int ci = class_of(args.begin, b);
  const LmEigClass &cl = args.cls[ci];
  const int mat = b - args.begin[ci];
  const int n = args.n;
  const int N = (n + 1) & ~1;   // even size for the pair schedule (a zero row/column pads an odd n)
  const int tid = threadIdx.x;

  // fixed-order sum of the matrix's partials; V = I
  const double *part = args.partials + (int64_t)(cl.part_base + mat * cl.nchunks) * kLmSlot;
  for (int e = tid; e < N * N; e += 256) {
    const int i = e / N, j = e - (e / N) * N;
    double s = 0.0;
    if (i < n && j < n)
      for (int c = 0; c < cl.nchunks; ++c) s += part[(int64_t)c * kLmSlot + i * kLmKP + j];
    a[i][j] = s;
    v[i][j] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();

  // cyclic Jacobi (Golub & Van Loan, "Matrix Computations", section 8.5):
  // each rotation J in rows / columns (p, q) with J_pp = J_qq = c,
  // J_pq = s, J_qp = -s zeroes a_pq in J^T A J; V <- V J.  A pair rotates
  // only while |a_pq| > 1e-15 sqrt(|a_pp a_qq|) (the relative test that
  // keeps small eigenvalues accurate); a sweep without any rotation ends the
  // iteration (at most kMaxSweeps; NaN input runs them all).
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    if (tid == 0) rotated = 0;
    __syncthreads();
    for (int r = 0; r < N - 1; ++r) {
      if (tid < N / 2) {
        int p, q;
        round_pair(N, r, tid, p, q);
        const double apq = a[p][q];
        double c = 1.0, s = 0.0;
        if (fabs(apq) > 1e-15 * sqrt(fabs(a[p][p] * a[q][q]))) {
          const double tau = (a[q][q] - a[p][p]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
          rotated = 1;
        }
        rot_p[tid] = p;
        rot_q[tid] = q;
        rot_c[tid] = c;
        rot_s[tid] = s;
      }
      __syncthreads();
      // A <- J^T A (rows p and q)
      for (int it = tid; it < (N / 2) * N; it += 256) {
        const int k = it / N, j = it - (it / N) * N;
        const int p = rot_p[k], q = rot_q[k];
        const double c = rot_c[k], s = rot_s[k];
        const double x = a[p][j], y = a[q][j];
        a[p][j] = c * x - s * y;
        a[q][j] = s * x + c * y;
      }
      __syncthreads();
      // A <- A J and V <- V J (columns p and q)
      for (int it = tid; it < (N / 2) * N; it += 256) {
        const int k = it / N, i = it - (it / N) * N;
        const int p = rot_p[k], q = rot_q[k];
        const double c = rot_c[k], s = rot_s[k];
        const double x = a[i][p], y = a[i][q];
        a[i][p] = c * x - s * y;
        a[i][q] = s * x + c * y;
        const double vx = v[i][p], vy = v[i][q];
        v[i][p] = c * vx - s * vy;
        v[i][q] = s * vx + c * vy;
      }
      __syncthreads();
    }
    const int done = (rotated == 0);   // read by every thread after the barrier above
    __syncthreads();                   // ... before thread 0 clears it again
    if (done) break;
  }

  // eigenvalues in descending order (ties by index)
  if (tid < N) {
    const double d = a[tid][tid];
    int rank = 0;
    for (int j = 0; j < N; ++j) {
      const double dj = a[j][j];
      rank += (dj > d || (dj == d && j < tid)) ? 1 : 0;
    }
    order[rank] = tid;
  }
  __syncthreads();
  const double dmax = a[order[0]][order[0]];
  const double floor_d = args.cutoff * dmax;
  float *out = cl.out + (int64_t)mat * cl.out_stride;
  if (args.mode == kLmOrth) {
    // out[j][i] = W[i][j], W[:, j] = v[:, order[j]] / sqrt(d_order[j]) for kept j
    for (int e = tid; e < kLmSlot; e += 256) {
      const int j = e / kLmKP, i = e - (e / kLmKP) * kLmKP;
      float w = 0.f;
      if (j < N && i < N) {
        const int o = order[j];
        const double d = a[o][o];
        if (dmax > 0.0 && d > floor_d) w = (float)(v[i][o] / sqrt(d));
      }
      out[e] = w;
    }
  } else {
    const int keep = min(args.rank, N);
    for (int e = tid; e < kLmSlot; e += 256) {
      const int i = e / kLmKP, j = e - (e / kLmKP) * kLmKP;
      double t = 0.0;
      if (i < N && j < N && dmax > 0.0) {
        for (int m = 0; m < keep; ++m) {
          const int o = order[m];
          const double d = a[o][o];
          if (d > floor_d) t += v[i][o] * v[j][o] / sqrt(d);
        }
      }
      out[e] = (float)t;
    }
  }
}

// ------------------------------------------------------------------ pad
__global__ __launch_bounds__(256) void lm_pad_kernel(LmPadArgs args) {
  const int b = (int)blockIdx.x;
  const int ci = class_of(args.begin, b);
  const LmPadClass &cl = args.cls[ci];
  const int64_t base = (int64_t)(b - args.begin[ci]) * kLmPadElems;
  const int64_t total = (int64_t)kLmKP * cl.lp;
  for (int m = threadIdx.x; m < kLmPadElems; m += 256) {
    const int64_t e = base + m;
    if (e >= total) break;
    const int j = (int)(e / cl.lp);
    const int t = (int)(e - (int64_t)j * cl.lp);
    cl.dst[e] = (j < args.kp && t < cl.l) ? args.src[(int64_t)j * args.ld + t] : 0.f;
  }
}

}  // namespace

hipError_t launch_lm_gram(const LmGramArgs &args, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_gram_kernel, dim3(blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

hipError_t launch_lm_eig(const LmEigArgs &args, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_eig_kernel, dim3(blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

hipError_t launch_lm_pad(const LmPadArgs &args, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_pad_kernel, dim3(blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

}  // namespace muon
