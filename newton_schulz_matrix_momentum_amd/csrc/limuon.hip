// Small-matrix stages of the LiMuon orthogonaliser for gfx950.
//
// LiMuon (digest "LiMuon: Light and Fast Muon Optimizer for Large Models",
// section "Метод") replaces Newton-Schulz by a randomized SVD of the
// momentum.  Its products against (k + p)-wide panels (the sketch X Omega,
// the power iterations X^T Q and X Z, the projection X^T Q, and the
// orthonormalising factors) and the small-matrix stages are implemented
// here; the final product (the weight update) runs in the grouped GEMM:
//
//   lm_thin_kernel  the products against a (k + p)-wide panel, with the
//                   fp64 Gram partials of the result fused in
//   lm_eig_kernel   one block per matrix: fixed-order sum of its partials,
//                   then either the orthonormalising factor of the panel
//                   (pivoted Cholesky of the Gram matrix in fp64, stopped at
//                   the panel's numerical rank, and the inverse of its
//                   triangular factor) or, from a cyclic Jacobi
//                   eigen-decomposition in fp64 (parallel round-robin pair
//                   order), the truncated inverse square root
//                   V_k D_k^{-1/2} V_k^T
//   lm_pad_kernel   the caller's Gaussian test matrix into zero-padded
//                   per-class buffers
//
// Working from Gram matrices in fp64 (the fp32 panels' products are exact in
// fp64) keeps the orthonormalisation rank-revealing: a direction whose
// pivot or eigenvalue falls under the cutoff is dropped instead of
// amplified.  Every reduction has a fixed order, so results are bitwise
// reproducible.
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

// s_waitcnt vmcnt(n), leaving expcnt and lgkmcnt alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]); n >= 32 waits for everything.
#define LM_VMCNT(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define LM_VMCASE(n) case n: __builtin_amdgcn_s_waitcnt(LM_VMCNT(n)); break;
__device__ __forceinline__ void lm_waitcnt_vm(int n) {
  switch (n) {
    LM_VMCASE(1) LM_VMCASE(2) LM_VMCASE(3) LM_VMCASE(4) LM_VMCASE(5) LM_VMCASE(6) LM_VMCASE(7) LM_VMCASE(8)
    LM_VMCASE(9) LM_VMCASE(10) LM_VMCASE(11) LM_VMCASE(12) LM_VMCASE(13) LM_VMCASE(14) LM_VMCASE(15)
    LM_VMCASE(16) LM_VMCASE(17) LM_VMCASE(18) LM_VMCASE(19) LM_VMCASE(20) LM_VMCASE(21) LM_VMCASE(22)
    LM_VMCASE(23) LM_VMCASE(24) LM_VMCASE(25) LM_VMCASE(26) LM_VMCASE(27) LM_VMCASE(28) LM_VMCASE(29)
    LM_VMCASE(30) LM_VMCASE(31)
    default: __builtin_amdgcn_s_waitcnt(LM_VMCNT(0)); break;
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ thin products
// C (64 rows of one matrix x NB) = A B^T, fp32.  The products of the
// randomized SVD read the whole of X (or X^T) against a narrow panel, so
// they are bound by streaming X: operands move global -> LDS by DMA in
// stages of 32 k (one 128-byte line per row: the block's 64 rows of A, then
// NB rows of B) through a ring of kThinRing stages (kThinRing - 1 stages in
// flight).  16-byte chunk c of row r is stored at chunk c ^ (r & 7).  Wave w
// computes rows 16 w .. 16 w + 15 against all NB columns with
// v_mfma_f32_16x16x4_f32 (a lane's 16-byte fragment holds 4 consecutive k,
// consumed by four MFMAs).  The epilogue writes C, optionally C^T, and
// optionally the fp64 Gram matrix of the block's rows of C (the next
// orthonormalisation's input), so no Gram pass re-reads the panel.
// A stage's work is a few LDS reads and 16 MFMAs per wave, so a block is
// bound by its per-stage latency (the wait, the barrier, the reads): many
// small blocks per CU stream faster than a few deep rings.  Two stages and
// six blocks per CU at a 32-wide panel (five at 64): 4.26 against 4.65 ms
// per LiMuon step of the Llama-shaped set with six stages and two blocks,
// 4.31 with three stages and four blocks.
#ifndef MUON_THIN_RING
#define MUON_THIN_RING 2
#endif
#ifndef MUON_THIN_BLOCKS
#define MUON_THIN_BLOCKS 6
#endif
constexpr int kThinRing = MUON_THIN_RING;
constexpr int kThinBlocks = MUON_THIN_BLOCKS;   // blocks per CU at a 32-wide panel (one fewer at 64)

template <int NB>
__global__ __launch_bounds__(256, NB == 32 ? kThinBlocks : (kThinBlocks > 1 ? kThinBlocks - 1 : 1)) void lm_thin_kernel(LmThinArgs args) {
  constexpr int ROWS = kThinRows + NB;      // rows per stage: A then B
  constexpr int CHUNKS = ROWS / 8;          // 1 KB DMA instructions per stage
  constexpr int STAGE = ROWS * 128;         // bytes per stage
  constexpr int FN = NB / 16;
  static_assert(kThinRing * STAGE * (NB == 32 ? kThinBlocks : (kThinBlocks > 1 ? kThinBlocks - 1 : 1)) <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[kThinRing * STAGE];
  const int b = (int)blockIdx.x;
  const int ci = class_of(args.begin, b);
  const LmThinClass &cl = args.cls[ci];
  const int local = b - args.begin[ci];
  const int mat = local / cl.tiles, tile = local - mat * cl.tiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char *A = (const char *)(cl.a + (int64_t)mat * cl.sa + (int64_t)tile * kThinRows * cl.lda);
  const char *B = (const char *)(cl.b + (int64_t)mat * cl.sb);
  const int64_t lda_b = (int64_t)cl.lda * 4, ldb_b = (int64_t)cl.ldb * 4;
  const int nk = cl.K / 32;
  const int my_chunks = (CHUNKS - wave + 3) / 4;   // DMA instructions of this wave per stage
  auto dma = [&](int kb) {
    char *dst = lds + (kb % kThinRing) * STAGE;
    for (int c = wave; c < CHUNKS; c += 4) {
      const int row = 8 * c + (lane >> 3);
      const int lch = (lane & 7) ^ (lane >> 3);          // logical chunk held at physical chunk lane & 7
      const char *src = row < kThinRows ? A + (int64_t)row * lda_b : B + (int64_t)(row - kThinRows) * ldb_b;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(src + (int64_t)kb * 128 + lch * 16),
                                       (void __attribute__((address_space(3))) *)(dst + c * 1024), 16, 0, 0);
    }
  };
  f32x4 acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int pre = min(kThinRing - 1, nk);
  for (int kb = 0; kb < pre; ++kb) dma(kb);
  const int fr = lane & 15;
  const int arow = 16 * wave + fr;
  for (int kb = 0; kb < nk; ++kb) {
    const int issued = min(nk, kb + kThinRing - 1);
    lm_waitcnt_vm((issued - kb - 1) * my_chunks);
    __syncthreads();   // every wave's part of stage kb has landed; stage kb - 1's slot is free
    if (kb + kThinRing - 1 < nk) dma(kb + kThinRing - 1);
    const char *slot = lds + (kb % kThinRing) * STAGE;
    // every fragment of the stage first, then the MFMAs
    u32x4 a[2], bv[2][FN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int lch = 4 * ks + (lane >> 4);
      a[ks] = *(const u32x4 *)(slot + arow * 128 + ((lch ^ (arow & 7)) * 16));
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int brow = kThinRows + 16 * j + fr;
        bv[ks][j] = *(const u32x4 *)(slot + brow * 128 + ((lch ^ (brow & 7)) * 16));
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[ks].x), __uint_as_float(bv[ks][j].x), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[ks].y), __uint_as_float(bv[ks][j].y), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[ks].z), __uint_as_float(bv[ks][j].z), acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[ks].w), __uint_as_float(bv[ks][j].w), acc[j], 0, 0, 0);
      }
  }
  // epilogue: lane holds C[16 w + 4 (lane / 16) + r][16 j + lane % 16]
  const int r0 = tile * kThinRows + 16 * wave + 4 * (lane >> 4);
  if (cl.c) {
    float *C = cl.c + (int64_t)mat * cl.sc;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) C[(int64_t)(r0 + r) * cl.ldc + 16 * j + fr] = acc[j][r];
  }
  if (cl.c2) {
    float *C2 = cl.c2 + (int64_t)mat * cl.sc2;
#pragma unroll
    for (int j = 0; j < FN; ++j) *(f32x4 *)(C2 + (int64_t)(16 * j + fr) * cl.ldc2 + r0) = acc[j];
  }
  if (cl.part_base < 0) return;   // uniform per class
  __syncthreads();                // every wave is done with the ring
  float *cb = (float *)lds;       // 64 x (NB + 1) floats
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) cb[(16 * wave + 4 * (lane >> 4) + r) * (NB + 1) + 16 * j + fr] = acc[j][r];
  __syncthreads();
  const int n = args.n, nn = n * n;
  double *out = args.partials + (int64_t)(cl.part_base + mat * cl.tiles + tile) * nn;
  for (int e = threadIdx.x; e < nn; e += 256) {
    const int i = e / n, j = e - (e / n) * n;
    double sum = 0.0;
    for (int r = 0; r < kThinRows; ++r) sum = fma((double)cb[r * (NB + 1) + i], (double)cb[r * (NB + 1) + j], sum);
    out[e] = sum;
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

// Orthonormalising factor from the Gram matrix G = P^T P of an n-column
// panel P (Golub & Van Loan, "Matrix Computations", section 4.2, Cholesky
// with symmetric pivoting): at step j the remaining index with the largest
// Schur-complement diagonal is the pivot p_j, L[:, j] = S[:, p_j] / sqrt(S_pp)
// and S <- S - L[:, j] L[:, j]^T; the factorisation stops when that diagonal
// falls to cutoff * max(diag G) (the panel's numerical rank r).  With the
// lower-triangular C[a][c] = L[p_a][c] (a, c < r), the selected columns
// satisfy P_sel^T P_sel = C C^T, so P W with W[p_a][m] = (C^-1)[m][a] has r
// orthonormal columns spanning P's range (the other columns of W are 0).
// Writes W^T (out[m][i] = W[i][m]).  Runs on the block's first n threads
// per step; s holds G on entry.
__device__ void lm_orth_cholesky(int n, double cutoff, double (*S)[kLmKP + 1], double (*L)[kLmKP + 1],
                                 double (*X)[kLmKP + 1], int *piv, int *chosen, int *ctl, double *tau_s,
                                 float *out) {
  const int tid = threadIdx.x, NT = (int)blockDim.x;
  for (int i = tid; i < kLmKP; i += NT) chosen[i] = 0;
  if (tid == 0) {
    double dmax = 0.0;
    bool bad = false;
    for (int i = 0; i < n; ++i) {
      const double d = S[i][i];
      bad = bad || !(d >= 0.0) || isinf(d);
      dmax = fmax(dmax, d);
    }
    ctl[1] = bad ? 1 : 0;              // non-finite (or negative) diagonal: NaN result
    *tau_s = cutoff * dmax;
  }
  __syncthreads();
  const double tau = *tau_s;
  int r = 0;
  if (ctl[1] == 0) {
    for (int j = 0; j < n; ++j) {
      if (tid < 64) {
        // pivot: the unchosen index with the largest diagonal (lowest index on ties)
        double best = (tid < n && !chosen[tid]) ? S[tid][tid] : -1.0;
        int p = (tid < n && !chosen[tid]) ? tid : kLmKP;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const double ob = __shfl_xor(best, off);
          const int op = __shfl_xor(p, off);
          if (ob > best || (ob == best && op < p)) { best = ob; p = op; }
        }
        if (tid == 0) {
          const bool go = p < n && best > tau && best > 0.0;
          piv[j] = go ? p : -1;
          if (go) chosen[p] = 1;
        }
      }
      __syncthreads();
      const int p = piv[j];
      if (p < 0) break;                  // uniform: every thread read the same piv[j]
      // L[:, j] = S[:, p] / sqrt(S_pp) and S <- S - L[:, j] L[:, j]^T on the
      // unchosen indices, in one pass: column p is not updated (p is chosen)
      const double inv = 1.0 / sqrt(S[p][p]);
      for (int e = tid; e < n * n; e += NT) {
        const int i = e / n, k = e - (e / n) * n;
        if (k == p) L[i][j] = (i == p) ? S[p][p] * inv : (chosen[i] ? 0.0 : S[i][p] * inv);
        else if (!chosen[i] && !chosen[k]) S[i][k] -= (S[i][p] * inv) * (S[k][p] * inv);
      }
      __syncthreads();
      r = j + 1;
    }
  }
  // X = C^-1 (lower triangular), column b by thread b: forward substitution
  if (tid < r) {
    const int b = tid;
    for (int a = 0; a < b; ++a) X[a][b] = 0.0;
    for (int a = b; a < r; ++a) {
      const double *Ca = L[piv[a]];
      double t = (a == b) ? 1.0 : 0.0;
      for (int c = b; c < a; ++c) t -= Ca[c] * X[c][b];
      X[a][b] = t / Ca[a];
    }
  }
  __syncthreads();
  // W^T staged in S (no longer needed): row m of W^T holds column m of W
  for (int e = tid; e < kLmSlot; e += NT) {
    const int m = e / kLmKP, i = e - (e / kLmKP) * kLmKP;
    S[m][i] = ctl[1] ? __builtin_nan("") : 0.0;
  }
  __syncthreads();
  for (int e = tid; e < r * r; e += NT) {
    const int m = e / r, a = e - (e / r) * r;
    if (a <= m) S[m][piv[a]] = X[m][a];
  }
  __syncthreads();
  for (int e = tid; e < kLmSlot; e += NT) {
    const int m = e / kLmKP, i = e - (e / kLmKP) * kLmKP;
    out[e] = (float)S[m][i];
  }
}

__global__ __launch_bounds__(256) void lm_eig_kernel(LmEigArgs args) {
  __shared__ double a[2][kLmKP][kLmKP + 1];   // double-buffered: each round reads one, writes the other
  __shared__ double v[kLmKP][kLmKP + 1];
  __shared__ double rot_c[kLmKP / 2], rot_s[kLmKP / 2];
  __shared__ int rot_p[kLmKP / 2], rot_q[kLmKP / 2];
  __shared__ int order[kLmKP];
  __shared__ int chosen[kLmKP];
  __shared__ int ctl[2];
  __shared__ double tau_s;
  __shared__ int rotated;
  const int b = (int)blockIdx.x;
  const int ci = class_of(args.begin, b);
  const LmEigClass &cl = args.cls[ci];
  const int mat = b - args.begin[ci];
  const int n = args.n;
  const int N = (n + 1) & ~1;   // even size for the pair schedule (a zero row/column pads an odd n)
  const int H = N / 2;          // pairs per round
  const int tid = threadIdx.x;
  const int NT = (int)blockDim.x;

  // fixed-order sum of the matrix's partials; V = I
  const int nn = n * n;
  const double *part = args.partials + (int64_t)(cl.part_base + mat * cl.nchunks) * nn;
  for (int e = tid; e < N * N; e += NT) {
    const int i = e / N, j = e - (e / N) * N;
    double s = 0.0;
    if (i < n && j < n) {
      // partials in chunk order; 8 loads in flight before their adds
      const double *pe = part + i * n + j;
      int c = 0;
      for (; c + 8 <= cl.nchunks; c += 8) {
        double x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = pe[(int64_t)(c + u) * nn];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += x[u];
      }
      for (; c < cl.nchunks; ++c) s += pe[(int64_t)c * nn];
    }
    a[0][i][j] = s;
    v[i][j] = (i == j) ? 1.0 : 0.0;
  }
  __syncthreads();
  if (args.mode == kLmOrth) {
    lm_orth_cholesky(n, args.cutoff, a[0], a[1], v, order, chosen, ctl, &tau_s,
                     cl.out + (int64_t)mat * cl.out_stride);
    return;
  }

  // cyclic Jacobi (Golub & Van Loan, "Matrix Computations", section 8.5):
  // a rotation J in rows / columns (p, q) with J_pp = J_qq = c, J_pq = s,
  // J_qp = -s zeroes a_pq in J^T A J.  A round applies N / 2 disjoint
  // rotations at once: each 2 x 2 block of rows (p_k, q_k) and columns
  // (p_m, q_m) becomes J_k^T A_km J_m, read from one buffer and written to
  // the other; V <- V J column pair by column pair.  A pair rotates only
  // while |a_pq| > 1e-15 sqrt(|a_pp a_qq|) (the relative test that keeps
  // small eigenvalues accurate); a sweep without any rotation ends the
  // iteration (at most kMaxSweeps; NaN input runs them all).
  int cur = 0;
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    if (tid == 0) rotated = 0;
    __syncthreads();
    for (int r = 0; r < N - 1; ++r) {
      for (int k = tid; k < H; k += NT) {
        int p, q;
        round_pair(N, r, k, p, q);
        const double apq = a[cur][p][q];
        double c = 1.0, s = 0.0;
        if (fabs(apq) > 1e-15 * sqrt(fabs(a[cur][p][p] * a[cur][q][q]))) {
          const double tau = (a[cur][q][q] - a[cur][p][p]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
          rotated = 1;
        }
        rot_p[k] = p;
        rot_q[k] = q;
        rot_c[k] = c;
        rot_s[k] = s;
      }
      __syncthreads();
      const int nxt = cur ^ 1;
      for (int it = tid; it < H * H + H * N; it += NT) {
        if (it < H * H) {
          const int k = it / H, m = it - (it / H) * H;
          const int p = rot_p[k], q = rot_q[k], pm = rot_p[m], qm = rot_q[m];
          const double ck = rot_c[k], sk = rot_s[k], cm = rot_c[m], sm = rot_s[m];
          const double x00 = a[cur][p][pm], x01 = a[cur][p][qm], x10 = a[cur][q][pm], x11 = a[cur][q][qm];
          // rows: J_k^T (first row c x - s y, second s x + c y)
          const double y00 = ck * x00 - sk * x10, y01 = ck * x01 - sk * x11;
          const double y10 = sk * x00 + ck * x10, y11 = sk * x01 + ck * x11;
          // columns: J_m
          a[nxt][p][pm] = cm * y00 - sm * y01;
          a[nxt][p][qm] = sm * y00 + cm * y01;
          a[nxt][q][pm] = cm * y10 - sm * y11;
          a[nxt][q][qm] = sm * y10 + cm * y11;
        } else {
          const int u = it - H * H;
          const int k = u / N, i = u - (u / N) * N;
          const int p = rot_p[k], q = rot_q[k];
          const double c = rot_c[k], s = rot_s[k];
          const double vx = v[i][p], vy = v[i][q];
          v[i][p] = c * vx - s * vy;
          v[i][q] = s * vx + c * vy;
        }
      }
      __syncthreads();
      cur = nxt;
    }
    const int done = (rotated == 0);   // read by every thread after the barrier above
    __syncthreads();                   // ... before thread 0 clears it again
    if (done) break;
  }

  // eigenvalues in descending order (ties by index)
  for (int i = tid; i < N; i += NT) {
    const double d = a[cur][i][i];
    int rank = 0;
    for (int j = 0; j < N; ++j) {
      const double dj = a[cur][j][j];
      rank += (dj > d || (dj == d && j < i)) ? 1 : 0;
    }
    order[rank] = i;
  }
  __syncthreads();
  const double dmax = a[cur][order[0]][order[0]];
  const double floor_d = args.cutoff * dmax;
  float *out = cl.out + (int64_t)mat * cl.out_stride;
  // T = U U^T with U[:, m] = v[:, order[m]] / d^(1/4) over the kept m
  // (reusing the other A buffer for U)
  const int keep = min(args.rank, N);
  double (*U)[kLmKP + 1] = a[cur ^ 1];
  for (int e = tid; e < N * keep; e += NT) {
    const int i = e / keep, m = e - (e / keep) * keep;
    const int o = order[m];
    const double d = a[cur][o][o];
    U[i][m] = (dmax > 0.0 && d > floor_d) ? v[i][o] / sqrt(sqrt(d)) : 0.0;
  }
  __syncthreads();
  for (int e = tid; e < kLmSlot; e += NT) {
    const int i = e / kLmKP, j = e - (e / kLmKP) * kLmKP;
    double t = 0.0;
    if (i < N && j < N)
      for (int m = 0; m < keep; ++m) t += U[i][m] * U[j][m];
    out[e] = (float)t;
  }
}

// ------------------------------------------------------------------ final
// W <- W - lr (gamma O + wd W) with O = P Z^T: a wide W (rows = s) takes
// W[r][c] = sum_m P[r][m] Z[c][m], a tall one W[r][c] = sum_m Z[r][m] P[c][m].
// The tile's 64 U rows and 64 V rows (kp columns each, rows padded to kp + 1
// floats: distinct banks for the 16 V rows a wave reads) are staged in LDS;
// thread t owns columns c0 + 4 (t % 16) .. + 3 of rows r0 + t / 16 + 16 q,
// q = 0..3, so every W access is a 16-byte vector along a row.  O is an
// fp32 sum over m in increasing order.
__global__ __launch_bounds__(256) void lm_final_kernel(LmFinalArgs args) {
  extern __shared__ float lm_final_smem[];   // U then V rows, kp + 1 floats each
  const int ld = args.kp + 1;
  float *su = lm_final_smem, *sv = lm_final_smem + kLmFinalTile * ld;
  const int b = (int)blockIdx.x;
  const int ci = class_of(args.begin, b);
  const LmFinalClass &cl = args.cls[ci];
  const int local = b - args.begin[ci];
  const int mat = local / cl.tiles, t = local - mat * cl.tiles;
  const FinalDesc fd = args.desc[cl.desc_base + mat];
  const int tcn = (fd.cols + kLmFinalTile - 1) / kLmFinalTile;
  const int r0 = (t / tcn) * kLmFinalTile, c0 = (t - (t / tcn) * tcn) * kLmFinalTile;
  const float *P = cl.p + (int64_t)mat * cl.sp, *Z = cl.z + (int64_t)mat * cl.sz;
  const float *U = fd.wide ? P : Z, *V = fd.wide ? Z : P;
  const int kp = args.kp;
  for (int e = threadIdx.x; e < kLmFinalTile * kp; e += 256) {
    const int r = e / kp, m = e - (e / kp) * kp;
    su[r * ld + m] = U[(int64_t)(r0 + r) * kLmKP + m];
    sv[r * ld + m] = V[(int64_t)(c0 + r) * kLmKP + m];
  }
  __syncthreads();
  const int cq = threadIdx.x & 15, rr = threadIdx.x >> 4;
  float o[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[q][e] = 0.f;
  for (int m = 0; m < kp; ++m) {
    float u[4], v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) u[q] = su[(rr + 16 * q) * ld + m];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = sv[(4 * cq + e) * ld + m];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[q][e] = fmaf(u[q], v[e], o[q][e]);
  }
  const float lr = args.lr, wd = args.wd, gm = fd.gamma;
  const int c = c0 + 4 * cq;
  const bool vec = (fd.cols & 3) == 0 && ((((uintptr_t)fd.weight) | ((uintptr_t)fd.ortho_out)) & 15) == 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + rr + 16 * q;
    if (r >= fd.rows) continue;
    float *w = fd.weight + (int64_t)r * fd.cols;
    float *oo = fd.ortho_out ? fd.ortho_out + (int64_t)r * fd.cols : nullptr;
    if (vec && c + 4 <= fd.cols) {
      float4 x = *(const float4 *)(w + c);
      x.x = x.x - lr * (gm * o[q][0] + wd * x.x);
      x.y = x.y - lr * (gm * o[q][1] + wd * x.y);
      x.z = x.z - lr * (gm * o[q][2] + wd * x.z);
      x.w = x.w - lr * (gm * o[q][3] + wd * x.w);
      *(float4 *)(w + c) = x;
      if (oo) *(float4 *)(oo + c) = make_float4(o[q][0], o[q][1], o[q][2], o[q][3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c + e < fd.cols) {
          const float x = w[c + e];
          w[c + e] = x - lr * (gm * o[q][e] + wd * x);
          if (oo) oo[c + e] = o[q][e];
        }
      }
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

hipError_t launch_lm_thin(const LmThinArgs &args, int nb, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (nb == 32) hipLaunchKernelGGL(lm_thin_kernel<32>, dim3(blocks), dim3(256), 0, s, args);
  else if (nb == 64) hipLaunchKernelGGL(lm_thin_kernel<64>, dim3(blocks), dim3(256), 0, s, args);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lm_eig(const LmEigArgs &args, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_eig_kernel, dim3(blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

hipError_t launch_lm_final(const LmFinalArgs &args, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const size_t smem = (size_t)2 * kLmFinalTile * (args.kp + 1) * sizeof(float);
  hipLaunchKernelGGL(lm_final_kernel, dim3(blocks), dim3(256), smem, s, args);
  return hipGetLastError();
}

hipError_t launch_lm_pad(const LmPadArgs &args, int blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_pad_kernel, dim3(blocks), dim3(256), 0, s, args);
  return hipGetLastError();
}

}  // namespace muon
