// Grouped MFMA matrix products for the Newton-Schulz iteration on gfx950.
//
// Every product of the iteration is written as C = A B^T with both operands
// stored row-major along k ("NT"): the Gram X X^T, the square A A of a
// symmetric matrix (A A = A A^T), and the update X^T B with B symmetric
// (Gram Newton-Schulz post: the Gram matrix and its polynomials are
// symmetric).  Both orientations of the iterate are kept in HBM, so no
// operand is ever transposed on the fly.
//
// One launch covers every matrix of a step that shares a tile shape ("grouped
// launch"): blockIdx selects (class, matrix, tile) from the kernel-argument
// table.  Symmetric results are computed on upper-triangular tiles only and
// mirrored (Gram Newton-Schulz post: half the entries suffice for products
// of symmetric matrices).  The epilogue fuses the polynomial step:
//   out = alpha * acc + beta * Cin + diag * [row == col < diag_limit]
// which covers A = X X^T, B = b A + c A^2, P = a I + b R + c R^2 and
// X' = a X + B X, plus the storage scale of fp16 buffers.
//
// Operands: fp16 / bf16 use v_mfma_f32_16x16x32_{f16,bf16}; fp32 uses
// v_mfma_f32_16x16x4_f32.  Accumulation is always fp32.  Each 64-lane
// wavefront owns a (BM/2) x (BN/2) sub-tile; k advances 128 bytes per LDS
// stage, double-buffered, with one barrier per stage.  LDS rows carry 16 bytes
// of padding so the 16-byte fragment reads of 8 consecutive rows fall into
// distinct banks.  All workspace buffers are zero-padded to tile multiples, so
// the main loop has no bounds checks.
#include "muon_kernels.h"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
  static __device__ __forceinline__ void run(const u32x4 &a, const u32x4 &b, f32x4 &c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<_Float16> {
  static __device__ __forceinline__ void run(const u32x4 &a, const u32x4 &b, f32x4 &c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  // A lane's 16-byte fragment holds 4 consecutive k; four 16x16x4 MFMAs
  // consume them (MFMA q pairs element q of A with element q of B, so the
  // k ordering inside the fragment is the same on both sides).
  static __device__ __forceinline__ void run(const u32x4 &a, const u32x4 &b, f32x4 &c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float load(const void *p, int64_t i) { return ((const float *)p)[i]; }
  static __device__ __forceinline__ void store(void *p, int64_t i, float v) { ((float *)p)[i] = v; }
  static __device__ __forceinline__ void store4(void *p, int64_t i, const float v[4]) {
    *(float4 *)((float *)p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <typename H> struct Store16 {
  static __device__ __forceinline__ uint16_t bits(float v) { return __builtin_bit_cast(uint16_t, (H)v); }
  static __device__ __forceinline__ float load(const void *p, int64_t i) {
    return (float)__builtin_bit_cast(H, ((const uint16_t *)p)[i]);
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, float v) { ((uint16_t *)p)[i] = bits(v); }
  static __device__ __forceinline__ void store4(void *p, int64_t i, const float v[4]) {
    uint2 u;
    u.x = (uint32_t)bits(v[0]) | ((uint32_t)bits(v[1]) << 16);
    u.y = (uint32_t)bits(v[2]) | ((uint32_t)bits(v[3]) << 16);
    *(uint2 *)((uint16_t *)p + i) = u;
  }
};
template <> struct Store<__bf16> : Store16<__bf16> {};
template <> struct Store<_Float16> : Store16<_Float16> {};

constexpr int kThreads = 256;
constexpr int kStageBytes = 128;               // k bytes per LDS stage per row
constexpr int kPitch = kStageBytes + 16;       // padded LDS row

template <typename T, int BM, int BN>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(GemmArgs args) {
  constexpr int ES = sizeof(T);
  constexpr int KS = kStageBytes / ES;         // k elements per stage
  constexpr int WM = BM / 2, WN = BN / 2;      // 2 x 2 waves
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_LD = BM * (kStageBytes / 16) / kThreads;  // 16-byte chunks per thread
  constexpr int B_LD = BN * (kStageBytes / 16) / kThreads;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the block");
  __shared__ __attribute__((aligned(16))) char lds[2][(BM + BN) * kPitch];

  // ---- locate (class, matrix, tile); uniform across the block
  const int tile = blockIdx.x;
  int ci = 0;
#pragma unroll 1
  for (int i = 1; i < args.nclass; ++i)
    if (tile >= args.cls[i].tile_begin) ci = i;
  const GemmClass &cl = args.cls[ci];
  const int local = tile - cl.tile_begin;
  const int mat = local / cl.tiles_per_mat;
  int t = local - mat * cl.tiles_per_mat;
  int tm, tn;
  if (cl.half) {
    tm = 0;
    int rowlen = cl.tiles_n;
#pragma unroll 1
    while (t >= rowlen) { t -= rowlen; ++tm; --rowlen; }
    tn = tm + t;
  } else {
    tm = t / cl.tiles_n;
    tn = t - tm * cl.tiles_n;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const char *A = (const char *)cl.a + ((int64_t)mat * cl.sa + (int64_t)tm * BM * cl.lda) * ES;
  const char *B = (const char *)cl.b + ((int64_t)mat * cl.sb + (int64_t)tn * BN * cl.ldb) * ES;
  const int64_t lda_b = (int64_t)cl.lda * ES, ldb_b = (int64_t)cl.ldb * ES;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = cl.K / KS;
  if (nk > 0) {
    u32x4 ra[A_LD], rb[B_LD];
    {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int q = tid + kThreads * i;
        ra[i] = *(const u32x4 *)(A + (q >> 3) * lda_b + (int64_t)0 * kStageBytes + (q & 7) * 16);
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int q = tid + kThreads * i;
        rb[i] = *(const u32x4 *)(B + (q >> 3) * ldb_b + (int64_t)0 * kStageBytes + (q & 7) * 16);
      }
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int q = tid + kThreads * i;
        *(u32x4 *)(&lds[0][(q >> 3) * kPitch + (q & 7) * 16]) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int q = tid + kThreads * i;
        *(u32x4 *)(&lds[0][(BM + (q >> 3)) * kPitch + (q & 7) * 16]) = rb[i];
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int kb = 0; kb < nk; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < nk) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int q = tid + kThreads * i;
        ra[i] = *(const u32x4 *)(A + (q >> 3) * lda_b + (int64_t)(kb + 1) * kStageBytes + (q & 7) * 16);
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int q = tid + kThreads * i;
        rb[i] = *(const u32x4 *)(B + (q >> 3) * ldb_b + (int64_t)(kb + 1) * kStageBytes + (q & 7) * 16);
      }
      }
      const char *la = &lds[buf][(wm * WM + (lane & 15)) * kPitch + (lane >> 4) * 16];
      const char *lb = &lds[buf][(BM + wn * WN + (lane & 15)) * kPitch + (lane >> 4) * 16];
#pragma unroll
      for (int ks = 0; ks < kStageBytes / 64; ++ks) {
        u32x4 fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[i] = *(const u32x4 *)(la + i * 16 * kPitch + ks * 64);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = *(const u32x4 *)(lb + j * 16 * kPitch + ks * 64);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) Mma<T>::run(fa[i], fb[j], acc[i][j]);
      }
      if (kb + 1 < nk) {
#pragma unroll
      for (int i = 0; i < A_LD; ++i) {
        const int q = tid + kThreads * i;
        *(u32x4 *)(&lds[buf ^ 1][(q >> 3) * kPitch + (q & 7) * 16]) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int q = tid + kThreads * i;
        *(u32x4 *)(&lds[buf ^ 1][(BM + (q >> 3)) * kPitch + (q & 7) * 16]) = rb[i];
      }
      }
      __syncthreads();
    }
  }

  // ---- epilogue.  MFMA 16x16 output layout: lane holds rows 4*(lane/16)+r,
  // column lane%16, r = 0..3.
  const float alpha = cl.alpha, beta = cl.beta, diag = cl.diag;
  void *C = cl.c ? (void *)((char *)cl.c + (int64_t)mat * cl.sc * ES) : nullptr;
  void *C2 = cl.c2 ? (void *)((char *)cl.c2 + (int64_t)mat * cl.sc2 * ES) : nullptr;
  const void *Cin = cl.cin ? (const void *)((const char *)cl.cin + (int64_t)mat * cl.scin * ES) : nullptr;
  const bool diag_tile = cl.half && tm == tn;
  const int row_base = tm * BM + wm * WM + 4 * (lane >> 4);
  const int col_base = tn * BN + wn * WN + (lane & 15);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r0 = row_base + i * 16;
      const int col = col_base + j * 16;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = alpha * acc[i][j][r];
        if (Cin) v[r] += beta * Store<T>::load(Cin, (int64_t)(r0 + r) * cl.ldcin + col);
        if (diag != 0.0f && r0 + r == col && col < cl.diag_limit) v[r] += diag;
      }
      if (C) {
        if (!cl.half) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Store<T>::store(C, (int64_t)(r0 + r) * cl.ldc + col, v[r]);
        } else if (!diag_tile) {
#pragma unroll
          for (int r = 0; r < 4; ++r) Store<T>::store(C, (int64_t)(r0 + r) * cl.ldc + col, v[r]);
          Store<T>::store4(C, (int64_t)col * cl.ldc + r0, v);   // mirror
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (col >= r0 + r) {
              Store<T>::store(C, (int64_t)(r0 + r) * cl.ldc + col, v[r]);
              Store<T>::store(C, (int64_t)col * cl.ldc + r0 + r, v[r]);
            }
          }
        }
      }
      if (C2) Store<T>::store4(C2, (int64_t)col * cl.ldc2 + r0, v);
    }
  }
}

template <typename T>
hipError_t launch_t(const GemmArgs &args, int tile, hipStream_t s) {
  switch (tile) {
    case 64: hipLaunchKernelGGL((ns_gemm_kernel<T, 64, 64>), dim3(args.total_tiles), dim3(kThreads), 0, s, args); break;
    case 128: hipLaunchKernelGGL((ns_gemm_kernel<T, 128, 128>), dim3(args.total_tiles), dim3(kThreads), 0, s, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &args, int dtype, int tile, hipStream_t s) {
  if (args.total_tiles <= 0) return hipSuccess;
  switch (dtype) {
    case kF32: return launch_t<float>(args, tile, s);
    case kF16: return launch_t<_Float16>(args, tile, s);
    case kBF16: return launch_t<__bf16>(args, tile, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace muon
