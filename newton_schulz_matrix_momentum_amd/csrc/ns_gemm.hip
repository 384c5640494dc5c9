// Grouped MFMA matrix products for the Newton-Schulz iteration on gfx950.
//
// Every product of the iteration is written as C = A B^T with both operands
// stored row-major along k ("NT"): the Gram X X^T, the square A A of a
// symmetric matrix (A A = A A^T), and the update X^T B with B symmetric
// (Gram Newton-Schulz post: the Gram matrix and its polynomials are
// symmetric).  Both orientations of the iterate are kept in HBM, so these
// products never transpose an operand; the fused update of short sides
// reads the iterate in its wide layout through gfx950's transposing LDS
// reads instead, and keeps that one layout.
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
// v_mfma_f32_16x16x4_f32.  Accumulation is always fp32.  16-bit block
// tiles: 64 x 64 (latency-bound small products), 128 x 128 and 256 x 256
// (global -> LDS DMA); fp32 products use register-staged 64 x 64 and
// 128 x 128 tiles; and for direct steps with short sides up to 192, one
// kernel forms the square A A inside the update product
// (ns_poly_update_kernel).  All
// workspace buffers are zero-padded to tile multiples, so the main loops have
// no bounds checks.
#include "muon_kernels.h"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(n), leaving expcnt and lgkmcnt alone.  gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].  n >= 64 waits
// for vmcnt(0) (always safe).
#define MUON_VMCNT(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
#define MUON_VMCASE(n) case n: __builtin_amdgcn_s_waitcnt(MUON_VMCNT(n)); break;
__device__ __forceinline__ void waitcnt_vm(int n) {
  switch (n) {
    MUON_VMCASE(1) MUON_VMCASE(2) MUON_VMCASE(3) MUON_VMCASE(4) MUON_VMCASE(5) MUON_VMCASE(6) MUON_VMCASE(7)
    MUON_VMCASE(8) MUON_VMCASE(9) MUON_VMCASE(10) MUON_VMCASE(11) MUON_VMCASE(12) MUON_VMCASE(13) MUON_VMCASE(14)
    MUON_VMCASE(15) MUON_VMCASE(16) MUON_VMCASE(17) MUON_VMCASE(18) MUON_VMCASE(19) MUON_VMCASE(20) MUON_VMCASE(21)
    MUON_VMCASE(22) MUON_VMCASE(23) MUON_VMCASE(24) MUON_VMCASE(25) MUON_VMCASE(26) MUON_VMCASE(27) MUON_VMCASE(28)
    MUON_VMCASE(29) MUON_VMCASE(30) MUON_VMCASE(31) MUON_VMCASE(32) MUON_VMCASE(33) MUON_VMCASE(34)
    MUON_VMCASE(35) MUON_VMCASE(36) MUON_VMCASE(37) MUON_VMCASE(38) MUON_VMCASE(39) MUON_VMCASE(40) MUON_VMCASE(41)
    MUON_VMCASE(42) MUON_VMCASE(43) MUON_VMCASE(44) MUON_VMCASE(45) MUON_VMCASE(46) MUON_VMCASE(47) MUON_VMCASE(48)
    MUON_VMCASE(49) MUON_VMCASE(50) MUON_VMCASE(51) MUON_VMCASE(52) MUON_VMCASE(53) MUON_VMCASE(54) MUON_VMCASE(55)
    MUON_VMCASE(56) MUON_VMCASE(57) MUON_VMCASE(58) MUON_VMCASE(59) MUON_VMCASE(60) MUON_VMCASE(61) MUON_VMCASE(62)
    MUON_VMCASE(63)
    default: __builtin_amdgcn_s_waitcnt(MUON_VMCNT(0)); break;
  }
}

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


// Compile-time loop: every index is a template constant, so register arrays
// indexed by it are never demoted to scratch memory.
template <int I> struct IntC { static constexpr int value = I; };
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<I + 1, N>(f);
  }
}

struct TileRef {
  int ci, mat, tm, tn;
};

// Tile rows per super-row in the order of a full (non-symmetric) product's
// tiles (4: measured against 1 and 8).
constexpr int kRowGroup = 4;

// Locate (class, matrix, tile) of this workgroup; uniform across the block.
// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2), in
// blockIdx order.  xcd_group == 0: remap so that each XCD walks one
// contiguous run of tiles, which share operand panels.  xcd_group = G > 0:
// every 8 G workgroups take 8 G consecutive tiles, G contiguous ones per XCD,
// so each class of the launch is spread over all XCDs (a launch mixing long-
// and short-K classes stays balanced); a last partial round keeps the
// identity order.  xcd_group == kXcdByClass: the contiguous runs walk an
// order that lists one eighth of every class per XCD (balanced and still
// contiguous within each class).  All three maps are bijections of [0, nb).
__device__ __forceinline__ TileRef locate_tile(const GemmArgs &args) {
  const int nb = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  int tile;
  if (args.xcd_group > 0) {
    const int G = args.xcd_group, chunk = 8 * G;
    const int q = b / chunk, u = b - q * chunk;
    tile = (b < nb / chunk * chunk) ? q * chunk + (u & 7) * G + (u >> 3) : b;
  } else {
    const int per_xcd = nb / 8, rem = nb % 8, xcd = b % 8, slot = b / 8;
    tile = (xcd < rem ? xcd * (per_xcd + 1) : rem * (per_xcd + 1) + (xcd - rem) * per_xcd) + slot;
    if (args.xcd_group == kXcdByClass) {
      // position `tile` of an order that lists eighth 0 of every class, then
      // eighth 1 of every class, ...: each XCD's contiguous run covers about
      // one eighth of each class
      const int v = tile;
      int x = 0;
#pragma unroll
      for (int i = 1; i < 8; ++i) x += (args.xcd_start[i] <= v) ? 1 : 0;
      int r = v - args.xcd_start[x];
      tile = 0;
      bool found = false;
#pragma unroll
      for (int c = 0; c < kGemmMaxClasses; ++c) {
        const int lo = args.xcd_lo[c][x], n = args.xcd_lo[c][x + 1] - lo;
        if (!found && r < n) {
          tile = args.tile_begin[c] + lo + r;
          found = true;
        }
        if (!found) r -= n;
      }
    }
  }
  // tile_begin[] is ascending with INT32_MAX past the last class: the class
  // index is the count of later entries <= tile (independent scalar loads)
  int ci = 0;
#pragma unroll
  for (int i = 1; i < kGemmMaxClasses; ++i) ci += (args.tile_begin[i] <= tile) ? 1 : 0;
  const GemmClass &cl = args.cls[ci];
  const int local = tile - args.tile_begin[ci];
  TileRef r;
  r.ci = ci;
  r.mat = local / cl.tiles_per_mat;
  int t = local - r.mat * cl.tiles_per_mat;
  if (cl.half) {
    int tm = 0, rowlen = cl.tiles_n;
#pragma unroll 1
    while (t >= rowlen) { t -= rowlen; ++tm; --rowlen; }
    r.tm = tm;
    r.tn = tm + t;
  } else {
    // super-rows of kRowGroup tile rows, walked column by column: the tiles
    // a workgroup's neighbours take share both A and B panels in L2
    const int per_group = kRowGroup * cl.tiles_n;
    const int g = t / per_group, u = t - g * per_group;
    const int rows = min(kRowGroup, cl.tiles_m - g * kRowGroup);
    r.tm = g * kRowGroup + u % rows;
    r.tn = u / rows;
  }
  return r;
}

// Load the epilogue input Cin for one wave's FM x FN accumulator grid (same
// layout as the accumulators), so its latency can overlap the main loop.
template <typename T, int FM, int FN>
__device__ __forceinline__ void load_cin(const GemmClass &cl, int mat, int row0, int col0, float (&cin)[FM][FN][4]) {
  constexpr int ES = sizeof(T);
  const int lane = threadIdx.x & 63;
  if (!cl.cin) return;
  const void *Cin = (const void *)((const char *)cl.cin + (int64_t)mat * cl.scin * ES);
  const int row_base = row0 + 4 * (lane >> 4);
  const int col_base = col0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cin[i][j][r] = Store<T>::load(Cin, (int64_t)(row_base + i * 16 + r) * cl.ldcin + col_base + j * 16);
}

// Direct epilogue for latency-bound small tiles: each lane stores its own
// accumulator values (MFMA 16x16 layout: rows 4 (lane / 16) + r, column
// lane % 16) straight to global memory, with no LDS hand-off.  Same results
// as epilogue_lds.  Top-left corner of the wave's grid: (row0, col0).
// PRE: Cin was prefetched into cin_pre by load_cin (else it is loaded here).
template <typename T, int FM, int FN, bool PRE = false>
__device__ __forceinline__ void epilogue(const GemmClass &cl, int mat, bool diag_tile, int row0, int col0,
                                         const f32x4 (&acc)[FM][FN], const float (&cin_pre)[FM][FN][4]) {
  constexpr int ES = sizeof(T);
  const int lane = threadIdx.x & 63;
  const float alpha = cl.alpha, beta = cl.beta, diag = cl.diag;
  void *C = cl.c ? (void *)((char *)cl.c + (int64_t)mat * cl.sc * ES) : nullptr;
  void *C2 = cl.c2 ? (void *)((char *)cl.c2 + (int64_t)mat * cl.sc2 * ES) : nullptr;
  const void *Cin = cl.cin ? (const void *)((const char *)cl.cin + (int64_t)mat * cl.scin * ES) : nullptr;
  const int row_base = row0 + 4 * (lane >> 4);
  const int col_base = col0 + (lane & 15);
  FinalDesc fd{};
  bool fvec = false;
  if (cl.final_mode) {
    fd = cl.desc[cl.desc_base + mat];
    fvec = (fd.cols & 3) == 0 && ((((uintptr_t)fd.weight) | ((uintptr_t)fd.ortho_out)) & 15) == 0;
  }
  static_for<0, FM>([&](auto ic) {
    static_for<0, FN>([&](auto jc) {
      constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
      const int r0 = row_base + i * 16;
      const int col = col_base + j * 16;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = alpha * acc[i][j][r];
        if (Cin) {
          if constexpr (PRE) v[r] += beta * cin_pre[i][j][r];
          else v[r] += beta * Store<T>::load(Cin, (int64_t)(r0 + r) * cl.ldcin + col);
        }
        if (diag != 0.0f && r0 + r == col && col < cl.diag_limit) v[r] += diag;
      }
      if (cl.final_mode) {
        // fused decoupled update: the tile is tall (rows = long side)
        const float lr = cl.lr, wd = cl.wd, gm = fd.gamma;
        if (!fd.wide) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = r0 + r;
            if (i < fd.rows && col < fd.cols) {
              const int64_t x = (int64_t)i * fd.cols + col;
              const float w = fd.weight[x];
              fd.weight[x] = w - lr * (gm * v[r] + wd * w);
              if (fd.ortho_out) fd.ortho_out[x] = v[r];
            }
          }
        } else if (col < fd.rows) {
          // W row `col`, columns r0 .. r0+3 (r0 is a multiple of 4)
          const int64_t x = (int64_t)col * fd.cols + r0;
          if (fvec && r0 + 4 <= fd.cols) {
            float4 w = *(const float4 *)(fd.weight + x);
            w.x = w.x - lr * (gm * v[0] + wd * w.x);
            w.y = w.y - lr * (gm * v[1] + wd * w.y);
            w.z = w.z - lr * (gm * v[2] + wd * w.z);
            w.w = w.w - lr * (gm * v[3] + wd * w.w);
            *(float4 *)(fd.weight + x) = w;
            if (fd.ortho_out) *(float4 *)(fd.ortho_out + x) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (r0 + r < fd.cols) {
                const float w = fd.weight[x + r];
                fd.weight[x + r] = w - lr * (gm * v[r] + wd * w);
                if (fd.ortho_out) fd.ortho_out[x + r] = v[r];
              }
            }
          }
        }
        return;
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
    });
  });
}

// s_waitcnt lgkmcnt(0) (LDS and scalar memory), vmcnt and expcnt untouched.
#define MUON_LGKM0 (0xF | (0x7 << 4) | (0x3 << 14))

// Barrier for LDS hand-offs inside the epilogue: this wave's LDS accesses
// have completed, then s_barrier.  No memory fence, so global stores already
// issued stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(MUON_LGKM0);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Floats of LDS the epilogue of a BM x BN block tile needs: a band of HB
// rows stored row-major (rows padded by 4 floats) and transposed.
template <int HB, int BN>
constexpr int epilogue_lds_floats() {
  return HB * (BN + 4) + BN * HB;
}

// One 16-byte chunk of the result, from 16-byte aligned floats, stored to
// global memory as T.
template <typename T> struct Pack;
template <> struct Pack<float> {
  static __device__ __forceinline__ void copy(float *dst, const float4 *src) { *(float4 *)dst = src[0]; }
};
template <typename H> struct Pack16 {
  static __device__ __forceinline__ uint32_t pair(float a, float b) {
    return (uint32_t)Store16<H>::bits(a) | ((uint32_t)Store16<H>::bits(b) << 16);
  }
  static __device__ __forceinline__ void copy(H *dst, const float4 *src) {
    u32x4 u;
    u.x = pair(src[0].x, src[0].y);
    u.y = pair(src[0].z, src[0].w);
    u.z = pair(src[1].x, src[1].y);
    u.w = pair(src[1].z, src[1].w);
    *(u32x4 *)dst = u;
  }
};
template <> struct Pack<__bf16> : Pack16<__bf16> {};
template <> struct Pack<_Float16> : Pack16<_Float16> {};

__device__ __forceinline__ float elem(const float4 *v, int e) {
  const float4 x = v[e >> 2];
  return (e & 3) == 0 ? x.x : (e & 3) == 1 ? x.y : (e & 3) == 2 ? x.z : x.w;
}

// Offset of (column c, band row r) in the transposed band: rows are stored
// in groups of 4 (one float4), and the groups of column c are permuted by
// (c / 8) % 8 so that float4 accesses of 8 consecutive 8-column chunks at one
// row group fall into distinct banks.
template <int HB>
__device__ __forceinline__ int tpos(int c, int r) {
  return c * HB + 4 * ((r >> 2) ^ ((c >> 3) & 7)) + (r & 3);
}

// Epilogue of one BM x BN block tile (NT threads; wave tiles of FM x FN
// 16 x 16 accumulator blocks with block-local origin (wrow, wcol)):
//   v = alpha * acc + beta * Cin + diag * [row == col < diag_limit]
// handed through LDS in bands of HB rows so that every global access is a
// 16-byte vector along a row.  Per band: the waves write alpha * acc (+ diag)
// from the MFMA layout (lane holds rows 4 (lane / 16) + r, column lane % 16)
// into a row-major copy; a row-major sweep, in units of 4 rows x 16 bytes,
// adds beta * Cin (read as 16-byte chunks in C's orientation), stores C rows
// and fills the transposed copy; a transposed sweep stores the mirrored tile
// of a symmetric product (upper-triangular tiles only; a diagonal tile keeps
// its upper triangle and mirrors it) or the transposed copy C2.  In final
// mode the sweeps apply the fp32 decoupled update of W instead: row-major for
// tall W, transposed for wide W.  On entry every wave must be done reading
// LDS for the main loop.
template <typename T, int BM, int BN, int HB, int NT, int FM, int FN>
__device__ __forceinline__ void epilogue_lds(const GemmClass &cl, int mat, int tm, int tn, int wrow, int wcol,
                                             f32x4 (&acc)[FM][FN], float *lds) {
  static_assert(BM % HB == 0 && HB % 16 == 0 && HB >= 32 && HB <= 64, "bands hold whole 16-row blocks");
  constexpr int ES = sizeof(T);
  constexpr int CE = 16 / ES;                 // elements per 16-byte chunk
  constexpr int CQ = CE / 4;                  // float4 per chunk
  constexpr int PR = BN + 4;                  // row-major pitch (floats)
  constexpr int CPR = BN / CE;                // chunks per row
  constexpr int UNITS = (HB / 4) * CPR;       // 4-row units per band
  static_assert(UNITS % NT == 0, "every thread takes the same number of units");
  constexpr int NU = UNITS / NT;
  float *lr = lds;                            // HB x PR, row-major band
  float *lt = lds + HB * PR;                  // BN x HB, transposed band (tpos)
  const int lane = threadIdx.x & 63;
  const int tid = threadIdx.x;
  const int row0 = tm * BM, col0 = tn * BN;   // block tile origin in the result
  const float alpha = cl.alpha, beta = cl.beta, diag = cl.diag;
  const T *Cin = cl.cin ? (const T *)((const char *)cl.cin + (int64_t)mat * cl.scin * ES) : nullptr;
  // alpha * acc + diag in place
  {
    const int rb = row0 + wrow + 4 * (lane >> 4);
    const int cb = col0 + wcol + (lane & 15);
    static_for<0, FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = cb + j * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = alpha * acc[i][j][r];
          if (diag != 0.0f && rb + i * 16 + r == col && col < cl.diag_limit) v += diag;
          acc[i][j][r] = v;
        }
      }
    });
  }
  const bool diag_tile = cl.half && tm == tn;
  FinalDesc fd{};
  bool fvec = false;
  if (cl.final_mode) {
    fd = cl.desc[cl.desc_base + mat];
    fvec = (fd.cols & 3) == 0 && ((((uintptr_t)fd.weight) | ((uintptr_t)fd.ortho_out)) & 15) == 0;
  }
  T *C = cl.c ? (T *)((char *)cl.c + (int64_t)mat * cl.sc * ES) : nullptr;
  T *C2 = cl.c2 ? (T *)((char *)cl.c2 + (int64_t)mat * cl.sc2 * ES) : nullptr;
  T *Ct = cl.half ? C : C2;                   // destination of the transposed sweep
  const int ldt = cl.half ? cl.ldc : cl.ldc2;
  const bool out_r = cl.final_mode ? !fd.wide : (C != nullptr);    // row-major sweep stores
  const bool out_t = cl.final_mode ? (fd.wide != 0) : (Ct != nullptr);
  // the MFMA layout fills the transposed copy directly unless beta * Cin must
  // be added first (then the row-major sweep fills it)
  const bool direct_t = out_t && !Cin;
  const float lrate = cl.lr, wd = cl.wd, gm = fd.gamma;

  // W <- W - lr (gamma o + wd W) for 4 consecutive elements of W's row wr
  auto update_w = [&](int wr, int wc, const float4 o4) {
    if (wr >= fd.rows || wc >= fd.cols) return;
    const float o[4] = {o4.x, o4.y, o4.z, o4.w};
    const int64_t x = (int64_t)wr * fd.cols + wc;
    if (fvec) {   // cols % 4 == 0, so wc + 4 <= cols
      float4 w = *(const float4 *)(fd.weight + x);
      w.x = w.x - lrate * (gm * o[0] + wd * w.x);
      w.y = w.y - lrate * (gm * o[1] + wd * w.y);
      w.z = w.z - lrate * (gm * o[2] + wd * w.z);
      w.w = w.w - lrate * (gm * o[3] + wd * w.w);
      *(float4 *)(fd.weight + x) = w;
      if (fd.ortho_out) *(float4 *)(fd.ortho_out + x) = o4;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (wc + e < fd.cols) {
          const float w = fd.weight[x + e];
          fd.weight[x + e] = w - lrate * (gm * o[e] + wd * w);
          if (fd.ortho_out) fd.ortho_out[x + e] = o[e];
        }
      }
    }
  };
  // W loads issued together before their stores, in batches of WB rows /
  // sweep units (the kernels run two waves per SIMD)
  constexpr int WB = NT >= 512 ? 1 : 2;
  // the same update for 4 consecutive W rows from wr, CQ float4 of columns
  // from wc each (o[i][h])
  auto update_w_rows = [&](int wr, int wc, const float4 (&o)[4][CQ]) {
    if (fvec && wr + 4 <= fd.rows && wc + 4 * CQ <= fd.cols) {
#pragma unroll
      for (int i0 = 0; i0 < 4; i0 += WB) {
      float4 w[WB][CQ];
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int h = 0; h < CQ; ++h) w[i][h] = *(const float4 *)(fd.weight + (int64_t)(wr + i0 + i) * fd.cols + wc + 4 * h);
#pragma unroll
      for (int ii = 0; ii < WB; ++ii)
#pragma unroll
        for (int h = 0; h < CQ; ++h) {
          const int i = i0 + ii;
          float4 x = w[ii][h];
          const float4 v = o[i][h];
          x.x = x.x - lrate * (gm * v.x + wd * x.x);
          x.y = x.y - lrate * (gm * v.y + wd * x.y);
          x.z = x.z - lrate * (gm * v.z + wd * x.z);
          x.w = x.w - lrate * (gm * v.w + wd * x.w);
          const int64_t at = (int64_t)(wr + i) * fd.cols + wc + 4 * h;
          *(float4 *)(fd.weight + at) = x;
          if (fd.ortho_out) *(float4 *)(fd.ortho_out + at) = v;
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < CQ; ++h) update_w(wr + i, wc + 4 * h, o[i][h]);
  };
  // wide W: unit n of the transposed sweep of band brow is W row col0 + c,
  // CE columns from row0 + brow + rr
  auto update_w_cols = [&](int brow, auto &src) {
    constexpr int NQ = sizeof(src) / sizeof(src[0]);
    bool all = fvec;
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int q = tid + n * NT;
      const int c = q / (HB / CE), rr = (q - c * (HB / CE)) * CE;
      all = all && col0 + c < fd.rows && row0 + brow + rr + CE <= fd.cols;
    }
    if (all) {
      constexpr int NB = WB < NQ ? WB : NQ;
#pragma unroll
      for (int n0 = 0; n0 < NQ; n0 += NB) {
      float4 w[NB][CQ];
#pragma unroll
      for (int nn = 0; nn < NB; ++nn) {
        const int q = tid + (n0 + nn) * NT;
        const int c = q / (HB / CE), rr = (q - c * (HB / CE)) * CE;
#pragma unroll
        for (int h = 0; h < CQ; ++h)
          w[nn][h] = *(const float4 *)(fd.weight + (int64_t)(col0 + c) * fd.cols + row0 + brow + rr + 4 * h);
      }
#pragma unroll
      for (int nn = 0; nn < NB; ++nn) {
        const int n = n0 + nn;
        const int q = tid + n * NT;
        const int c = q / (HB / CE), rr = (q - c * (HB / CE)) * CE;
#pragma unroll
        for (int h = 0; h < CQ; ++h) {
          float4 x = w[nn][h];
          const float4 v = src[n][h];
          x.x = x.x - lrate * (gm * v.x + wd * x.x);
          x.y = x.y - lrate * (gm * v.y + wd * x.y);
          x.z = x.z - lrate * (gm * v.z + wd * x.z);
          x.w = x.w - lrate * (gm * v.w + wd * x.w);
          const int64_t at = (int64_t)(col0 + c) * fd.cols + row0 + brow + rr + 4 * h;
          *(float4 *)(fd.weight + at) = x;
          if (fd.ortho_out) *(float4 *)(fd.ortho_out + at) = v;
        }
      }
      }
      return;
    }
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int q = tid + n * NT;
      const int c = q / (HB / CE), rr = (q - c * (HB / CE)) * CE;
#pragma unroll
      for (int h = 0; h < CQ; ++h) update_w(col0 + c, row0 + brow + rr + 4 * h, src[n][h]);
    }
  };

  // this thread's Cin chunks of band p (4 rows x 16 bytes per unit)
  auto load_cin_band = [&](int p, u32x4 (&dst)[NU][4]) {
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = tid + k * NT;
      const int rg = u / CPR, c = (u - rg * CPR) * CE;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[k][i] = *(const u32x4 *)(Cin + (int64_t)(row0 + p * HB + 4 * rg + i) * cl.ldcin + col0 + c);
    }
  };
  // every band's Cin is loaded before the first store: the vector memory
  // counter retires in order, so a load issued after a store could only be
  // awaited together with that store
  u32x4 cin_all[BM / HB][NU][4];
  if (Cin) static_for<0, BM / HB>([&](auto pc) { load_cin_band(decltype(pc)::value, cin_all[decltype(pc)::value]); });

  // bands unrolled: each band's accumulators are dead once staged
  static_for<0, BM / HB>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    const int brow = p * HB;   // block-local first row of the band
    lds_barrier();   // previous band (or the main loop) is done with LDS
    static_for<0, FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rloc = wrow + i * 16 - brow;   // band-local first row of block i
      if (rloc >= 0 && rloc < HB) {
        const int rr = rloc + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = wcol + j * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) lr[(rr + r) * PR + c] = acc[i][j][r];
          if (direct_t) *(float4 *)&lt[tpos<HB>(c, rr)] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    });
    lds_barrier();
    auto &cinv = cin_all[p];
    // row-major sweep: units of 4 rows x one 16-byte chunk
#pragma unroll
    for (int k = 0; k < NU; ++k) {
      const int u = tid + k * NT;
      const int rg = u / CPR, c = (u - rg * CPR) * CE;
      float4 v[4][CQ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < CQ; ++h) v[i][h] = *(const float4 *)&lr[(4 * rg + i) * PR + c + 4 * h];
      if (Cin) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 w = cinv[k][i];
          if constexpr (ES == 4) {
            v[i][0].x += beta * __uint_as_float(w.x);
            v[i][0].y += beta * __uint_as_float(w.y);
            v[i][0].z += beta * __uint_as_float(w.z);
            v[i][0].w += beta * __uint_as_float(w.w);
          } else {
            auto lo = [](uint32_t x) { return (float)__builtin_bit_cast(T, (uint16_t)(x & 0xFFFFu)); };
            auto hi = [](uint32_t x) { return (float)__builtin_bit_cast(T, (uint16_t)(x >> 16)); };
            v[i][0].x += beta * lo(w.x);
            v[i][0].y += beta * hi(w.x);
            v[i][0].z += beta * lo(w.y);
            v[i][0].w += beta * hi(w.y);
            v[i][1].x += beta * lo(w.z);
            v[i][1].y += beta * hi(w.z);
            v[i][1].z += beta * lo(w.w);
            v[i][1].w += beta * hi(w.w);
          }
        }
        if (out_t) {   // column c + e, rows 4 rg .. 4 rg + 3
#pragma unroll
          for (int e = 0; e < CE; ++e)
            *(float4 *)&lt[tpos<HB>(c + e, 4 * rg)] =
                make_float4(elem(v[0], e), elem(v[1], e), elem(v[2], e), elem(v[3], e));
        }
      }
      if (!out_r) continue;
      if (cl.final_mode) {
        // tall W: rows row0 + brow + 4 rg + i, 4 h columns from col0 + c
        update_w_rows(row0 + brow + 4 * rg, col0 + c, v);
        continue;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int R = brow + 4 * rg + i;   // block-local row
        T *dst = C + (int64_t)(row0 + R) * cl.ldc + col0 + c;
        if (!diag_tile || c >= R) {
          Pack<T>::copy(dst, v[i]);
        } else if (c + CE > R) {   // the chunk crossing the diagonal: upper part only
#pragma unroll
          for (int e = 0; e < CE; ++e)
            if (c + e >= R) Store<T>::store(dst, e, elem(v[i], e));
        }
      }
    }
    if (!out_t) return;
    if (!direct_t) lds_barrier();   // the transposed copy was filled by the sweep above
    if (cl.final_mode) {
      // wide W: row col0 + c, CE columns from row0 + brow + rr; every W load
      // of the thread is issued before its first store
      static_assert((BN * HB / CE) % NT == 0, "whole transposed sweep per thread");
      constexpr int NQ = BN * HB / CE / NT;
      float4 src[NQ][CQ];
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int q = tid + n * NT;
        const int c = q / (HB / CE), rr = (q - c * (HB / CE)) * CE;
#pragma unroll
        for (int h = 0; h < CQ; ++h) src[n][h] = *(const float4 *)&lt[tpos<HB>(c, rr + 4 * h)];
      }
      update_w_cols(brow, src);
      return;
    }
    // transposed sweep: chunks of CE band rows of one column
#pragma unroll 1
    for (int q = tid; q < BN * HB / CE; q += NT) {
      const int c = q / (HB / CE), rr = (q - c * (HB / CE)) * CE;
      float4 src[CQ];
#pragma unroll
      for (int h = 0; h < CQ; ++h) src[h] = *(const float4 *)&lt[tpos<HB>(c, rr + 4 * h)];
      T *dst = Ct + (int64_t)(col0 + c) * ldt + row0 + brow + rr;
      const int R0 = brow + rr;   // block-local row of the chunk's first element
      if (!diag_tile || c >= R0 + CE - 1) {
        Pack<T>::copy(dst, src);
      } else if (c >= R0) {       // mirror only the upper-triangular sources
#pragma unroll
        for (int e = 0; e < CE; ++e)
          if (c >= R0 + e) Store<T>::store(dst, e, elem(src, e));
      }
    }
  });
}

// Epilogue of the 16-bit 128 x 128 and 256 x 256 block tiles (2 BM
// threads): the same values as epilogue_lds, in bands of 128 rows.  The accumulators
// (alpha * acc + diag) are staged row-major in LDS; then each thread takes
// one 8 x 8 unit of the band (lanes arranged 8 x 8, so 8 lanes cover one
// 128-byte line in either orientation), adds beta * Cin, stores the unit's 8
// rows as 16-byte vectors and transposes the packed 16-bit values in
// registers for the 8 transposed (mirror / C2) 16-byte stores: no transposed
// LDS copy and one barrier per band fewer.  In final mode the unit updates
// 8 rows of a tall W, or 8 rows of a wide W from the unit's columns.  Every
// Cin chunk is loaded before the first store (the memory counter retires in
// order).  On entry every wave must be done reading LDS for the main loop.
template <typename T, int BM, int FM, int FN>
__device__ __forceinline__ void epilogue_u8(const GemmClass &cl, int mat, int tm, int tn, int wrow, int wcol,
                                            f32x4 (&acc)[FM][FN], float *lds) {
  static_assert(sizeof(T) == 2, "16-bit results");
  static_assert(BM == 128 || BM == 256, "bands of 128 rows, 8 x 8 units over 2 BM threads");
  constexpr int BN = BM, HB = 128;
  constexpr int WPR = BM / 64;                // waves per 64-column-unit row of the band
  constexpr int PR = BN + 4;                  // row-major pitch (floats)
  float *lr = lds;                            // HB x PR
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = tm * BM, col0 = tn * BN;
  const float alpha = cl.alpha, beta = cl.beta, diag = cl.diag;
  const T *Cin = cl.cin ? (const T *)((const char *)cl.cin + (int64_t)mat * cl.scin * 2) : nullptr;
  {
    const int rb = row0 + wrow + 4 * (lane >> 4);
    const int cb = col0 + wcol + (lane & 15);
    static_for<0, FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = cb + j * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = alpha * acc[i][j][r];
          if (diag != 0.0f && rb + i * 16 + r == col && col < cl.diag_limit) v += diag;
          acc[i][j][r] = v;
        }
      }
    });
  }
  const bool diag_tile = cl.half && tm == tn;
  FinalDesc fd{};
  bool fvec = false;
  if (cl.final_mode) {
    fd = cl.desc[cl.desc_base + mat];
    fvec = (fd.cols & 3) == 0 && ((((uintptr_t)fd.weight) | ((uintptr_t)fd.ortho_out)) & 15) == 0;
  }
  T *C = cl.c ? (T *)((char *)cl.c + (int64_t)mat * cl.sc * 2) : nullptr;
  T *C2 = cl.c2 ? (T *)((char *)cl.c2 + (int64_t)mat * cl.sc2 * 2) : nullptr;
  T *Ct = cl.half ? C : C2;                   // destination of the transposed stores
  const int ldt = cl.half ? cl.ldc : cl.ldc2;
  const float lrate = cl.lr, wd = cl.wd, gm = fd.gamma;
  // this thread's unit: columns 8 cg .. 8 cg + 7, band rows 8 rg .. 8 rg + 7
  const int cg = (wave % WPR) * 8 + (lane & 7);
  const int rg = (wave / WPR) * 8 + (lane >> 3);
  const int c0 = 8 * cg;
  u32x4 cin[BM / HB][8];
  if (Cin) {
#pragma unroll
    for (int p = 0; p < BM / HB; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        cin[p][i] = *(const u32x4 *)(Cin + (int64_t)(row0 + p * HB + 8 * rg + i) * cl.ldcin + col0 + c0);
  }
  // W <- W - lr (gamma o + wd W) on 8 consecutive elements of W's row wr from wc
  auto update_w8 = [&](int wr, int wc, const float (&o)[8]) {
    if (wr >= fd.rows) return;
    float *w = fd.weight + (int64_t)wr * fd.cols + wc;
    float *oo = fd.ortho_out ? fd.ortho_out + (int64_t)wr * fd.cols + wc : nullptr;
    if (fvec && wc + 8 <= fd.cols) {
      float4 a = *(const float4 *)w, b = *(const float4 *)(w + 4);
      a.x = a.x - lrate * (gm * o[0] + wd * a.x);
      a.y = a.y - lrate * (gm * o[1] + wd * a.y);
      a.z = a.z - lrate * (gm * o[2] + wd * a.z);
      a.w = a.w - lrate * (gm * o[3] + wd * a.w);
      b.x = b.x - lrate * (gm * o[4] + wd * b.x);
      b.y = b.y - lrate * (gm * o[5] + wd * b.y);
      b.z = b.z - lrate * (gm * o[6] + wd * b.z);
      b.w = b.w - lrate * (gm * o[7] + wd * b.w);
      *(float4 *)w = a;
      *(float4 *)(w + 4) = b;
      if (oo) {
        *(float4 *)oo = make_float4(o[0], o[1], o[2], o[3]);
        *(float4 *)(oo + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (wc + e < fd.cols) {
          const float x = w[e];
          w[e] = x - lrate * (gm * o[e] + wd * x);
          if (oo) oo[e] = o[e];
        }
      }
    }
  };

  static_for<0, BM / HB>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    const int brow = p * HB;
    lds_barrier();   // the previous band (or the main loop) is done with LDS
    static_for<0, FM>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int rloc = wrow + i * 16 - brow;   // band-local first row of block i
      if (rloc >= 0 && rloc < HB) {
        const int rr = rloc + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = wcol + j * 16 + (lane & 15);
#pragma unroll
          for (int r = 0; r < 4; ++r) lr[(rr + r) * PR + c] = acc[i][j][r];
        }
      }
    });
    lds_barrier();
    const int R0 = brow + 8 * rg;   // block-local first row of the unit
    uint32_t pk[8][4];               // the unit as T: row i, columns 2k, 2k + 1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float *src = lr + (8 * rg + i) * PR + c0;
      const float4 a = *(const float4 *)src, b = *(const float4 *)(src + 4);
      float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      if (Cin) {
        const u32x4 w = cin[p][i];
        auto lo = [](uint32_t x) { return (float)__builtin_bit_cast(T, (uint16_t)(x & 0xFFFFu)); };
        auto hi = [](uint32_t x) { return (float)__builtin_bit_cast(T, (uint16_t)(x >> 16)); };
        v[0] += beta * lo(w.x);
        v[1] += beta * hi(w.x);
        v[2] += beta * lo(w.y);
        v[3] += beta * hi(w.y);
        v[4] += beta * lo(w.z);
        v[5] += beta * hi(w.z);
        v[6] += beta * lo(w.w);
        v[7] += beta * hi(w.w);
      }
      if (cl.final_mode) {   // kept in place for the W pass below
        *(float4 *)src = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(src + 4) = make_float4(v[4], v[5], v[6], v[7]);
        continue;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) pk[i][k] = Pack16<T>::pair(v[2 * k], v[2 * k + 1]);
      if (C) {
        const int R = R0 + i;
        T *dst = C + (int64_t)(row0 + R) * cl.ldc + col0 + c0;
        if (!diag_tile || c0 >= R) {
          *(u32x4 *)dst = u32x4{pk[i][0], pk[i][1], pk[i][2], pk[i][3]};
        } else if (c0 + 8 > R) {   // the chunk crossing the diagonal: upper part only
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c0 + e >= R) ((uint16_t *)dst)[e] = (uint16_t)(pk[i][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
    if (cl.final_mode) {
      // 8 W rows of 8 elements from the unit's own staged values: a tall W
      // takes the unit's rows (W row row0 + R0 + q, columns col0 + c0 ..), a
      // wide W its columns (W row col0 + c0 + q, columns row0 + R0 ..); in
      // batches of QB rows with every W load issued before the stores (the
      // staged values are read from LDS after the loads)
      constexpr int QB = BM == 256 ? 1 : 4;   // registers: two waves per SIMD on the 256 tile
      const bool tall = !fd.wide;
      const int wr0 = tall ? row0 + R0 : col0 + c0, wc = tall ? col0 + c0 : row0 + R0;
      auto staged = [&](int q, float (&o)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = tall ? lr[(8 * rg + q) * PR + c0 + e] : lr[(8 * rg + e) * PR + c0 + q];
      };
#pragma unroll
      for (int q0 = 0; q0 < 8; q0 += QB) {
        if (fvec && wr0 + q0 + QB <= fd.rows && wc + 8 <= fd.cols) {
          float4 w[QB][2];
#pragma unroll
          for (int qq = 0; qq < QB; ++qq) {
            const float *wp = fd.weight + (int64_t)(wr0 + q0 + qq) * fd.cols + wc;
            w[qq][0] = *(const float4 *)wp;
            w[qq][1] = *(const float4 *)(wp + 4);
          }
#pragma unroll
          for (int qq = 0; qq < QB; ++qq) {
            float x[8];
            staged(q0 + qq, x);
            float4 a = w[qq][0], b = w[qq][1];
            a.x = a.x - lrate * (gm * x[0] + wd * a.x);
            a.y = a.y - lrate * (gm * x[1] + wd * a.y);
            a.z = a.z - lrate * (gm * x[2] + wd * a.z);
            a.w = a.w - lrate * (gm * x[3] + wd * a.w);
            b.x = b.x - lrate * (gm * x[4] + wd * b.x);
            b.y = b.y - lrate * (gm * x[5] + wd * b.y);
            b.z = b.z - lrate * (gm * x[6] + wd * b.z);
            b.w = b.w - lrate * (gm * x[7] + wd * b.w);
            const int64_t at = (int64_t)(wr0 + q0 + qq) * fd.cols + wc;
            *(float4 *)(fd.weight + at) = a;
            *(float4 *)(fd.weight + at + 4) = b;
            if (fd.ortho_out) {
              *(float4 *)(fd.ortho_out + at) = make_float4(x[0], x[1], x[2], x[3]);
              *(float4 *)(fd.ortho_out + at + 4) = make_float4(x[4], x[5], x[6], x[7]);
            }
          }
        } else {
#pragma unroll
          for (int qq = 0; qq < QB; ++qq) {
            float x[8];
            staged(q0 + qq, x);
            update_w8(wr0 + q0 + qq, wc, x);
          }
        }
      }
      return;
    }
    if (!Ct) return;
    // transposed stores: column c0 + e, rows R0 .. R0 + 7
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = 16 * (e & 1);
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (pk[i][e >> 1] >> sh) & 0xFFFFu;
      T *dst = Ct + (int64_t)(col0 + c0 + e) * ldt + row0 + R0;
      const int c = c0 + e;
      if (!diag_tile || c >= R0 + 7) {
        *(u32x4 *)dst = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      } else if (c >= R0) {       // mirror only the upper-triangular sources
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c >= R0 + i) ((uint16_t *)dst)[i] = (uint16_t)h[i];
      }
    }
  });
}

// Register-staged BM x BN block tile (64 or 128; every fp32 product and the
// 16-bit 128 tile): four waves of (BM/2) x (BN/2); k advances 128 bytes per
// LDS stage, double-buffered through registers, with one barrier per stage.
// LDS rows carry 16 bytes of padding so the 16-byte fragment reads of 8
// consecutive rows fall into distinct banks.
constexpr int kThreads = 256;
constexpr int kStageBytes = 128;               // k bytes per LDS stage per row
constexpr int kPitch = kStageBytes + 16;       // padded LDS row

template <typename T, int BM, int BN>
__global__ __launch_bounds__(kThreads, 2) void ns_gemm_kernel(GemmArgs args) {
  constexpr int ES = sizeof(T);
  constexpr int KS = kStageBytes / ES;         // k elements per stage
  constexpr int WM = BM / 2, WN = BN / 2;      // 2 x 2 waves
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_LD = BM * (kStageBytes / 16) / kThreads;  // 16-byte chunks per thread
  constexpr int B_LD = BN * (kStageBytes / 16) / kThreads;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the block");
  __shared__ __attribute__((aligned(16))) char lds[2][(BM + BN) * kPitch];

  const TileRef tr = locate_tile(args);
  const GemmClass &cl = args.cls[tr.ci];
  const int mat = tr.mat, tm = tr.tm, tn = tr.tn;

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

  static_assert(epilogue_lds_floats<64, BN>() * 4 <= (int)sizeof(lds), "epilogue bands must fit the LDS stages");
  const float no_cin[FM][FN][4] = {};
  if constexpr (BM == 64) {   // latency-bound small tiles: no LDS hand-off
    epilogue<T, FM, FN>(cl, mat, cl.half && tm == tn, tm * BM + wm * WM, tn * BN + wn * WN, acc, no_cin);
  } else if constexpr (ES == 2 && BM == 128 && BN == 128) {
    static_assert(128 * (BN + 4) * 4 <= (int)sizeof(lds) && kThreads == 2 * BM, "epilogue_u8 fits");
    epilogue_u8<T, BM, FM, FN>(cl, mat, tm, tn, wm * WM, wn * WN, acc, (float *)&lds[0][0]);
  } else {
    epilogue_lds<T, BM, BN, 64, kThreads, FM, FN>(cl, mat, tm, tn, wm * WM, wn * WN, acc, (float *)&lds[0][0]);
  }
}


// ---------------------------------------------------------------------------
// Stage formats shared by the 16-bit DMA kernels.
#ifndef MUON_A_AHEAD
#define MUON_A_AHEAD 3
#endif
constexpr int kAAhead = MUON_A_AHEAD;     // A fragments read this many 16-row blocks ahead
#ifndef MUON_WIDE_DEFER
#define MUON_WIDE_DEFER 1
#endif
constexpr int kWideDefer = MUON_WIDE_DEFER;   // fragment groups whose MFMAs run after the stage barrier
#ifndef MUON_WIDE_DMA_SPREAD
#define MUON_WIDE_DMA_SPREAD 1
#endif
// 256 tile: DMA instructions per fragment group when a stage's DMA is spread
// over the previous stage instead of issued at its start (0: at its start)
constexpr int kWideSpreadPer = MUON_WIDE_DMA_SPREAD;

// ---------------------------------------------------------------------------
// TILE x TILE block tile for fp16 / bf16 (TILE = 256: eight waves, two per
// SIMD, of 128 x 64 each, one block per CU; TILE = 128: four waves of 64 x 64,
// two blocks per CU): the second wave on a SIMD issues MFMAs while the first
// waits at a barrier or on LDS.
//
// Operands move global -> LDS with global_load_lds_dwordx4 (no register
// staging).  A stage holds 64 k = 128 bytes of every row of the TILE-row A
// and B panels (64 KB at TILE = 256); each group of 8 lanes of a DMA
// instruction fetches one whole 128-byte line (8 rows x 128 bytes per
// instruction), which halves the L1 -> L2 requests per byte relative to
// 64-byte row segments.  Two stages form the ring; the DMA of stage kb+2 is
// issued once every wave is done with stage kb, so a stage has one stage of
// compute to land.
// LDS rows are not padded: 16-byte chunk c of row r is stored at chunk
// c ^ (r & 7), so the fragment reads of 8 consecutive rows at one logical
// chunk cover all 32 banks.  Within a stage the A fragments are streamed
// kAAhead 16-row blocks ahead and the second k-step's B fragments are read
// during the first.
constexpr int kWideRowBytes = 128;                                  // 64 x 16-bit k per stage

template <typename T, int TILE>
__global__ __launch_bounds__(TILE * 2, TILE == 256 ? 1 : 2) void ns_gemm_wide_kernel(GemmArgs args) {
  static_assert(sizeof(T) == 2, "16-bit operands only");
  static_assert(TILE == 128 || TILE == 256, "128 or 256 tiles");
  constexpr int WN_WAVES = TILE / 64;            // 2 x WN_WAVES waves
  constexpr int NWAVES = 2 * WN_WAVES;
  constexpr int WTM = TILE / 2, WTN = 64;        // wave tile
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int NG = 2 * FM;                     // fragment groups per stage (2 k-steps)
  static_assert(NG % (kAAhead + 1) == 0, "A fragment ring must divide the fragment groups");
  constexpr int kWideStage = (TILE + TILE) * kWideRowBytes;
  constexpr int DMA_PER_WAVE = TILE / 8 / NWAVES;   // 1 KB DMA instructions per operand per stage
  constexpr int PER_STAGE = 2 * DMA_PER_WAVE;    // DMA instructions per stage and wave
  // the 128 tile's 8 groups per stage leave too little lead for a spread DMA
  constexpr int SPREAD = TILE == 256 ? kWideSpreadPer : 0;
  constexpr bool kWideSpread = SPREAD > 0;
  static_assert(SPREAD == 0 || (PER_STAGE % SPREAD == 0 && PER_STAGE / SPREAD <= NG), "spread DMA");
  constexpr int kEpiBytes = 128 * (TILE + 4) * 4;   // epilogue_u8's staging band
  constexpr int kLdsBytes = 2 * kWideStage > kEpiBytes ? 2 * kWideStage : kEpiBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];

  const TileRef tr = locate_tile(args);
  const GemmClass &cl = args.cls[tr.ci];
  const int mat = tr.mat, tm = tr.tm, tn = tr.tn;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: scalar arithmetic
  const int wm = wave / WN_WAVES, wn = wave % WN_WAVES;

  const char *A = (const char *)cl.a + ((int64_t)mat * cl.sa + (int64_t)tm * TILE * cl.lda) * 2;
  const char *B = (const char *)cl.b + ((int64_t)mat * cl.sb + (int64_t)tn * TILE * cl.ldb) * 2;
  const int64_t lda_b = (int64_t)cl.lda * 2, ldb_b = (int64_t)cl.ldb * 2;

  // DMA: wave w moves rows [8 DMA_PER_WAVE w, +8 DMA_PER_WAVE) of A and of
  // B, 8 rows per instruction; lane L covers row L / 8 of the group and
  // physical chunk L % 8, which holds logical chunk (L % 8) ^ (L / 8).  The
  // source address is a wave-uniform base (scalar registers) plus a 32-bit
  // lane offset: one vector add per load, and the LDS destination (M0) is
  // scalar arithmetic.
  const int dma_row = lane >> 3;
  const int dma_chunk = (lane & 7) ^ dma_row;
  const char *a_base = A + (int64_t)(wave * 8 * DMA_PER_WAVE) * lda_b;
  const char *b_base = B + (int64_t)(wave * 8 * DMA_PER_WAVE) * ldb_b;
  const uint32_t a_off = (uint32_t)(dma_row * lda_b + dma_chunk * 16);
  const uint32_t b_off = (uint32_t)(dma_row * ldb_b + dma_chunk * 16);

  // fragment of k-step ks (32 k) for row block base + lane % 16: logical
  // chunk 4 ks + lane / 16, physical chunk logical ^ (lane % 8)
  const int fr_row = lane & 15;
  const int a_frag = (wm * WTM + fr_row) * kWideRowBytes;
  // a diagonal tile of a symmetric product (the same panel as A and B) moves
  // the panel once and reads B's fragments from A's rows
  const bool same_ab = tm == tn && cl.a == cl.b && cl.sa == cl.sb && cl.lda == cl.ldb;
  const int b_frag = ((same_ab ? 0 : TILE) + wn * WTN + fr_row) * kWideRowBytes;
  const int chunk0 = (((lane >> 4)) ^ (lane & 7)) * 16;       // ks = 0
  const int chunk1 = ((4 + (lane >> 4)) ^ (lane & 7)) * 16;   // ks = 1

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = cl.K / (kWideRowBytes / 2);
  if (nk > 0) {
    // DMA instruction q of stage kb (q < DMA_PER_WAVE: A rows, else B rows)
    auto dma_piece = [&](int kb, int q) {
      char *dst = lds + (kb & 1) * kWideStage + wave * DMA_PER_WAVE * 1024;
      const bool is_a = q < DMA_PER_WAVE;
      if (!is_a && same_ab) return;
      const int j = is_a ? q : q - DMA_PER_WAVE;
      // the empty asm keeps each row group's base in scalar registers, so
      // the compiler cannot fold the lane offset into per-lane addresses
      const char *sp = is_a ? a_base + (int64_t)j * 8 * lda_b + (int64_t)kb * kWideRowBytes
                            : b_base + (int64_t)j * 8 * ldb_b + (int64_t)kb * kWideRowBytes;
      asm volatile("" : "+s"(sp));
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(sp + (is_a ? a_off : b_off)),
                                       (void __attribute__((address_space(3))) *)(dst + (is_a ? 0 : TILE * kWideRowBytes) + j * 1024),
                                       16, 0, 0);
    };
    auto dma = [&](int kb) {
#pragma unroll
      for (int q = 0; q < PER_STAGE; ++q) dma_piece(kb, q);
    };
    // fragment group g = FM ks + i: A row block i at k-step ks
    auto rd_a = [&](const char *slot, int g) -> u32x4 {
      return *(const u32x4 *)(slot + a_frag + (g % FM) * 16 * kWideRowBytes + ((g / FM) ? chunk1 : chunk0));
    };
    constexpr int NQ = kAAhead + 1;             // A fragment ring entries
    constexpr int D = kWideDefer;
    static_assert(D >= 0 && D < NQ && D <= FM, "deferred groups: k-step 1 only, within the A ring");
    // The deferred groups NG-D .. NG-1 hold ring entries NQ-D .. NQ-1 (NG is a
    // multiple of NQ); the next stage's first PRE A fragments go to the others.
    constexpr int PRE = kAAhead < NQ - D ? kAAhead : NQ - D;
    u32x4 b0[FN], b1[FN], a_q[NQ];
    auto mfma_group = [&](auto gc) {
      constexpr int g = decltype(gc)::value;
#pragma unroll
      for (int j = 0; j < FN; ++j) Mma<T>::run(a_q[g % NQ], (g < FM) ? b0[j] : b1[j], acc[g % FM][j]);
    };
    auto stage_head = [&](const char *slot, int lo, int hi) {
#pragma unroll
      for (int q = 0; q < kAAhead; ++q)
        if (q >= lo && q < hi) a_q[q] = rd_a(slot, q);
    };
    dma(0);
    if constexpr (!kWideSpread) {
      if (nk > 1) dma(1);
    }
    // stage 0 landed: only stage 1's DMA (half of it on a diagonal tile) may be outstanding
    waitcnt_vm(!kWideSpread && nk > 1 ? (same_ab ? DMA_PER_WAVE : PER_STAGE) : 0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = *(const u32x4 *)(lds + b_frag + j * 16 * kWideRowBytes + chunk0);
    stage_head(lds, 0, kAAhead);
#pragma unroll 1
    for (int kb = 0; kb < nk; ++kb) {
      const char *slot = lds + (kb & 1) * kWideStage;
      static_for<0, NG>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        // spread: stage kb+1's DMA goes out SPREAD instructions per group over
        // the first groups (its slot was freed by the previous barrier)
        if constexpr (kWideSpread && g < PER_STAGE / (SPREAD > 0 ? SPREAD : 1)) {
          if (kb + 1 < nk) {
#pragma unroll
            for (int q = 0; q < SPREAD; ++q) dma_piece(kb + 1, g * SPREAD + q);
          }
        }
        if constexpr (g + kAAhead < NG) a_q[(g + kAAhead) % NQ] = rd_a(slot, g + kAAhead);
        if constexpr (g < FN) b1[g] = *(const u32x4 *)(slot + b_frag + g * 16 * kWideRowBytes + chunk1);
        __builtin_amdgcn_sched_barrier(0);   // reads issue before the MFMAs that hide them
        if constexpr (g < NG - D) mfma_group(gc);
        __builtin_amdgcn_sched_barrier(0);
      });
      // every fragment read of stage kb has returned (the deferred groups'
      // operands are in registers), stage kb+1 has landed (its DMA is the
      // only one outstanding) and every wave is past both: slot kb is free
      // for stage kb+2 (issued right here, or spread over the next stage)
      if constexpr (D > 0) __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      waitcnt_vm(0);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!kWideSpread) {
        if (kb + 2 < nk) dma(kb + 2);
      }
      // stage kb+1's first fragments go out before the deferred MFMAs of
      // stage kb, which cover their latency
      const char *next = lds + ((kb + 1) & 1) * kWideStage;
      const bool more = kb + 1 < nk;
      if (more) {
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = *(const u32x4 *)(next + b_frag + j * 16 * kWideRowBytes + chunk0);
        stage_head(next, 0, PRE);
      }
      // MFMAs have no memory effects and would float back above the barrier:
      // their A operands pass through an empty asm that stays after the reads
      static_assert(D <= 2, "two deferred groups at most");
      if constexpr (D >= 1) asm volatile("" : "+v"(a_q[NQ - 1]) :: "memory");
      if constexpr (D >= 2) asm volatile("" : "+v"(a_q[NQ - 2]) :: "memory");
      __builtin_amdgcn_sched_barrier(0);
      static_for<NG - D, NG>([&](auto gc) { mfma_group(gc); });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PRE < kAAhead) {
        if (more) stage_head(next, PRE, kAAhead);
      }
    }
  }
  static_assert(NWAVES * 64 == 2 * TILE, "epilogue_u8 takes 2 TILE threads");
  epilogue_u8<T, TILE, FM, FN>(cl, mat, tm, tn, wm * WTM, wn * WTN, acc, (float *)lds);
}

// ---------------------------------------------------------------------------
// 64 x 64 block tile for fp16 / bf16 at small sizes, where a step is a chain
// of memory latencies rather than MFMA work.  Four waves of 32 x 32.  The
// operands move global -> LDS by DMA in 64-k stages of 128-byte rows (A and
// B: 16 KB), so each 8-lane group of a DMA instruction fetches one whole
// 128-byte line (8 rows x 128 bytes per instruction); 16-byte chunk c of row
// r stored at c ^ (r & 7).  Ring of RING stages: RING <= 8 holds the whole K
// and is filled up front (a K <= 64 RING panel costs one memory round trip);
// longer K refill the ring of 8, two stages consumed per barrier.  Cin is
// prefetched before the K loop.
constexpr int kSmallTile = 64;
constexpr int kSmallStage = 2 * kSmallTile * kWideRowBytes;   // 16 KB
constexpr int kSmallGroup = 2;

template <typename T, int RING>
__global__ __launch_bounds__(kThreads) void ns_gemm_small_kernel(GemmArgs args) {
  static_assert(sizeof(T) == 2, "16-bit operands only");
  static_assert(RING < 8 || RING >= 2 * kSmallGroup, "refilling ring needs two groups of look-ahead");
  constexpr int FM = 2, FN = 2;
  constexpr int PER_STAGE = 4;   // DMA instructions per stage and wave
  __shared__ __attribute__((aligned(1024))) char lds[RING * kSmallStage];

  const TileRef tr = locate_tile(args);
  const GemmClass &cl = args.cls[tr.ci];
  const int mat = tr.mat, tm = tr.tm, tn = tr.tn;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const char *A = (const char *)cl.a + ((int64_t)mat * cl.sa + (int64_t)tm * kSmallTile * cl.lda) * 2;
  const char *B = (const char *)cl.b + ((int64_t)mat * cl.sb + (int64_t)tn * kSmallTile * cl.ldb) * 2;
  const int64_t lda_b = (int64_t)cl.lda * 2, ldb_b = (int64_t)cl.ldb * 2;

  // DMA: wave w moves rows [16 w, 16 w + 16) of A and of B, 8 rows per
  // instruction; lane L covers row L / 8 of the group and physical chunk
  // L % 8, which holds logical chunk (L % 8) ^ (L / 8).
  const int dma_row = lane >> 3;
  const int dma_chunk = (lane & 7) ^ dma_row;
  const char *a_src = A + (int64_t)(wave * 16 + dma_row) * lda_b + dma_chunk * 16;
  const char *b_src = B + (int64_t)(wave * 16 + dma_row) * ldb_b + dma_chunk * 16;

  const int fr_row = lane & 15;
  const int a_frag = (wm * 32 + fr_row) * kWideRowBytes;
  const int b_frag = (kSmallTile + wn * 32 + fr_row) * kWideRowBytes;
  const int chunk0 = (((lane >> 4)) ^ (lane & 7)) * 16;
  const int chunk1 = ((4 + (lane >> 4)) ^ (lane & 7)) * 16;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float cin[FM][FN][4];
  load_cin<T, FM, FN>(cl, mat, tm * kSmallTile + wm * 32, tn * kSmallTile + wn * 32, cin);

  const int nk = cl.K / (kWideRowBytes / 2);
  if (nk > 0) {
    auto dma = [&](int kb) {
      char *dst = lds + (kb % RING) * kSmallStage + wave * 2048;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_global_load_lds((const void *)(a_src + (int64_t)j * 8 * lda_b + (int64_t)kb * kWideRowBytes),
                                         (void __attribute__((address_space(3))) *)(dst + j * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(b_src + (int64_t)j * 8 * ldb_b + (int64_t)kb * kWideRowBytes),
                                         (void __attribute__((address_space(3))) *)(dst + kSmallTile * kWideRowBytes + j * 1024),
                                         16, 0, 0);
      }
    };
    const int first = min(nk, RING);
#pragma unroll 1
    for (int kb = 0; kb < first; ++kb) dma(kb);
    int issued = first;   // stages [0, issued) have been requested
    const int ngroups = (nk + kSmallGroup - 1) / kSmallGroup;
#pragma unroll 1
    for (int g = 0; g < ngroups; ++g) {
      const int s0 = g * kSmallGroup, s1 = min(nk, s0 + kSmallGroup);
      // stages after this group may stay in flight
      waitcnt_vm(PER_STAGE * (issued - s1));
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // every wave is past group g-1: refill its slots with the stages RING ahead
      if constexpr (RING >= 8) {
        if (g > 0) {
          const int r1 = min(nk, s0 + RING);
#pragma unroll 1
          for (; issued < r1; ++issued) dma(issued);
        }
      }
#pragma unroll 1
      for (int kb = s0; kb < s1; ++kb) {
        const char *st = lds + (kb % RING) * kSmallStage;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int ch = ks ? chunk1 : chunk0;
          u32x4 fa[FM], fb[FN];
#pragma unroll
          for (int i = 0; i < FM; ++i) fa[i] = *(const u32x4 *)(st + a_frag + i * 16 * kWideRowBytes + ch);
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[j] = *(const u32x4 *)(st + b_frag + j * 16 * kWideRowBytes + ch);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) Mma<T>::run(fa[i], fb[j], acc[i][j]);
        }
      }
    }
  }
  epilogue<T, FM, FN, true>(cl, mat, cl.half && tm == tn, tm * kSmallTile + wm * 32, tn * kSmallTile + wn * 32, acc,
                            cin);
}

// ---------------------------------------------------------------------------
// Fused polynomial update of a direct Newton-Schulz step for short sides
// s <= 192 (padded to SP):
//   X'^T = alpha X^T B + beta X^T,   B = sq_alpha A A + sq_beta A,
// with A = X X^T symmetric (MONA summary, section 2 "Kernalgoritme": the quintic step a X + (b A + c A^2) X).
// At these sizes every launch is a chain of memory latencies, so the square
// A A is not a launch of its own: each block loads all of A (SP x SP) into
// LDS, forms its 64-row panel of B there (rounded to T exactly as the
// separate square product stores it), and then runs the update product for a
// group of up to poly_max_group(SP) output tiles that share the panel.
//
// X is read in its wide layout (s x l, the buffer the Gram product X X^T
// reads), so the iterate is kept in one orientation only.  Output row tile t
// of X'^T needs the 64 columns [64 t, 64 t + 64) of X over all SP rows: one
// 128-byte row per k.  Its MFMA operand (8 consecutive k of one column per
// lane) comes from two transposing LDS reads (ds_read_b64_tr_b16: within
// each 16-lane group, lane l receives element l % 4 of the 8 bytes that lane
// 4 e + l / 4 addressed, as its element e).
//
// LDS (128-byte rows, chunk c of row r at c ^ (r & 7)):
//   region 0  all of A (SP / 64 stages of SP rows); once the panel is formed:
//             X tiles 2 and 3 of the group and the epilogue's staging tiles
//   panel     SP / 64 stages of 64 rows (rows of B for this block's columns)
//   X         tiles 0 and 1 of the group (SP rows of 64 columns each)
// The panel product is computed transposed, P^T = A A_panel^T (A symmetric),
// so each lane's accumulator holds 4 consecutive k of one panel row and is
// written with one 8-byte LDS store.  Every X tile has landed before the
// first global store, so the vmcnt-counted DMA waits never count stores.
//
// Epilogue per output tile: v = alpha acc + beta X^T (X read from LDS).
// When X' alone is stored, each lane writes its 4 consecutive long-side
// entries of one X' row as one 8-byte vector, straight from the accumulator
// layout.  Otherwise (the weight update, or X'^T also wanted ahead of a
// cubic step) v is staged as fp32 in a 64 x 64 tile (two staging tiles
// alternate, so one barrier per output tile suffices); a transposed sweep
// stores X' (or applies the fp32 weight update of a wide W) and a row-major
// sweep stores X'^T (or the update of a tall W), 16 bytes per access.  The
// next tile's operands are read from LDS while the current one is finished.
template <int SP>
struct PolyLayout {
  static constexpr int A_BYTES = SP * SP * 2;
  static constexpr int P_BYTES = SP * 128;              // 64 rows over all k
  static constexpr int MAXG = SP == 192 ? 4 : 2;        // tiles 2, 3 need room in region 0
  static constexpr int S_BYTES = 64 * 64 * 4;            // one fp32 staging tile
  // staging tiles: SP = 192: region 0 after X^T tiles 2, 3, and the X^T tile 0
  // buffer once tile 0 is done; otherwise the first two slots of region 0
  static constexpr int S0_OFF = SP == 192 ? 2 * P_BYTES : 0;
  static constexpr int R0_BYTES = SP == 192 ? A_BYTES : (A_BYTES > 2 * S_BYTES ? A_BYTES : 2 * S_BYTES);
  static constexpr int TOTAL = R0_BYTES + 3 * P_BYTES;
  static_assert(MAXG <= kPolyMaxGroup, "group bound");
  static_assert(SP != 192 || (S0_OFF + S_BYTES <= A_BYTES && S_BYTES <= P_BYTES), "staging fits");
};

// Staging position of (row r, column c) of a 64 x 64 fp32 tile: 16-column
// groups permuted per row so that MFMA-layout writes (4 rows 4 apart x 16
// columns) and column reads of 16-row groups hit distinct banks, while each
// 16-column group of a row stays contiguous for row reads.
__device__ __forceinline__ int spos(int r, int c) { return r * 64 + (c ^ ((((r >> 2) ^ (r >> 4)) & 3) << 4)); }

template <typename T, int SP>
__global__ __launch_bounds__(kThreads) void ns_poly_update_kernel(GemmArgs args) {
  static_assert(sizeof(T) == 2, "16-bit operands only");
  static_assert(SP == 64 || SP == 128 || SP == 192, "short side padded to 64, 128 or 192");
  typedef PolyLayout<SP> L;
  constexpr int NST = SP / 64;          // k stages
  constexpr int NKS = 2 * NST;          // 32-k MFMA steps
  constexpr int FM1 = SP / 64;          // 16-row blocks per wave in the panel product (SP / 4 rows)
  constexpr int A_DMA = SP / 32;        // DMA instructions per wave and stage of A (8 rows each)
  constexpr int X_DMA = SP / 32;        // DMA instructions per wave for one X tile (8 rows each)
  __shared__ __attribute__((aligned(1024))) char lds[L::TOTAL];
  char *const la = lds;
  char *const lp = lds + L::R0_BYTES;
  char *const lx = lp + L::P_BYTES;

  const TileRef tr = locate_tile(args);
  const GemmClass &cl = args.cls[tr.ci];
  const int mat = tr.mat, tn = tr.tn;
  const int tm0 = tr.tm * cl.m_group;
  const int nt = min(cl.m_group, cl.m_tiles - tm0);   // in [1, MAXG] by construction
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const char *Am = (const char *)cl.b + (int64_t)mat * cl.sb * 2;
  const char *Xm = (const char *)cl.a + (int64_t)mat * cl.sa * 2;   // X, wide: SP rows of lda
  const int64_t lda_b = (int64_t)cl.lda * 2, ldb_b = (int64_t)cl.ldb * 2;
  const int dma_row = lane >> 3;
  const int dma_chunk = (lane & 7) ^ dma_row;

  // all of A, stage by stage: wave w moves rows [w SP/4, (w+1) SP/4)
#pragma unroll
  for (int kb = 0; kb < NST; ++kb) {
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
      const int r0 = wave * (SP / 4) + j * 8;
      __builtin_amdgcn_global_load_lds(
          (const void *)(Am + (int64_t)(r0 + dma_row) * ldb_b + kb * kWideRowBytes + dma_chunk * 16),
          (void __attribute__((address_space(3))) *)(la + kb * SP * kWideRowBytes + r0 * kWideRowBytes), 16, 0, 0);
    }
  }
  // LDS home of X tile t of the group
  auto xbuf = [&](int t) -> char * { return t < 2 ? lx + t * L::P_BYTES : la + (t - 2) * L::P_BYTES; };
  // X tile of output row tile tm0 + t: columns [64 (tm0 + t), +64) of X rows
  // 0 .. SP-1; wave w moves rows [w SP/4, (w+1) SP/4)
  auto dma_x = [&](int t) {
    const char *src = Xm + (int64_t)(tm0 + t) * kWideRowBytes;
    char *dst = xbuf(t);
#pragma unroll
    for (int j = 0; j < X_DMA; ++j) {
      const int r0 = wave * (SP / 4) + j * 8;
      __builtin_amdgcn_global_load_lds((const void *)(src + (int64_t)(r0 + dma_row) * lda_b + dma_chunk * 16),
                                       (void __attribute__((address_space(3))) *)(dst + r0 * kWideRowBytes), 16, 0, 0);
    }
  };
  dma_x(0);
  const int early = nt > 1 ? 2 : 1;
  if (nt > 1) dma_x(1);

  const int fr_row = lane & 15;
  const int chunk0 = ((lane >> 4) ^ (lane & 7)) * 16;
  const int chunk1 = ((4 + (lane >> 4)) ^ (lane & 7)) * 16;
  auto kchunk = [&](int ks) { return (ks & 1) ? chunk1 : chunk0; };   // 32-k half of a stage

  // ---- panel product: P^T[c][r] = sum_k A[c][k] A[r][k], r in this block's column tile
  {
    f32x4 acc[FM1][4];
#pragma unroll
    for (int i = 0; i < FM1; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int crow = wave * (SP / 4);
    u32x4 fa[2][FM1], fb[2][4];
    auto load = [&](int ks, int b) {
      const char *st = la + (ks >> 1) * SP * kWideRowBytes;
      const int ch = kchunk(ks);
#pragma unroll
      for (int i = 0; i < FM1; ++i) fa[b][i] = *(const u32x4 *)(st + (crow + i * 16 + fr_row) * kWideRowBytes + ch);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[b][j] = *(const u32x4 *)(st + (tn * 64 + j * 16 + fr_row) * kWideRowBytes + ch);
    };
    static_for<0, NST>([&](auto sc) {
      constexpr int kb = decltype(sc)::value;
      // stage kb of A has landed (later stages and the X^T tiles may be in flight)
      waitcnt_vm(A_DMA * (NST - 1 - kb) + X_DMA * early);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // both halves' fragments are read up front; the second half's reads
      // overlap the first half's MFMAs
      load(2 * kb, 0);
      load(2 * kb + 1, 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < FM1; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) Mma<T>::run(fa[h][i], fb[h][j], acc[i][j]);
    });
    // B[r][c .. c+3] = sq_alpha P + sq_beta A[r][c .. c+3], rounded to T, into the panel
    const float sa = cl.sq_alpha, sb = cl.sq_beta;
#pragma unroll
    for (int i = 0; i < FM1; ++i) {
      const int c = crow + i * 16 + 4 * (lane >> 4);
      const int coff = (c & 63) >> 3;   // 16-byte chunk of k = c within its stage row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = j * 16 + fr_row;   // panel row; A row tn * 64 + rr
        const int r = tn * 64 + rr;
        const uint2 av = *(const uint2 *)(la + (c >> 6) * SP * kWideRowBytes + r * kWideRowBytes +
                                          ((coff ^ (r & 7)) << 4) + (c & 7) * 2);
        const float a0 = (float)__builtin_bit_cast(T, (uint16_t)(av.x & 0xFFFF));
        const float a1 = (float)__builtin_bit_cast(T, (uint16_t)(av.x >> 16));
        const float a2 = (float)__builtin_bit_cast(T, (uint16_t)(av.y & 0xFFFF));
        const float a3 = (float)__builtin_bit_cast(T, (uint16_t)(av.y >> 16));
        // same rounding as the epilogue of a separate product: fma(beta, Cin,
        // alpha * acc) in fp32, then to T (the empty asm keeps the compiler
        // from fusing the fma with the conversion into one rounding)
        float v0 = __builtin_fmaf(sb, a0, sa * acc[i][j][0]), v1 = __builtin_fmaf(sb, a1, sa * acc[i][j][1]);
        float v2 = __builtin_fmaf(sb, a2, sa * acc[i][j][2]), v3 = __builtin_fmaf(sb, a3, sa * acc[i][j][3]);
        asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
        uint2 bv;
        bv.x = Pack16<T>::pair(v0, v1);
        bv.y = Pack16<T>::pair(v2, v3);
        *(uint2 *)(lp + (c >> 6) * kSmallTile * kWideRowBytes + rr * kWideRowBytes + ((coff ^ (rr & 7)) << 4) +
                   (c & 7) * 2) = bv;
      }
    }
  }
  lds_barrier();   // panel complete; region 0 (A) is free
  if constexpr (L::MAXG > 2) {
    if (nt > 2) dma_x(2);
    if (nt > 3) dma_x(3);
  }
  waitcnt_vm(0);   // every X tile of the group has landed
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- update product and epilogue for each output row tile of the group
  constexpr int FM = 2, FN = 2;
  const int b_frag = (wn * 32 + fr_row) * kWideRowBytes;
  const float alpha = cl.alpha, beta = cl.beta;
  FinalDesc fd{};
  bool fvec = false;
  if (cl.final_mode) {
    fd = cl.desc[cl.desc_base + mat];
    fvec = (fd.cols & 3) == 0 && ((((uintptr_t)fd.weight) | ((uintptr_t)fd.ortho_out)) & 15) == 0;
  }
  void *C = cl.c ? (void *)((char *)cl.c + (int64_t)mat * cl.sc * 2) : nullptr;
  void *C2 = cl.c2 ? (void *)((char *)cl.c2 + (int64_t)mat * cl.sc2 * 2) : nullptr;
  // operands of a whole tile (every k step) and its X^T entries for Cin, read
  // from LDS one tile ahead so the reads overlap the previous tile's epilogue.
  // A operand (output row m = wm 32 + 16 i + l, k = 32 ks + 8 g + 0..7, lane
  // = 16 g + l): transposing read h covers k + 4 h .. 4 h + 3; lane 16 g + j
  // addresses X row 32 ks + 8 g + 4 h + j / 4, columns m0 + 4 (j % 4) .. + 3.
  u32x4 fa[NKS][FM], fb[NKS][FN];
  uint2 cu[FM][FN];
  const int tj = lane & 15, tg = lane >> 4;
  int tr_off[2][FM];   // byte offset within a 32-k step, per half h and row block i
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = 8 * tg + 4 * h + (tj >> 2);      // row within the 32-k step (r & 7 = 4 h + tj / 4)
      const int c = wm * 32 + i * 16 + 4 * (tj & 3);  // first of 4 columns
      tr_off[h][i] = r * kWideRowBytes + (((c >> 3) ^ (r & 7)) << 4) + (c & 7) * 2;
    }
  auto load_tile = [&](int t) {
    const char *xb = xbuf(t);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const char *sx = xb + ks * 32 * kWideRowBytes;
      const char *sp = lp + (ks >> 1) * kSmallTile * kWideRowBytes;
      const int ch = kchunk(ks);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(sx + tr_off[0][i]));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4 *)(sx + tr_off[1][i]));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        fa[ks][i] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[ks][j] = *(const u32x4 *)(sp + b_frag + j * 16 * kWideRowBytes + ch);
    }
    // the tile's own X^T entries X^T[ir .. ir+3][jc] = X[tn 64 + jc][ir .. ir+3]:
    // one 8-byte read each
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int ir = wm * 32 + i * 16 + 4 * (lane >> 4);
        const int kr = tn * 64 + wn * 32 + j * 16 + (lane & 15);
        cu[i][j] = *(const uint2 *)(xb + kr * kWideRowBytes + (((ir >> 3) ^ (kr & 7)) << 4) + (ir & 7) * 2);
      }
  };
  load_tile(0);
  static_for<0, L::MAXG>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    if (t < nt) {
      f32x4 acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) Mma<T>::run(fa[ks][i], fb[ks][j], acc[i][j]);
      float cin[FM][FN][4];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = (q < 2) ? cu[i][j].x : cu[i][j].y;
            cin[i][j][q] = (float)__builtin_bit_cast(T, (uint16_t)((q & 1) ? (w >> 16) : (w & 0xFFFF)));
          }
      if (t + 1 < nt) load_tile(t + 1);
      if (!cl.final_mode && !C) {
        // X' alone: a lane's 4 accumulator rows are 4 consecutive long-side
        // entries of one X' row, stored as one 8-byte vector (the same fp32
        // fma and rounding as the staged path; the empty asm keeps the fma
        // and the conversion two roundings)
        if (C2) {
          const int row0 = (tm0 + t) * kSmallTile, col0 = tn * kSmallTile;
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int ir = wm * 32 + i * 16 + 4 * (lane >> 4);
              const int jc = wn * 32 + j * 16 + (lane & 15);
              float v0 = __builtin_fmaf(beta, cin[i][j][0], alpha * acc[i][j][0]);
              float v1 = __builtin_fmaf(beta, cin[i][j][1], alpha * acc[i][j][1]);
              float v2 = __builtin_fmaf(beta, cin[i][j][2], alpha * acc[i][j][2]);
              float v3 = __builtin_fmaf(beta, cin[i][j][3], alpha * acc[i][j][3]);
              asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
              uint2 u;
              u.x = Pack16<T>::pair(v0, v1);
              u.y = Pack16<T>::pair(v2, v3);
              *(uint2 *)((T *)C2 + (int64_t)(col0 + jc) * cl.ldc2 + row0 + ir) = u;
            }
        }
      } else {
        // v = alpha acc + beta X^T, staged (alternating staging tiles: the
        // previous barrier already ordered the sweeps of tile t - 2)
        float *stg = (t & 1) ? (SP == 192 ? (float *)lx : (float *)(la + L::S_BYTES)) : (float *)(la + L::S0_OFF);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int ir = wm * 32 + i * 16 + 4 * (lane >> 4) + q;
              const int jc = wn * 32 + j * 16 + (lane & 15);
              stg[spos(ir, jc)] = __builtin_fmaf(beta, cin[i][j][q], alpha * acc[i][j][q]);
            }
        lds_barrier();
        const int row0 = (tm0 + t) * kSmallTile;   // tile rows index the long side
        const int col0 = tn * kSmallTile;          // tile columns index the short side
        // row-major sweep: thread -> (tile row tid / 4, 16 columns)
        {
          const int r = tid >> 2, c0 = (tid & 3) * 16;
          float v[16];
          const float *src = stg + spos(r, c0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float4 x = *(const float4 *)(src + 4 * e);
            v[4 * e] = x.x; v[4 * e + 1] = x.y; v[4 * e + 2] = x.z; v[4 * e + 3] = x.w;
          }
          if (!cl.final_mode) {
            if (C) {
              T *dst = (T *)C + (int64_t)(row0 + r) * cl.ldc + col0 + c0;
              Pack<T>::copy(dst, (const float4 *)v);
              Pack<T>::copy(dst + 8, (const float4 *)(v + 8));
            }
          } else if (!fd.wide && row0 + r < fd.rows) {
            const int i = row0 + r, j0 = col0 + c0;
            const float lr = cl.lr, wd = cl.wd, gm = fd.gamma;
            float *wrow = fd.weight + (int64_t)i * fd.cols;
            float *orow = fd.ortho_out ? fd.ortho_out + (int64_t)i * fd.cols : nullptr;
            if (fvec && j0 + 16 <= fd.cols) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float4 w = *(const float4 *)(wrow + j0 + 4 * e);
                w.x = w.x - lr * (gm * v[4 * e] + wd * w.x);
                w.y = w.y - lr * (gm * v[4 * e + 1] + wd * w.y);
                w.z = w.z - lr * (gm * v[4 * e + 2] + wd * w.z);
                w.w = w.w - lr * (gm * v[4 * e + 3] + wd * w.w);
                *(float4 *)(wrow + j0 + 4 * e) = w;
                if (orow) *(float4 *)(orow + j0 + 4 * e) = make_float4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                if (j0 + e < fd.cols) {
                  const float w = wrow[j0 + e];
                  wrow[j0 + e] = w - lr * (gm * v[e] + wd * w);
                  if (orow) orow[j0 + e] = v[e];
                }
              }
            }
          }
        }
        // transposed sweep: thread -> (tile column tid / 4, 16 rows)
        if (!cl.final_mode ? (C2 != nullptr) : (bool)fd.wide) {
          const int c = tid >> 2, r0 = (tid & 3) * 16;
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] = stg[spos(r0 + e, c)];
          if (!cl.final_mode) {
            T *dst = (T *)C2 + (int64_t)(col0 + c) * cl.ldc2 + row0 + r0;
            Pack<T>::copy(dst, (const float4 *)v);
            Pack<T>::copy(dst + 8, (const float4 *)(v + 8));
          } else if (col0 + c < fd.rows) {
            // wide W: row col0 + c, columns row0 + r0 ..
            const int i = col0 + c, j0 = row0 + r0;
            const float lr = cl.lr, wd = cl.wd, gm = fd.gamma;
            float *wrow = fd.weight + (int64_t)i * fd.cols;
            float *orow = fd.ortho_out ? fd.ortho_out + (int64_t)i * fd.cols : nullptr;
            if (fvec && j0 + 16 <= fd.cols) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float4 w = *(const float4 *)(wrow + j0 + 4 * e);
                w.x = w.x - lr * (gm * v[4 * e] + wd * w.x);
                w.y = w.y - lr * (gm * v[4 * e + 1] + wd * w.y);
                w.z = w.z - lr * (gm * v[4 * e + 2] + wd * w.z);
                w.w = w.w - lr * (gm * v[4 * e + 3] + wd * w.w);
                *(float4 *)(wrow + j0 + 4 * e) = w;
                if (orow) *(float4 *)(orow + j0 + 4 * e) = make_float4(v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                if (j0 + e < fd.cols) {
                  const float w = wrow[j0 + e];
                  wrow[j0 + e] = w - lr * (gm * v[e] + wd * w);
                  if (orow) orow[j0 + e] = v[e];
                }
              }
            }
          }
        }
      }
    }
  });
}

template <typename T>
hipError_t launch_t(const GemmArgs &args, int tile, hipStream_t s) {
  switch (tile) {
    case 64:
      if constexpr (sizeof(T) == 2) {
        // ring just deep enough for the longest K of the launch (8 stages
        // and refills beyond), so more blocks fit per CU
        int kmax = 0;
        for (int c = 0; c < args.nclass; ++c) kmax = max(kmax, args.cls[c].K);
        const int nk = kmax / (kWideRowBytes / 2);
        const dim3 g(args.total_tiles), b(kThreads);
        if (nk <= 1) hipLaunchKernelGGL((ns_gemm_small_kernel<T, 1>), g, b, 0, s, args);
        else if (nk <= 2) hipLaunchKernelGGL((ns_gemm_small_kernel<T, 2>), g, b, 0, s, args);
        else if (nk <= 3) hipLaunchKernelGGL((ns_gemm_small_kernel<T, 3>), g, b, 0, s, args);
        else if (nk <= 4) hipLaunchKernelGGL((ns_gemm_small_kernel<T, 4>), g, b, 0, s, args);
        else if (nk <= 6) hipLaunchKernelGGL((ns_gemm_small_kernel<T, 6>), g, b, 0, s, args);
        else hipLaunchKernelGGL((ns_gemm_small_kernel<T, 8>), g, b, 0, s, args);
      } else {
        hipLaunchKernelGGL((ns_gemm_kernel<T, 64, 64>), dim3(args.total_tiles), dim3(kThreads), 0, s, args);
      }
      break;
    case 128:
      if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((ns_gemm_wide_kernel<T, 128>), dim3(args.total_tiles), dim3(256), 0, s, args);
      else
        hipLaunchKernelGGL((ns_gemm_kernel<T, 128, 128>), dim3(args.total_tiles), dim3(kThreads), 0, s, args);
      break;
    case 256:
      if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((ns_gemm_wide_kernel<T, 256>), dim3(args.total_tiles), dim3(512), 0, s, args);
        break;
      } else {
        return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_poly_t(const GemmArgs &args, int sp, hipStream_t s) {
  const dim3 g(args.total_tiles), b(kThreads);
  switch (sp) {
    case 64: hipLaunchKernelGGL((ns_poly_update_kernel<T, 64>), g, b, 0, s, args); break;
    case 128: hipLaunchKernelGGL((ns_poly_update_kernel<T, 128>), g, b, 0, s, args); break;
    case 192: hipLaunchKernelGGL((ns_poly_update_kernel<T, 192>), g, b, 0, s, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int poly_blocks_per_cu(int sp) {
  const int bytes = sp == 64 ? PolyLayout<64>::TOTAL : sp == 128 ? PolyLayout<128>::TOTAL : PolyLayout<192>::TOTAL;
  const int n = 160 * 1024 / bytes;
  return n < 1 ? 1 : (n > 8 ? 8 : n);
}

int poly_max_group(int sp) {
  return sp == 64 ? PolyLayout<64>::MAXG : sp == 128 ? PolyLayout<128>::MAXG : PolyLayout<192>::MAXG;
}

hipError_t launch_poly_update(const GemmArgs &args, int dtype, int sp, hipStream_t s) {
  if (args.total_tiles <= 0) return hipSuccess;
  for (int c = 0; c < args.nclass; ++c)
    if (args.cls[c].K != sp || args.cls[c].m_group < 1 || args.cls[c].m_group > poly_max_group(sp) ||
        args.cls[c].diag != 0.0f)
      return hipErrorInvalidValue;
  switch (dtype) {
    case kF16: return launch_poly_t<_Float16>(args, sp, s);
    case kBF16: return launch_poly_t<__bf16>(args, sp, s);
    default: return hipErrorInvalidValue;
  }
}

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
