// HBM-bound stages of the Muon / MONA step for gfx950.
//
//   E1  MONA difference + EMA, heavy-ball momentum, Frobenius partials
//       (MONA summary, section 2 "Kernalgoritme", steps 1-4)
//   norm_finalize  per-matrix 1 / (sqrt(d) ||M||_F), fixed summation order
//   E2  X0 = M / (sqrt(d) ||M||_F) rounded to the Newton-Schulz dtype, stored
//       in both orientations, or in the one the products read (Gram
//       Newton-Schulz post: the divisor keeps the Gram's eigenvalues inside
//       [0, 1])
//   E3  W = W - lr (gamma O + lambda W)  (MONA summary, step 4)
//
// All loads and stores are 16-byte vectors where alignment allows; every
// reduction runs in a fixed order, so results are bitwise reproducible.
#include "muon_kernels.h"

#include <math.h>

namespace muon {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_to_f32(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

template <int DT> struct Elem;
template <> struct Elem<kF32> {
  typedef float raw;
  static __device__ __forceinline__ float to_f32(raw v) { return v; }
  static __device__ __forceinline__ raw from_f32(float v) { return v; }
};
template <> struct Elem<kBF16> {
  typedef uint16_t raw;
  static __device__ __forceinline__ float to_f32(raw v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ raw from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<kF16> {
  typedef uint16_t raw;
  static __device__ __forceinline__ float to_f32(raw v) { return f16_to_f32(v); }
  static __device__ __forceinline__ raw from_f32(float v) { return f32_to_f16(v); }
};

// Four consecutive elements of a given dtype: 16 bytes (fp32) or 8 bytes.
template <int DT> struct Vec4;
template <> struct Vec4<kF32> {
  typedef float4 type;
  static __device__ __forceinline__ void unpack(const type &v, float o[4]) { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
  static __device__ __forceinline__ type pack(const float o[4]) { return make_float4(o[0], o[1], o[2], o[3]); }
};
template <int DT> struct Vec4Half {
  typedef uint2 type;
  static __device__ __forceinline__ void unpack(const type &v, float o[4]) {
    o[0] = Elem<DT>::to_f32((uint16_t)(v.x & 0xffffu));
    o[1] = Elem<DT>::to_f32((uint16_t)(v.x >> 16));
    o[2] = Elem<DT>::to_f32((uint16_t)(v.y & 0xffffu));
    o[3] = Elem<DT>::to_f32((uint16_t)(v.y >> 16));
  }
  static __device__ __forceinline__ type pack(const float o[4]) {
    type v;
    v.x = (uint32_t)Elem<DT>::from_f32(o[0]) | ((uint32_t)Elem<DT>::from_f32(o[1]) << 16);
    v.y = (uint32_t)Elem<DT>::from_f32(o[2]) | ((uint32_t)Elem<DT>::from_f32(o[3]) << 16);
    return v;
  }
};
template <> struct Vec4<kBF16> : Vec4Half<kBF16> {};
template <> struct Vec4<kF16> : Vec4Half<kF16> {};

// Streaming accesses (`nt`: non-temporal loads and stores) for calls whose
// state is far larger than the caches: measured on MI355X, a non-temporal
// read stream sustains about 7.1 TB/s against 6.4 for a plain one, and E1
// runs 7-11% faster on the Llama-shaped and tall-matrix sets; a call whose
// momentum fits in the caches keeps plain accesses (E2 re-reads M from
// cache there).  The choice is a template parameter of the kernels.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
// Loads and stores of clang vector types (the non-temporal builtins keep
// their hint on these; through HIP's float4 / uint2 structs it was lost).
template <bool NT, typename V> __device__ __forceinline__ V ld(const void *p) {
  if (NT) return __builtin_nontemporal_load((const V *)p);
  return *(const V *)p;
}
template <bool NT, typename V> __device__ __forceinline__ void st(void *p, V v) {
  if (NT) __builtin_nontemporal_store(v, (V *)p);
  else *(V *)p = v;
}
// four gradient (or previous-gradient) elements: 16 bytes of fp32 or 8 bytes
// of a 16-bit dtype
template <int DT> struct GV {
  typedef u32x2v type;
  static __device__ __forceinline__ void unpack(type v, float o[4]) {
    o[0] = Elem<DT>::to_f32((uint16_t)(v.x & 0xffffu));
    o[1] = Elem<DT>::to_f32((uint16_t)(v.x >> 16));
    o[2] = Elem<DT>::to_f32((uint16_t)(v.y & 0xffffu));
    o[3] = Elem<DT>::to_f32((uint16_t)(v.y >> 16));
  }
};
template <> struct GV<kF32> {
  typedef f32x4v type;
  static __device__ __forceinline__ void unpack(type v, float o[4]) { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
};

__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Matrix owning block `b`: begin[] is ascending with INT32_MAX past the
// last matrix, so the owner's index is the number of later entries <= b.
template <int N>
__device__ __forceinline__ int find_mat(const int32_t (&begin)[N], int b) {
  int mi = 0;
#pragma unroll
  for (int i = 1; i < N; ++i) mi += (begin[i] <= b) ? 1 : 0;
  return mi;
}

// ------------------------------------------------------------------ E1
// MODE: kE1Plain (Muon), kE1Mona (A and G_prev in their own buffers) or
// kE1Lite (MONA-Lite: one bfloat16 state C = beta_a A - (1 - beta_a) G, MONA
// summary "Efficiëntie en Implementatie"; A_k = C_{k-1} + (1 - beta_a) G_k).
// `s` is A (MONA) or C (Lite) on entry and on exit; `prev` is G_{k-1} (MONA).
template <int MODE>
__device__ __forceinline__ void e1_elem(float g, float &m, float &s, float prev, const E1Args &args) {
  if (MODE == kE1Mona) {
    const float d = args.first_step ? 0.0f : (g - prev);
    s = args.beta_a * s + (1.0f - args.beta_a) * d;
    g = g + args.alpha * s;
  } else if (MODE == kE1Lite) {
    const float a = args.first_step ? 0.0f : s + (1.0f - args.beta_a) * g;
    s = args.beta_a * a - (1.0f - args.beta_a) * g;
    g = g + args.alpha * a;
  }
  m = args.mu * m + g;
}

template <int GDT, int MODE, bool NT>
__global__ __launch_bounds__(kE1Threads) void e1_kernel(E1Args args) {
  typedef typename Elem<GDT>::raw graw;
  typedef typename Vec4<GDT>::type gvec;
  constexpr bool MONA = MODE == kE1Mona, LITE = MODE == kE1Lite;
  constexpr int G = kE1ElemsPerThread / 4;   // groups of 4 elements per thread
  const int mi = find_mat(args.begin, (int)blockIdx.x);
  const E1Mat &mt = args.mats[mi];
  const int64_t blk = (int64_t)blockIdx.x - args.begin[mi];
  const int64_t base = blk * kE1BlockElems;
  if (blk == 0 && threadIdx.x == 0 && mt.desc_idx >= 0) {
    FinalDesc d;
    d.weight = mt.weight;
    d.ortho_out = mt.ortho_out;
    d.rows = mt.rows;
    d.cols = mt.cols;
    d.gamma = mt.gamma;
    d.wide = mt.rows <= mt.cols ? 1 : 0;
    args.desc[mt.desc_idx] = d;
  }
  const int64_t numel = mt.numel;
  const graw *grad = (const graw *)mt.grad;
  graw *prev = (graw *)mt.prev;
  float *mom = mt.mom;
  float *acc = mt.accel;
  uint16_t *lite = (uint16_t *)mt.lite;
  const bool vec_ok = ((((uintptr_t)grad) | ((uintptr_t)mom) | ((uintptr_t)acc) | ((uintptr_t)prev)) & 15) == 0 &&
                      (sizeof(graw) == 4 || ((((uintptr_t)grad) | ((uintptr_t)prev)) & 7) == 0) &&
                      (((uintptr_t)lite) & 7) == 0;
  float sq = 0.0f;
  if (vec_ok) {
    // Groups of 4 elements, predicated on lying inside the matrix; every load
    // of the thread is issued before the first use (no serial tail loop).
    typedef typename GV<GDT>::type gx;
    gx gv[G], pv[G];
    f32x4v mv[G], av[G];
    u32x2v lv[G];
#pragma unroll
    for (int it = 0; it < G; ++it) {
      const int64_t e = base + ((int64_t)it * kE1Threads + threadIdx.x) * 4;
      if (e + 4 <= numel) {
        gv[it] = ld<NT, gx>(grad + e);
        mv[it] = ld<NT, f32x4v>(mom + e);
        if (MONA) {
          av[it] = ld<NT, f32x4v>(acc + e);
          if (!args.first_step) pv[it] = ld<NT, gx>(prev + e);
        }
        if (LITE && !args.first_step) lv[it] = ld<NT, u32x2v>(lite + e);
      }
    }
#pragma unroll
    for (int it = 0; it < G; ++it) {
      const int64_t e = base + ((int64_t)it * kE1Threads + threadIdx.x) * 4;
      if (e + 4 <= numel) {
        float g[4], m[4] = {mv[it].x, mv[it].y, mv[it].z, mv[it].w}, a[4] = {0, 0, 0, 0}, p[4] = {0, 0, 0, 0};
        GV<GDT>::unpack(gv[it], g);
        if (MONA) {
          a[0] = av[it].x; a[1] = av[it].y; a[2] = av[it].z; a[3] = av[it].w;
          if (!args.first_step) GV<GDT>::unpack(pv[it], p);
        }
        if (LITE && !args.first_step) GV<kBF16>::unpack(lv[it], a);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          e1_elem<MODE>(g[q], m[q], a[q], p[q], args);
          sq += m[q] * m[q];
        }
        st<NT, f32x4v>(mom + e, f32x4v{m[0], m[1], m[2], m[3]});
        if (MONA) {
          st<NT, f32x4v>(acc + e, f32x4v{a[0], a[1], a[2], a[3]});
          st<NT, gx>(prev + e, gv[it]);  // exact copy of the stored gradient
        }
        if (LITE) st<NT, u32x2v>(lite + e, __builtin_bit_cast(u32x2v, Vec4<kBF16>::pack(a)));
      } else if (e < numel) {
        // the matrix's last numel % 4 elements
        for (int64_t j = e; j < numel; ++j) {
          const graw graw_v = grad[j];
          float m = mom[j], a = 0.0f, pp = 0.0f;
          if (MONA) {
            a = acc[j];
            if (!args.first_step) pp = Elem<GDT>::to_f32(prev[j]);
          }
          if (LITE && !args.first_step) a = bf16_to_f32(lite[j]);
          e1_elem<MODE>(Elem<GDT>::to_f32(graw_v), m, a, pp, args);
          sq += m * m;
          mom[j] = m;
          if (MONA) {
            acc[j] = a;
            prev[j] = graw_v;
          }
          if (LITE) lite[j] = f32_to_bf16(a);
        }
      }
    }
  } else {
    // unaligned buffers: element by element
    for (int64_t j = base + threadIdx.x; j < numel && j < base + kE1BlockElems; j += kE1Threads) {
      const graw graw_v = grad[j];
      const float g = Elem<GDT>::to_f32(graw_v);
      float m = mom[j];
      float a = 0.0f, p = 0.0f;
      if (MONA) {
        a = acc[j];
        if (!args.first_step) p = Elem<GDT>::to_f32(prev[j]);
      }
      if (LITE && !args.first_step) a = bf16_to_f32(lite[j]);
      e1_elem<MODE>(g, m, a, p, args);
      sq += m * m;
      mom[j] = m;
      if (MONA) {
        acc[j] = a;
        prev[j] = graw_v;
      }
      if (LITE) lite[j] = f32_to_bf16(a);
    }
  }
  // fixed-order block reduction: lanes (fp64 butterfly), then waves in order
  __shared__ double wsum[kE1Threads / 64];
  double s = wave_sum((double)sq);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kE1Threads / 64; ++w) t += wsum[w];
    args.partials[mt.partial_off + blk] = t;
  }
}

// ------------------------------------------------------------------ norm
__global__ __launch_bounds__(256) void norm_kernel(NormArgs args) {
  const NormMat &mt = args.mats[blockIdx.x];
  double s = 0.0;
  for (int i = threadIdx.x; i < mt.nparts; i += 256) s += args.partials[mt.partial_off + i];
  __shared__ double wsum[4];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double t = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    // zero matrix => X0 = 0 (no epsilon); Inf/NaN propagate through the product
    const double scale = (t == 0.0) ? 0.0 : (double)args.inv_sqrt_d / sqrt(t);
    args.scales[mt.scale_idx] = (float)(scale * (double)args.store_scale);
  }
}

// ------------------------------------------------------------------ E2
// Per-matrix scale: reduced here from few partials (the same fixed order in
// every block of the matrix: one partial per lane, fp64 butterfly), else
// read from norm_kernel's output.
__device__ __forceinline__ float e2_scale(const E2Args &args, const E2Mat &mt) {
  if (mt.nparts > 0) {
    __shared__ float sh_scale;
    if (threadIdx.x < 64) {
      double p = ((int)threadIdx.x < mt.nparts) ? args.partials[mt.partial_off + threadIdx.x] : 0.0;
      p = wave_sum(p);
      if (threadIdx.x == 0) {
        // zero matrix => X0 = 0 (no epsilon); Inf/NaN propagate
        const double sc = (p == 0.0) ? 0.0 : (double)args.inv_sqrt_d / sqrt(p);
        sh_scale = (float)(sc * (double)args.store_scale);
      }
    }
    __syncthreads();
    return sh_scale;
  }
  return args.scales[mt.scale_idx];
}

// fp32 X0: 64 x 64 tiles, each thread 4 rows x 4 columns (16-byte loads and
// stores in both orientations).
// E2's loads of M stay plain by default: measured on the large sets,
// non-temporal loads made E2 15-20% slower (M was just written by E1).  X0's
// stores stay plain too: the first product reads X0 right away.
#ifndef MUON_E2_NT_LOADS
#define MUON_E2_NT_LOADS 0
#endif

template <int NDT>
__global__ __launch_bounds__(256) void e2_kernel(E2Args args) {
  typedef typename Elem<NDT>::raw nraw;
  typedef typename Vec4<NDT>::type nvec;
  __shared__ float tile[kE2Tile][kE2Tile + 1];
  const int b = blockIdx.x;
  const int mi = find_mat(args.begin, b);
  const E2Mat &mt = args.mats[mi];
  const int t = b - args.begin[mi];
  const int tr = t / mt.tiles_c, tc = t - tr * mt.tiles_c;
  const int r0 = tr * kE2Tile, c0 = tc * kE2Tile;
  // M loads first: their latency overlaps the scale reduction below
  const int cg = (threadIdx.x & 15) * 4;   // column group within the tile
  const int rr = threadIdx.x >> 4;         // 0..15
  const bool vec_ok = ((mt.cols & 3) == 0) && ((((uintptr_t)mt.mom) & 15) == 0);
  float v[4][4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = r0 + rr + 16 * it;
    const int c = c0 + cg;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[it][q] = 0.f;
    if (r < mt.rows) {
      const float *src = mt.mom + (int64_t)r * mt.cols;
      if (vec_ok && c + 4 <= mt.cols) {
        const float4 x = *(const float4 *)(src + c);
        v[it][0] = x.x; v[it][1] = x.y; v[it][2] = x.z; v[it][3] = x.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c + q < mt.cols) v[it][q] = src[c + q];
      }
    }
  }
  const float scale = e2_scale(args, mt);
  nraw *nat = (nraw *)mt.nat;
  nraw *trn = (nraw *)mt.trn;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = r0 + rr + 16 * it;
    const int c = c0 + cg;
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // round once to the storage dtype; the LDS copy holds the rounded value
      o[q] = Elem<NDT>::to_f32(Elem<NDT>::from_f32(v[it][q] * scale));
      tile[rr + 16 * it][cg + q] = o[q];
    }
    if (nat) *(nvec *)(nat + (int64_t)r * mt.ld_nat + c) = Vec4<NDT>::pack(o);
  }
  if (!trn) return;   // uniform per matrix
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int tcol = rr + 16 * it;       // column of M = row of the transposed buffer
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = tile[cg + q][tcol];
    *(nvec *)(trn + (int64_t)(c0 + tcol) * mt.ld_trn + r0 + cg) = Vec4<NDT>::pack(o);
  }
}


// 16-bit X0: 64 x 64 tiles.  Each thread loads 4 rows x 4 columns of M (16
// threads cover a row's 256 bytes), rounds them once and leaves them in LDS;
// then both layouts are written from LDS as 16-byte vectors of 8 values, 8
// threads per 128-byte line: rows of X0 (row-major) and rows of X0^T
// (columns of the tile).
__device__ __forceinline__ void store16(void *p, u32x4v v) { *(u32x4v *)p = v; }

template <int NDT, bool NT>
__global__ __launch_bounds__(256) void e2_kernel16(E2Args args) {
  __shared__ float tile[kE2Tile][kE2Tile + 1];
  const int b = blockIdx.x;
  const int mi = find_mat(args.begin, b);
  const E2Mat &mt = args.mats[mi];
  const int t = b - args.begin[mi];
  const int tr = t / mt.tiles_c, tc = t - tr * mt.tiles_c;
  const int r0 = tr * kE2Tile, c0 = tc * kE2Tile;
  const int cg = (threadIdx.x & 15) * 4;   // column group within the tile
  const int rr = threadIdx.x >> 4;         // 0..15
  const bool vec_ok = ((mt.cols & 3) == 0) && ((((uintptr_t)mt.mom) & 15) == 0);
  float v[4][4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = r0 + rr + 16 * it;
    const int c = c0 + cg;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[it][q] = 0.f;
    if (r < mt.rows) {
      const float *src = mt.mom + (int64_t)r * mt.cols;
      if (vec_ok && c + 4 <= mt.cols) {
        const f32x4v x = ld<NT && MUON_E2_NT_LOADS, f32x4v>(src + c);
        v[it][0] = x.x; v[it][1] = x.y; v[it][2] = x.z; v[it][3] = x.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c + q < mt.cols) v[it][q] = src[c + q];
      }
    }
  }
  const float scale = e2_scale(args, mt);
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int q = 0; q < 4; ++q)   // round once to the storage dtype; LDS holds the rounded value
      tile[rr + 16 * it][cg + q] = Elem<NDT>::to_f32(Elem<NDT>::from_f32(v[it][q] * scale));
  __syncthreads();
  uint16_t *nat = (uint16_t *)mt.nat;
  uint16_t *trn = (uint16_t *)mt.trn;
  const int l8 = threadIdx.x >> 3;          // 0..31: a row (or column) of the tile, per pass
  const int e8 = (threadIdx.x & 7) * 8;     // first of the 8 values this thread stores
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int line = l8 + 32 * h;
    uint32_t pn[4], pt[4];
#pragma unroll
    for (int q = 0; q < 8; q += 2) {
      pn[q / 2] = (uint32_t)Elem<NDT>::from_f32(tile[line][e8 + q]) |
                  ((uint32_t)Elem<NDT>::from_f32(tile[line][e8 + q + 1]) << 16);
      pt[q / 2] = (uint32_t)Elem<NDT>::from_f32(tile[e8 + q][line]) |
                  ((uint32_t)Elem<NDT>::from_f32(tile[e8 + q + 1][line]) << 16);
    }
    if (nat) store16(nat + (int64_t)(r0 + line) * mt.ld_nat + c0 + e8, u32x4v{pn[0], pn[1], pn[2], pn[3]});
    if (trn) store16(trn + (int64_t)(c0 + line) * mt.ld_trn + r0 + e8, u32x4v{pt[0], pt[1], pt[2], pt[3]});
  }
}

// ------------------------------------------------------------------ E3
template <int NDT>
__global__ __launch_bounds__(kE3Threads) void e3_kernel(E3Args args) {
  typedef typename Elem<NDT>::raw nraw;
  typedef typename Vec4<NDT>::type nvec;
  constexpr int G = kE3BlockElems / (kE3Threads * 4);
  const int mi = find_mat(args.begin, (int)blockIdx.x);
  const E3Mat &mt = args.mats[mi];
  const int64_t base = ((int64_t)blockIdx.x - args.begin[mi]) * kE3BlockElems;
  const nraw *o = (const nraw *)mt.o;
  const float lr = args.lr, wd = args.wd, gamma = mt.gamma, inv = mt.inv_o_scale;
  if (mt.vec_ok) {
    // cols % 4 == 0, so groups of 4 never straddle a row; every load of the
    // thread is issued before the first use
    nvec ovv[G];
    float4 wvv[G];
#pragma unroll
    for (int it = 0; it < G; ++it) {
      const int64_t e = base + ((int64_t)it * kE3Threads + threadIdx.x) * 4;
      if (e < mt.numel) {
        const int64_t i = e / mt.cols;
        const int64_t j = e - i * mt.cols;
        ovv[it] = *(const nvec *)(o + i * mt.ld_o + j);
        wvv[it] = *(const float4 *)(mt.weight + e);
      }
    }
#pragma unroll
    for (int it = 0; it < G; ++it) {
      const int64_t e = base + ((int64_t)it * kE3Threads + threadIdx.x) * 4;
      if (e >= mt.numel) continue;
      float ov[4];
      Vec4<NDT>::unpack(ovv[it], ov);
      float wv[4] = {wvv[it].x, wvv[it].y, wvv[it].z, wvv[it].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ov[q] *= inv;
        wv[q] = wv[q] - lr * (gamma * ov[q] + wd * wv[q]);
      }
      *(float4 *)(mt.weight + e) = make_float4(wv[0], wv[1], wv[2], wv[3]);
      if (mt.ortho_out) *(float4 *)(mt.ortho_out + e) = make_float4(ov[0], ov[1], ov[2], ov[3]);
    }
  } else {
    for (int64_t x = base + threadIdx.x; x < mt.numel && x < base + kE3BlockElems; x += kE3Threads) {
      const int64_t i = x / mt.cols;
      const int64_t j = x - i * mt.cols;
      const float ov = Elem<NDT>::to_f32(o[i * mt.ld_o + j]) * inv;
      const float w = mt.weight[x];
      mt.weight[x] = w - lr * (gamma * ov + wd * w);
      if (mt.ortho_out) mt.ortho_out[x] = ov;
    }
  }
}

// ------------------------------------------------------------------ AdamW
// Decoupled AdamW (MONA summary, "Ontwerprichtlijnen": vector parameters
// keep AdamW; the update is the textbook one of Loshchilov & Hutter 2019,
// Algorithm 2):  m = b1 m + (1-b1) g ; v = b2 v + (1-b2) g^2 ;
// p = p - lr wd p - (lr / (1-b1^t)) m / (sqrt(v) / sqrt(1-b2^t) + eps).
template <int GDT>
__device__ __forceinline__ void adam_elem(float g, float &p, float &m, float &v, const AdamArgs &a) {
  m = a.beta1 * m + a.one_minus_beta1 * g;
  v = a.beta2 * v + a.one_minus_beta2 * (g * g);
  const float denom = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
  p = p - a.decay * p - a.step_size * (m / denom);
}

template <int GDT>
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(AdamArgs args) {
  typedef typename Elem<GDT>::raw graw;
  typedef typename Vec4<GDT>::type gvec;
  constexpr int G = kAdamBlockElems / kAdamThreads / 4;   // groups of 4 per thread
  const int ti = find_mat(args.begin, (int)blockIdx.x);
  const AdamTensor &t = args.t[ti];
  const int64_t base = ((int64_t)blockIdx.x - args.begin[ti]) * kAdamBlockElems;
  const graw *grad = (const graw *)t.grad;
  if (t.vec_ok) {
    gvec gv[G];
    float4 pv[G], mv[G], vv[G];
#pragma unroll
    for (int it = 0; it < G; ++it) {
      const int64_t e = base + ((int64_t)it * kAdamThreads + threadIdx.x) * 4;
      if (e + 4 <= t.numel) {
        gv[it] = *(const gvec *)(grad + e);
        pv[it] = *(const float4 *)(t.param + e);
        mv[it] = *(const float4 *)(t.m + e);
        vv[it] = *(const float4 *)(t.v + e);
      }
    }
#pragma unroll
    for (int it = 0; it < G; ++it) {
      const int64_t e = base + ((int64_t)it * kAdamThreads + threadIdx.x) * 4;
      if (e + 4 <= t.numel) {
        float g[4], p[4] = {pv[it].x, pv[it].y, pv[it].z, pv[it].w}, m[4] = {mv[it].x, mv[it].y, mv[it].z, mv[it].w},
              v[4] = {vv[it].x, vv[it].y, vv[it].z, vv[it].w};
        Vec4<GDT>::unpack(gv[it], g);
#pragma unroll
        for (int q = 0; q < 4; ++q) adam_elem<GDT>(g[q], p[q], m[q], v[q], args);
        *(float4 *)(t.param + e) = make_float4(p[0], p[1], p[2], p[3]);
        *(float4 *)(t.m + e) = make_float4(m[0], m[1], m[2], m[3]);
        *(float4 *)(t.v + e) = make_float4(v[0], v[1], v[2], v[3]);
      } else if (e < t.numel) {
        for (int64_t j = e; j < t.numel; ++j) {
          float p = t.param[j], m = t.m[j], v = t.v[j];
          adam_elem<GDT>(Elem<GDT>::to_f32(grad[j]), p, m, v, args);
          t.param[j] = p;
          t.m[j] = m;
          t.v[j] = v;
        }
      }
    }
  } else {
    for (int64_t j = base + threadIdx.x; j < t.numel && j < base + kAdamBlockElems; j += kAdamThreads) {
      float p = t.param[j], m = t.m[j], v = t.v[j];
      adam_elem<GDT>(Elem<GDT>::to_f32(grad[j]), p, m, v, args);
      t.param[j] = p;
      t.m[j] = m;
      t.v[j] = v;
    }
  }
}

}  // namespace

hipError_t launch_e1(const E1Args &args, int blocks, hipStream_t s) {
  const dim3 g(blocks), b(kE1Threads);
#define MUON_E1(GDT, MODE)                                                                \
  if (args.stream) hipLaunchKernelGGL((e1_kernel<GDT, MODE, true>), g, b, 0, s, args);   \
  else hipLaunchKernelGGL((e1_kernel<GDT, MODE, false>), g, b, 0, s, args);              \
  break;
  switch (args.grad_dtype * 3 + args.mode) {
    case kF32 * 3 + kE1Plain: MUON_E1(kF32, kE1Plain)
    case kF32 * 3 + kE1Mona: MUON_E1(kF32, kE1Mona)
    case kF32 * 3 + kE1Lite: MUON_E1(kF32, kE1Lite)
    case kF16 * 3 + kE1Plain: MUON_E1(kF16, kE1Plain)
    case kF16 * 3 + kE1Mona: MUON_E1(kF16, kE1Mona)
    case kF16 * 3 + kE1Lite: MUON_E1(kF16, kE1Lite)
    case kBF16 * 3 + kE1Plain: MUON_E1(kBF16, kE1Plain)
    case kBF16 * 3 + kE1Mona: MUON_E1(kBF16, kE1Mona)
    case kBF16 * 3 + kE1Lite: MUON_E1(kBF16, kE1Lite)
    default: return hipErrorInvalidValue;
  }
#undef MUON_E1
  return hipGetLastError();
}

hipError_t launch_norm(const NormArgs &args, hipStream_t s) {
  hipLaunchKernelGGL(norm_kernel, dim3(args.nmat), dim3(256), 0, s, args);
  return hipGetLastError();
}

hipError_t launch_e2(const E2Args &args, int blocks, hipStream_t s) {
  switch (args.ns_dtype) {
    case kF32: hipLaunchKernelGGL(e2_kernel<kF32>, dim3(blocks), dim3(256), 0, s, args); break;
    case kF16:
      if (args.stream) hipLaunchKernelGGL((e2_kernel16<kF16, true>), dim3(blocks), dim3(256), 0, s, args);
      else hipLaunchKernelGGL((e2_kernel16<kF16, false>), dim3(blocks), dim3(256), 0, s, args);
      break;
    case kBF16:
      if (args.stream) hipLaunchKernelGGL((e2_kernel16<kBF16, true>), dim3(blocks), dim3(256), 0, s, args);
      else hipLaunchKernelGGL((e2_kernel16<kBF16, false>), dim3(blocks), dim3(256), 0, s, args);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_e3(const E3Args &args, int blocks, hipStream_t s) {
  switch (args.ns_dtype) {
    case kF32: hipLaunchKernelGGL(e3_kernel<kF32>, dim3(blocks), dim3(kE3Threads), 0, s, args); break;
    case kF16: hipLaunchKernelGGL(e3_kernel<kF16>, dim3(blocks), dim3(kE3Threads), 0, s, args); break;
    case kBF16: hipLaunchKernelGGL(e3_kernel<kBF16>, dim3(blocks), dim3(kE3Threads), 0, s, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamArgs &args, int blocks, hipStream_t s) {
  switch (args.grad_dtype) {
    case kF32: hipLaunchKernelGGL(adamw_kernel<kF32>, dim3(blocks), dim3(kAdamThreads), 0, s, args); break;
    case kF16: hipLaunchKernelGGL(adamw_kernel<kF16>, dim3(blocks), dim3(kAdamThreads), 0, s, args); break;
    case kBF16: hipLaunchKernelGGL(adamw_kernel<kBF16>, dim3(blocks), dim3(kAdamThreads), 0, s, args); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
