// Host side of libmuon: argument checks, workspace layout and the stage
// schedules of the Muon / MONA step (C ABI declared in include/muon.h).
//
// Order of a step (MONA summary, section 2 "Kernalgoritme"; the acceleration
// comes before orthogonalisation per "Ontwerprichtlijnen"):
//   E1    MONA + momentum + Frobenius partials          (HBM-bound)
//   norm  per-matrix 1 / (sqrt(d) ||M||_F)
//   E2    X0 in the Newton-Schulz dtype, both orientations (HBM-bound)
//   NS    direct:  per step  A = X X^T (half) ; B = b A + c A^2 (half) ;
//                            X^T <- a X^T + X^T B      (writes X and X^T)
//         Gram:    R = X X^T ; per step P = a I + b R + c R^2 ; Q <- Q P ;
//                  R <- (R P) P ; restarts re-form Y <- Y Q / sqrt(d) and R ;
//                  O = Y Q        (Gram Newton-Schulz post, main body)
//   E3    W <- W - lr (gamma O + lambda W)               (HBM-bound)
//
// Matrices are grouped into classes of equal (short side s, long side l);
// wide and tall matrices of the same (s, l) share a class because the
// iteration works on both orientations of the iterate.  Every NS launch
// covers all classes that use the same tile size.
#include "muon.h"
#include "muon_kernels.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

using namespace muon;

namespace {

thread_local std::string g_last_error;

muon_status fail(muon_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr int kMaxSteps = 64;
static_assert(sizeof(GemmArgs) <= 4096 && sizeof(E1Args) <= 4096 && sizeof(E2Args) <= 4096 &&
                  sizeof(E3Args) <= 4096 && sizeof(NormArgs) <= 4096 && sizeof(AdamArgs) <= 4096 &&
                  sizeof(LmThinArgs) <= 4096 && sizeof(LmEigArgs) <= 4096 && sizeof(LmPadArgs) <= 4096 &&
                  sizeof(LmFinalArgs) <= 4096,
              "kernel arguments must stay within 4 KB");
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxNumel = (int64_t(1) << 31) - 1;

int elem_size(int dt) { return dt == kF32 ? 4 : 2; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Settings {
  int grad_dtype = kF32;
  int ns_dtype = kF32;
  std::vector<double> coeffs;   // 3 * K
  double divisor = 1.0;
  int restart_every = 0;
  int64_t step = 0;
  // LiMuon
  const float *sketch = nullptr;
  int64_t sketch_ld = 0;
  int rank = 0, oversample = 0, power_iters = 0;
  double rcond = 0.0;
};

// LiMuon buffers of a class (indices into ClassInfo::lm): the padded test
// matrix (shared by the class) and the (k + p)-wide panels of each matrix.
enum LmBuf { kLmOmt = 0, kLmY, kLmQ, kLmQ2, kLmQt, kLmZ, kLmZ2, kLmZ2t, kLmW, kLmT, kLmP, kLmBufs };

struct ClassInfo {
  int64_t s = 0, l = 0;
  int tile = 64;
  int64_t Sp = 0, Lp = 0;
  int desc_base = 0;               // first FinalDesc slot of the class
  std::vector<int> members;
  size_t X[2] = {0, 0}, XT[2] = {0, 0};
  size_t sq[5] = {0, 0, 0, 0, 0};   // direct: A, B ; gram: R, T, P, Q, Qspare
  size_t lm[kLmBufs] = {};         // LiMuon panels
  int lm_part_base = 0;            // first fp64 Gram partial slot (LiMuon)
  int lm_chunks_s = 0, lm_chunks_l = 0;   // Gram partials (64-row tiles) of an s-row / l-row panel
};

struct Plan {
  int n = 0;
  int K = 0;
  muon_variant variant = MUON_NS_DIRECT;
  Settings set;
  std::vector<ClassInfo> classes;
  std::vector<int> cls_of, idx_in_cls;
  std::vector<int> e1_blocks, partial_off;
  size_t off_partials = 0, off_scales = 0, off_desc = 0, total = 0;
  size_t off_lm_parts = 0;         // LiMuon fp64 Gram partials
};

bool is_limuon(const Plan &plan) { return plan.variant == MUON_LIMUON; }
// The step ends in an orthogonalisation product that applies the update
// (otherwise E3 applies it to X0).
bool has_products(const Plan &plan) { return is_limuon(plan) || plan.K > 0; }

bool is_finite(double v) { return std::isfinite(v); }

// Largest square block tile whose zero padding of the short side stays under
// 7% (the padded s x s products grow with its square); small sides use 64.
#ifndef MUON_PAD_LIMIT
#define MUON_PAD_LIMIT 1.07
#endif
int pick_tile(int64_t s, int64_t l, int ns_dtype) {
  (void)l;
  for (int t : {256, 128}) {
    if (t == 256 && ns_dtype == kF32) continue;   // the 256 tile is 16-bit only
    if (s < 2 * t) continue;
    if ((double)round_up(s, t) <= MUON_PAD_LIMIT * (double)s) return t;
  }
  return 64;
}

muon_status read_options(const muon_options *o, int ns_steps, muon_variant v, Settings &s) {
  s = Settings();
  muon_options d;
  muon_options_init(&d);
  if (!o) o = &d;
  if (o->grad_dtype != MUON_F32 && o->grad_dtype != MUON_F16 && o->grad_dtype != MUON_BF16)
    return fail(MUON_ERR_UNSUPPORTED, "unknown grad_dtype %d", (int)o->grad_dtype);
  if (o->ns_dtype != MUON_F32 && o->ns_dtype != MUON_F16 && o->ns_dtype != MUON_BF16)
    return fail(MUON_ERR_UNSUPPORTED, "unknown ns_dtype %d", (int)o->ns_dtype);
  // muon_dtype values equal the internal DType values.
  s.grad_dtype = (int)o->grad_dtype;
  s.ns_dtype = (int)o->ns_dtype;
  if (!is_finite(o->divisor) || o->divisor < 1.0f) return fail(MUON_ERR_INVALID_ARG, "divisor must be finite and >= 1 (got %g)", (double)o->divisor);
  if (o->restart_every < 0) return fail(MUON_ERR_INVALID_ARG, "restart_every must be >= 0");
  if (o->step < 0) return fail(MUON_ERR_INVALID_ARG, "step must be >= 0");
  s.divisor = o->divisor;
  s.restart_every = o->restart_every;
  s.step = o->step;
  if (v == MUON_LIMUON) {
    if (s.ns_dtype != kF32)
      return fail(MUON_ERR_UNSUPPORTED, "LiMuon runs its products with fp32 operands: ns_dtype must be MUON_F32");
    if (!o->sketch) return fail(MUON_ERR_INVALID_ARG, "LiMuon needs a sketch (Gaussian test matrix)");
    if (o->rank < 1) return fail(MUON_ERR_INVALID_ARG, "LiMuon rank must be >= 1 (got %d)", (int)o->rank);
    if (o->oversample < 0) return fail(MUON_ERR_INVALID_ARG, "LiMuon oversample must be >= 0");
    if ((int64_t)o->rank + o->oversample > kLmKP)
      return fail(MUON_ERR_INVALID_ARG, "LiMuon rank + oversample must be <= %d (got %d)", kLmKP,
                  (int)(o->rank + o->oversample));
    if (o->power_iters < 0 || o->power_iters > 16) return fail(MUON_ERR_INVALID_ARG, "LiMuon power_iters must lie in [0, 16]");
    if (!is_finite(o->rcond) || o->rcond < 0.0f || o->rcond >= 1.0f)
      return fail(MUON_ERR_INVALID_ARG, "LiMuon rcond must lie in [0, 1)");
    s.sketch = o->sketch;
    s.sketch_ld = o->sketch_ld;
    s.rank = o->rank;
    s.oversample = o->oversample;
    s.power_iters = o->power_iters;
    s.rcond = o->rcond;
  }
  s.coeffs.resize(3 * (size_t)ns_steps);
  for (int k = 0; k < ns_steps; ++k) {
    for (int j = 0; j < 3; ++j) {
      double v;
      if (o->coeffs) {
        v = o->coeffs[3 * k + j];
        if (!is_finite(v)) return fail(MUON_ERR_INVALID_ARG, "coeffs[%d][%d] is not finite", k, j);
      } else {
        static const double q[3] = {15.0 / 8.0, -5.0 / 4.0, 3.0 / 8.0};
        v = q[j];
      }
      s.coeffs[3 * k + j] = v;
    }
  }
  return MUON_OK;
}

struct Range {
  uintptr_t lo, hi;
  int param;
  const char *what;
};

muon_status check_params(const muon_param *p, int n, const Settings &set) {
  std::vector<Range> ranges;
  ranges.reserve((size_t)n * 6 + 1);
  if (set.sketch) {
    int64_t lmax = 0;
    for (int i = 0; i < n; ++i) lmax = std::max(lmax, std::max(p[i].rows, p[i].cols));
    if (set.sketch_ld < std::max<int64_t>(lmax, 1))
      return fail(MUON_ERR_INVALID_ARG, "sketch_ld %lld is below the longest side %lld", (long long)set.sketch_ld,
                  (long long)lmax);
    if (set.sketch_ld > kMaxDim) return fail(MUON_ERR_UNSUPPORTED, "sketch_ld exceeds the supported size");
    const uint64_t kp = (uint64_t)(set.rank + set.oversample);
    ranges.push_back({(uintptr_t)set.sketch, (uintptr_t)set.sketch + kp * (uint64_t)set.sketch_ld * 4, -1, "sketch"});
  }
  for (int i = 0; i < n; ++i) {
    const muon_param &q = p[i];
    if (!q.weight || !q.grad || !q.momentum) return fail(MUON_ERR_INVALID_ARG, "param %d: weight, grad and momentum must be non-NULL", i);
    if ((q.accel == nullptr) != (q.prev_grad == nullptr))
      return fail(MUON_ERR_INVALID_ARG, "param %d: accel and prev_grad must both be given or both be NULL", i);
    if (q.mona_lite && q.accel)
      return fail(MUON_ERR_INVALID_ARG, "param %d: mona_lite cannot be combined with accel / prev_grad", i);
    if (q.rows < 1 || q.cols < 1) return fail(MUON_ERR_INVALID_ARG, "param %d: rows and cols must be >= 1", i);
    if (q.rows > kMaxDim || q.cols > kMaxDim || q.rows * q.cols > kMaxNumel)
      return fail(MUON_ERR_UNSUPPORTED, "param %d: %lld x %lld exceeds the supported size", i, (long long)q.rows, (long long)q.cols);
    if (!is_finite(q.gamma)) return fail(MUON_ERR_INVALID_ARG, "param %d: gamma is not finite", i);
    const uint64_t ne = (uint64_t)(q.rows * q.cols);
    const uint64_t gb = ne * (uint64_t)elem_size(set.grad_dtype);
    ranges.push_back({(uintptr_t)q.weight, (uintptr_t)q.weight + ne * 4, i, "weight"});
    ranges.push_back({(uintptr_t)q.grad, (uintptr_t)q.grad + gb, i, "grad"});
    ranges.push_back({(uintptr_t)q.momentum, (uintptr_t)q.momentum + ne * 4, i, "momentum"});
    if (q.accel) {
      ranges.push_back({(uintptr_t)q.accel, (uintptr_t)q.accel + ne * 4, i, "accel"});
      ranges.push_back({(uintptr_t)q.prev_grad, (uintptr_t)q.prev_grad + gb, i, "prev_grad"});
    }
    if (q.ortho_out) ranges.push_back({(uintptr_t)q.ortho_out, (uintptr_t)q.ortho_out + ne * 4, i, "ortho_out"});
    if (q.mona_lite) ranges.push_back({(uintptr_t)q.mona_lite, (uintptr_t)q.mona_lite + ne * 2, i, "mona_lite"});
  }
  std::sort(ranges.begin(), ranges.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
  for (size_t i = 1; i < ranges.size(); ++i) {
    const Range &a = ranges[i - 1], &b = ranges[i];
    // two read-only grads may not overlap either: every buffer is distinct
    if (b.lo < a.hi)
      return fail(MUON_ERR_INVALID_ARG, "buffers overlap: param %d %s and param %d %s", a.param, a.what, b.param, b.what);
  }
  return MUON_OK;
}

muon_status build_plan(const muon_param *p, int n, int ns_steps, muon_variant v, const muon_options *o, Plan &plan) {
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && !p) return fail(MUON_ERR_INVALID_ARG, "params is NULL");
  if (ns_steps < 0 || ns_steps > kMaxSteps) return fail(MUON_ERR_INVALID_ARG, "ns_steps must be in [0, %d]", kMaxSteps);
  if (v != MUON_NS_DIRECT && v != MUON_NS_GRAM && v != MUON_LIMUON)
    return fail(MUON_ERR_INVALID_ARG, "unknown variant %d", (int)v);
  muon_status st = read_options(o, ns_steps, v, plan.set);
  if (st != MUON_OK) return st;
  st = check_params(p, n, plan.set);
  if (st != MUON_OK) return st;
  plan.n = n;
  plan.K = ns_steps;
  plan.variant = v;
  plan.cls_of.assign(n, -1);
  plan.idx_in_cls.assign(n, -1);
  plan.e1_blocks.assign(n, 0);
  plan.partial_off.assign(n, 0);
  int64_t parts = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t s = std::min(p[i].rows, p[i].cols), l = std::max(p[i].rows, p[i].cols);
    int c = -1;
    for (size_t k = 0; k < plan.classes.size(); ++k)
      if (plan.classes[k].s == s && plan.classes[k].l == l) c = (int)k;
    if (c < 0) {
      ClassInfo ci;
      ci.s = s;
      ci.l = l;
      // (LiMuon: fp32, so 64 or 128; the 128 tile's staged epilogue writes
      // the weight update of its last product along W's rows)
      ci.tile = pick_tile(s, l, plan.set.ns_dtype);
      ci.Sp = round_up(s, ci.tile);
      ci.Lp = round_up(l, ci.tile);
      plan.classes.push_back(ci);
      c = (int)plan.classes.size() - 1;
    }
    plan.cls_of[i] = c;
    plan.idx_in_cls[i] = (int)plan.classes[c].members.size();
    plan.classes[c].members.push_back(i);
    const int64_t ne = p[i].rows * p[i].cols;
    plan.e1_blocks[i] = (int)((ne + kE1BlockElems - 1) / kE1BlockElems);
    plan.partial_off[i] = (int)parts;
    parts += plan.e1_blocks[i];
  }
  size_t off = 0;
  plan.off_partials = off;
  off = align256(off + (size_t)parts * sizeof(double));
  plan.off_scales = off;
  off = align256(off + (size_t)std::max(n, 1) * sizeof(float));
  plan.off_desc = off;
  off = align256(off + (size_t)std::max(n, 1) * sizeof(FinalDesc));
  {
    int base = 0;
    for (ClassInfo &c : plan.classes) {
      c.desc_base = base;
      base += (int)c.members.size();
    }
  }
  const size_t es = (size_t)elem_size(plan.set.ns_dtype);
  if (v == MUON_LIMUON) {
    // X0 in both orientations, the class's padded test matrix, the panels,
    // and the fp64 Gram partials (one set per matrix, enough chunks for an
    // l-row panel)
    int slots = 0;
    for (ClassInfo &c : plan.classes) {
      const size_t cnt = c.members.size();
      const size_t rect = (size_t)c.Sp * (size_t)c.Lp * es * cnt;
      c.X[0] = off; off = align256(off + rect);
      c.XT[0] = off; off = align256(off + rect);
      c.X[1] = c.X[0];
      c.XT[1] = c.XT[0];
      const size_t kp = (size_t)kLmKP;
      const size_t sizes[kLmBufs] = {kp * (size_t)c.Lp * 4,                                     // omt (shared)
                                     (size_t)c.Sp * kp * 4 * cnt, (size_t)c.Sp * kp * 4 * cnt,   // y, q
                                     (size_t)c.Sp * kp * 4 * cnt, (size_t)c.Sp * kp * 4 * cnt,   // q2, qt
                                     (size_t)c.Lp * kp * 4 * cnt, (size_t)c.Lp * kp * 4 * cnt,   // z, z2
                                     (size_t)c.Lp * kp * 4 * cnt,                                // z2t
                                     kp * kp * 4 * cnt, kp * kp * 4 * cnt,                       // w, t
                                     (size_t)c.Sp * kp * 4 * cnt};                               // p
      for (int j = 0; j < kLmBufs; ++j) { c.lm[j] = off; off = align256(off + sizes[j]); }
      c.lm_chunks_s = (int)(c.Sp / kThinRows);
      c.lm_chunks_l = (int)(c.Lp / kThinRows);
      c.lm_part_base = slots;
      slots += (int)cnt * c.lm_chunks_l;
    }
    const size_t kp = (size_t)(plan.set.rank + plan.set.oversample);
    plan.off_lm_parts = off;
    off = align256(off + (size_t)slots * kp * kp * sizeof(double));
  } else {
    for (ClassInfo &c : plan.classes) {
      const size_t cnt = c.members.size();
      const size_t rect = (size_t)c.Sp * (size_t)c.Lp * es * cnt;
      const size_t sqb = (size_t)c.Sp * (size_t)c.Sp * es * cnt;
      for (int j = 0; j < 2; ++j) {
        c.X[j] = off; off = align256(off + rect);
        c.XT[j] = off; off = align256(off + rect);
      }
      const int nsq = (v == MUON_NS_DIRECT) ? 2 : 5;
      for (int j = 0; j < nsq; ++j) { c.sq[j] = off; off = align256(off + sqb); }
    }
  }
  plan.total = std::max<size_t>(off, 256);
  return MUON_OK;
}

// ---------------------------------------------------------------- scales
// fp16 buffers are stored multiplied by a power of two chosen from a bound on
// their entries, so that small entries stay in fp16's normal range; the
// scaling is exact and undone in the next epilogue.  bf16 and fp32 have
// fp32's exponent range and use 1.
struct Scaler {
  bool active;
  double pick(double bound) const {
    if (!active) return 1.0;
    if (!(bound > 0.0) || !std::isfinite(bound)) return 1.0;
    int e = (int)std::floor(std::log2(32768.0 / bound));
    e = std::max(-14, std::min(24, e));
    return std::ldexp(1.0, e);
  }
};

// sup over x in [0, hi] of |f(x)|, f one of: 0 p(x)=a x+b x^3+c x^5,
// 1 q(x)=a+b x^2+c x^4, 2 h(x)=b x^2+c x^4, 3 x p(x)
double sup_poly(double a, double b, double c, double hi, int which) {
  double best = 0.0;
  const int N = 4096;
  for (int i = 0; i <= N; ++i) {
    const double x = hi * (double)i / N, x2 = x * x;
    double f;
    switch (which) {
      case 0: f = x * (a + x2 * (b + c * x2)); break;
      case 1: f = a + x2 * (b + c * x2); break;
      case 2: f = x2 * (b + c * x2); break;
      default: f = x2 * (a + x2 * (b + c * x2)); break;
    }
    best = std::max(best, std::fabs(f));
  }
  return best * 1.0001;
}

bool restart_due(int k, int r) { return r > 0 && k > 1 && (k - 1) % r == 0; }

// Optional HIP-event timing (muon_trace): one interval per launch, or per
// run of consecutive launches of one stage (group mode; the run's end event
// is recorded when the run closes, so no event separates its launches).
struct Tracer {
  muon_trace *t;
  hipStream_t s;
  int open = -1;   // group mode: interval still accepting launches
  hipError_t close() {
    if (!t || open < 0) return hipSuccess;
    const int i = open;
    open = -1;
    return hipEventRecord((hipEvent_t)t->events[2 * i + 1], s);
  }
  template <typename F>
  hipError_t run(int stage, double work, F &&launch) {
    if (!t) return launch();
    if (t->group && open >= 0 && t->stages[open] == stage) {
      hipError_t e = launch();
      if (e != hipSuccess) return e;
      t->work[open] += work;
      t->launches[open] += 1;
      return hipSuccess;
    }
    hipError_t e = close();
    if (e != hipSuccess) return e;
    const int i = t->count;
    const bool rec = i < t->capacity;
    if (rec) {
      e = hipEventRecord((hipEvent_t)t->events[2 * i], s);
      if (e != hipSuccess) return e;
    }
    e = launch();
    if (e != hipSuccess) return e;
    if (rec) {
      t->stages[i] = stage;
      t->work[i] = work;
      if (t->launches) t->launches[i] = 1;
      if (t->group) {
        open = i;
      } else {
        e = hipEventRecord((hipEvent_t)t->events[2 * i + 1], s);
        if (e != hipSuccess) return e;
      }
    }
    t->count++;
    return hipSuccess;
  }
};

// Workgroup -> tile order of a launch (GemmArgs::xcd_group), measured with
// the bench on each workload: 256-tile launches deal every class over all
// XCDs (an eighth of each class per XCD when the launch holds several
// classes, runs of 16 tiles when it holds one); the 64 and 128 tiles and the
// fused update (tile 0 here) keep one contiguous run per XCD.
void set_order(GemmArgs &a, int tile) {
  a.xcd_group = tile != 256 ? 0 : (a.nclass > 1 ? kXcdByClass : kXcdGroup);
  if (a.xcd_group == kXcdByClass) set_xcd_order(a);
}

// One NS product for every class: built per class, launched grouped by tile.
// per_flops[c] is the algorithmic FLOP count of one matrix of class c (true,
// unpadded sizes; a half product counts only its upper triangle).
struct StageBuilder {
  const Plan &plan;
  char *ws;
  Tracer &tr;
  std::vector<GemmClass> per_class;
  std::vector<double> per_flops;
  std::vector<char> skip;   // classes launched elsewhere in this stage
  explicit StageBuilder(const Plan &p, char *w, Tracer &t) : plan(p), ws(w), tr(t) {
    per_class.resize(p.classes.size());
    per_flops.assign(p.classes.size(), 0.0);
    skip.assign(p.classes.size(), 0);
  }
  hipError_t launch() {
    for (int tile : {64, 128, 256}) {
      GemmArgs args;
      auto reset = [&]() {
        std::memset(&args, 0, sizeof(args));
        for (int i = 0; i < kGemmMaxClasses; ++i) args.tile_begin[i] = INT32_MAX;
      };
      reset();
      double flops = 0.0;
      auto go = [&]() -> hipError_t {
        GemmArgs a = args;
        set_order(a, tile);
        const int dt = plan.set.ns_dtype;
        return tr.run(MUON_STAGE_GEMM, flops, [&]() { return launch_gemm(a, dt, tile, tr.s); });
      };
      for (size_t c = 0; c < per_class.size(); ++c) {
        if (plan.classes[c].tile != tile || skip[c]) continue;
        GemmClass g = per_class[c];
        if (args.nclass == kGemmMaxClasses) {
          hipError_t e = go();
          if (e != hipSuccess) return e;
          reset();
          flops = 0.0;
        }
        args.tile_begin[args.nclass] = args.total_tiles;
        args.cls[args.nclass++] = g;
        args.total_tiles += g.tiles_per_mat * g.count;
        flops += per_flops[c] * (double)g.count;
      }
      if (args.nclass > 0) {
        hipError_t e = go();
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  }
};

// Algorithmic FLOPs: half product of an s x s result over k: s (s + 1) k;
// full s x l result over s: 2 s^2 l.
double half_flops(const ClassInfo &c, int64_t k) { return (double)c.s * (double)(c.s + 1) * (double)k; }
double full_flops(const ClassInfo &c) { return 2.0 * (double)c.s * (double)c.s * (double)c.l; }

// Fill a GemmClass for class c: C (m x n) = alpha * A B^T + beta * Cin + diag I.
GemmClass make_gemm(const ClassInfo &c, size_t es, char *ws, size_t a, int64_t a_rows, int64_t a_ld,
                    size_t b, int64_t b_rows, int64_t b_ld, int64_t K, bool half) {
  GemmClass g;
  std::memset(&g, 0, sizeof(g));
  g.a = ws + a;
  g.b = ws + b;
  g.sa = a_rows * a_ld;
  g.sb = b_rows * b_ld;
  g.lda = (int32_t)a_ld;
  g.ldb = (int32_t)b_ld;
  g.K = (int32_t)K;
  g.tiles_m = (int32_t)(a_rows / c.tile);
  g.tiles_n = (int32_t)(b_rows / c.tile);
  g.half = half ? 1 : 0;
  g.tiles_per_mat = half ? g.tiles_m * (g.tiles_m + 1) / 2 : g.tiles_m * g.tiles_n;
  g.count = (int32_t)c.members.size();
  g.diag_limit = (int32_t)c.s;
  g.alpha = 1.0f;
  (void)es;
  return g;
}

void set_out(GemmClass &g, char *ws, size_t cbuf, int64_t c_rows, int64_t c_ld, bool has_c) {
  if (has_c) {
    g.c = ws + cbuf;
    g.sc = c_rows * c_ld;
    g.ldc = (int32_t)c_ld;
  }
}
void set_out2(GemmClass &g, char *ws, size_t cbuf, int64_t c_rows, int64_t c_ld) {
  g.c2 = ws + cbuf;
  g.sc2 = c_rows * c_ld;
  g.ldc2 = (int32_t)c_ld;
}
void set_in(GemmClass &g, char *ws, size_t cbuf, int64_t c_rows, int64_t c_ld) {
  g.cin = ws + cbuf;
  g.scin = c_rows * c_ld;
  g.ldcin = (int32_t)c_ld;
}

// Turn the iteration's last product into the fused decoupled update.
void set_final(GemmClass &g, const Plan &plan, const ClassInfo &cl, char *ws, float lr, float wd) {
  g.c = nullptr;
  g.c2 = nullptr;
  g.final_mode = 1;
  g.desc_base = cl.desc_base;
  g.desc = (const FinalDesc *)(ws + plan.off_desc);
  g.lr = lr;
  g.wd = wd;
}

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(MUON_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Output of the NS schedule: which buffer holds O and its storage scale.
struct NsResult {
  int cur;          // index into X / XT ping-pong
  double scale;     // storage scale of O
};

// Scalars of the direct iteration's products, step by step, with the
// storage scales of fp16 buffers and the restart factors folded in.  The
// last update yields O in true scale.
struct DirectStep {
  double syrk_alpha;          // A = syrk_alpha X X^T   (B itself when cubic)
  double sq_alpha, sq_beta;   // B = sq_alpha A A + sq_beta A
  double upd_alpha, upd_beta; // X'^T = upd_alpha X^T B + upd_beta X^T
  bool cubic;
};

std::vector<DirectStep> direct_steps(const Plan &plan, double sx0) {
  const Scaler S{plan.set.ns_dtype == kF16};
  const double d = plan.set.divisor;
  double sigma = 1.0 / std::sqrt(d);
  double sX = sx0;
  std::vector<DirectStep> out;
  for (int k = 1; k <= plan.K; ++k) {
    const double a = plan.set.coeffs[3 * (k - 1)], b = plan.set.coeffs[3 * (k - 1) + 1], c = plan.set.coeffs[3 * (k - 1) + 2];
    const double rs = restart_due(k, plan.set.restart_every) ? 1.0 / std::sqrt(d) : 1.0;
    sigma *= rs;
    DirectStep st{};
    st.cubic = (c == 0.0);
    const double sA = S.pick(sigma * sigma);
    const double sB = S.pick(sup_poly(0.0, b, c, sigma, 2));
    if (st.cubic) {
      st.syrk_alpha = sB * b * rs * rs / (sX * sX);
    } else {
      st.syrk_alpha = sA * rs * rs / (sX * sX);
      st.sq_alpha = c * sB / (sA * sA);
      st.sq_beta = b * sB / sA;
    }
    const double sigma_new = sup_poly(a, b, c, sigma, 0);
    const double sXn = (k == plan.K) ? 1.0 : S.pick(sigma_new);
    st.upd_alpha = sXn * rs / (sX * sB);
    st.upd_beta = a * rs * sXn / sX;
    out.push_back(st);
    sigma = sigma_new;
    sX = sXn;
  }
  return out;
}

// Direct steps of classes with a short side of at most 192 (16-bit, 64
// tiles) form B = b A + c A^2 inside the update launch
// (ns_poly_update_kernel) instead of in a launch of its own: at these sizes
// a launch costs more than the redundant panel products.  That kernel reads
// the iterate in its wide layout X only, so X^T is written only for a cubic
// step's separate update product (c = 0: no square to fuse).
bool poly_fused(const Plan &plan, const ClassInfo &cl) {
  return plan.set.ns_dtype != kF32 && cl.tile == 64 && cl.Sp <= 192;
}

bool step_cubic(const Plan &plan, int k) { return plan.set.coeffs[3 * (k - 1) + 2] == 0.0f; }

// X0^T is needed only when the first product to read the iterate is a
// separate update product: Gram, or a direct first step that is cubic or not
// fused.
bool needs_x0_transposed(const Plan &plan, const ClassInfo &cl) {
  return !(plan.variant == MUON_NS_DIRECT && plan.K > 0 && poly_fused(plan, cl) && !step_cubic(plan, 1));
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Launch the fused update of every poly_fused class, one launch per padded
// short side.  Output row tiles are grouped per block (sharing the block's
// panel of B) just enough for the launch to fit the device in one wave of
// blocks.
hipError_t launch_poly_stage(const Plan &plan, Tracer &tr, const std::vector<GemmClass> &gc,
                             const std::vector<double> &flops, const std::vector<char> &use) {
  for (int sp : {64, 128, 192}) {
    int64_t pairs = 0;
    for (size_t c = 0; c < gc.size(); ++c)
      if (use[c] && plan.classes[c].Sp == sp) pairs += (int64_t)gc[c].count * gc[c].m_tiles * gc[c].tiles_n;
    if (pairs == 0) continue;
    const int64_t cap = (int64_t)device_cus() * poly_blocks_per_cu(sp);
    const int group = (int)std::min<int64_t>(poly_max_group(sp), std::max<int64_t>(1, (pairs + cap - 1) / cap));
    GemmArgs args;
    double work = 0.0;
    auto reset = [&]() {
      std::memset(&args, 0, sizeof(args));
      for (int i = 0; i < kGemmMaxClasses; ++i) args.tile_begin[i] = INT32_MAX;
      work = 0.0;
    };
    auto go = [&]() -> hipError_t {
      GemmArgs a = args;
      set_order(a, 0);
      const int dt = plan.set.ns_dtype;
      return tr.run(MUON_STAGE_GEMM, work, [&]() { return launch_poly_update(a, dt, sp, tr.s); });
    };
    reset();
    for (size_t c = 0; c < gc.size(); ++c) {
      if (!use[c] || plan.classes[c].Sp != sp) continue;
      GemmClass g = gc[c];
      g.m_group = group;
      g.tiles_m = (g.m_tiles + group - 1) / group;
      g.tiles_per_mat = g.tiles_m * g.tiles_n;
      if (args.nclass == kGemmMaxClasses) {
        hipError_t e = go();
        if (e != hipSuccess) return e;
        reset();
      }
      args.tile_begin[args.nclass] = args.total_tiles;
      args.cls[args.nclass++] = g;
      args.total_tiles += g.tiles_per_mat * g.count;
      work += flops[c] * (double)g.count;
    }
    if (args.nclass > 0) {
      hipError_t e = go();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

muon_status run_direct(const Plan &plan, char *ws, Tracer &st, double sx0, float lr, float wd, NsResult &res) {
  const size_t es = (size_t)elem_size(plan.set.ns_dtype);
  const std::vector<DirectStep> steps = direct_steps(plan, sx0);
  int cur = 0;
  for (int k = 1; k <= plan.K; ++k) {
    const DirectStep &ds = steps[k - 1];
    // A = X X^T (or B = b X X^T directly when c == 0)
    {
      StageBuilder sb(plan, ws, st);
      for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
        const ClassInfo &cl = plan.classes[ci];
        GemmClass g = make_gemm(cl, es, ws, cl.X[cur], cl.Sp, cl.Lp, cl.X[cur], cl.Sp, cl.Lp, cl.Lp, true);
        set_out(g, ws, ds.cubic ? cl.sq[1] : cl.sq[0], cl.Sp, cl.Sp, true);
        g.alpha = (float)ds.syrk_alpha;
        sb.per_class[ci] = g;
        sb.per_flops[ci] = half_flops(cl, cl.l);
      }
      HIP_TRY(sb.launch());
    }
    // B = b A + c A^2 (fused into the update for poly_fused classes)
    std::vector<char> fuse(plan.classes.size(), 0);
    bool any_fused = false;
    if (!ds.cubic)
      for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
        fuse[ci] = poly_fused(plan, plan.classes[ci]) ? 1 : 0;
        any_fused = any_fused || fuse[ci];
      }
    if (!ds.cubic) {
      StageBuilder sb(plan, ws, st);
      sb.skip = fuse;
      for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
        const ClassInfo &cl = plan.classes[ci];
        GemmClass g = make_gemm(cl, es, ws, cl.sq[0], cl.Sp, cl.Sp, cl.sq[0], cl.Sp, cl.Sp, cl.Sp, true);
        set_out(g, ws, cl.sq[1], cl.Sp, cl.Sp, true);
        set_in(g, ws, cl.sq[0], cl.Sp, cl.Sp);
        g.alpha = (float)ds.sq_alpha;
        g.beta = (float)ds.sq_beta;
        sb.per_class[ci] = g;
        sb.per_flops[ci] = half_flops(cl, cl.s);
      }
      HIP_TRY(sb.launch());
    }
    // X^T <- a X^T + X^T B, also written transposed into X; the last step's
    // O (true scale) goes straight into the weight update
    {
      StageBuilder sb(plan, ws, st);
      sb.skip = fuse;
      std::vector<GemmClass> pg(plan.classes.size());
      std::vector<double> pf(plan.classes.size(), 0.0);
      for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
        const ClassInfo &cl = plan.classes[ci];
        GemmClass g = make_gemm(cl, es, ws, cl.XT[cur], cl.Lp, cl.Sp, cl.sq[1], cl.Sp, cl.Sp, cl.Sp, false);
        set_out(g, ws, cl.XT[1 - cur], cl.Lp, cl.Sp, true);
        set_out2(g, ws, cl.X[1 - cur], cl.Sp, cl.Lp);
        set_in(g, ws, cl.XT[cur], cl.Lp, cl.Sp);
        if (k == plan.K) set_final(g, plan, cl, ws, lr, wd);
        g.alpha = (float)ds.upd_alpha;
        g.beta = (float)ds.upd_beta;
        sb.per_class[ci] = g;
        sb.per_flops[ci] = full_flops(cl);
        if (fuse[ci]) {
          // same product with A in place of B (the block forms its panel of
          // B) and X in place of X^T; X'^T only for a following cubic step
          g.a = ws + cl.X[cur];
          g.sa = cl.Sp * cl.Lp;
          g.lda = (int32_t)cl.Lp;
          g.cin = nullptr;
          if (k < plan.K && !step_cubic(plan, k + 1)) g.c = nullptr;
          g.b = ws + cl.sq[0];
          g.sq_alpha = (float)ds.sq_alpha;
          g.sq_beta = (float)ds.sq_beta;
          g.m_tiles = (int32_t)(cl.Lp / 64);
          pg[ci] = g;
          pf[ci] = full_flops(cl) + half_flops(cl, cl.s);
        }
      }
      if (any_fused) HIP_TRY(launch_poly_stage(plan, st, pg, pf, fuse));
      HIP_TRY(sb.launch());
    }
    cur = 1 - cur;
  }
  res.cur = cur;
  res.scale = 1.0;
  return MUON_OK;
}

muon_status run_gram(const Plan &plan, char *ws, Tracer &st, double sx0, float lr, float wd, NsResult &res) {
  const size_t es = (size_t)elem_size(plan.set.ns_dtype);
  const Scaler S{plan.set.ns_dtype == kF16};
  const double d = plan.set.divisor;
  const int r = plan.set.restart_every;
  double sigma = 1.0 / std::sqrt(d);
  double sY = sx0;
  int cur = 0;
  // square-buffer roles (indices into ClassInfo::sq), rotated on the host
  const int iR = 0, iT = 1;
  int iP = 2, iQ = 3, iQs = 4;
  double sR = 1.0, sQ = 1.0, qbound = 1.0;
  bool q_is_identity = true;

  auto form_gram = [&]() -> muon_status {
    sR = S.pick(sigma * sigma);
    StageBuilder sb(plan, ws, st);
    for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
      const ClassInfo &cl = plan.classes[ci];
      GemmClass g = make_gemm(cl, es, ws, cl.X[cur], cl.Sp, cl.Lp, cl.X[cur], cl.Sp, cl.Lp, cl.Lp, true);
      set_out(g, ws, cl.sq[iR], cl.Sp, cl.Sp, true);
      g.alpha = (float)(sR / (sY * sY));
      sb.per_class[ci] = g;
      sb.per_flops[ci] = half_flops(cl, cl.l);
    }
    HIP_TRY(sb.launch());
    return MUON_OK;
  };
  // Y_new = alpha * Y Q, written as Y (tall) and X = Y^T (wide); the final
  // O = Y Q goes straight into the weight update instead
  auto apply_q = [&](double extra, double out_scale, bool final_product = false) -> muon_status {
    StageBuilder sb(plan, ws, st);
    for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
      const ClassInfo &cl = plan.classes[ci];
      GemmClass g = make_gemm(cl, es, ws, cl.XT[cur], cl.Lp, cl.Sp, cl.sq[iQ], cl.Sp, cl.Sp, cl.Sp, false);
      set_out(g, ws, cl.XT[1 - cur], cl.Lp, cl.Sp, true);
      set_out2(g, ws, cl.X[1 - cur], cl.Sp, cl.Lp);
      if (final_product) set_final(g, plan, cl, ws, lr, wd);
      g.alpha = (float)(extra * out_scale / (sY * sQ));
      sb.per_class[ci] = g;
      sb.per_flops[ci] = full_flops(cl);
    }
    HIP_TRY(sb.launch());
    return MUON_OK;
  };
  // C = alpha * L Rt^T for square s x s operands (half product)
  auto square_product = [&](int il, int ir, int iout, double alpha) -> muon_status {
    StageBuilder sb(plan, ws, st);
    for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
      const ClassInfo &cl = plan.classes[ci];
      GemmClass g = make_gemm(cl, es, ws, cl.sq[il], cl.Sp, cl.Sp, cl.sq[ir], cl.Sp, cl.Sp, cl.Sp, true);
      set_out(g, ws, cl.sq[iout], cl.Sp, cl.Sp, true);
      g.alpha = (float)alpha;
      sb.per_class[ci] = g;
      sb.per_flops[ci] = half_flops(cl, cl.s);
    }
    HIP_TRY(sb.launch());
    return MUON_OK;
  };

  muon_status stt = form_gram();
  if (stt != MUON_OK) return stt;
  for (int k = 1; k <= plan.K; ++k) {
    const double a = plan.set.coeffs[3 * (k - 1)], b = plan.set.coeffs[3 * (k - 1) + 1], c = plan.set.coeffs[3 * (k - 1) + 2];
    if (restart_due(k, r)) {
      const double sigma_new = sigma / std::sqrt(d);
      const double sYn = S.pick(sigma_new);
      stt = apply_q(1.0 / std::sqrt(d), sYn);
      if (stt != MUON_OK) return stt;
      cur = 1 - cur;
      sigma = sigma_new;
      sY = sYn;
      stt = form_gram();
      if (stt != MUON_OK) return stt;
      q_is_identity = true;
      qbound = 1.0;
    }
    // P = a I + b R + c R^2   (K = 0 product when c == 0: epilogue only)
    const double pbound = sup_poly(a, b, c, sigma, 1);
    const double sP = S.pick(pbound);
    {
      StageBuilder sb(plan, ws, st);
      for (size_t ci = 0; ci < plan.classes.size(); ++ci) {
        const ClassInfo &cl = plan.classes[ci];
        GemmClass g = make_gemm(cl, es, ws, cl.sq[iR], cl.Sp, cl.Sp, cl.sq[iR], cl.Sp, cl.Sp, c != 0.0 ? cl.Sp : 0, true);
        set_out(g, ws, cl.sq[iP], cl.Sp, cl.Sp, true);
        set_in(g, ws, cl.sq[iR], cl.Sp, cl.Sp);
        g.alpha = (float)(c * sP / (sR * sR));
        g.beta = (float)(b * sP / sR);
        g.diag = (float)(a * sP);
        sb.per_class[ci] = g;
        sb.per_flops[ci] = c != 0.0 ? half_flops(cl, cl.s) : 0.0;
      }
      HIP_TRY(sb.launch());
    }
    // Q <- Q P.  P's buffer stays valid for the R update below; when Q was
    // the identity, P's buffer becomes Q and the old Q buffer takes the next P.
    const int pb = iP;
    if (q_is_identity) {
      std::swap(iQ, iP);
      sQ = sP;
      qbound = pbound;
      q_is_identity = false;
    } else {
      qbound *= pbound;
      const double sQn = S.pick(qbound);
      stt = square_product(iQ, pb, iQs, sQn / (sQ * sP));
      if (stt != MUON_OK) return stt;
      std::swap(iQ, iQs);
      sQ = sQn;
    }
    const double sigma_new = sup_poly(a, b, c, sigma, 0);
    // R <- (R P) P, unless this is the last step before a restart or the end
    const bool need_r = k < plan.K && !restart_due(k + 1, r);
    if (need_r) {
      const double sT = S.pick(sup_poly(a, b, c, sigma, 3));
      stt = square_product(iR, pb, iT, sT / (sR * sP));
      if (stt != MUON_OK) return stt;
      const double sRn = S.pick(sigma_new * sigma_new);
      stt = square_product(iT, pb, iR, sRn / (sT * sP));
      if (stt != MUON_OK) return stt;
      sR = sRn;
    }
    sigma = sigma_new;
  }
  if (plan.K > 0) {
    // O = Y Q, fused with the weight update (true scale)
    stt = apply_q(1.0, 1.0, true);
    if (stt != MUON_OK) return stt;
    cur = 1 - cur;
    sY = 1.0;
  }
  res.cur = cur;
  res.scale = sY;
  return MUON_OK;
}

// ---------------------------------------------------------------- LiMuon
// Randomized SVD of X (X0 in its wide orientation, s x l) in place of
// Newton-Schulz (LiMuon digest, "Метод"; Halko, Martinsson & Tropp 2011,
// Algorithms 4.4 and 5.1), with kp = k + p test vectors (panels nb = 32 or
// 64 columns wide, stored kLmKP wide):
//   Y = X Omega ; Q = orth(Y)
//   q times: Z = orth(X^T Q) ; Q = orth(X Z)     (the last Q orthonormalised twice)
//   B^T = X^T Q ; H = B B^T = V D V^T ; T = V_k D_k^{-1/2} V_k^T
//   O = (Q T) B, fused with the weight update (lm_final_kernel)
// orth(P) = P W from the fp64 Gram matrix P^T P: Cholesky with symmetric
// pivoting, stopped where the pivot falls to 1e-12 of the largest diagonal,
// and the inverse of the triangular factor.  Every product against a panel
// runs in lm_thin_kernel, which also writes the fp64 Gram partials of its
// result.
muon_status run_limuon(const Plan &plan, char *ws, Tracer &st, float lr, float wd) {
  const int kp = plan.set.rank + plan.set.oversample;
  const int nb = kp <= 32 ? 32 : 64;
  const int KP = kLmKP;
  double *parts = (double *)(ws + plan.off_lm_parts);
  const int pan_s = 0, pan_l = 1;   // panel kinds: s rows or l rows

  // pad the caller's test matrix into each class's [KP x Lp] buffer
  {
    LmPadArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
    a.src = plan.set.sketch;
    a.ld = plan.set.sketch_ld;
    a.kp = kp;
    int blocks = 0;
    double bytes = 0.0;
    auto go = [&]() -> muon_status {
      if (a.nclass == 0) return MUON_OK;
      HIP_TRY(st.run(MUON_STAGE_SMALL, bytes, [&]() { return launch_lm_pad(a, blocks, st.s); }));
      a.nclass = 0;
      blocks = 0;
      bytes = 0.0;
      for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
      return MUON_OK;
    };
    for (const ClassInfo &cl : plan.classes) {
      if (a.nclass == kLmMaxClasses) {
        muon_status e = go();
        if (e != MUON_OK) return e;
      }
      LmPadClass &c = a.cls[a.nclass];
      c.dst = (float *)(ws + cl.lm[kLmOmt]);
      c.l = (int32_t)cl.l;
      c.lp = (int32_t)cl.Lp;
      c.blocks = (int32_t)(((int64_t)KP * cl.Lp + kLmPadElems - 1) / kLmPadElems);
      a.begin[a.nclass++] = blocks;
      blocks += c.blocks;
      bytes += (double)kp * (double)cl.l * 4.0 + (double)KP * (double)cl.Lp * 4.0;
    }
    muon_status e = go();
    if (e != MUON_OK) return e;
  }

  // One thin product per class: C = A B^T over K, A's rows `kind` (s or l
  // padded), optionally C^T and the Gram partials of C.
  struct Thin {
    const float *a;
    int64_t sa, lda;
    const float *b;
    int64_t sb, ldb;
    int64_t K;
    int kind;
    float *c, *c2;
    int64_t sc, ldc, sc2, ldc2;
    bool gram;
    double flops;
  };
  auto thin = [&](auto &&make) -> muon_status {
    LmThinArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
    a.n = kp;
    a.partials = parts;
    int blocks = 0;
    double flops = 0.0;
    auto go = [&]() -> muon_status {
      if (a.nclass == 0) return MUON_OK;
      HIP_TRY(st.run(MUON_STAGE_GEMM, flops, [&]() { return launch_lm_thin(a, nb, blocks, st.s); }));
      a.nclass = 0;
      blocks = 0;
      flops = 0.0;
      for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
      return MUON_OK;
    };
    for (const ClassInfo &cl : plan.classes) {
      if (a.nclass == kLmMaxClasses) {
        muon_status e = go();
        if (e != MUON_OK) return e;
      }
      const Thin t = make(cl);
      LmThinClass &c = a.cls[a.nclass];
      c.a = t.a;
      c.sa = t.sa;
      c.lda = (int32_t)t.lda;
      c.b = t.b;
      c.sb = t.sb;
      c.ldb = (int32_t)t.ldb;
      c.c = t.c;
      c.c2 = t.c2;
      c.sc = t.sc;
      c.ldc = (int32_t)t.ldc;
      c.sc2 = t.sc2;
      c.ldc2 = (int32_t)t.ldc2;
      c.K = (int32_t)t.K;
      c.tiles = t.kind == pan_s ? cl.lm_chunks_s : cl.lm_chunks_l;
      c.count = (int32_t)cl.members.size();
      c.part_base = t.gram ? cl.lm_part_base : -1;
      a.begin[a.nclass++] = blocks;
      blocks += c.count * c.tiles;
      flops += t.flops * (double)c.count;
    }
    return go();
  };
  auto eig = [&](int kind, int mode, int out_buf) -> muon_status {
    LmEigArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
    a.n = kp;
    a.mode = mode;
    a.rank = plan.set.rank;
    a.cutoff = mode == kLmOrth ? 1e-12 : plan.set.rcond * plan.set.rcond;
    a.partials = parts;
    int blocks = 0;
    auto go = [&]() -> muon_status {
      if (a.nclass == 0) return MUON_OK;
      HIP_TRY(st.run(MUON_STAGE_SMALL, 0.0, [&]() { return launch_lm_eig(a, blocks, st.s); }));
      a.nclass = 0;
      blocks = 0;
      for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
      return MUON_OK;
    };
    for (const ClassInfo &cl : plan.classes) {
      if (a.nclass == kLmMaxClasses) {
        muon_status e = go();
        if (e != MUON_OK) return e;
      }
      LmEigClass &c = a.cls[a.nclass];
      c.out = (float *)(ws + cl.lm[out_buf]);
      c.out_stride = (int64_t)KP * KP;
      c.count = (int32_t)cl.members.size();
      c.nchunks = kind == pan_s ? cl.lm_chunks_s : cl.lm_chunks_l;
      c.part_base = cl.lm_part_base;
      a.begin[a.nclass++] = blocks;
      blocks += c.count;
    }
    return go();
  };
  auto buf = [&](const ClassInfo &cl, int i) { return (float *)(ws + cl.lm[i]); };
  // panel (rows x KP) times a KP x KP factor stored as its transpose's rows
  auto apply = [&](int in_buf, int kind, int w_buf, int out_buf, int out_t_buf, bool gram) -> muon_status {
    return thin([&](const ClassInfo &cl) {
      const int64_t rows = kind == pan_s ? cl.Sp : cl.Lp;
      Thin t{};
      t.a = buf(cl, in_buf); t.sa = rows * KP; t.lda = KP;
      t.b = buf(cl, w_buf); t.sb = (int64_t)KP * KP; t.ldb = KP;
      t.K = nb; t.kind = kind;
      t.c = buf(cl, out_buf); t.sc = rows * KP; t.ldc = KP;
      if (out_t_buf >= 0) { t.c2 = buf(cl, out_t_buf); t.sc2 = (int64_t)KP * rows; t.ldc2 = rows; }
      t.gram = gram;
      t.flops = 2.0 * (double)(kind == pan_s ? cl.s : cl.l) * kp * kp;
      return t;
    });
  };
  // X (s x l) times an l-row panel given as its transpose [KP x Lp]
  auto x_times = [&](int bt_buf, bool shared_b, int out_buf) -> muon_status {
    return thin([&](const ClassInfo &cl) {
      Thin t{};
      t.a = (const float *)(ws + cl.X[0]); t.sa = cl.Sp * cl.Lp; t.lda = cl.Lp;
      t.b = buf(cl, bt_buf); t.sb = shared_b ? 0 : (int64_t)KP * cl.Lp; t.ldb = cl.Lp;
      t.K = cl.Lp; t.kind = pan_s;
      t.c = buf(cl, out_buf); t.sc = cl.Sp * KP; t.ldc = KP;
      t.gram = true;
      t.flops = 2.0 * (double)cl.s * (double)cl.l * kp;
      return t;
    });
  };
  // X^T (l x s) times an s-row panel given as its transpose [KP x Sp]
  auto xt_times = [&](int bt_buf, int out_buf) -> muon_status {
    return thin([&](const ClassInfo &cl) {
      Thin t{};
      t.a = (const float *)(ws + cl.XT[0]); t.sa = cl.Lp * cl.Sp; t.lda = cl.Sp;
      t.b = buf(cl, bt_buf); t.sb = (int64_t)KP * cl.Sp; t.ldb = cl.Sp;
      t.K = cl.Sp; t.kind = pan_l;
      t.c = buf(cl, out_buf); t.sc = cl.Lp * KP; t.ldc = KP;
      t.gram = true;
      t.flops = 2.0 * (double)cl.s * (double)cl.l * kp;
      return t;
    });
  };
  // orth of an s-row panel into Q (and Q^T), once or twice
  auto orth_s = [&](int in_buf, bool twice) -> muon_status {
    muon_status e = eig(pan_s, kLmOrth, kLmW);
    if (e != MUON_OK) return e;
    if (!twice) return apply(in_buf, pan_s, kLmW, kLmQ, kLmQt, false);
    if ((e = apply(in_buf, pan_s, kLmW, kLmQ2, -1, true)) != MUON_OK) return e;
    if ((e = eig(pan_s, kLmOrth, kLmW)) != MUON_OK) return e;
    return apply(kLmQ2, pan_s, kLmW, kLmQ, kLmQt, false);
  };

  muon_status e;
  const int q = plan.set.power_iters;
  if ((e = x_times(kLmOmt, true, kLmY)) != MUON_OK) return e;          // Y = X Omega (+ Gram)
  if ((e = orth_s(kLmY, q == 0)) != MUON_OK) return e;
  for (int it = 0; it < q; ++it) {
    if ((e = xt_times(kLmQt, kLmZ)) != MUON_OK) return e;              // Z = X^T Q (+ Gram)
    if ((e = eig(pan_l, kLmOrth, kLmW)) != MUON_OK) return e;
    if ((e = apply(kLmZ, pan_l, kLmW, kLmZ2, kLmZ2t, false)) != MUON_OK) return e;
    if ((e = x_times(kLmZ2t, false, kLmY)) != MUON_OK) return e;       // Y = X Z (+ Gram)
    if ((e = orth_s(kLmY, it + 1 == q)) != MUON_OK) return e;
  }
  if ((e = xt_times(kLmQt, kLmZ)) != MUON_OK) return e;                // B^T = X^T Q (+ Gram: B B^T)
  if ((e = eig(pan_l, kLmTrunc, kLmT)) != MUON_OK) return e;
  if ((e = apply(kLmQ, pan_s, kLmT, kLmP, -1, false)) != MUON_OK) return e;   // P = Q T
  // O = P Z^T (Z = B^T) and the weight update, tile by tile of W
  {
    LmFinalArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
    a.kp = kp;
    a.lr = lr;
    a.wd = wd;
    a.desc = (const FinalDesc *)(ws + plan.off_desc);
    int blocks = 0;
    double flops = 0.0;
    auto go = [&]() -> muon_status {
      if (a.nclass == 0) return MUON_OK;
      HIP_TRY(st.run(MUON_STAGE_GEMM, flops, [&]() { return launch_lm_final(a, blocks, st.s); }));
      a.nclass = 0;
      blocks = 0;
      flops = 0.0;
      for (int j = 0; j < kLmMaxClasses; ++j) a.begin[j] = INT32_MAX;
      return MUON_OK;
    };
    for (const ClassInfo &cl : plan.classes) {
      if (a.nclass == kLmMaxClasses) {
        muon_status e2 = go();
        if (e2 != MUON_OK) return e2;
      }
      LmFinalClass &c = a.cls[a.nclass];
      c.p = buf(cl, kLmP);
      c.z = buf(cl, kLmZ);
      c.sp = cl.Sp * KP;
      c.sz = cl.Lp * KP;
      c.desc_base = cl.desc_base;
      c.count = (int32_t)cl.members.size();
      c.tiles = (int32_t)(((cl.s + kLmFinalTile - 1) / kLmFinalTile) * ((cl.l + kLmFinalTile - 1) / kLmFinalTile));
      a.begin[a.nclass++] = blocks;
      blocks += c.count * c.tiles;
      flops += 2.0 * (double)cl.s * (double)cl.l * kp * (double)c.count;
    }
    if ((e = go()) != MUON_OK) return e;
  }
  return MUON_OK;
}

}  // namespace

muon_status muon::record_error(muon_status s, const char *msg) {
  g_last_error = msg ? msg : "";
  return s;
}

extern "C" {

void muon_options_init(muon_options *o) {
  if (!o) return;
  o->grad_dtype = MUON_F32;
  o->ns_dtype = MUON_F32;
  o->coeffs = nullptr;
  o->divisor = 1.0f;
  o->restart_every = 0;
  o->step = 0;
  o->trace = nullptr;
  o->sketch = nullptr;
  o->sketch_ld = 0;
  o->rank = 0;
  o->oversample = 8;
  o->power_iters = 1;
  o->rcond = 1e-4f;
}

size_t muon_workspace_size(const muon_param *params, int n, int ns_steps, muon_variant variant,
                           const muon_options *opts) {
  Plan plan;
  if (build_plan(params, n, ns_steps, variant, opts, plan) != MUON_OK) return 0;
  g_last_error.clear();
  return plan.total;
}

muon_status muon_debug_square_buffer(const muon_param *params, int n, int ns_steps, muon_variant variant,
                                     const muon_options *opts, int index, int which, size_t *offset, int64_t *ld,
                                     int64_t *side) {
  if (!offset || !ld || !side) return fail(MUON_ERR_INVALID_ARG, "offset, ld and side must be non-NULL");
  Plan plan;
  muon_status st = build_plan(params, n, ns_steps, variant, opts, plan);
  if (st != MUON_OK) return st;
  if (index < 0 || index >= n) return fail(MUON_ERR_INVALID_ARG, "index %d out of [0, %d)", index, n);
  const int nsq = variant == MUON_NS_DIRECT ? 2 : variant == MUON_NS_GRAM ? 5 : 0;
  if (which < 0 || which >= nsq) return fail(MUON_ERR_INVALID_ARG, "which %d out of [0, %d)", which, nsq);
  const ClassInfo &cl = plan.classes[plan.cls_of[index]];
  const size_t es = (size_t)elem_size(plan.set.ns_dtype);
  *offset = cl.sq[which] + (size_t)plan.idx_in_cls[index] * (size_t)cl.Sp * (size_t)cl.Sp * es;
  *ld = cl.Sp;
  *side = cl.s;
  g_last_error.clear();
  return MUON_OK;
}

muon_status muon_step(const muon_param *params, int n, float lr, float mu, float beta_a, float alpha, float lambda,
                      int ns_steps, muon_variant variant, const muon_options *opts, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!is_finite(lr) || !is_finite(mu) || !is_finite(beta_a) || !is_finite(alpha) || !is_finite(lambda))
    return fail(MUON_ERR_INVALID_ARG, "lr, mu, beta_a, alpha and lambda must be finite");
  Plan plan;
  muon_status st = build_plan(params, n, ns_steps, variant, opts, plan);
  if (st != MUON_OK) return st;
  if (n == 0) {
    g_last_error.clear();
    return MUON_OK;
  }
  if (!workspace) return fail(MUON_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255) != 0) return fail(MUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan.total)
    return fail(MUON_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, plan.total);
  hipStream_t hs = (hipStream_t)stream;
  char *ws = (char *)workspace;
  muon_trace *trace = opts ? opts->trace : nullptr;
  if (trace) {
    if (trace->capacity > 0 && (!trace->events || !trace->stages || !trace->work || (trace->group && !trace->launches)))
      return fail(MUON_ERR_INVALID_ARG, "trace arrays are NULL");
    trace->count = 0;
  }
  Tracer tr{trace, hs};
  const Settings &set = plan.set;
  double *partials = (double *)(ws + plan.off_partials);
  // Streaming (non-temporal) accesses in E1 / E2 when the call's momentum is
  // far larger than the device's caches (256 MB of last-level cache).
  int64_t total_elems = 0;
  for (int i = 0; i < n; ++i) total_elems += params[i].rows * params[i].cols;
  const int32_t stream_ew = total_elems * 4 > (int64_t(512) << 20) ? 1 : 0;
  float *scales = (float *)(ws + plan.off_scales);

  // ---- E1, launched separately for plain, MONA and MONA-Lite matrices
  for (int mode = kE1Plain; mode <= kE1Lite; ++mode) {
    E1Args a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kE1MaxMats; ++j) a.begin[j] = INT32_MAX;
    a.grad_dtype = set.grad_dtype;
    a.mode = mode;
    a.first_step = set.step == 0 ? 1 : 0;
    a.mu = mu;
    a.beta_a = beta_a;
    a.alpha = alpha;
    a.stream = stream_ew;
    a.partials = partials;
    a.desc = (FinalDesc *)(ws + plan.off_desc);
    int blocks = 0;
    double bytes = 0.0;
    auto flush = [&]() -> muon_status {
      if (a.nmat == 0) return MUON_OK;
      HIP_TRY(tr.run(MUON_STAGE_E1, bytes, [&]() { return launch_e1(a, blocks, hs); }));
      a.nmat = 0;
      for (int j = 0; j < kE1MaxMats; ++j) a.begin[j] = INT32_MAX;
      blocks = 0;
      bytes = 0.0;
      return MUON_OK;
    };
    for (int i = 0; i < n; ++i) {
      const int m_i = params[i].mona_lite ? kE1Lite : params[i].accel ? kE1Mona : kE1Plain;
      if (m_i != mode) continue;
      if (a.nmat == kE1MaxMats) {
        st = flush();
        if (st != MUON_OK) return st;
      }
      E1Mat &m = a.mats[a.nmat++];
      m.grad = params[i].grad;
      m.mom = params[i].momentum;
      m.accel = params[i].accel;
      m.prev = params[i].prev_grad;
      m.lite = params[i].mona_lite;
      m.numel = params[i].rows * params[i].cols;
      a.begin[a.nmat - 1] = blocks;
      m.partial_off = plan.partial_off[i];
      m.weight = params[i].weight;
      m.ortho_out = params[i].ortho_out;
      m.rows = (int32_t)params[i].rows;
      m.cols = (int32_t)params[i].cols;
      m.gamma = params[i].gamma;
      m.desc_idx = has_products(plan) ? plan.classes[plan.cls_of[i]].desc_base + plan.idx_in_cls[i] : -1;
      blocks += plan.e1_blocks[i];
      {
        // G read, M read+write; MONA: A read+write, G_prev written (and read
        // after step 0); MONA-Lite: C written (and read after step 0)
        const double gs = (double)elem_size(set.grad_dtype);
        double per = gs + 8.0;
        if (mode == kE1Mona) per += 8.0 + gs + (set.step == 0 ? 0.0 : gs);
        if (mode == kE1Lite) per += 2.0 + (set.step == 0 ? 0.0 : 2.0);
        bytes += per * (double)m.numel;
      }
    }
    st = flush();
    if (st != MUON_OK) return st;
  }
  HIP_TRY(tr.close());   // a traced run of launches ends where its stage ends

  // ---- norm finalize
  const Scaler S{set.ns_dtype == kF16};
  const double sx0 = S.pick(1.0 / std::sqrt(set.divisor));
  {
    NormArgs a;
    std::memset(&a, 0, sizeof(a));
    a.inv_sqrt_d = (float)(1.0 / std::sqrt(set.divisor));
    a.store_scale = (float)sx0;
    a.partials = partials;
    a.scales = scales;
    for (int i = 0; i < n; ++i) {
      if (plan.e1_blocks[i] <= kE2InlineParts) continue;   // reduced inside E2
      if (a.nmat == kNormMaxMats) {
        HIP_TRY(tr.run(MUON_STAGE_NORM, 0.0, [&]() { return launch_norm(a, hs); }));
        a.nmat = 0;
      }
      NormMat &m = a.mats[a.nmat++];
      m.partial_off = plan.partial_off[i];
      m.nparts = plan.e1_blocks[i];
      m.scale_idx = i;
    }
    if (a.nmat) HIP_TRY(tr.run(MUON_STAGE_NORM, 0.0, [&]() { return launch_norm(a, hs); }));
    HIP_TRY(tr.close());
  }

  // ---- E2: X0 into X[0] / XT[0]
  const size_t es = (size_t)elem_size(set.ns_dtype);
  {
    E2Args a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kE2MaxMats; ++j) a.begin[j] = INT32_MAX;
    a.ns_dtype = set.ns_dtype;
    a.scales = scales;
    a.partials = partials;
    a.inv_sqrt_d = (float)(1.0 / std::sqrt(set.divisor));
    a.store_scale = (float)sx0;
    a.stream = stream_ew;
    int blocks = 0;
    double bytes = 0.0;
    for (int i = 0; i < n; ++i) {
      if (a.nmat == kE2MaxMats) {
        HIP_TRY(tr.run(MUON_STAGE_E2, bytes, [&]() { return launch_e2(a, blocks, hs); }));
        a.nmat = 0;
        blocks = 0;
        bytes = 0.0;
        for (int j = 0; j < kE2MaxMats; ++j) a.begin[j] = INT32_MAX;
      }
      const ClassInfo &cl = plan.classes[plan.cls_of[i]];
      const size_t j = (size_t)plan.idx_in_cls[i];
      const bool wide = params[i].rows <= params[i].cols;
      const size_t rect = (size_t)cl.Sp * (size_t)cl.Lp * es;
      E2Mat &m = a.mats[a.nmat++];
      m.mom = params[i].momentum;
      m.nat = ws + (wide ? cl.X[0] : cl.XT[0]) + j * rect;
      m.trn = ws + (wide ? cl.XT[0] : cl.X[0]) + j * rect;
      const bool both = needs_x0_transposed(plan, cl);
      if (!both) (wide ? m.trn : m.nat) = nullptr;   // X^T (the tall layout) is not read
      m.rows = (int32_t)params[i].rows;
      m.cols = (int32_t)params[i].cols;
      const int64_t prow = wide ? cl.Sp : cl.Lp, pcol = wide ? cl.Lp : cl.Sp;
      m.ld_nat = (int32_t)pcol;
      m.ld_trn = (int32_t)prow;
      m.tiles_c = (int32_t)(pcol / kE2Tile);
      a.begin[a.nmat - 1] = blocks;
      m.scale_idx = i;
      if (plan.e1_blocks[i] <= kE2InlineParts) {
        m.partial_off = plan.partial_off[i];
        m.nparts = plan.e1_blocks[i];
      }
      blocks += (int)((prow / kE2Tile) * (pcol / kE2Tile));
      // M read (fp32), X0 written in one or both orientations
      bytes += (4.0 + (both ? 2.0 : 1.0) * (double)es) * (double)(params[i].rows * params[i].cols);
    }
    if (a.nmat) HIP_TRY(tr.run(MUON_STAGE_E2, bytes, [&]() { return launch_e2(a, blocks, hs); }));
    HIP_TRY(tr.close());
  }

  // ---- Newton-Schulz (or LiMuon's randomized SVD)
  NsResult res{0, sx0};
  if (is_limuon(plan)) {
    st = run_limuon(plan, ws, tr, lr, lambda);
    if (st != MUON_OK) return st;
    HIP_TRY(tr.close());
  } else if (plan.K > 0) {
    st = (variant == MUON_NS_DIRECT) ? run_direct(plan, ws, tr, sx0, lr, lambda, res)
                                     : run_gram(plan, ws, tr, sx0, lr, lambda, res);
    if (st != MUON_OK) return st;
    HIP_TRY(tr.close());
  }

  // ---- E3: only without Newton-Schulz steps (O = X0); otherwise the last
  // product applied the update in its epilogue
  if (!has_products(plan)) {
    E3Args a;
    std::memset(&a, 0, sizeof(a));
    for (int j = 0; j < kE3MaxMats; ++j) a.begin[j] = INT32_MAX;
    a.ns_dtype = set.ns_dtype;
    a.lr = lr;
    a.wd = lambda;
    int blocks = 0;
    double bytes = 0.0;
    for (int i = 0; i < n; ++i) {
      if (a.nmat == kE3MaxMats) {
        HIP_TRY(tr.run(MUON_STAGE_E3, bytes, [&]() { return launch_e3(a, blocks, hs); }));
        a.nmat = 0;
        blocks = 0;
        bytes = 0.0;
        for (int j = 0; j < kE3MaxMats; ++j) a.begin[j] = INT32_MAX;
      }
      const ClassInfo &cl = plan.classes[plan.cls_of[i]];
      const size_t j = (size_t)plan.idx_in_cls[i];
      const bool wide = params[i].rows <= params[i].cols;
      const size_t rect = (size_t)cl.Sp * (size_t)cl.Lp * es;
      E3Mat &m = a.mats[a.nmat++];
      m.weight = params[i].weight;
      m.o = ws + (wide ? cl.X[res.cur] : cl.XT[res.cur]) + j * rect;
      m.ortho_out = params[i].ortho_out;
      m.numel = params[i].rows * params[i].cols;
      m.cols = (int32_t)params[i].cols;
      m.ld_o = (int32_t)(wide ? cl.Lp : cl.Sp);
      m.gamma = params[i].gamma;
      m.inv_o_scale = (float)(1.0 / res.scale);
      a.begin[a.nmat - 1] = blocks;
      m.vec_ok = ((params[i].cols & 3) == 0) && ((((uintptr_t)params[i].weight) | ((uintptr_t)params[i].ortho_out)) & 15) == 0;
      blocks += (int)((m.numel + kE3BlockElems - 1) / kE3BlockElems);
      // W read+write, O read (and the optional fp32 copy written)
      bytes += (8.0 + (double)es + (m.ortho_out ? 4.0 : 0.0)) * (double)m.numel;
    }
    if (a.nmat) HIP_TRY(tr.run(MUON_STAGE_E3, bytes, [&]() { return launch_e3(a, blocks, hs); }));
  }
  HIP_TRY(tr.close());
  g_last_error.clear();
  return MUON_OK;
}

muon_status muon_adamw_step(const muon_adamw_param *params, int n, muon_dtype grad_dtype, float lr, float beta1,
                            float beta2, float eps, float weight_decay, int64_t step, muon_trace *trace,
                            void *stream) {
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && !params) return fail(MUON_ERR_INVALID_ARG, "params is NULL");
  if (grad_dtype != MUON_F32 && grad_dtype != MUON_F16 && grad_dtype != MUON_BF16)
    return fail(MUON_ERR_UNSUPPORTED, "unknown grad_dtype %d", (int)grad_dtype);
  if (!is_finite(lr) || !is_finite(beta1) || !is_finite(beta2) || !is_finite(eps) || !is_finite(weight_decay))
    return fail(MUON_ERR_INVALID_ARG, "lr, beta1, beta2, eps and weight_decay must be finite");
  if (beta1 < 0.0f || beta1 >= 1.0f || beta2 < 0.0f || beta2 >= 1.0f)
    return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
  if (eps < 0.0f) return fail(MUON_ERR_INVALID_ARG, "eps must be >= 0");
  if (step < 0) return fail(MUON_ERR_INVALID_ARG, "step must be >= 0");
  if (trace && trace->capacity > 0 && (!trace->events || !trace->stages || !trace->work || (trace->group && !trace->launches)))
    return fail(MUON_ERR_INVALID_ARG, "trace arrays are NULL");
  const int gs = elem_size((int)grad_dtype);
  std::vector<Range> ranges;
  ranges.reserve((size_t)n * 4);
  for (int i = 0; i < n; ++i) {
    const muon_adamw_param &q = params[i];
    if (!q.param || !q.grad || !q.exp_avg || !q.exp_avg_sq)
      return fail(MUON_ERR_INVALID_ARG, "adamw param %d: param, grad, exp_avg and exp_avg_sq must be non-NULL", i);
    if (q.numel < 1) return fail(MUON_ERR_INVALID_ARG, "adamw param %d: numel must be >= 1", i);
    if (q.numel > kMaxNumel) return fail(MUON_ERR_UNSUPPORTED, "adamw param %d: %lld elements exceed the supported size", i, (long long)q.numel);
    const uint64_t ne = (uint64_t)q.numel;
    ranges.push_back({(uintptr_t)q.param, (uintptr_t)q.param + ne * 4, i, "param"});
    ranges.push_back({(uintptr_t)q.grad, (uintptr_t)q.grad + ne * (uint64_t)gs, i, "grad"});
    ranges.push_back({(uintptr_t)q.exp_avg, (uintptr_t)q.exp_avg + ne * 4, i, "exp_avg"});
    ranges.push_back({(uintptr_t)q.exp_avg_sq, (uintptr_t)q.exp_avg_sq + ne * 4, i, "exp_avg_sq"});
  }
  std::sort(ranges.begin(), ranges.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].lo < ranges[i - 1].hi)
      return fail(MUON_ERR_INVALID_ARG, "buffers overlap: adamw param %d %s and adamw param %d %s", ranges[i - 1].param,
                  ranges[i - 1].what, ranges[i].param, ranges[i].what);
  if (trace) trace->count = 0;
  if (n == 0) {
    g_last_error.clear();
    return MUON_OK;
  }
  hipStream_t hs = (hipStream_t)stream;
  Tracer tr{trace, hs};
  AdamArgs a;
  std::memset(&a, 0, sizeof(a));
  const double t = (double)step + 1.0;
  a.grad_dtype = (int32_t)grad_dtype;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.one_minus_beta1 = (float)(1.0 - (double)beta1);
  a.one_minus_beta2 = (float)(1.0 - (double)beta2);
  a.step_size = (float)((double)lr / (1.0 - std::pow((double)beta1, t)));
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow((double)beta2, t)));
  a.eps = eps;
  a.decay = (float)((double)lr * (double)weight_decay);
  int blocks = 0;
  double bytes = 0.0;
  auto reset = [&]() {
    a.nt = 0;
    for (int j = 0; j < kAdamMaxTensors; ++j) a.begin[j] = INT32_MAX;
    blocks = 0;
    bytes = 0.0;
  };
  reset();
  for (int i = 0; i < n; ++i) {
    if (a.nt == kAdamMaxTensors) {
      HIP_TRY(tr.run(MUON_STAGE_ADAMW, bytes, [&]() { return launch_adamw(a, blocks, hs); }));
      reset();
    }
    const muon_adamw_param &q = params[i];
    AdamTensor &d = a.t[a.nt];
    d.param = q.param;
    d.grad = q.grad;
    d.m = q.exp_avg;
    d.v = q.exp_avg_sq;
    d.numel = q.numel;
    d.vec_ok = (((((uintptr_t)q.param) | ((uintptr_t)q.exp_avg) | ((uintptr_t)q.exp_avg_sq)) & 15) == 0 &&
                (((uintptr_t)q.grad) & (gs == 4 ? 15 : 7)) == 0) ? 1 : 0;
    a.begin[a.nt] = blocks;
    a.nt++;
    blocks += (int)((q.numel + kAdamBlockElems - 1) / kAdamBlockElems);
    bytes += (24.0 + (double)gs) * (double)q.numel;   // p, m, v read + written, g read
  }
  if (a.nt) HIP_TRY(tr.run(MUON_STAGE_ADAMW, bytes, [&]() { return launch_adamw(a, blocks, hs); }));
  HIP_TRY(tr.close());
  g_last_error.clear();
  return MUON_OK;
}

const char *muon_status_string(muon_status s) {
  switch (s) {
    case MUON_OK: return "ok";
    case MUON_ERR_INVALID_ARG: return "invalid argument";
    case MUON_ERR_UNSUPPORTED: return "unsupported";
    case MUON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MUON_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char *muon_last_error(void) { return g_last_error.c_str(); }

const char *muon_version(void) { return "libmuon 0.1.0 gfx950"; }

}  // extern "C"
