"""The host code (argument checks, workspace planning, schedules, the static
entry point's size check) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer, driven through every validation path and the
planning of every workload (no GPU: the kernels are replaced by launch
stubs, and every call here fails or returns before a HIP call)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "newton_schulz_matrix_momentum_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

STUBS = r'''
#include "muon_kernels.h"
namespace muon {
#define STUB(name, T) hipError_t name(const T &, int, hipStream_t) { return hipErrorNotSupported; }
STUB(launch_e1, E1Args) STUB(launch_e2, E2Args) STUB(launch_e3, E3Args) STUB(launch_adamw, AdamArgs)
STUB(launch_lm_eig, LmEigArgs) STUB(launch_lm_pad, LmPadArgs) STUB(launch_lm_final, LmFinalArgs)
hipError_t launch_lm_thin(const LmThinArgs &, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_norm(const NormArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm(const GemmArgs &, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_poly_update(const GemmArgs &, int, int, hipStream_t) { return hipErrorNotSupported; }
int poly_blocks_per_cu(int) { return 1; }
int poly_max_group(int) { return 1; }
}
'''

DRIVER = r'''
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "muon.h"
#define BASE ((uintptr_t)1 << 40)
static muon_param P(int i, int64_t r, int64_t c, int mona) {
  muon_param p; memset(&p, 0, sizeof(p));
  uintptr_t step = (uintptr_t)1 << 34;
  p.weight = (float *)(BASE + (uintptr_t)(8 * i) * step); p.grad = (void *)(BASE + (uintptr_t)(8 * i + 1) * step);
  p.momentum = (float *)(BASE + (uintptr_t)(8 * i + 2) * step);
  if (mona) { p.accel = (float *)(BASE + (uintptr_t)(8 * i + 3) * step); p.prev_grad = (void *)(BASE + (uintptr_t)(8 * i + 4) * step); }
  p.rows = r; p.cols = c; p.gamma = 1.0f;
  return p;
}
int main(void) {
  static muon_param ps[200];
  int n = 0, bad = 0;
  /* every workload shape mix: NanoChat, Llama, Gram-tall, MoE, odd sizes */
  int64_t shapes[][2] = {{192,192},{192,768},{768,192},{1024,1024},{1024,2816},{2816,1024},{4096,16384},
                         {16384,4096},{2048,1408},{1408,2048},{2048,2048},{1,77},{77,1},{64,256},{130,70},
                         {520,1100},{70001,3}};
  for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); ++k) ps[n] = P(n, shapes[k][0], shapes[k][1], (int)(k & 1)), ++n;
  muon_options o; muon_options_init(&o);
  for (int v = 0; v <= 2; ++v)
    for (int dt = 0; dt <= 2; ++dt) {
      o.ns_dtype = (muon_dtype)dt; o.grad_dtype = MUON_BF16;
      o.sketch = (const float *)(BASE - ((uintptr_t)1 << 32)); o.sketch_ld = 70001; o.rank = 8; o.oversample = 8;
      o.divisor = 1.03f; o.restart_every = 3;
      size_t ws = muon_workspace_size(ps, n, 5, (muon_variant)v, &o);
      int ok = (v == 2 && dt != 0) ? ws == 0 : ws > 0;
      if (!ok) { printf("workspace v=%d dt=%d: %zu (%s)\n", v, dt, ws, muon_last_error()); bad++; }
      for (int i = 0; i < n && v < 2; ++i) {
        size_t off; int64_t ld, side;
        if (muon_debug_square_buffer(ps, n, 5, (muon_variant)v, &o, i, 0, &off, &ld, &side) != MUON_OK || off >= ws) bad++;
      }
      /* too small a workspace: fails before any launch */
      if (ws && muon_step(ps, n, 0.02f, 0.95f, 0.9f, 0.5f, 0.01f, 5, (muon_variant)v, &o,
                          (void *)(BASE * 3), ws - 1, 0) != MUON_ERR_WORKSPACE_TOO_SMALL) bad++;
      if (muon_step_static(ps, n, 0.02f, 0.95f, 0.9f, 0.5f, 0.01f, 5, (muon_variant)v, &o, 0) == MUON_OK) bad++;
    }
  /* invalid arguments */
  muon_param q = P(0, 8, 16, 1); q.prev_grad = 0;
  if (muon_step(&q, 1, 0.02f, 0.95f, 0.9f, 0.5f, 0.01f, 5, MUON_NS_DIRECT, 0, (void *)BASE, 1 << 20, 0) != MUON_ERR_INVALID_ARG) bad++;
  q = P(0, 8, 16, 0); q.momentum = q.weight + 3;
  if (muon_step(&q, 1, 0.02f, 0.95f, 0.9f, 0.5f, 0.01f, 5, MUON_NS_DIRECT, 0, (void *)BASE, 1 << 20, 0) != MUON_ERR_INVALID_ARG) bad++;
  float coeffs[3 * 64]; for (int i = 0; i < 3 * 64; ++i) coeffs[i] = 1.0f;
  o.coeffs = coeffs; o.ns_dtype = MUON_F16;
  if (muon_workspace_size(ps, n, 64, MUON_NS_GRAM, &o) == 0) bad++;
  if (muon_workspace_size(ps, n, 65, MUON_NS_GRAM, &o) != 0) bad++;
  muon_adamw_param a; memset(&a, 0, sizeof(a));
  if (muon_adamw_step(&a, 1, MUON_BF16, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.0f, 0, 0, 0) != MUON_ERR_INVALID_ARG) bad++;
  printf("%s %d\n", bad ? "FAIL" : "OK", bad);
  return bad != 0;
}
'''


def test_host_code_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the ROCm headers are missing")
    (tmp_path / "stubs.cpp").write_text(STUBS)
    (tmp_path / "driver.c").write_text(DRIVER)
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + INCLUDE, "-I" + CSRC]
    objs = []
    for name, src in (("host", os.path.join(CSRC, "muon_host.cpp")), ("stubs", str(tmp_path / "stubs.cpp"))):
        obj = str(tmp_path / (name + ".o"))
        r = subprocess.run([gxx, "-x", "c++"] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    # the static entry point without its device array: the size check runs first
    static_src = open(os.path.join(CSRC, "muon_static.hip")).read()
    static_src = static_src.replace("static __device__ __align__(256) unsigned char scratch[MUON_STATIC_WORKSPACE_BYTES];",
                                    "static unsigned char scratch[1];")
    assert "static unsigned char scratch[1];" in static_src
    (tmp_path / "static.cpp").write_text(static_src.replace("HIP_SYMBOL(scratch)", "(const void *)scratch"))
    obj = str(tmp_path / "static.o")
    r = subprocess.run([gxx, "-x", "c++"] + flags + ["-c", str(tmp_path / "static.cpp"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    objs.append(obj)
    exe = str(tmp_path / "driver")
    r = subprocess.run([gxx, "-x", "c"] + [f for f in flags if f != "-std=c++17"] + ["-c", str(tmp_path / "driver.c"),
                       "-o", str(tmp_path / "driver.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([gxx, "-fsanitize=address,undefined", str(tmp_path / "driver.o")] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # verify_asan_link_order=0: the process may start with other preloaded
    # libraries ahead of the ASan runtime (the driver links it directly)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "OK 0" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
