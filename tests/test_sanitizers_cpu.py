"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C
oracle (every function, on exactly sized heap buffers, including the empty and
one-element shapes and every optional input) and the C ABI's argument
validator (including sizes whose products overflow int64). Built with gcc/g++
for the host only; nothing here touches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

ORACLE_DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include "ss_oracle.c"

static unsigned rng = 12345u;
static double uni(void) { rng = rng * 1664525u + 1013904223u; return ((rng >> 8) / 16777216.0) * 2.0 - 1.0; }
/* exactly n doubles (one if n == 0, never read then): overruns hit the redzone */
static double* arr(int64_t n) {
  double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
  for (int64_t i = 0; i < n; ++i) p[i] = uni();
  return p;
}
static uint8_t* mask(int64_t n, int every) {
  uint8_t* p = (uint8_t*)malloc((size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = every ? 1 : (uni() > 0.7);
  return p;
}
#define CHECK(e) do { int rc_ = (e); if (rc_ != 0) { fprintf(stderr, "%s -> %d\n", #e, rc_); return 1; } } while (0)

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 0}, {1, 1, 1, 1}, {2, 3, 4, 17}, {1, 2, 16, 33}, {2, 1, 64, 5}, {3, 2, 3, 2}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int64_t B = shapes[s][0], C = shapes[s][1], N = shapes[s][2], L = shapes[s][3];
    const int64_t tok = B * C * L, bc = B * N * L, st = B * C * N;
    double *x = arr(tok), *dt = arr(tok), *z = arr(tok), *A = arr(C * N), *Bm = arr(bc), *Cm = arr(bc);
    double *D = arr(C), *bias = arr(C), *h0 = arr(st), *y = arr(tok), *hl = arr(st), *states = arr(tok * N);
    uint8_t *r0 = mask(B * L, 0), *r1 = mask(B * L, 1);
    for (int v = 0; v < 4; ++v) {
      CHECK(oracle_scan(B, C, N, L, x, dt, A, Bm, Cm, v & 1 ? D : NULL, v & 1 ? z : NULL, v & 2 ? bias : NULL,
                        v & 2 ? h0 : NULL, v == 3 ? r1 : (v == 2 ? r0 : NULL), v & 1, y, hl, v ? states : NULL, 0,
                        B * C));
    }
    double *state = arr(st), *xd = arr(B * C), *dd = arr(B * C), *zd = arr(B * C), *Bd = arr(B * N),
           *Cd = arr(B * N), *yd = arr(B * C);
    CHECK(oracle_update(B, C, N, state, xd, dd, A, Bd, Cd, D, zd, bias, 1, yd, 0, B * C));
    CHECK(oracle_update(B, C, N, state, xd, dd, A, Bd, Cd, NULL, NULL, NULL, 0, yd, 0, B * C));
    for (int per = 0; per < 2; ++per) {
      double* M = arr(B * C * L * L * (per ? N : 1));
      CHECK(oracle_effective_attention(B, C, N, L, dt, A, Bm, Cm, per ? bias : NULL, 1, per, per, M, 0, B * C));
      free(M);
    }
    for (int64_t W = 1; W <= 8; W += 3) {
      double* w = arr(C * W);
      CHECK(oracle_conv1d_silu(B, C, L, W, x, w, W > 1 ? bias : NULL, W > 4 ? r0 : NULL, y, 0, B * C));
      free(w);
    }
    for (int64_t R = 1; R <= 5; R += 4) {
      double *w = arr(C * R), *delta = arr(B * L * R);
      CHECK(oracle_dt_proj(B, C, L, R, w, delta, R > 1 ? bias : NULL, R > 1, y, 0, B * C));
      free(w);
      free(delta);
    }
    {
      const int64_t dk = N, dv = C + 1;
      double *q = arr(B * L * dk), *k = arr(B * L * dk), *vv = arr(B * L * dv), *g = arr(B * L);
      double *s0 = arr(B * dk * dv), *yg = arr(B * L * dv), *fs = arr(B * dk * dv);
      CHECK(oracle_gated_scan(B, L, dk, dv, q, k, vv, g, s0, yg, fs, 0, B));
      CHECK(oracle_gated_scan(B, L, dk, dv, q, k, vv, g, NULL, yg, NULL, 0, B));
      free(q); free(k); free(vv); free(g); free(s0); free(yg); free(fs);
    }
    free(x); free(dt); free(z); free(A); free(Bm); free(Cm); free(D); free(bias); free(h0); free(y); free(hl);
    free(states); free(r0); free(r1); free(state); free(xd); free(dd); free(zd); free(Bd); free(Cd); free(yd);
  }
  /* rejected arguments return an error code, touching nothing */
  if (oracle_scan(1, 1, 0, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL, 0, 1) == 0)
    return 2;
  puts("oracle ok");
  return 0;
}
"""

VALIDATOR_DRIVER = r"""
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include "ss_validate.h"

int main() {
  const int64_t big = INT64_MAX, M = 1 << 20;
  const int64_t sizes[] = {-1, 0, 1, 7, 64, 1 << 20, (int64_t)1 << 40, big / 2, big};
  int n = 0;
  for (int64_t b : sizes)
    for (int64_t c : sizes)
      for (int64_t l : sizes)
        for (int64_t nn : {(int64_t)1, (int64_t)16, (int64_t)64, (int64_t)65}) {
          bool noop = false;
          ss_scan_args a{};
          a.batch = b; a.channels = c; a.state_dim = nn; a.seqlen = l; a.io_dtype = SS_BF16;
          a.x = (void*)(1 * M); a.dt = (void*)(2 * M); a.A = (const float*)(3 * M); a.B = (void*)(4 * M);
          a.C = (void*)(5 * M); a.y = (void*)(6 * M); a.h0 = (const float*)(7 * M); a.h_last = (float*)(7 * M);
          n += ss::validate_scan(a, &noop) == SS_OK;
          n += ss::validate_scan_states(a, (const float*)(8 * M), l / 2) == SS_OK;
          ss_update_args u{};
          u.batch = b; u.channels = c; u.state_dim = nn; u.io_dtype = SS_F32; u.state = (float*)(1 * M);
          u.x = (void*)(2 * M); u.dt = (void*)(3 * M); u.A = (const float*)(4 * M); u.B = (void*)(5 * M);
          u.C = (void*)(6 * M); u.y = (void*)(7 * M);
          n += ss::validate_update(u, &noop) == SS_OK;
          ss::GatedArgs g{b, l, nn, c, SS_BF16, SS_F32, (void*)(1 * M), (void*)(2 * M), (void*)(3 * M),
                          (const float*)(4 * M), nullptr, (void*)(5 * M), nullptr};
          n += ss::validate_gated(g, &noop) == SS_OK;
          ss::AttnArgs at{b, c, nn, l, SS_BF16, (void*)(1 * M), (const float*)(2 * M), (void*)(3 * M),
                          (void*)(4 * M), nullptr, 1, 0, 1, (float*)(6 * M)};
          n += ss::validate_attention(at, &noop) == SS_OK;
          ss::ConvArgs cv{b, c, l, 4, SS_BF16, (void*)(1 * M), (const float*)(2 * M), nullptr, nullptr, (void*)(4 * M)};
          n += ss::validate_conv(cv, &noop) == SS_OK;
          ss::ProjArgs pj{b, c, l, nn, SS_BF16, (void*)(1 * M), (void*)(2 * M), nullptr, 1, (void*)(4 * M)};
          n += ss::validate_proj(pj, &noop) == SS_OK;
        }
  std::printf("validator ok (%d accepted)\n", n);
  return 0;
}
"""


def _run(cmd, **kw):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)


def _sanitizers_work(tmp_path, compiler):
    """gcc/g++ here must link the sanitizer runtimes."""
    src = tmp_path / ("probe.c" if compiler == "gcc" else "probe.cpp")
    src.write_text("int main(void){return 0;}\n")
    r = _run([compiler, *SAN, str(src), "-o", str(tmp_path / "probe")])
    return r.returncode == 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    if not _sanitizers_work(tmp_path, "gcc"):
        pytest.skip("gcc cannot link the address/undefined sanitizer runtimes here")
    src = tmp_path / "oracle_driver.c"
    src.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_driver"
    r = _run(["gcc", "-std=c11", "-Wall", "-Wextra", *SAN, "-I", os.path.join(ROOT, "oracle"), str(src), "-o",
              str(exe), "-lm"])
    assert r.returncode == 0, r.stdout
    r = _run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"}, timeout=300)
    assert r.returncode == 0 and "oracle ok" in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not installed")
def test_validator_under_asan_ubsan(tmp_path):
    if not _sanitizers_work(tmp_path, "g++"):
        pytest.skip("g++ cannot link the address/undefined sanitizer runtimes here")
    src = tmp_path / "validator_driver.cpp"
    src.write_text(VALIDATOR_DRIVER)
    exe = tmp_path / "validator_driver"
    r = _run(["g++", "-std=c++17", "-Wall", *SAN, "-I", os.path.join(ROOT, "include"), "-I",
              os.path.join(ROOT, "selective_state_space_ss_amd", "csrc"), str(src), "-o", str(exe)])
    assert r.returncode == 0, r.stdout
    r = _run([str(exe)], timeout=300)
    assert r.returncode == 0 and "validator ok" in r.stdout, r.stdout
