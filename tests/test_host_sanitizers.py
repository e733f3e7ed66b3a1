"""Host code of libkivi.so under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt (into a temporary folder, not in-tree) with the
sanitizers on its host code only (`-Xarch_host`; the GPU code is built as
usual), and a C driver built with the same sanitizers calls every entry
point with geometries and counters drawn from a list of extreme values
(negative, zero, off-by-one around the supported sizes, 2^24, INT_MAX).
Every call is given a NULL cache buffer or an invalid argument, so each must
return an error status from host validation before any HIP call: the
driver fails on KIVI_OK or KIVI_E_HIP, and the sanitizers on any memory error
or undefined behaviour (signed overflow in the size arithmetic, invalid enum
loads).  No GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
build = pytest.importorskip("decode_attention_channel_amd.build")

DRIVER = r"""
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "kivi.h"

static const int V[] = {INT_MIN, -4097, -1, 0, 1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 64, 127,
                        128, 129, 160, 4096, 4097, 65535, 65536, 1 << 20, 1 << 24,
                        (1 << 24) + 32, 1 << 30, INT_MAX};
#define NV ((int)(sizeof V / sizeof V[0]))
static unsigned long long st = 88172645463325252ull;   /* xorshift64 */
static int pick(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return V[st % NV]; }

int main(int argc, char **argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  long long calls = 0, valid_layouts = 0;
  size_t b[KIVI_NUM_BUFS];
  int32_t mp, fl, di[8];
  uint16_t d16[8];
  float df[8];
  for (int it = 0; it < iters; ++it) {
    kivi_geom g;
    memset(&g, 0, sizeof g);
    g.batch = pick(); g.kv_heads = pick(); g.q_per_kv = pick();
    g.head_dim = (it & 1) ? 128 : pick();
    g.bits = (it & 2) ? ((it & 4) ? 4 : 2) : pick();
    g.group = (it & 8) ? 32 : pick();
    g.residual = pick(); g.max_tokens = pick();
    g.meta_format = it % 5 == 0 ? pick() : (it >> 4) & 1;
    g.flags = it % 7 == 0 ? pick() : (it >> 5) & 1;
    if (kivi_cache_layout(&g, b) == KIVI_OK) ++valid_layouts;
    (void)kivi_decode_workspace_bytes(&g, pick(), pick());
    (void)kivi_paged_layout(&g, pick(), pick(), b, &mp);
    kivi_cache c;
    memset(&c, 0, sizeof c);
    c.n_q = pick(); c.n_res = pick(); c.res_start = pick();
    kivi_paged_cache pc;
    memset(&pc, 0, sizeof pc);
    pc.page_groups = pick(); pc.num_pages = pick();
    kivi_status s[12];
    s[0] = kivi_quantize_prefill(&g, &c, d16, d16, pick(), NULL);
    s[1] = kivi_append_token(&g, &c, d16, d16, NULL);
    s[2] = kivi_flush_residual(&g, &c, &fl, NULL);
    s[3] = kivi_decode_attention(&g, &c, d16, df, 0.1f, df, 64, NULL);
    s[4] = kivi_decode_step(&g, &c, d16, d16, d16, df, 0.1f, df, 64, &fl, NULL);
    s[5] = kivi_decode_step_noalloc(&g, &c, d16, d16, d16, df, 0.1f, &fl, NULL);
    s[6] = kivi_dense_decode_attention(&g, NULL, d16, pick(), d16, df, 0.1f, df, 64, NULL);
    s[7] = kivi_ragged_prefill(&g, &c, d16, d16, pick(), di, di, NULL);
    s[8] = kivi_ragged_decode_step(&g, &c, di, di, d16, d16, d16, df, 0.1f, df, 64, NULL);
    s[9] = kivi_paged_prefill(&g, &pc, d16, d16, pick(), di, di, NULL);
    s[10] = kivi_paged_decode_step(&g, &pc, di, di, d16, d16, d16, df, 0.1f, df, 64, NULL);
    s[11] = kivi_cache_layout(NULL, b);
    for (int i = 0; i < 12; ++i, ++calls)
      if (s[i] == KIVI_OK || s[i] == KIVI_E_HIP) {
        printf("iteration %d call %d: status %d\n", it, i, (int)s[i]);
        return 1;
      }
  }
  for (int k = -5; k < 20; ++k) (void)kivi_status_string((kivi_status)k);
  printf("ok %lld %lld\n", calls, valid_layouts);
  return 0;
}
"""


def test_host_validation_is_sanitizer_clean(tmp_path):
    hipcc = build.HIPCC
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("hipcc / clang not available")
    lib = tmp_path / "libkivi.so"
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in build.FLAGS if f not in ("-O3", "-Rpass-analysis=kernel-resource-usage")]
    subprocess.run([hipcc, *flags, "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"),
                    "-I", build.CSRC, "-o", str(lib),
                    *[os.path.join(build.CSRC, s) for s in build.SOURCES]],
                   check=True, capture_output=True, text=True)
    src, exe = tmp_path / "driver.c", tmp_path / "driver"
    src.write_text(DRIVER)
    subprocess.run([clang, "-std=c99", "-g", "-O1", "-fsanitize=address,undefined",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    str(src), "-L", str(tmp_path), "-lkivi", "-Wl,-rpath," + str(tmp_path)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe), "20000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    ok, calls, valid = r.stdout.split()
    assert ok == "ok" and int(calls) == 12 * 20000 and int(valid) > 0
