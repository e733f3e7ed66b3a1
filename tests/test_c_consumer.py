"""The C ABI from a plain C99 program: include/kivi.h compiles as strict C
(gcc -std=c99 -pedantic -Werror) and a program linked against libkivi.so
gets the buffer sizes, workspace bytes and host-side error statuses that the
Python binding reports.  Only calls that return before any device work are
made, so this runs without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
kivi = pytest.importorskip("decode_attention_channel_amd.kivi")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "kivi.h"

static kivi_geom geom(int bits, int meta) {
  kivi_geom g;
  memset(&g, 0, sizeof g);
  g.batch = 2; g.kv_heads = 3; g.q_per_kv = 4; g.head_dim = 128; g.bits = bits;
  g.group = 32; g.residual = 128; g.max_tokens = 1024; g.meta_format = meta;
  return g;
}

int main(void) {
  int bits, meta;
  for (bits = 2; bits <= 4; bits += 2)
    for (meta = 0; meta <= 1; ++meta) {
      kivi_geom g = geom(bits, meta);
      size_t b[KIVI_NUM_BUFS];
      kivi_status s = kivi_cache_layout(&g, b);
      printf("layout %d %d %d %zu %zu %zu\n", bits, meta, (int)s, b[KIVI_BUF_RECORDS],
             b[KIVI_BUF_K_RES], b[KIVI_BUF_V_RES]);
      printf("ws %d %d %zu %zu\n", bits, meta, kivi_decode_workspace_bytes(&g, 1024, 160),
             kivi_decode_workspace_bytes(&g, 0, 1));
    }
  {
    /* host-side rejections: nothing reaches the device */
    kivi_geom g = geom(3, 0);
    kivi_cache c;
    size_t b[KIVI_NUM_BUFS];
    memset(&c, 0, sizeof c);
    printf("status bits3 %d\n", (int)kivi_cache_layout(&g, b));
    g = geom(2, 0);
    printf("status nullgeom %d\n", (int)kivi_cache_layout(NULL, b));
    printf("status nullcache %d\n",
           (int)kivi_quantize_prefill(&g, &c, NULL, NULL, 256, NULL));
    printf("string %s\n", kivi_status_string(KIVI_E_WORKSPACE));
  }
  return 0;
}
"""


def test_plain_c_program_uses_the_abi(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lib = kivi.library_path()
    src, exe = tmp_path / "consumer.c", tmp_path / "consumer"
    src.write_text(PROGRAM)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src),
                    "-L", os.path.dirname(lib), "-lkivi",
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    lines = out.splitlines()
    by_key = {}
    for ln in lines:
        f = ln.split()
        by_key[tuple(f[:3]) if f[0] in ("layout", "ws") else tuple(f[:2])] = f
    for bits in (2, 4):
        for meta in (kivi.META_FP32, kivi.META_FP16_BF16):
            g = kivi.Geom(2, 3, 4, bits=bits, max_tokens=1024, meta_format=meta)
            f = by_key[("layout", str(bits), str(meta))]
            assert int(f[3]) == 0
            assert [int(x) for x in f[4:7]] == list(kivi.cache_layout(g))
            f = by_key[("ws", str(bits), str(meta))]
            assert int(f[3]) == kivi.workspace_bytes(g, 1024, 160)
            assert int(f[4]) == kivi.workspace_bytes(g, 0, 1)
    # the statuses kivi.h assigns to these rejections
    assert by_key[("status", "bits3")][2] == "3"       # KIVI_E_UNSUPPORTED
    assert by_key[("status", "nullgeom")][2] == "1"    # KIVI_E_NULL
    assert by_key[("status", "nullcache")][2] == "1"   # KIVI_E_NULL (cache buffers unset)
    assert out.splitlines()[-1] == "string decode workspace NULL or too small"
