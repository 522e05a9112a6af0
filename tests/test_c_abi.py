"""The C ABI as a C program sees it (no GPU): include/ks.h and
include/ks_measure.h compile as C99 with warnings as errors, every declared
function is taken by address and linked from libks.so, and calls that fail
argument validation, or have nothing to do, return their documented status
without touching the device."""
import os
import shutil
import subprocess

import pytest

import kv_cache_compaction_amd as ks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "ks.h"
#include "ks_measure.h"

static int fail(const char* what, int got, int want) {
  fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, ks_last_error());
  return 1;
}

int main(void) {
  int bad = 0;
  /* every declared function, by address */
  void (*fns[])(void) = { %FNS% };
  for (size_t i = 0; i < sizeof(fns) / sizeof(fns[0]); ++i)
    if (!fns[i]) bad |= fail("null function", 0, 1);
  if (strncmp(ks_version(), "libks", 5) != 0) bad |= fail("version", 0, 1);
  /* nothing to do: B == 0 */
  int st = ks_compact_block_table(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 32, NULL);
  if (st != KS_OK) bad |= fail("compact B=0", st, KS_OK);
  st = ks_evict_attn_fwd_rope(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 4, 2,
                              128, KS_BF16, 0.1f, 10000.0f, NULL, 0, NULL);
  if (st != KS_OK) bad |= fail("fused forward B=0", st, KS_OK);
  /* refused before any launch */
  void* p = (void*)(size_t)4096;
  st = ks_evict_attn_fwd(p, p, p, p, p, p, 1, 64, 3, 2, 128, KS_BF16, 0.1f, p, 1 << 20, NULL);
  if (st != KS_ERR_INVALID_ARG) bad |= fail("Hq not a multiple of Hkv", st, KS_ERR_INVALID_ARG);
  st = ks_evict_attn_bwd(p, p, p, p, p, p, p, p, p, p, 1, 64, 4, 2, 128, KS_F32, 0.1f, p,
                         1 << 20, NULL);
  if (st != KS_ERR_UNSUPPORTED) bad |= fail("fp32 backward", st, KS_ERR_UNSUPPORTED);
  size_t need = ks_paged_decode_workspace(4, 32, 128, 100);
  if (need == 0) bad |= fail("decode workspace query", 0, 1);
  st = ks_paged_decode(p, p, p, p, p, p, NULL, 4, 32, 8, 128, 100, 10, KS_BF16, 0.1f, p,
                       need - 1, NULL);
  if (st != KS_ERR_WORKSPACE) bad |= fail("short workspace", st, KS_ERR_WORKSPACE);
  if (ks_paged_decode_noalloc_max_scratch() == 0) bad |= fail("scratch size", 0, 1);
  puts(bad ? "FAIL" : "OK");
  return bad;
}
"""


def _declared():
    names = set()
    for h in ("ks.h", "ks_measure.h"):
        names.update(ks.header_functions(os.path.join(INC, h)))
    return sorted(names)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_headers_compile_as_c_and_link(tmp_path):
    names = _declared()
    assert "ks_evict_attn_bwd_rope" in names and "ks_measure_mfma_bf16" in names
    src = PROGRAM.replace("%FNS%", ", ".join(f"(void (*)(void)){n}" for n in names))
    c = tmp_path / "abi.c"
    c.write_text(src)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(ks.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{INC}", str(c), "-o", str(exe),
           f"-L{libdir}", "-l:libks.so", f"-Wl,-rpath,{libdir}"]
    out = subprocess.run(cmd, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "OK", run.stdout + run.stderr
