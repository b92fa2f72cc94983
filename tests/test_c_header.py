"""The boundary is plain C: a C99 program that includes include/fa.h compiles with gcc -Wall -Wextra
-Werror -pedantic, links against libfa.so, and gets status codes (no HIP call) for bad arguments of
every entry point.  Runs on the CPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

import transformer_attention_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fa.h"

static int expect(const char* what, int got, int want) {
  if (got != want) {
    printf("%s: got %d (%s), want %d\n", what, got, fa_status_str(got), want);
    return 1;
  }
  return 0;
}

int main(void) {
  int bad = 0;
  float lse_host[4];
  const int32_t cu[2] = {0, 4};
  if (fa_version() < 1) bad = 1;
  if (strlen(fa_status_str(FA_ERR_ALIAS)) == 0) bad = 1;
  bad |= expect("fa_fwd null q", fa_fwd(NULL, (void*)16, (void*)32, (void*)48, lse_host, 1, 1, 4, 64,
                                        FA_LAYOUT_BHSD, 1, 0.125f, FA_DTYPE_BF16, NULL), FA_ERR_NULL);
  bad |= expect("fa_fwd bad layout", fa_fwd((void*)16, (void*)32, (void*)48, (void*)64, lse_host, 1, 1, 4, 64, 7, 1,
                                            0.125f, FA_DTYPE_BF16, NULL), FA_ERR_BAD_LAYOUT);
  bad |= expect("fa_fwd_ex window without causal",
                fa_fwd_ex((void*)16, (void*)32, (void*)48, (void*)64, lse_host, 1, 1, 4, 4, 64, FA_LAYOUT_BHSD, 0, 3, 0,
                          0, 4, 0.125f, FA_DTYPE_BF16, NULL), FA_ERR_BAD_RANGE);
  bad |= expect("fa_merge no parts", fa_merge((void*)16, lse_host, 0, (void*)64, lse_host, 1, 1, 4, 64,
                                              FA_LAYOUT_BHSD, FA_DTYPE_BF16, NULL), FA_ERR_BAD_DIM);
  bad |= expect("fa_fwd_varlen D=80", fa_fwd_varlen((void*)16, (void*)32, (void*)48, (void*)64, lse_host, cu, cu, 1, 1,
                                                    4, 4, 4, 80, 1, 0.125f, FA_DTYPE_BF16, NULL), FA_ERR_UNSUPPORTED);
  bad |= expect("fa_bwd bad dtype", fa_bwd((void*)16, (void*)32, (void*)48, (void*)64, lse_host, (void*)80, (void*)96,
                                           (void*)112, (void*)128, lse_host, 1, 1, 4, 64, FA_LAYOUT_BHSD, 1, 0.125f, 9,
                                           NULL), FA_ERR_BAD_DTYPE);
  bad |= expect("fa_bwd_ex chunk out of range",
                fa_bwd_ex((void*)16, (void*)32, (void*)48, (void*)64, lse_host, (void*)80, (void*)96, (void*)112,
                          (void*)128, lse_host, 1, 1, 4, 4, 64, FA_LAYOUT_BHSD, 1, -1, 0, 3, 2, 0.125f, FA_DTYPE_BF16,
                          NULL), FA_ERR_BAD_RANGE);
  bad |= expect("fa_bwd_varlen null offsets",
                fa_bwd_varlen((void*)16, (void*)32, (void*)48, (void*)64, lse_host, (void*)80, (void*)96, (void*)112,
                              (void*)128, lse_host, NULL, cu, 1, 1, 4, 4, 4, 4, 64, 1, 0.125f, FA_DTYPE_BF16, NULL),
                FA_ERR_NULL);
  bad |= expect("fa_bwd_noalloc beyond the scratch array",
                fa_bwd_noalloc((void*)16, (void*)32, (void*)48, (void*)64, lse_host, (void*)80, (void*)96, (void*)112,
                               (void*)128, 1, 1, (int64_t)FA_NOALLOC_MAX_ROWS + 1, 64, FA_LAYOUT_BHSD, 1, 0.125f,
                               FA_DTYPE_BF16, NULL), FA_ERR_SCRATCH_LIMIT);
  bad |= expect("fa_bwd_atomic fp32",
                fa_bwd_atomic((void*)16, (void*)32, (void*)48, (void*)64, lse_host, (void*)80, (void*)96, (void*)112,
                              (void*)128, lse_host, (float*)144, 1, 1, 4, 64, FA_LAYOUT_BHSD, 1, 0.125f, FA_DTYPE_FP32,
                              NULL), FA_ERR_UNSUPPORTED);
  printf(bad ? "FAIL\n" : "OK version %d\n", fa_version());
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_c_program_compiles_links_and_gets_status_codes():
    lib = fa.library_path()
    if not os.path.exists(lib):
        pytest.skip("libfa.so is not built")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "use_fa.c")
        exe = os.path.join(d, "use_fa")
        open(src, "w").write(PROGRAM)
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), src,
               "-o", exe, "-L", os.path.dirname(lib), "-lfa", "-Wl,-rpath," + os.path.dirname(lib)]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
        assert out.returncode == 0, out.stdout + out.stderr
        assert out.stdout.startswith("OK version %d" % fa.version())
