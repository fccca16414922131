"""include/plx.h is plain C: a C99 program that includes it, links against
libplx.so and calls the host-side entry points (version, status strings,
workspace sizes, argument validation) compiles and runs without a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "parallax_local_linear_plx_amd")

PROGRAM = r"""
#include <stdio.h>
#include "plx.h"

int main(void) {
  if (plx_abi_version() != PLX_ABI_VERSION) return 1;
  if (plx_status_string(PLX_ERR_WORKSPACE) == NULL) return 2;
  /* validation happens before any device call */
  if (plx_fwd_prefill(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 1, 64, 0.125f,
                      PLX_BF16, NULL) != PLX_ERR_INVALID_ARG) return 3;
  if (plx_fwd_prefill_ex(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 1, 64, 0.125f,
                         PLX_UNIFORM_WEIGHTS | PLX_NO_INTERCEPT, PLX_BF16, NULL) != PLX_ERR_INVALID_ARG)
    return 4;
  if (plx_decode_workspace_size(2, 4, 2, 1024, 128, 4) != (size_t)2 * 4 * 4 * (2 * 128 + 4) * 4) return 5;
  if (plx_bwd_workspace_size(1, 1, 1, 0, 64) != 0) return 6;
  if (plx_qkvr_proj(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 1, 1, 64, PLX_BF16, NULL) !=
      PLX_ERR_INVALID_ARG) return 7;
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_header_compiles_as_c99_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libplx.so")):
        pytest.fail("libplx.so is not built")
    src = tmp_path / "use_plx.c"
    exe = tmp_path / "use_plx"
    src.write_text(PROGRAM)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", LIBDIR, "-lplx", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", (res.returncode, res.stdout, res.stderr)
