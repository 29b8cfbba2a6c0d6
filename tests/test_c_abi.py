"""The boundary is plain C: the header compiles as C99 and a C program links against the
library and runs its host-only calls (no GPU)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "long_context_approximate_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "spava.h"

int main(void) {
  spava_shape s;
  size_t sel = 0, attn = 0, ovl = 0, qry = 0;
  memset(&s, 0, sizeof s);
  s.seq_len = 131072; s.num_hosts = 8; s.num_q_heads = 28; s.num_kv_heads = 4;
  s.head_dim = 128; s.anchor_len = 4096; s.passing_len = 2048; s.window = 128;
  s.dtype = SPAVA_BF16; s.sm_scale = 0.0;
  s.q_stride_tok = 28 * 128; s.q_stride_head = 128;
  s.kv_stride_tok = 4 * 128; s.kv_stride_head = 128;
  s.o_stride_tok = 28 * 128; s.o_stride_head = 128;
  if (spava_abi_version() != 2) return 1;
  if (spava_validate_shape(&s) != SPAVA_OK) return 2;       /* zeroed options: defaults */
  s.schedule = SPAVA_SCHED_ZIGZAG; s.select_logits = SPAVA_LOGITS_RECOMPUTE;
  if (spava_validate_shape(&s) != SPAVA_OK) return 10;
  s.schedule = 7;
  if (spava_validate_shape(&s) != SPAVA_ERR_OPTION) return 11;
  s.schedule = SPAVA_SCHED_LONGEST_FIRST; s.select_logits = SPAVA_LOGITS_AUTO;
  if (spava_select_workspace_bytes(&s, &sel) != SPAVA_OK) return 3;
  if (spava_attn_workspace_bytes(&s, &attn) != SPAVA_OK) return 4;
  if (spava_layer_overlap_workspace_bytes(&s, &ovl) != SPAVA_OK) return 5;
  if (spava_query_workspace_bytes(&s, 256, &qry) != SPAVA_OK) return 6;
  if (spava_approx_attn_fwd(&s, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != SPAVA_ERR_NULL)
    return 7;
  s.seq_len = 131071;
  if (spava_validate_shape(&s) != SPAVA_ERR_SHAPE) return 8;
  printf("%zu %zu %zu %zu %s\n", sel, attn, ovl, qry, spava_status_string(SPAVA_ERR_SHAPE));
  return 0;
}
"""


@pytest.fixture(scope="module")
def cc():
    c = shutil.which("gcc") or shutil.which("cc")
    if c is None:
        pytest.skip("no C compiler")
    return c


def test_header_is_strict_c99(cc, tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "spava.h"\nint main(void) { return spava_abi_version() == 1 ? 0 : 1; }\n')
    res = subprocess.run([cc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                          "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_c_program_links_and_runs_host_calls(cc, tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libspava.so")):
        pytest.skip("libspava.so not built")
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    res = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                          str(src), "-L", LIB_DIR, "-lspava", f"-Wl,-rpath,{LIB_DIR}", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    sel, attn, ovl, qry = (int(v) for v in run.stdout.split()[:4])
    assert sel > 3_000_000_000 and attn > 0 and ovl >= sel + attn and qry > 0
