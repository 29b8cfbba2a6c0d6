"""Host-side sanitizer run of the C ABI (CPU only).

The library is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer on its host
code (device code is built as usual), loaded into a fresh Python process with the
sanitizer runtime preloaded, and every host-only path is driven: shape validation
(including extreme sizes, where the size and launch arithmetic could overflow),
workspace queries and the argument checks of every entry point. Any sanitizer report
fails the test. No GPU is touched.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


DRIVER = textwrap.dedent(r"""
    import ctypes, itertools, sys
    sys.path.insert(0, ROOT)
    from long_context_approximate_amd import spava
    lib = spava.load(LIB)
    FAKE = 0x10000
    big = 2**31 - 1
    values = {
        "seq_len": [1, 4096, 3000, (1 << 30) * 4, (1 << 24), (2**31 - 1) * 16, 2**62],
        "num_hosts": [1, 3, 4, 64, 2**31 - 1],
        "num_q_heads": [1, 8, 28, 65535, 65536, big],
        "num_kv_heads": [1, 2, 4, big],
        "head_dim": [64, 128, 96],
        "anchor_len": [0, 100, big],
        "passing_len": [0, 64, big],
        "window": [1, 32, big],
    }
    n = ctypes.c_size_t()
    count = 0
    for combo in itertools.product(*values.values()):
        kw = dict(zip(values.keys(), combo))
        for dtype in (0, 1):
            sh = spava.make_shape(dtype=dtype, **kw)
            s = ctypes.byref(sh)
            st = lib.spava_validate_shape(s)
            lib.spava_select_workspace_bytes(s, ctypes.byref(n))
            lib.spava_attn_workspace_bytes(s, ctypes.byref(n))
            lib.spava_layer_overlap_workspace_bytes(s, ctypes.byref(n))
            for nq in (1, 256, 1 << 30, (1 << 30) + 1):
                lib.spava_query_workspace_bytes(s, nq, ctypes.byref(n))
                lib.spava_select_query_workspace_bytes(s, nq, ctypes.byref(n))
            # Entry points with a missing pointer: must return before any HIP call.
            lib.spava_select_passing(s, None, FAKE, FAKE, None, FAKE, 1 << 40, None)
            lib.spava_approx_attn_fwd(s, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 40, None)
            lib.spava_layer_overlap_fwd(s, None, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40,
                                        None, None)
            lib.spava_query_attn_fwd(s, 16, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                                     None)
            lib.spava_select_passing_query(s, 16, None, FAKE, FAKE, None, FAKE, 1 << 40, None)
            lib.spava_select_passing_noalloc(s, None, FAKE, FAKE, None, None)
            count += 1
    for code in range(-1, 10):
        lib.spava_status_string(code)
    print("driven", count)
""")


def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if not os.path.exists(HIPCC) or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not available")
    csrc = os.path.join(ROOT, "long_context_approximate_amd", "csrc")
    from long_context_approximate_amd.build import SOURCES
    lib = str(tmp_path / "libspava_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-o", lib, *[os.path.join(csrc, f) for f in SOURCES]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    script = tmp_path / "drive.py"
    script.write_text(f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + DRIVER)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, env=env,
                         timeout=600)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert "driven" in run.stdout
