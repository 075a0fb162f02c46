"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the C ABI's
argument validation and launch planning (CPU only, no GPU).

The library is rebuilt with the host half of every source instrumented
(device code is not: the sanitizers apply to the host pass only) and
driven through ctypes in a child process that preloads the sanitizer
runtime: every entry point with rejected arguments (null, misaligned,
negative, oversized, unsupported), empty calls, workspace-size queries at
extreme sizes, and -- on a host without a GPU -- calls that pass
validation, run the split planners and fail at the launch.  Any report
from either sanitizer fails the test.
"""

import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_mqa_gqa_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _asan_runtime():
    pats = ["/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"]
    for p in pats:
        hits = sorted(glob.glob(p))
        if hits:
            return hits[-1]
    return None


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


DRIVER = r'''
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
sig = {
  "mqa_prefill_workspace_size": (sz, [i, i, i, i, i, i]),
  "mqa_prefill": (i, [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]),
  "mqa_prefill_ex_workspace_size": (sz, [i, i, i, i, i, i, i, i]),
  "mqa_prefill_ex": (i, [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]),
  "mqa_decode_workspace_size": (sz, [i, i, i, i, i]),
  "mqa_decode": (i, [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]),
  "mla_decode_workspace_size": (sz, [i, i, i]),
  "mla_decode_absorbed": (i, [vp, vp, vp, vp, vp, i, i, i, f, i, i, vp, sz, vp]),
  "mla_decode_sparse_workspace_size": (sz, [i, i, i]),
  "mla_decode_sparse": (i, [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp, sz, vp]),
  "mla_absorb_query": (i, [vp, vp, vp, vp, vp, vp, i, i, i, vp]),
  "mla_cache_append": (i, [vp, vp, vp, vp, vp, vp, i, i, i, vp]),
  "mla_output_project": (i, [vp, vp, vp, i, i, i, i, vp]),
  "mqa_status_string": (ctypes.c_char_p, [i]),
  "mqa_last_hip_error_name": (ctypes.c_char_p, []),
}
for n, (r, a) in sig.items():
    fn = getattr(lib, n); fn.restype = r; fn.argtypes = a
P, MIS, N = 4096, 4104, None
BIG = 2 ** 31 - 1
launch_ok = sys.argv[2] == "1"
n_calls = 0
def call(n, *a, expect=None):
    global n_calls
    st = getattr(lib, n)(*a); n_calls += 1
    if expect is not None and st != expect:
        raise SystemExit(f"{n}{a}: status {st}, expected {expect}")
    return st
# workspace queries at ordinary and extreme sizes
for B in (0, 1, 7, BIG):
    for T in (0, 1, 4097, BIG):
        for d in (1, 128, 192, 512, BIG):
            call("mqa_prefill_workspace_size", B, 16, 1, T, d, 1)
            call("mqa_prefill_ex_workspace_size", B, 16, 1, T, T, d, 128, 1)
            call("mqa_decode_workspace_size", B, 16, 1, T, d)
        call("mla_decode_workspace_size", B, 128, T)
        call("mla_decode_sparse_workspace_size", B, 128, T)
# prefill rejections
for args, exp in [
    ((P, P, P, P, N, 1, 16, 3, 64, 512, .05, 1, 1, 1, P, 1 << 40, N), -1),
    ((P, P, P, P, N, -1, 16, 1, 64, 512, .05, 1, 1, 1, P, 1 << 40, N), -1),
    ((N, P, P, P, N, 1, 16, 1, 64, 512, .05, 1, 1, 1, P, 1 << 40, N), -1),
    ((P, P, P, MIS, N, 1, 16, 1, 64, 512, .05, 1, 1, 1, P, 1 << 40, N), -1),
    ((P, P, P, P, N, 1, 16, 1, 64, 512, float("nan"), 1, 1, 1, P, 1 << 40, N), -1),
    ((P, P, P, P, N, 1, 16, 1, 64, 256, .05, 1, 1, 1, P, 1 << 40, N), -2),
    ((P, P, P, P, N, 1, 16, 1, 64, 512, .05, 1, 1, 1, N, 0, N), -3),
    ((P, P, P, P, N, 1, 16, 1, BIG, 512, .05, 1, 1, 1, P, 1 << 40, N), -2),
    ((P, P, P, P, N, 1, 16, 1, 64, BIG, .05, 1, 0, 0, N, 0, N), -2),
    ((N, N, N, N, N, 0, 16, 1, 64, 512, .05, 1, 1, 1, N, 0, N), 0),
]:
    call("mqa_prefill", *args, expect=exp)
call("mqa_prefill_ex", P, P, P, P, N, 1, 16, 1, 65, 64, 512, 512, .05, 1, 1, 1, P, 1 << 40, N, expect=-1)
call("mqa_prefill_ex", P, P, P, P, N, 1, 16, 1, 0, 64, 512, 512, .05, 1, 1, 1, N, 0, N, expect=0)
call("mqa_prefill_ex", P, P, P, P, N, 1, 16, 1, 5, 0, 512, 512, .05, 0, 1, 1, N, 0, N, expect=-1)
call("mqa_prefill_ex", P, P, P, P, N, 1, 16, 1, 5, 9, 512, 128, .05, 1, 1, 1, P, 1 << 40, N, expect=-2)
# decode / MLA rejections
call("mqa_decode", P, P, P, P, P, N, 2, 16, 1, 64, 512, .05, 1, 1, P, 1 << 40, N)
call("mqa_decode", P, P, P, N, P, N, 2, 16, 1, 64, 512, .05, 1, 1, P, 1 << 40, N, expect=-1)
call("mqa_decode", P, P, P, P, P, N, 2, 64, 1, 64, 128, .05, 1, 1, P, 1 << 40, N, expect=-2)
call("mqa_decode", P, P, P, P, P, N, 2, 16, 1, 0, 512, .05, 1, 1, P, 1 << 40, N, expect=-1)
call("mqa_decode", P, P, P, P, P, N, 2, 16, 1, 64, 512, .05, 1, 1, P, 16, N, expect=-3)
call("mla_decode_absorbed", P, P, P, P, N, 2, 24, 64, .07, 1, 1, P, 1 << 40, N, expect=-2)
call("mla_decode_absorbed", P, P, P, P, N, 2, 128, BIG, .07, 1, 1, P, 1 << 40, N, expect=-2)
call("mla_decode_absorbed", P, P, P, P, N, 2, 128, 64, .07, 1, 1, P, 8, N, expect=-3)
call("mla_decode_sparse", P, P, P, P, N, 2, 128, 64, 0, .07, 1, 1, P, 1 << 40, N, expect=-1)
call("mla_decode_sparse", P, P, P, P, N, 2, 128, 64, BIG, .07, 1, 1, P, 16, N, expect=-3)
call("mla_absorb_query", P, P, P, P, P, MIS, 2, 128, 1, N, expect=-1)
call("mla_cache_append", P, P, P, P, P, P, 2, 0, 1, N, expect=-1)
call("mla_output_project", P, P, P, 2, 128, 0, 0, N, expect=-2)
for s in range(-6, 3):
    assert lib.mqa_status_string(s)
# valid calls: the planners run; on a host without a GPU the launch fails
if launch_ok:
    ws = 1 << 40
    call("mqa_prefill", P, P, P, P, N, 2, 16, 1, 4096, 512, .05, 1, 1, 1, P, ws, N, expect=-4)
    call("mqa_prefill", P, P, P, P, P, 1, 64, 8, 8192, 128, .05, 1, 1, 0, P, ws, N, expect=-4)
    call("mqa_prefill_ex", P, P, P, P, N, 1, 128, 128, 8192, 8192, 192, 128, .07, 1, 1, 1, P, ws, N, expect=-4)
    call("mqa_prefill", P, P, P, P, P, 1, 16, 1, 128, 512, .05, 1, 0, 0, N, 0, N, expect=-4)
    call("mqa_decode", P, P, P, P, P, P, 128, 64, 8, 16384, 128, .08, 1, 1, P, ws, N, expect=-4)
    call("mla_decode_absorbed", P, P, P, P, P, 32, 128, 32768, .07, 1, 1, P, ws, N, expect=-4)
    call("mla_decode_sparse", P, P, P, P, P, 32, 128, 32768, 2048, .07, 1, 1, P, ws, N, expect=-4)
    call("mla_absorb_query", P, P, P, P, P, P, 32, 128, 1, N, expect=-4)
    call("mla_cache_append", P, P, P, P, P, P, 32, 32768, 1, N, expect=-4)
    call("mla_output_project", P, P, P, 32, 128, 1, 0, N, expect=-4)
    assert lib.mqa_last_hip_error_name() != b"hipSuccess"
print(f"ok {n_calls}")
'''


@pytest.mark.skipif(_asan_runtime() is None or not os.path.exists(HIPCC), reason="needs hipcc and the clang ASan runtime")
def test_abi_under_host_asan_and_ubsan():
    rt = _asan_runtime()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "libmqa_attn_asan.so")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared", "-shared-libasan",
               "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *srcs, "-o", so]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        env = dict(os.environ)
        env["LD_PRELOAD"] = rt
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        run = subprocess.run([sys.executable, "-c", DRIVER, so, "0" if _gpu_present() else "1"],
                             capture_output=True, text=True, env=env, timeout=300)
        out = run.stdout + run.stderr
        assert run.returncode == 0, out[-4000:]
        assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert run.stdout.strip().startswith("ok"), out[-4000:]
