"""The C-ABI checks of test_abi.py against a build whose host code (the argument
validation and error reporting of csrc/abi.hip) is compiled with AddressSanitizer.

The device code and the other kernels' objects are the regular build's; only abi.hip is
recompiled with the sanitizer on its host side, linked against the shared sanitizer
runtime, which the child interpreter preloads.  No GPU is touched: every call in
test_abi.py fails validation before any HIP call.  Needs no GPU, only hipcc."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sliding_window_attention_amd import build as bld  # noqa: E402

OUT = os.path.join(bld.BUILD_DIR, "asan")
LIB = os.path.join(OUT, "libswasink_asan.so")


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build():
    os.makedirs(OUT, exist_ok=True)
    objs = [o for o in glob.glob(os.path.join(bld.BUILD_DIR, "*.o")) if not os.path.basename(o).startswith("abi.")]
    if len(objs) < len(bld.sources()) - 1:  # the regular build provides the other objects
        bld.build(verbose=False)
        objs = [o for o in glob.glob(os.path.join(bld.BUILD_DIR, "*.o")) if not os.path.basename(o).startswith("abi.")]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    abi_o = os.path.join(OUT, "abi.o")
    r = subprocess.run([bld.hipcc(), *bld.HIPCC_FLAGS, *host_san, "-c", os.path.join(bld.CSRC, "abi.hip"),
                        "-o", abi_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([bld.hipcc(), f"--offload-arch={bld.ARCH}", "-shared", "-fPIC", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-o", LIB, abi_o, *sorted(objs)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_abi_checks_pass_under_address_sanitizer():
    rt = _runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    _build()
    env = dict(os.environ, SWASINK_LIBRARY=LIB, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + os.environ.get("LD_LIBRARY_PATH", ""),
               CUDA_VISIBLE_DEVICES="", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-m", "not gpu", "-p", "no:cacheprovider"], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
