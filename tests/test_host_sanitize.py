"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: lh_api.hip (every entry point's argument checks,
status codes and error messages) is rebuilt with host-only sanitizers
(-Xarch_host, so no GPU code is instrumented), linked with the library's
other objects, and tests/test_boundary.py runs against it in a child
process with the sanitizer runtime preloaded.  None of those calls reaches
a kernel launch, so this needs no GPU."""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "nvfp4_scale_calibration_amd")
HIPCC = "/opt/rocm/bin/hipcc"
OTHERS = ["lh_dense.o", "lh_hessian.o", "lh_quant.o", "lh_sweep.o"]


def _asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


@pytest.mark.skipif(not os.path.exists(HIPCC) or _asan_runtime() is None, reason="hipcc or its ASan runtime missing")
def test_host_validation_is_clean_under_sanitizers():
    objs = [os.path.join(PKG, "_build", o) for o in OTHERS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run __graft_entry__.build())")
    with tempfile.TemporaryDirectory() as d:
        api_o = os.path.join(d, "lh_api.o")
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
        subprocess.run([HIPCC, *flags, "-c", os.path.join(PKG, "csrc", "lh_api.hip"), "-o", api_o], check=True,
                       capture_output=True)
        pkg = os.path.join(d, "pkg", "nvfp4_scale_calibration_amd")
        os.makedirs(pkg)
        shutil.copy(os.path.join(PKG, "__init__.py"), pkg)
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", os.path.join(pkg, "liblh.so"),
                        api_o, *objs], check=True, capture_output=True)
        env = dict(os.environ, PYTHONPATH=os.path.join(d, "pkg") + os.pathsep + ROOT, LD_PRELOAD=_asan_runtime(),
                   ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
        which = subprocess.run([sys.executable, "-c", "import nvfp4_scale_calibration_amd as m; print(m.LIB_PATH)"],
                               env=env, capture_output=True, text=True, cwd=d)
        assert which.returncode == 0, which.stderr[-3000:]
        assert which.stdout.strip() == os.path.join(pkg, "liblh.so"), which.stdout
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_boundary.py")], env=env, capture_output=True,
                           text=True, cwd=d, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
