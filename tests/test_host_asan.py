"""The C ABI's host-side argument validation under AddressSanitizer.

The library is linked once more with its host-side C code (api.hip) built
with the sanitizer (on the host pass only: the device code is built as
usual), and tests/host_asan/driver.cpp calls every entry point with
arguments that validation must reject.  Any out-of-bounds read of an argument
array, use of freed memory or overflow on those paths aborts the driver.
CPU only: the driver hands the library fake device addresses, so it never
runs where a GPU is visible."""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fmha_mqa_fwd_amd")


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def _build_module():
    spec = importlib.util.spec_from_file_location("_fmha_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(_gpu_visible(), reason="passes fake device addresses: host-only check")
@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_validation_paths_are_clean_under_asan(tmp_path):
    b = _build_module()
    hipcc = b._hipcc()
    objs = [os.path.join(b.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in b.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_asan.o")
    subprocess.run([hipcc, *b.COMMON_FLAGS, *b.SOURCE_FLAGS.get("api.hip", []), *san, "-g",
                    "-c", os.path.join(b.CSRC, "api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    lib = str(tmp_path / "libfmha_asan.so")
    others = [o for o, s in zip(objs, b.SOURCES) if s != "api.hip"]
    subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *san, "-o", lib,
                    api_o, *others], check=True, capture_output=True)
    drv = str(tmp_path / "driver")
    subprocess.run([hipcc, "-x", "c++", *san, "-g", "-I", b.INCLUDE,
                    os.path.join(ROOT, "tests", "host_asan", "driver.cpp"), "-x", "none", lib,
                    f"-Wl,-rpath,{tmp_path}", "-o", drv], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "AddressSanitizer: ok" in r.stdout
