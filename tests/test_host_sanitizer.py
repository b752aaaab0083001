"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/abi_driver.cpp calls every entry point with arguments the
validation must reject (so that no kernel is ever launched) and the
workspace-size functions at extreme sizes.  hs_api.cpp is rebuilt with the
sanitizers on its host code only and linked with the library's other
objects; the driver then runs on the CPU with no GPU visible.  Any
sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "decode_indexer_logits_amd" / "csrc"
DRIVER = ROOT / "tests" / "sanitize" / "abi_driver.cpp"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.timeout(600)
@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.skipif(_gpu_visible(), reason="host-only check: runs where no GPU is visible")
def test_c_abi_validation_under_asan_and_ubsan(tmp_path):
    from decode_indexer_logits_amd import build as b
    hipcc = _hipcc()
    # the library's kernel objects, unsanitized (built if missing)
    objs = [b.BUILD / (Path(s).stem + ".o") for s in b.SOURCES if s != "hs_api.cpp"]
    if not all(o.exists() for o in objs):
        b.build()
    api_o = tmp_path / "hs_api_san.o"
    cmd = [hipcc, "-x", "hip", *b.FLAGS, *SAN, "-c", str(CSRC / "hs_api.cpp"), "-o", str(api_o)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # the driver is plain host C++; clang links with the sanitizer runtimes
    clang = str(Path(hipcc).resolve().parent.parent / "lib" / "llvm" / "bin" / "clang++")
    host_san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer"]
    drv_o = tmp_path / "abi_driver.o"
    r = subprocess.run([clang, "-std=c++17", "-O1", *host_san, "-c", str(DRIVER), "-o", str(drv_o)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = tmp_path / "abi_driver"
    rocm_lib = Path(hipcc).resolve().parent.parent / "lib"
    cmd = [clang, *host_san, str(drv_o), str(api_o), *map(str, objs), f"-L{rocm_lib}",
           "-lamdhip64", f"-Wl,-rpath,{rocm_lib}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
