"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host C/C++ (CPU
only).

* the oracle (oracle/da2_oracle.c) with tests/sanitize/oracle_driver.c:
  partitions of every frame up to 40 x 40, plans, tiered attention with every
  tier value, the text prefix, a traced row and the dense reference on small
  grid and ragged problems; leaks are reported too;
* the library's host side (da2_host.cpp, da2_partition.cpp) with
  tests/sanitize/host_driver.cpp: layouts of every frame up to 48 x 48 with
  and without a prefix, slot tables, workspace carving, plan objects over a
  fake workspace address and every argument check that returns before a
  launch (the kernel launchers are stubs that abort if reached).

Any sanitizer report fails the program, and so the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "video_diffusion_dit_frame_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(map(str, cmd)), r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "da2_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not available")
def test_host_library_under_asan_ubsan(tmp_path):
    # host-side sanitizers only: each sanitizer flag goes to the host pass
    flags = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-x", "hip",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "da2_host.cpp"), os.path.join(CSRC, "da2_partition.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(flags + ["-c", src, "-o", obj], timeout=600)
        objs.append(obj)
    exe = str(tmp_path / "host_san")
    # the link: a plain host link of the sanitized objects
    _run([CLANG, "-fsanitize=address,undefined"] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert "host driver ok" in r.stdout
