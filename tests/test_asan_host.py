"""AddressSanitizer / UndefinedBehaviorSanitizer runs of the library's host
code: the MACKO encoder and 8-bit quantiser (macko_encode.cpp, built for the
host only) and the oracle's encoder (oracle.c), driven by
tests/asan/macko_host_asan.cpp on seeded random inputs and on every error
path, with output buffers of exactly the reported size (the driver also
compares the two encoders bit for bit); and the element-block FE planner
(fem_blocks.cpp), driven by tests/asan/fem_blocks_host_asan.cpp on several
meshes and the error paths, with buffers of exactly the documented
upper-bound sizes.  No GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_matrix_vector_amd", "csrc")
CLANG = shutil.which("amdclang++") or "/opt/rocm/bin/amdclang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


@pytest.mark.skipif(not (os.path.exists(CLANG) and shutil.which("gcc")), reason="needs amdclang++ and gcc")
def test_macko_host_code_under_asan(tmp_path):
    out = tmp_path / "asan"
    common = ["-g", "-O1", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in ("macko_encode.cpp", "api_common.hip"):
        o = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip", "--offload-host-only", "--offload-arch=gfx950"]
        r = subprocess.run([CLANG, *lang, "-std=c++17", *common, *SAN, "-c", os.path.join(CSRC, src), "-o", o],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(o)
    orc = str(tmp_path / "oracle.o")
    r = subprocess.run(["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address",
                        "-fsanitize=undefined", "-c", os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([CLANG, "-x", "c++", "-std=c++17", *common, "-fsanitize=address", "-fsanitize=undefined",
                        "-c", os.path.join(ROOT, "tests", "asan", "macko_host_asan.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([CLANG, "-fsanitize=address", "-fsanitize=undefined", *objs, orc, drv, "-o", str(out),
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(out)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout, r.stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="needs amdclang++")
def test_fem_blocks_planner_under_asan(tmp_path):
    out = tmp_path / "asan_fb"
    common = ["-g", "-O1", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src in ("fem_blocks.cpp", "api_common.hip"):
        o = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip", "--offload-host-only", "--offload-arch=gfx950"]
        r = subprocess.run([CLANG, *lang, "-std=c++17", *common, *SAN, "-c", os.path.join(CSRC, src), "-o", o],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(o)
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([CLANG, "-x", "c++", "-std=c++17", *common, "-fsanitize=address", "-fsanitize=undefined",
                        "-c", os.path.join(ROOT, "tests", "asan", "fem_blocks_host_asan.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([CLANG, "-fsanitize=address", "-fsanitize=undefined", *objs, drv, "-o", str(out),
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lpthread", "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(out)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "0 failures" in r.stdout, r.stdout
