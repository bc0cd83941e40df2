"""The library's host code (argument validation, chunk layout, launch planning,
AUTO, the graph-replay cache) built for the CPU with AddressSanitizer,
LeakSanitizer and UndefinedBehaviorSanitizer, linked against a fake HIP
runtime (tests/host_fake/fake_hip.cpp) that stands in for device memory,
streams, events, graphs and the kernel launchers.  The driver
(tests/host_fake/driver.cpp) checks every rejected call launches nothing,
every accepted call launches the expected kernel sequence with a grid that
covers its work, graph replay repeats the direct launches exactly, and
ar_destroy / ar_set_graphs(0) release every stream, event and graph.  No GPU
is used; the sanitizers instrument host code only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_allreduce_rs_amd", "csrc")
FAKE = os.path.join(ROOT, "tests", "host_fake")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs the ROCm toolchain")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def test_host_code_under_sanitizers(tmp_path):
    common = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-x", "hip",
              "--cuda-host-only", f"-I{ROOT}/include", f"-I{CSRC}", f"-I{FAKE}"] + SAN
    objs = []
    for src in (os.path.join(CSRC, "ar_api.cpp"), os.path.join(CSRC, "dispatch.hip"),
                os.path.join(FAKE, "fake_hip.cpp"), os.path.join(FAKE, "driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC] + common + ["-c", src, "-o", obj],
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, f"compile {src}:\n{r.stderr[-4000:]}"
        objs.append(obj)
    exe = str(tmp_path / "host_driver")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-o", exe] + objs,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"link:\n{r.stderr[-4000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ALL OK" in r.stdout, out[-6000:]
