"""The C ABI's host code (argument checks, workspace layout, tracing, error
strings) built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel launchers replaced by stubs
(tests/sanitize/host_stubs.cpp), and driven through the cases of
test_abi.py by tests/sanitize/host_checks.cpp.  CPU only: the sanitizers are
applied to host code only (-Xarch_host before each -fsanitize=), and no
pointer the driver passes is dereferenced."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_paged_kv_scatter_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"

FLAGS = ["-O1", "-g", "-std=c++20", "-fno-omit-frame-pointer", "--offload-arch=gfx950",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-command-line-argument"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_checks_under_asan_and_ubsan(tmp_path):
    objs = []
    for src in (os.path.join(CSRC, "rpa_api.cpp"), os.path.join(SAN, "host_stubs.cpp"),
                os.path.join(SAN, "host_checks.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, "-x", "hip", *FLAGS, "-c", src, "-o", obj],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main(); leaks are not what is checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host checks:" in r.stdout and "passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
