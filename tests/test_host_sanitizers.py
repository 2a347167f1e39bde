"""The library's host code (argument validation, workspace carving, launch planning)
built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/host_sanitize/driver.cpp.  The device code is compiled as usual and never
launched: every call in the driver returns before the first HIP call, so this runs on
a machine without a GPU.  The sanitizers apply to host code only (each -fsanitize
option follows -Xarch_host)."""
import concurrent.futures as cf
import os
import subprocess

import pytest

from hybrid_attention_ssm_proj_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
       "-g"]


def _hipcc():
    try:
        return b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")


def test_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        cmd = [hipcc, *b.flags(), *SAN, "-c", src, "-o", obj]
        if src.endswith("hymba.cpp"):
            cmd.insert(1, "-xhip")
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
        return obj

    srcs = [os.path.join(b.CSRC, s) for s in b.SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"))
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_checks")
    link = [hipcc, f"--offload-arch={b.ARCH}", *SAN, "-o", exe, *objs]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    # leaks in the HIP runtime's process-lifetime state are not this library's; the
    # harness may preload a library ahead of the sanitizer runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout, r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
