"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every csrc/*.hip file is compiled with the sanitizers on the host side only (each -fsanitize=
sits right after -Xarch_host; the device code is built as usual and never runs) and linked with
tests/host/lh_host_checks.cpp, a driver that plans valid and invalid configurations, reads
every status string and has each entry point reject bad arguments -- all answered on the host
before any launch.  The build is cached under _build/host_sanitize, keyed by the sources.
"""

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_sparse_attention_lh_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "host", "lh_host_checks.cpp")
OUT = os.path.join(ROOT, "_build", "host_sanitize")
SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
       "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
FLAGS = ["--offload-arch=gfx950", "-O0", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")] + SAN


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _key(files):
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _build():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    deps = srcs + sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    deps += [os.path.join(ROOT, "include", "lh_api.h"), DRIVER]
    exe = os.path.join(OUT, f"lh_host_checks_{_key(deps)}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT, exist_ok=True)
    cc = _hipcc()

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([cc, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    r = subprocess.run([cc, "-O0", "-g", "-std=c++17", *SAN[:6], "-I", os.path.join(ROOT, "include"),
                        "-x", "c++", DRIVER, "-x", "none", *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_host_code_is_clean_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "host checks passed" in r.stdout
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
