"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

  * the C oracle (oracle/oracle.c, gcc), driven by tests/sanitize/oracle_main.c
    over every function on small inputs;
  * the library's host code -- argument validation, planning and workspace
    sizing in ic_api.cpp and the launch wrappers -- driven by
    tests/sanitize/api_main.cpp over every entry point with arguments that
    the validation rejects (so nothing reaches a launch). The sanitizers
    apply to the host side of each compile only; device code is built as
    usual.

Builds go to _build/sanitize/ and are reused while the sources are unchanged.
"""
import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cross_layer_index_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
LIB_SOURCES = ["ic_api.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "gate.hip", "write.hip", "calib.hip"]
# sanitizers on the host side of each compile (each flag after -Xarch_host)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in paths:
        h.update(open(p, "rb").read())
    for p in sorted(os.listdir(CSRC)):
        if p.endswith(".h"):
            h.update(open(os.path.join(CSRC, p), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "ic.h"), "rb").read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd[:3])} ... failed:\n{r.stderr[-3000:]}")


def _check_output(r, what):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, f"{what}: sanitizer report\n{text[-4000:]}"
    assert r.returncode == 0, f"{what}: exit {r.returncode}\n{text[-4000:]}"
    assert "ok:" in r.stdout, text[-2000:]


def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_main.c")]
    exe = os.path.join(OUT, "oracle_main-" + _digest(srcs, SAN))
    if not os.path.exists(exe):
        _run(["gcc", "-O1", "-g", "-std=c11", *SAN, *srcs, "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    _check_output(subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300), "oracle")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_host_api_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    srcs = [os.path.join(CSRC, f) for f in LIB_SOURCES]
    main = os.path.join(ROOT, "tests", "sanitize", "api_main.cpp")
    tag = _digest(srcs + [main], flags + SAN)
    exe = os.path.join(OUT, "api_main-" + tag)
    if not os.path.exists(exe):
        objs = [os.path.join(OUT, f"{f}.{tag}.o") for f in LIB_SOURCES]
        with ThreadPoolExecutor(max_workers=4) as ex:
            list(ex.map(lambda so: _run([HIPCC, *flags, "-x", "hip", "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
        mobj = os.path.join(OUT, f"api_main.{tag}.o")
        _run([CLANGXX, "-O1", "-g", "-std=c++17", *SAN, f"-I{os.path.join(ROOT, 'include')}", "-c", main, "-o", mobj])
        _run([CLANGXX, *SAN, *objs, mobj, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    # leaks are not checked here: the HIP runtime's own start-up allocations
    # would be reported, and they are not this code's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    _check_output(subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300), "host API")
