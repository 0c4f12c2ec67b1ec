"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds into a temporary directory, with -fsanitize=address,undefined on
the host side:
  * the library -- its host code being the argument validation, the split
    and piece rules, workspace sizing, the block-sparse mask encoder and the
    kernel selector (nothing in these tests launches a kernel);
  * the oracle (serial: no OpenMP under the sanitizer).
Then runs the host ABI tests, the binding's rejection tests and the oracle
pins against those builds in a subprocess with the sanitizer runtime
preloaded (the Python interpreter itself is not instrumented).  A copy of
the oracle with a planted one-element heap overflow checks that the
sanitizer is live.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduction_attention_amd", "csrc")
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "bsr_rows.hip", "mla.hip", "scratch.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm clang toolchain not found")


def _runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return path


def _build_oracle(src, out):
    subprocess.run([CLANG, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-o", out, src, "-lm"], check=True)


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitized")
    lib = str(d / "libattn_san.so")
    flags = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]
    # one compiler process per source, then one link
    objs, procs = [], []
    for f in SOURCES:
        obj = str(d / (f + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(flags + ["-c", "-x", "hip", os.path.join(CSRC, f), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate()[0]
        assert p.returncode == 0, out[-3000:]
    r = subprocess.run(flags + ["-shared"] + objs + ["-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    ora = str(d / "liboracle_san.so")
    _build_oracle(os.path.join(ROOT, "oracle", "oracle.c"), ora)
    return dict(dir=d, lib=lib, oracle=ora, runtime=_runtime())


def _run_pytest(builds, oracle, args, tag):
    """pytest in a subprocess against the sanitized builds; sanitizer reports
    go to files <dir>/<tag>.<pid> (pytest's output capture would swallow
    them when the sanitizer ends the process).  Returns (result, reports)."""
    log = builds["dir"] / tag
    env = dict(os.environ, LD_PRELOAD=builds["runtime"], ATTN_LIBRARY_PATH=builds["lib"],
               ORACLE_LIBRARY_VARIANT=oracle, OMP_NUM_THREADS="1",
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + args, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    reports = "".join(open(builds["dir"] / f).read() for f in os.listdir(builds["dir"])
                      if f.startswith(tag + "."))
    return r, reports


def test_host_code_and_oracle_under_sanitizers(builds):
    r, reports = _run_pytest(builds, builds["oracle"],
                             [os.path.join(ROOT, "tests", t) for t in
                              ("test_abi_host.py", "test_oracle_pins.py", "test_zz_no_alloc.py")],
                             "clean")
    assert r.returncode == 0 and not reports, r.stdout[-3000:] + r.stderr[-3000:] + reports[-3000:]
    assert " passed" in r.stdout


def test_sanitizer_catches_a_planted_overflow(builds):
    """The per-thread scratch of the oracle one element short: the query
    row's last element is written past the allocation."""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old = "malloc(sizeof(double) * (size_t)((max_kv > 0 ? max_kv : 1) + D))"
    assert src.count(old) == 1
    bad = builds["dir"] / "oracle_overflow.c"
    bad.write_text(src.replace(old, "malloc(sizeof(double) * (size_t)((max_kv > 0 ? max_kv : 1) + D - 1))"))
    ora = str(builds["dir"] / "liboracle_overflow.so")
    _build_oracle(str(bad), ora)
    r, reports = _run_pytest(builds, ora, [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                                           "-k", "golden"], "planted")
    assert r.returncode != 0
    assert "heap-buffer-overflow" in reports, reports[-3000:]
