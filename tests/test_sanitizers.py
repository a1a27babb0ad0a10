"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the oracle (oracle.c, gcc -fsanitize=address,undefined, aborting on the first report) runs
  its pins with gcc's sanitizer runtimes preloaded;
* the library's host side (pa_api.cpp: argument validation, size queries, the no-allocation
  entry point's checks; clang -fsanitize=address,undefined through hipcc's -Xarch_host) runs
  the C-ABI tests with clang's ASan runtime preloaded.

Each run is a child process (the runtimes must be loaded first); the test checks that the
sanitized library is the one the child mapped, that every test passed, and that no sanitizer
report was printed.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer",
           "SUMMARY: UndefinedBehaviorSanitizer")


def _run(env_extra, preload, tests, lib_env, lib_path):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:protect_shadow_gap=0"
    env["OMP_NUM_THREADS"] = "4"
    env[lib_env] = lib_path
    # the child first proves which library it maps, then runs the tests unsandboxed by pytest's
    # output capture (a report printed before an abort must reach this process)
    probe = ("import sys; sys.path.insert(0, %r); import oracle; from mqa_split_kv_amd import binding; "
             "oracle.lib() if %r == 'ORACLE_LIB' else binding.lib(); "
             "print([l.split()[-1] for l in open('/proc/self/maps') if %r in l][:1])"
             % (ROOT, lib_env, os.path.basename(lib_path)))
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert os.path.basename(lib_path) in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu"]
                       + tests, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert not any(k in out for k in REPORTS), out[-4000:]
    assert " passed" in out


def test_oracle_pins_under_asan_ubsan():
    import oracle
    lib = oracle.build(force=True, sanitize=True)
    gcc_rt = [subprocess.run(["gcc", "-print-file-name=%s" % n], capture_output=True, text=True).stdout.strip()
              for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in gcc_rt):
        pytest.skip("gcc sanitizer runtimes not installed")
    _run({}, ":".join(gcc_rt), ["tests/test_oracle.py", "tests/test_oracle_variants.py",
                                "tests/test_oracle_append.py", "tests/test_plan_oracle.py",
                                "tests/test_accounting.py"], "ORACLE_LIB", lib)


def test_abi_host_code_under_asan_ubsan():
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt or not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc or clang's ASan runtime not installed")
    from mqa_split_kv_amd import build
    lib = build.build_sanitized()
    _run({}, rt[0], ["tests/test_abi.py"], "PA_DECODE_LIB", lib)
