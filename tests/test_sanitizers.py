"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU: the oracle
(gcc) under its pins, and the library's host-side argument validation
(hipcc, sanitizers on the host compilation only) under the C-ABI tests.
Each runs the existing tests in a subprocess with the sanitizer runtime
preloaded; any report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(env_extra, tests):
    env = dict(os.environ, **ENV_SAN, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    src = os.path.join(ROOT, "oracle", "kvq_oracle.c")
    lib = str(tmp_path / "libkvq_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", *SAN,
                    src, "-o", lib, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    out = _run({"KVQ_ORACLE_LIB": lib, "LD_PRELOAD": asan},
               ["tests/test_oracle_pins.py", "-k", "not envelope_search_sanity"])
    print(out.strip().splitlines()[-1])


def test_host_validation_under_asan_and_ubsan(tmp_path):
    from decode_attention_int2_amd import build
    lib = build.build(lib=str(tmp_path / "libkvq_san.so"), build_dir=str(tmp_path / "obj"), host_flags=SAN)
    clang_rt = subprocess.run([os.path.join(os.path.dirname(build.HIPCC), "..", "llvm", "bin", "clang"),
                               "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True).stdout
    clang_rt = clang_rt.strip()
    if not os.path.exists(clang_rt):
        pytest.skip("no clang AddressSanitizer runtime")
    out = _run({"KVQ_LIB": lib, "LD_PRELOAD": clang_rt}, ["tests/test_abi.py"])
    print(out.strip().splitlines()[-1])
