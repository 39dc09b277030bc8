"""The host layer of libnvfp4 (argument checks, workspace layout, dispatch)
and the C oracle under AddressSanitizer + UndefinedBehaviorSanitizer, on the
CPU.

The host-ABI tests (tests/test_abi_cpu.py) run against the sanitizer build
of the library (host code instrumented, device code unchanged), and the
oracle's CPU tests against a sanitizer build of nvfp4_oracle.c, each in a
child process with the matching runtime preloaded.  Any sanitizer report
fails the run (UBSan does not recover; ASan stops at the first error)."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    return r.returncode, out


def test_host_abi_under_asan_ubsan():
    from precision_moe_gemm_amd import build
    lib = build.build_sanitized()
    rc, out = _run({"LD_PRELOAD": build.sanitizer_runtime(), "NVFP4_LIB_PATH": lib},
                   ["tests/test_abi_cpu.py"])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert rc == 0, out[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "libnvfp4_oracle_san.so"))
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    rc, out = _run({"LD_PRELOAD": oracle.sanitizer_runtime(), "NVFP4_ORACLE_LIB": lib}, tests)
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert rc == 0, out[-4000:]
