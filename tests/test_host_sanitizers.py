"""Host AddressSanitizer + UndefinedBehaviorSanitizer run (CPU only) of the
C ABI's validation code and of the C oracle: gdn_api.hip's host code and
oracle/gdn_oracle.c are rebuilt with -fsanitize=address,undefined (every
report fatal), and the host ABI tests and the oracle pins run against those
builds in a subprocess with the clang sanitizer runtime preloaded.  Memory
errors in argument checking (the grouped calls validate every shape before
anything runs: "MTP inference: review and commit structure", Review fixes)
or in the oracle would end that run with a sanitizer report."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not RUNTIME or not os.path.exists(HIPCC), reason="clang sanitizer runtime or hipcc missing")
def test_abi_validation_and_oracle_pins_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    from gated_deltanet_recurrence_conv_amd import build
    gdn = build.build_host_sanitized(str(tmp_path / "libgdn_san.so"))
    ora = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(LD_PRELOAD=RUNTIME[-1], GDN_LIB=gdn, GDN_ORACLE_LIB=ora,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    # no conftest (it imports torch, which the sanitized process does not
    # need); the binding and ceiling checks import torch too and are left out
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "--noconftest",
           "-k", "not binding and not ceiling",
           os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    proc = subprocess.run(cmd, env=env, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                          timeout=600)
    tail = "\n".join(proc.stdout.splitlines()[-30:])
    assert proc.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in proc.stdout and "runtime error:" not in proc.stdout, tail
    assert " passed" in proc.stdout, tail
