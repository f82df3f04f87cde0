"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only), driven through every function on small and degenerate
inputs by tests/csrc/oracle_sanitize_main.c: no out-of-bounds access, leak or
undefined operation, and the pack/unpack round trips hold."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _sanitizers_work(td):
    probe = os.path.join(td, "p.c")
    with open(probe, "w") as f:
        f.write("int main(void){return 0;}\n")
    r = subprocess.run(["gcc", "-fsanitize=address,undefined", probe, "-o",
                        os.path.join(td, "p")], capture_output=True)
    return r.returncode == 0


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as td:
        if not _sanitizers_work(td):
            pytest.skip("this gcc cannot link the sanitizer runtimes")
        exe = os.path.join(td, "orc_asan")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off",
                        "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all",
                        os.path.join(HERE, "csrc", "oracle_sanitize_main.c"),
                        os.path.join(ROOT, "oracle", "bitlinear_oracle.c"), "-lm", "-o", exe],
                       check=True)
        # verify_asan_link_order=0: a library the environment preloads may
        # precede the ASan runtime; that does not change what ASan checks here
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
