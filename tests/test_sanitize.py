"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle (oracle/oracle.cpp) and the storage tier (csrc/store.cpp) built with
g++ -fsanitize=address,undefined into tests/sanitize_driver.cpp, which runs
every oracle routine and the threaded storage reads; any sanitizer report
makes the run fail. Host code only: nothing here touches a GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_oracle_and_store_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "sanitize_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "sanitize_driver.cpp"),
           os.path.join(ROOT, "sparse_moe_decode_amd", "csrc", "store.cpp"),
           "-pthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # verify_asan_link_order=0: a library preloaded by the environment may
    # precede the sanitizer runtime in the load order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    data = tmp_path / "store"
    data.mkdir()
    r = subprocess.run([str(exe), str(data)], capture_output=True, text=True, env=env,
                       timeout=240)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-6000:])
