"""The host planner under the address and undefined-behaviour sanitizers:
tests/planner_sanitize.cpp drives batch sanitising, both ubatch splits, the
cell search, rollback of failed ubatches, seq_rm / seq_cp / seq_keep and
defrag with random valid and invalid input (8 context shapes: unified or
not, one or two sequence-mask words, two sizes) and checks the cell tables'
invariants after every step.  Host code only, built with g++."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "planner_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "llama_decode_ubatch_amd", "csrc"),
           os.path.join(ROOT, "tests", "planner_sanitize.cpp"),
           os.path.join(ROOT, "llama_decode_ubatch_amd", "csrc", "planner.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([str(exe), "3000"], capture_output=True, text=True, timeout=300, env=env)
    print(p.stdout, p.stderr[-4000:])
    assert p.returncode == 0, p.stderr[-4000:]
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr
    assert "0 invariant failures" in p.stdout
