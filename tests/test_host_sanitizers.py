"""The host-side sources (plan builders, balance, draft tree, block pool) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven by
randomised valid and invalid calls: every call returns a status and the
sanitizers find no out-of-bounds access, leak or undefined operation."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tree_structured_attention_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(HERE, "host_fuzz", "fuzz.cpp"), os.path.join(HERE, "host_fuzz", "stub.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "errors.cpp"), os.path.join(CSRC, "draft.cpp"),
           os.path.join(CSRC, "kv_pool.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitizer" in (r.stderr or "").lower() and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime libraries are not installed")
    assert r.returncode == 0, r.stderr[-3000:]
    run = subprocess.run([exe, "1500"], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "ok=" in run.stdout
