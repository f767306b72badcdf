"""CPU checks of the build and of loud failure when the HIP library is absent."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_flags_forbid_packed_fp32_and_target_gfx950():
    from speculative_decode_verify_amd import build
    flags = " ".join(build.HIPCC_FLAGS)
    assert "--offload-arch=gfx950" in flags
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in flags


def test_missing_library_raises_instead_of_falling_back(tmp_path):
    """A copy of the package without lib/ must raise on first use."""
    import shutil
    pkg = tmp_path / "speculative_decode_verify_amd"
    shutil.copytree(os.path.join(ROOT, "speculative_decode_verify_amd"), pkg,
                    ignore=shutil.ignore_patterns("lib", "__pycache__"))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import speculative_decode_verify_amd as va\n"
        "try:\n"
        "    va.Plan(rows=8, live_rows=1, q_heads=6, kv_heads=1, head_dim=64, kv_capacity=10)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n" % str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "missing" in r.stdout


def test_product_does_not_import_oracle():
    """Only tests, smoke() and bench.py's CPU leg may touch the oracle."""
    pkg = os.path.join(ROOT, "speculative_decode_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracles", ""), f


def test_bench_refuses_more_than_one_gpu():
    """bench.py --gpus N with N > 1 exits with a message before touching a
    GPU: the verification call is a single-GPU kernel."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
