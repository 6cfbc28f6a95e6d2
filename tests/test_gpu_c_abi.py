"""The C ABI driven by a plain C program (tests/c_abi_roundtrip.c, compiled by
__graft_entry__.build() with gcc against include/entropack.h and the HIP runtime): no Python and
no PyTorch on the path. The program checks a lossless FP32 round trip itself; its lossy BF16
decode is compared here with the oracle, bit for bit."""
import os
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_program_round_trip(tmp_path):
    exe = os.path.join(HERE, "c_abi_roundtrip.bin")
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} is missing: __graft_entry__.build() compiles it")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr + r.stdout
    assert "bit-exact" in r.stdout
    stream = (tmp_path / "lossy.epk").read_bytes()
    got = np.fromfile(tmp_path / "lossy_bf16.bin", dtype=np.uint16).reshape(300, 700)
    want, _ = oracle.decompress(stream, oracle.BF16)
    assert np.array_equal(got, want)
