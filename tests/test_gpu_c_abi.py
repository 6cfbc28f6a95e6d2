"""The C ABI driven by a plain C program (tests/c_abi_roundtrip.c, compiled by
__graft_entry__.build() with gcc against include/entropack.h and the HIP runtime): no Python and
no PyTorch on the path. The program checks a lossless FP32 round trip itself, that the row tile
layout decodes to the same weights as layout 0, and that the grouped linear forward gives the same
bits as one forward per layer; both lossy BF16 decodes are compared here with the oracle, bit for
bit, and the forwards with the fp64 product of the oracle's weights."""
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
    rows = (tmp_path / "rows.epk").read_bytes()
    assert oracle.info(rows)["layout"] == 1
    got_rows = np.fromfile(tmp_path / "rows_bf16.bin", dtype=np.uint16).reshape(300, 700)
    want_rows, _ = oracle.decompress(rows, oracle.BF16)
    assert np.array_equal(got_rows, want_rows) and np.array_equal(want_rows, want)
    assert "grouped forward" in r.stdout
    x = np.fromfile(tmp_path / "x_bf16.bin", dtype=np.uint16).reshape(8, 512)
    x64 = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for l, n in enumerate((96, 40)):
        wq, _ = oracle.decompress((tmp_path / f"layer{l}.epk").read_bytes(), oracle.BF16)
        ref = x64 @ (wq.astype(np.uint32) << 16).view(np.float32).astype(np.float64).T
        y = np.fromfile(tmp_path / f"y{l}_bf16.bin", dtype=np.uint16).reshape(8, n)
        got = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 5e-3
