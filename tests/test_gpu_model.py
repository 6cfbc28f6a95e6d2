"""Whole-model use of the compressed linear layer with a per-layer bitrate allocation ("EntroPack
PyTorch Guide", "Replace one linear layer before a whole model": keep a map of the changed modules
and the original model for rollback; "Separate reconstruction metrics from application metrics":
inspect per-layer results, record the allocation).

A small DiT-like block with random weights (no trained weights are available): its four linear
layers get bitrates from plan_model under a 5.0 bpp budget, are swapped for compressed layers,
and the block's output is compared with the same block carrying the oracle-decoded weights in
fp32 (the path's own error: BF16 activations between layers, within 3e-2 relative L2); the
per-layer weight errors measured from the GPU decode are compared with the plan's estimates;
rollback restores the original outputs exactly."""
import numpy as np
import pytest
import torch

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import plan as P
from decode_tile_interleaved_rans_amd import workloads as W

pytestmark = pytest.mark.gpu


class Block(torch.nn.Module):
    def __init__(self, d=512, hidden=2048):
        super().__init__()
        self.qkv = torch.nn.Linear(d, 3 * d)
        self.proj = torch.nn.Linear(d, d)
        self.up = torch.nn.Linear(d, hidden)
        self.down = torch.nn.Linear(hidden, d)
        self.d = d

    def forward(self, x):
        q, k, v = self.qkv(x).split(self.d, dim=-1)
        a = torch.softmax((q.float() @ k.float().T) / self.d ** 0.5, dim=-1).to(v.dtype) @ v
        h = x + self.proj(a)
        return h + self.down(torch.nn.functional.gelu(self.up(h)))


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_planned_block_replacement_and_rollback(tmp_path):
    torch.manual_seed(0)
    blk = Block().cuda()
    with torch.no_grad():
        for m in (blk.qkv, blk.proj, blk.up, blk.down):
            m.weight.normal_(0, 0.02)
            m.bias.normal_(0, 0.01)
    x = torch.from_numpy(W.bf16_bits_to_f32(W.activations(64, 512, 3))).cuda()
    with torch.no_grad():
        y0 = blk(x).cpu().numpy()
    weights = {n: m.weight for n, m in blk.named_modules() if isinstance(m, torch.nn.Linear)}
    rec, streams = P.plan_model(weights, 5.0, sensitivity={"down": 4.0}, grid=(3.5, 4.0, 4.5, 5.0, 5.5, 6.0, 7.0))
    P.save_plan(rec, tmp_path / "plan.json")
    assert rec["achieved_bpp"] <= 5.0
    t = {l["name"]: l["target_bpp"] for l in rec["layers"]}
    assert t["down"] >= max(t["qkv"], t["proj"], t["up"])       # the sensitive layer gets the most bits
    # per-layer weight error: GPU decode against the original weight, next to the plan's estimate
    for l in rec["layers"]:
        wd = ep.decompress(streams[l["name"]], torch.bfloat16).float().cpu().numpy()
        w = weights[l["name"]].detach().cpu().numpy()
        measured = ((wd - w) ** 2).sum() / (w ** 2).sum()
        assert 0.7 <= measured / l["est_rel_mse"] <= 1.3, (l["name"], measured, l["est_rel_mse"])
    # reference: the same block with the oracle-decoded weights, in fp32
    ref = Block().cuda()
    ref.load_state_dict(blk.state_dict())
    with torch.no_grad():
        for n, s in streams.items():
            dec = W.bf16_bits_to_f32(oracle.decompress(s, oracle.BF16, n_threads=16)[0])
            getattr(ref, n).weight.copy_(torch.from_numpy(dec))
            getattr(ref, n).bias.copy_(getattr(ref, n).bias.to(torch.bfloat16).float())
        yr = ref(x).cpu().numpy()
    originals = P.replace_linears(blk, streams)
    assert set(originals) == set(streams)
    with torch.no_grad():
        yc = blk(x.to(torch.bfloat16)).float().cpu().numpy()
    torch.cuda.synchronize()
    assert rel_l2(yc, yr) < 3e-2
    assert rel_l2(yc, y0) < 0.1                                   # lossy weights at about 5 bpp
    P.restore_linears(blk, originals)
    with torch.no_grad():
        assert np.array_equal(blk(x).cpu().numpy(), y0)
