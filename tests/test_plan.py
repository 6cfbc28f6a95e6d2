"""Per-layer bitrate allocation (host tooling): a budget shared over layers whose errors matter
differently ("EntroPack 開源", section "目標大小與實際占用要分開"), recorded with its rationale
("EntroPack PyTorch Guide", section "Separate reconstruction metrics from application metrics").

Pins: the high-resolution error model G(E8) step^2 against the error the oracle's decode actually
has; the reverse water-filling closed form (two equal layers whose sensitivities differ by 16
differ by half of log2(16) = 2 bits); equal layers get equal or neighbouring rates; the budget holds and larger
budgets never lower a layer's rate."""
import json

import numpy as np
import pytest

import oracle
import decode_tile_interleaved_rans_amd as ep
from decode_tile_interleaved_rans_amd import plan as P
from decode_tile_interleaved_rans_amd import workloads as W


def gauss(R, C, seed):
    return np.random.default_rng(seed).normal(0, 0.02, (R, C)).astype(np.float32)


@pytest.mark.parametrize("target", [4.0, 5.0, 6.0])
def test_error_model_matches_oracle_decode(target):
    w = gauss(256, 1024, 1)
    cands, streams = P.layer_candidates(w, grid=(target,))
    c, s = cands[0], streams[0]
    assert s == oracle.compress(w, target, prob_bits=ep.LAYER_PROB_BITS, layout=ep.LAYER_LAYOUT)[0]
    q, _ = oracle.decode_symbols(s)
    d = oracle.info(s)
    scale = np.sqrt((w.astype(np.float64) ** 2).mean(1))
    rec = q * (d["step"] / 2) * scale[:, None]
    measured = ((rec - w) ** 2).sum() / (w.astype(np.float64) ** 2).sum()
    assert c.step == pytest.approx(d["step"])
    assert 0.85 <= measured / c.rel_mse <= 1.15, (measured, c.rel_mse)


def test_equal_layers_share_the_rate():
    ws = {f"l{i}": gauss(64, 512, 7) for i in range(3)}
    rec, streams = P.plan_model(ws, 4.5, grid=(3.5, 4.0, 4.5, 5.0))
    targets = [l["target_bpp"] for l in rec["layers"]]
    # equal layers end on the same candidate or, where the leftover budget buys one upgrade but
    # not three, on neighbouring ones
    assert max(targets) - min(targets) <= 0.5
    assert rec["achieved_bpp"] <= 4.5
    assert set(streams) == set(ws)


def test_reverse_water_filling_closed_form():
    w = gauss(128, 1024, 3)
    ws = {"sensitive": w, "robust": w.copy()}
    grid = tuple(np.arange(3.0, 7.01, 0.25))
    rec, _ = P.plan_model(ws, 5.0, sensitivity={"sensitive": 16.0, "robust": 1.0}, grid=grid)
    t = {l["name"]: l["target_bpp"] for l in rec["layers"]}
    assert 1.5 <= t["sensitive"] - t["robust"] <= 2.5, t
    assert rec["achieved_bpp"] <= 5.0


def test_budget_monotone_and_infeasible():
    ws = {"a": gauss(64, 512, 1), "b": W.bf16_bits_to_f32(W.student_t(64, 768, 2)).copy(), "c": gauss(32, 256, 3)}
    sens = {"a": 1.0, "b": 3.0, "c": 0.5}
    grid = (2.5, 3.0, 3.5, 4.0, 4.5, 5.0, 6.0)
    prev = None
    for budget in (3.5, 4.0, 4.5, 5.5):
        rec, _ = P.plan_model(ws, budget, sensitivity=sens, grid=grid)
        assert rec["achieved_bpp"] <= budget + 1e-9
        rates = {l["name"]: l["actual_bpp"] for l in rec["layers"]}
        if prev is not None:
            assert all(rates[n] >= prev[n] - 1e-9 for n in rates), (prev, rates)
        prev = rates
    with pytest.raises(ValueError):
        P.plan_model(ws, 1.0, grid=grid)


def test_record_is_json_with_rationale(tmp_path):
    ws = {"x": gauss(64, 512, 9)}
    rec, _ = P.plan_model(ws, 6.0, grid=(4.0, 5.0))
    path = tmp_path / "plan.json"
    P.save_plan(rec, path)
    back = json.load(open(path))
    assert back["rationale"] and back["layers"][0]["name"] == "x" and back["layers"][0]["bytes"] > 0
