"""Per-layer bitrate allocation and whole-model replacement of linear layers.

Layers differ in how much their error matters, so they need not share one setting, and the spare
space of a memory budget can go to the layers with the most impact ("EntroPack 開源：模型壓縮不必
只選 4 位元，如何配合顯示記憶體預算？", section "目標大小與實際占用要分開"). An allocation across
layers has to be recorded with its rationale, per-layer results have to be inspectable, and a
whole-model replacement keeps a map of the changed modules and the original model for rollback
("EntroPack PyTorch Guide", sections "Separate reconstruction metrics from application metrics"
and "Replace one linear layer before a whole model").

Reading (the pages fix no rule): the allocation minimizes sum_l a_l n_l D_l subject to
sum_l n_l b_l <= B, where n_l is the layer's weight count, b_l its actual stored bits per weight
(metadata included), a_l a sensitivity weight (1 unless given; for instance measured from the
model's outputs) and D_l its relative squared weight error. D_l is taken from the high-resolution
model of E8 quantization of unit-RMS rows, D = G(E8) step^2 with G(E8) = 0.0716821, using the
step the host encoder picks for each candidate target; every candidate is a real encode, so b_l
is exact. The discrete problem is solved by Lagrangian relaxation: each layer takes the candidate
minimizing a_l D + lambda b, with the smallest multiplier lambda (bisection) whose choices fit the
budget. These choices lie on each layer's lower convex hull, and a larger budget never lowers a
layer's rate; budget left below the next hull step stays unused.

Host-side tooling: the encoder runs in the compiled library; nothing here is on the GPU decode
path.
"""
from __future__ import annotations

import json
import math
from dataclasses import dataclass

import numpy as np

from . import BF16, F32, LAYER_LAYOUT, LAYER_PROB_BITS, compress, stream_info

E8_G = 0.0716821                     # normalized second moment of the E8 lattice
DEFAULT_GRID = tuple(np.round(np.arange(2.0, 8.0001, 0.25), 4))


@dataclass
class Candidate:
    target: float
    actual_bpp: float
    step: float
    rel_mse: float                   # model estimate G(E8) step^2
    nbytes: int


def _weight_array(w):
    """(array, dtype code) for compress(): float32 arrays as they are, torch tensors via their
    BF16/F32 bits."""
    if hasattr(w, "detach"):
        import torch
        t = w.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        return t.float().numpy(), F32
    a = np.ascontiguousarray(w)
    return (a, BF16) if a.dtype == np.uint16 else (a.astype(np.float32, copy=False), F32)


def layer_candidates(w, grid=DEFAULT_GRID, prob_bits: int = LAYER_PROB_BITS, tile_rows: int = 16, n_threads: int = 0,
                     layout: int = LAYER_LAYOUT):
    """Encode one weight at every target of the grid (the tile layout of compressed layers by
    default); returns the candidates (real stream sizes and steps) and the streams."""
    arr, code = _weight_array(w)
    out, streams = [], []
    for t in grid:
        s, bpp = compress(arr, float(t), dtype=code, prob_bits=prob_bits, tile_rows=tile_rows, n_threads=n_threads,
                          layout=layout)
        step = stream_info(s)["step"]
        out.append(Candidate(float(t), float(bpp), float(step), E8_G * float(step) ** 2, len(s)))
        streams.append(s)
    return out, streams


def _pick(cands, a, lam):
    return min(range(len(cands)), key=lambda i: (a * cands[i].rel_mse + lam * cands[i].actual_bpp, cands[i].actual_bpp))


def allocate(cands_by_layer: dict, sizes: dict, budget_bpp: float, sensitivity: dict | None = None):
    """Choose one candidate per layer. cands_by_layer: name -> candidates; sizes: name -> weight
    count; budget_bpp: allowed average stored bits per weight over all layers. Returns name ->
    index into that layer's candidates. Raises ValueError when even the cheapest candidates
    exceed the budget."""
    names = list(cands_by_layer)
    a = {n: float((sensitivity or {}).get(n, 1.0)) for n in names}
    n_tot = float(sum(sizes[n] for n in names))
    budget = budget_bpp * n_tot

    def total_bits(ch):
        return sum(sizes[n] * cands_by_layer[n][ch[n]].actual_bpp for n in names)

    cheapest = {n: min(range(len(cands_by_layer[n])), key=lambda i: cands_by_layer[n][i].actual_bpp) for n in names}
    if total_bits(cheapest) > budget:
        raise ValueError("budget below the smallest candidate of every layer")
    # Lagrangian: a larger multiplier favours fewer bits; find the smallest one that fits
    lo, hi = 0.0, 1.0
    while total_bits({n: _pick(cands_by_layer[n], a[n], hi) for n in names}) > budget and hi < 1e12:
        hi *= 4.0
    if total_bits({n: _pick(cands_by_layer[n], a[n], hi) for n in names}) > budget:
        choice = dict(cheapest)
    else:
        for _ in range(80):
            mid = math.sqrt(lo * hi) if lo > 0 else hi / 1024.0
            if total_bits({n: _pick(cands_by_layer[n], a[n], mid) for n in names}) <= budget:
                hi = mid
            else:
                lo = mid
            if hi - lo <= 1e-12 * hi:
                break
        choice = {n: _pick(cands_by_layer[n], a[n], hi) for n in names}
    return choice


def plan_model(weights: dict, budget_bpp: float, sensitivity: dict | None = None, grid=DEFAULT_GRID,
               prob_bits: int = LAYER_PROB_BITS, tile_rows: int = 16, n_threads: int = 0):
    """Allocate bitrates over named weights under an average budget of budget_bpp stored bits per
    weight. Returns (record, streams): the record is JSON-serializable (per-layer target, actual
    bits per weight, bytes, step, estimated relative error, sensitivity, totals and the
    rationale); streams maps each name to its chosen compressed stream."""
    cands, streams, sizes, shapes = {}, {}, {}, {}
    for name, w in weights.items():
        c, s = layer_candidates(w, grid, prob_bits, tile_rows, n_threads)
        cands[name], streams[name] = c, s
        shp = tuple(int(v) for v in w.shape)
        sizes[name], shapes[name] = shp[0] * shp[1], shp
    choice = allocate(cands, sizes, budget_bpp, sensitivity)
    layers = []
    for name in weights:
        c = cands[name][choice[name]]
        layers.append({"name": name, "shape": list(shapes[name]),
                       "sensitivity": float((sensitivity or {}).get(name, 1.0)),
                       "target_bpp": c.target, "actual_bpp": round(c.actual_bpp, 6), "bytes": c.nbytes,
                       "step": c.step, "est_rel_mse": c.rel_mse})
    n_tot = sum(sizes.values())
    record = {
        "budget_bpp": budget_bpp,
        "achieved_bpp": round(8.0 * sum(l["bytes"] for l in layers) / n_tot, 6),
        "est_weighted_rel_mse": sum(l["sensitivity"] * sizes[l["name"]] * l["est_rel_mse"] for l in layers) / n_tot,
        "grid": [float(g) for g in grid],
        "rationale": ("minimum of sum_l a_l n_l G(E8) step_l^2 (relative squared error of unit-RMS rows under "
                      "high-resolution E8 quantization, a_l the sensitivity weight) subject to sum_l n_l bpp_l <= "
                      "budget, over real encodes at the grid's targets; Lagrangian choice with the smallest "
                      "multiplier that fits"),
        "layers": layers,
    }
    return record, {name: streams[name][choice[name]] for name in weights}


def save_plan(record: dict, path) -> None:
    with open(path, "w") as f:
        json.dump(record, f, indent=1)


def replace_linears(model, streams: dict, compute: str = "bf16"):
    """Swap the named nn.Linear submodules of a model for compressed layers built from the given
    streams (names as in model.named_modules()). Returns the map name -> original module, which
    keeps the originals for comparison and rollback."""
    import torch
    from . import CompressedLinear

    class _Compressed(torch.nn.Module):
        def __init__(self, layer):
            super().__init__()
            self.layer = layer

        def forward(self, x):
            return self.layer(x)

    originals = {}
    mods = dict(model.named_modules())
    for name, s in streams.items():
        lin = mods[name]
        if not isinstance(lin, torch.nn.Linear):
            raise TypeError(f"{name} is not an nn.Linear")
        bias = None
        if lin.bias is not None:
            bias = lin.bias.detach().to(device="cuda", dtype=torch.bfloat16).contiguous()
        parent_name, _, child = name.rpartition(".")
        parent = mods[parent_name] if parent_name else model
        setattr(parent, child, _Compressed(CompressedLinear(s, bias, compute)))
        originals[name] = lin
    return originals


def restore_linears(model, originals: dict) -> None:
    """Undo replace_linears."""
    mods = dict(model.named_modules())
    for name, lin in originals.items():
        parent_name, _, child = name.rpartition(".")
        setattr(mods[parent_name] if parent_name else model, child, lin)
