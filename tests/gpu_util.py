"""Helpers shared by the GPU tests: run the HIP layer, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, Workspace, layer_call, to_device

MARGIN = 1e-4        # selection must match the oracle where the k-th vs (k+1)-th key gap exceeds this
MAX_REL = 1e-2       # max |y - y_ref| <= MAX_REL * max |y_ref|
L2_REL = 5e-3        # ||y - y_ref|| <= L2_REL * ||y_ref||
W_ABS = 1e-5         # routing weights (fp32 sigmoid and normalisation)


def say(msg: str):
    print(msg, flush=True)


def run(inp: dict, flags: int = 0, w: DeviceWeights | None = None, x: torch.Tensor | None = None):
    """Run route -> build -> forward on the GPU.  Returns (workspace, weights)."""
    dims = inp["dims"]
    if w is None:
        w = DeviceWeights.upload(inp)
    if x is None:
        x = to_device(inp["x"], "cuda")
    ws = Workspace(dims, flags)
    layer_call(x, w, ws)
    torch.cuda.synchronize()
    return ws, w


def routing_arrays(ws: Workspace) -> dict:
    dims = ws.dims
    E, P = dims.E, dims.T * dims.k
    out = {}
    for name, count in (("counts", E + 1), ("offsets", E + 1), ("sorted_pair", P), ("pair_pos", P),
                        ("row_expert", P), ("group_order", E + 1), ("mt_prefix", E + 2)):
        out[name] = ws.routing_view(name, count).cpu().numpy()
    return out


def oracle_selection(inp: dict, tokens) -> dict:
    """The oracle's router and selection alone (no expert pass): scores s, keys s + b, ids, margins."""
    xb = inp["x"][tokens]
    s = oracle.sigmoid(oracle.router_logits(xb, inp["w_router"]))
    ids, margin = oracle.select_experts(s, inp["bias"], inp["dims"].k)
    key = s + np.asarray(inp["bias"], dtype=np.float64)[None, :]
    return dict(s=s, key=key, ids=ids, margin=margin)


def check_near_tie_selection(sel: dict, ids_gpu: np.ndarray, i: int, label, token) -> None:
    """For a token inside the margin: the GPU's k experts are distinct, in range, and differ from the
    oracle's only in experts whose oracle key lies within MARGIN of the oracle's k-th key."""
    k = ids_gpu.shape[1]
    E = sel["key"].shape[1]
    g = ids_gpu[i].tolist()
    assert len(set(g)) == k and all(0 <= e < E for e in g), (label, token, g)
    key = sel["key"][i]
    kth = key[sel["ids"][i][-1]]
    for e in set(g) ^ set(sel["ids"][i].tolist()):
        assert abs(key[e] - kth) <= MARGIN, (label, token, e, key[e], kth)


def check_parity(inp: dict, ws: Workspace, tokens=None, label: str = "", residual=None, forward=None,
                 y=None) -> dict:
    """Parity rule: selection sets exact where margin > MARGIN; elsewhere the GPU's set may differ from
    the oracle's only among experts whose oracle key is within MARGIN of the k-th key, and the oracle is
    evaluated on the GPU's selection (weights from the oracle's fp64 scores); then max-abs and
    relative-L2 bounds over all checked tokens, and routing weights within W_ABS.
    forward: the oracle's layer function (default oracle.forward); y: the output tensor (default ws.y)."""
    dims = inp["dims"]
    tokens = np.arange(dims.T) if tokens is None else np.asarray(tokens)
    ids_gpu = ws.topk_ids.cpu().numpy()[tokens]
    w_gpu = ws.topk_w.cpu().numpy()[tokens]
    y_gpu = (ws.y if y is None else y).cpu().numpy()[tokens].astype(np.float64)
    sel = oracle_selection(inp, tokens)
    close = ~(sel["margin"] > MARGIN)
    for i in range(len(tokens)):
        if close[i]:
            check_near_tie_selection(sel, ids_gpu, i, label, int(tokens[i]))
        else:
            assert sorted(ids_gpu[i]) == sorted(sel["ids"][i]), (label, int(tokens[i]), ids_gpu[i], sel["ids"][i])
    ov = {int(tokens[i]): ids_gpu[i] for i in np.nonzero(close)[0]}
    # one expert pass of the oracle, on the GPU's selection where the margin is too small to decide
    if forward is None:
        ref = oracle.forward(inp, tokens=tokens, ids_override=ov or None, residual=residual)
    else:
        ref = forward(inp, tokens=tokens, ids_override=ov or None)
    # weights: compare by expert id
    for i in range(len(tokens)):
        ref_w = dict(zip(ref["ids"][i].tolist(), ref["w"][i].tolist()))
        for e, wv in zip(ids_gpu[i].tolist(), w_gpu[i].tolist()):
            assert abs(wv - ref_w[e]) <= W_ABS, (label, int(tokens[i]), e, wv, ref_w[e])
    assert np.all(np.isfinite(y_gpu)), label
    yr = ref["y"]
    err = y_gpu - yr
    max_rel = np.abs(err).max() / np.abs(yr).max()
    l2_rel = np.linalg.norm(err) / np.linalg.norm(yr)
    say(f"[parity] {label}: tokens={len(tokens)} near-ties={int(close.sum())} max_rel={max_rel:.3e} l2_rel={l2_rel:.3e}")
    assert max_rel <= MAX_REL, (label, max_rel)
    assert l2_rel <= L2_REL, (label, l2_rel)
    return dict(max_rel=max_rel, l2_rel=l2_rel, near_ties=int(close.sum()))


def check_routing_build(ws: Workspace):
    """Integer outputs of the routing build, bit-exact against the oracle's CPU construction on the GPU's ids."""
    dims = ws.dims
    ids = ws.topk_ids.cpu().numpy()
    got = routing_arrays(ws)
    ref = oracle.routing_build(ids, dims.E)
    np.testing.assert_array_equal(got["counts"][:dims.E], ref["counts"])
    assert got["counts"][dims.E] == dims.T
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["sorted_pair"], ref["sorted_pair"])
    np.testing.assert_array_equal(got["pair_pos"], ref["pair_pos"])
    np.testing.assert_array_equal(got["row_expert"], ref["row_expert"])
    if ws.flags & abi.MOE_FLAG_ID_ORDER:
        order = np.arange(dims.E + 1)
    else:
        order = oracle.group_order(ref["counts"], dims.T)
    np.testing.assert_array_equal(got["group_order"], order)
    sizes = np.array([dims.T if g == dims.E else ref["counts"][g] for g in order])
    tiles = (sizes + 95) // 96  # M-tile rows of the grouped GEMM
    np.testing.assert_array_equal(got["mt_prefix"], np.concatenate([[0], np.cumsum(tiles)]))
