"""GPU expert selection through moe_route alone: slot order, ties and weights against the oracle.

The selection rule (sigmoid scores, bias added for selection only, the k largest keys listed by
descending key, equal keys to the lower expert id, weights = unbiased scores normalised to 1) is
the oracle's select_experts / routing_weights.  Both router forms are covered: the GEMV router
(one logit array) and the MFMA router (eight partial logit arrays), and every key-register count
of the top-k (E up to 1024, k up to 32).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, Workspace, layer_call_fused, to_device
from gpu_util import MARGIN, W_ABS, say

pytestmark = pytest.mark.gpu

PATHS = {"gemv_router": abi.MOE_FLAG_FORCE_GEMV, "mfma_router": abi.MOE_FLAG_FORCE_GROUPED}
SHAPES = [(20, 4), (64, 10), (100, 1), (256, 10), (256, 32), (1000, 16), (1024, 32)]


def route(inp: dict, flags: int):
    dims = inp["dims"]
    ws = Workspace(dims, flags)
    abi.moe_route(dims, to_device(inp["x"], "cuda"), to_device(inp["w_router"], "cuda"),
                  to_device(inp["bias"], "cuda"), ws.topk_ids, ws.topk_w, ws.routing, flags=flags)
    torch.cuda.synchronize()
    return ws.topk_ids.cpu().numpy(), ws.topk_w.cpu().numpy()


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("E,k", SHAPES, ids=[f"E{e}k{k}" for e, k in SHAPES])
def test_exact_ties_go_to_the_lower_id(E, k, path):
    # W_r = 0: every logit is exactly 0 and every score exactly 1/2 on both sides; the biases are
    # multiples of 1/64 from a set of 8 values, so s + b is exact in fp32 and fp64 and most keys tie.
    dims = synth.Dims(T=6, d=64, E=E, k=k, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=7 + E + k, weights=False)
    rng = np.random.default_rng(E * 100 + k)
    inp["w_router"] = np.zeros((E, dims.d), dtype=np.float32)
    inp["bias"] = (rng.integers(0, 8, size=E) / 64.0).astype(np.float32)
    say(f"[case] ties E={E} k={k} {path}")
    ids, w = route(inp, PATHS[path])
    s = np.full((dims.T, E), 0.5)
    ref_ids, _ = oracle.select_experts(s, inp["bias"], k)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_allclose(w, oracle.routing_weights(s, ref_ids), rtol=0, atol=W_ABS)


@pytest.mark.parametrize("tie", [False, True], ids=["distinct", "tie_at_k"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("E,k", [(64, 10), (256, 10), (1024, 32)], ids=["E64k10", "E256k10", "E1024k32"])
def test_one_ulp_apart_at_the_kth_place(E, k, path, tie):
    # W_r = 0 again (every score exactly 1/2) and biases j * 2^-24 for a permutation j of 0 .. E-1: the
    # keys 1/2 + j * 2^-24 are exact in fp32 and fp64 and neighbours are one fp32 ulp apart, so the
    # k-th and (k+1)-th largest keys differ only in the last bit.  With tie, the (k+1)-th largest key is
    # raised to equal the k-th, so that two keys share the k-th place (the lower id is taken).
    dims = synth.Dims(T=6, d=64, E=E, k=k, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=17 + E + k, weights=False)
    rng = np.random.default_rng(E * 7 + k + tie)
    j = rng.permutation(E).astype(np.float64)
    if tie:
        j[np.argsort(-j)[k]] += 1.0
    inp["w_router"] = np.zeros((E, dims.d), dtype=np.float32)
    inp["bias"] = (j * 2.0 ** -24).astype(np.float32)
    assert np.array_equal(inp["bias"].astype(np.float64), j * 2.0 ** -24)
    say(f"[case] one-ulp gaps E={E} k={k} {path} tie={tie}")
    ids, w = route(inp, PATHS[path])
    s = np.full((dims.T, E), 0.5)
    ref_ids, _ = oracle.select_experts(s, inp["bias"], k)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_allclose(w, oracle.routing_weights(s, ref_ids), rtol=0, atol=W_ABS)


def _search_bias(case: str, E: int, k: int, rng) -> np.ndarray:
    """Biases that, with every score exactly 1/2, put the keys where each start of the search applies."""
    if case == "all_equal":  # every key the same: the k lowest ids
        return np.full(E, 0.125, dtype=np.float32)
    if case == "k_high":  # exactly k keys in [1, 2) and the rest below 1/2: taken without a search step
        b = -0.375 + rng.permutation(E) * 2.0 ** -12
        b[rng.choice(E, size=k, replace=False)] = 0.75 + np.arange(k) * 2.0 ** -8
        return b.astype(np.float32)
    # one key in [4, 8) and every other below 1: fewer than k keys at or above 2, a search from the top bit
    b = rng.permutation(E) * 2.0 ** -12 - 0.4375
    b[rng.integers(E)] = 3.5
    return b.astype(np.float32)


SEARCH_SHAPES = [(20, 4), (64, 10), (256, 10), (1000, 16)]


@pytest.mark.parametrize("case", ["all_equal", "k_high", "few_high"])
@pytest.mark.parametrize("E,k", SEARCH_SHAPES, ids=[f"E{e}k{k}" for e, k in SEARCH_SHAPES])
def test_search_starts(E, k, case):
    # W_r = 0 (every score exactly 1/2, every key exact in fp32 and fp64).  The search for the k-th key
    # starts from the leading bits shared by the keys at or above the binade below the largest one:
    # all_equal leaves nothing to search, k_high has exactly k such keys, few_high too few (the search
    # then starts at the top bit).  The top-k launch on both router paths and the selection inside the
    # whole-layer call (small-T path) must give the oracle's ids, in slot order, and its weights.
    dims = synth.Dims(T=6, d=128, E=E, k=k, I=64, I_shared=64)
    inp = synth.make_inputs(dims, seed=31 + E + k)
    rng = np.random.default_rng(E * 3 + k + len(case))
    inp["w_router"] = np.zeros((E, dims.d), dtype=np.float32)
    inp["bias"] = _search_bias(case, E, k, rng)
    s = np.full((dims.T, E), 0.5)
    ref_ids, _ = oracle.select_experts(s, inp["bias"], k)
    ref_w = oracle.routing_weights(s, ref_ids)
    for path, flags in PATHS.items():
        say(f"[case] search start {case} E={E} k={k} {path}")
        ids, w = route(inp, flags)
        np.testing.assert_array_equal(ids, ref_ids)
        np.testing.assert_allclose(w, ref_w, rtol=0, atol=W_ABS)
    say(f"[case] search start {case} E={E} k={k} whole-layer call")
    ws = Workspace(dims, 0)
    layer_call_fused(to_device(inp["x"], "cuda"), DeviceWeights.upload(inp), ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ws.topk_ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(ws.topk_w.cpu().numpy(), ref_w, rtol=0, atol=W_ABS)


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("E,k", SHAPES, ids=[f"E{e}k{k}" for e, k in SHAPES])
def test_slot_order_matches_oracle(E, k, path):
    dims = synth.Dims(T=40, d=256, E=E, k=k, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=11 + E + k, weights=False)
    say(f"[case] order E={E} k={k} {path}")
    ids, w = route(inp, PATHS[path])
    s = oracle.sigmoid(oracle.router_logits(inp["x"], inp["w_router"]))
    ref_ids, margin = oracle.select_experts(s, inp["bias"], k)
    key = s + inp["bias"].astype(np.float64)[None, :]
    ordered = 0
    for t in range(dims.T):
        if not margin[t] > MARGIN:
            continue  # the k-th and (k+1)-th keys are too close for an fp32 router to be held to
        assert sorted(ids[t]) == sorted(ref_ids[t]), (t, ids[t], ref_ids[t])
        gaps = -np.diff(key[t, ref_ids[t]])
        if gaps.size == 0 or gaps.min() > MARGIN:  # neighbours far enough apart: the order is fixed
            np.testing.assert_array_equal(ids[t], ref_ids[t])
            ordered += 1
        ref_w = oracle.routing_weights(s[t:t + 1], ids[t:t + 1])[0]
        np.testing.assert_allclose(w[t], ref_w, rtol=0, atol=W_ABS)
    say(f"[route] E={E} k={k} {path}: order checked on {ordered}/{dims.T} tokens")
    assert ordered > 0 or k == 1


@pytest.mark.parametrize("d", [512, 1024, 4096])
@pytest.mark.parametrize("T", [2000, 2048, 4096, 4100])
def test_large_t_router_tile(T, d):
    """The 128-token router tiles: over 128 experts with two K halves (T = 2048; 2000: a ragged last tile)
    and over all 256 experts (T = 4096; 4100: a ragged last tile of 4 tokens), with K parts of 2, 4 and 16
    K steps."""
    dims = synth.Dims(T=T, d=d, E=256, k=10, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=T + d, weights=False)
    say(f"[case] large-T router T={T} d={d}")
    ids, w = route(inp, abi.MOE_FLAG_FORCE_GROUPED)
    s = oracle.sigmoid(oracle.router_logits(inp["x"], inp["w_router"]))
    ref_ids, margin = oracle.select_experts(s, inp["bias"], dims.k)
    clear = margin > MARGIN
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(np.sort(ids[clear], 1), np.sort(ref_ids[clear], 1))
    ref_w = oracle.routing_weights(s, ids)
    np.testing.assert_allclose(w, ref_w, rtol=0, atol=W_ABS)


BUILDS = [(40, 1024, 32, 0), (40, 1024, 32, abi.MOE_FLAG_ID_ORDER), (700, 1024, 2, 0), (2000, 16, 2, 0),
          (64, 256, 10, abi.MOE_FLAG_ID_ORDER), (2048, 256, 10, 0)]


@pytest.mark.parametrize("T,E,k,extra", BUILDS, ids=[f"T{t}E{e}k{k}f{f}" for t, e, k, f in BUILDS])
def test_routing_build_forms(T, E, k, extra):
    """The routing build in one workgroup (at most 4096 pairs, token bitmasks in LDS: E * ceil(T/32) <=
    20480 words) and in two launches (700 tokens x 1024 experts; 20480 pairs), against the oracle's
    CSR construction bit for bit, including E = 1024 (1025 groups for 1024 threads) and the id-order
    schedule."""
    from gpu_util import check_routing_build
    flags = abi.MOE_FLAG_FORCE_GROUPED | extra
    dims = synth.Dims(T=T, d=64, E=E, k=k, I=32, I_shared=32)
    inp = synth.make_inputs(dims, seed=T + E + k, weights=False)
    say(f"[case] build T={T} E={E} k={k} flags={flags}")
    ws = Workspace(dims, flags)
    abi.moe_route(dims, to_device(inp["x"], "cuda"), to_device(inp["w_router"], "cuda"),
                  to_device(inp["bias"], "cuda"), ws.topk_ids, ws.topk_w, ws.routing, flags=flags)
    abi.moe_build_descriptors(dims, ws.topk_ids, ws.routing, flags=flags)
    torch.cuda.synchronize()
    check_routing_build(ws)
