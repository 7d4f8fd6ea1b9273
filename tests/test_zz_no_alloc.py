"""GPU: moe_layer_forward_noalloc (routing workspace and scratch in the library's own device array)
against moe_layer_forward with caller-owned workspaces, through the C ABI: the same topk_ids, topk_w and
y bit for bit, on calls in a row that each shrink the input (the array keeps the last call's contents),
on both execution paths, with and without a residual; and the first call held to the oracle."""
import numpy as np
import pytest
import torch

import synth
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, Workspace, layer_call_fused, to_device
from gpu_util import check_parity, say

pytestmark = pytest.mark.gpu


def _noalloc(dims, x, w, flags=0, residual=None):
    T, k, d = dims.T, dims.k, dims.d
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    tw = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    abi.moe_layer_forward_noalloc(dims, x, w["w_router"], w["bias"], w, y, ids, tw, residual=residual, flags=flags)
    return ids, tw, y


def _same(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("residual", [False, True], ids=["plain", "residual"])
def test_noalloc_matches_layer_forward_on_shrinking_calls(residual):
    E, k = 32, 4
    # grouped path (T = 150), then the small-T path (T = 6), then T = 1: each call smaller than the last
    shapes = [(150, 512, 256, 128, 0), (6, 512, 256, 128, 0), (1, 256, 128, 64, abi.MOE_FLAG_FORCE_GEMV)]
    for i, (T, d, I, Is, flags) in enumerate(shapes):
        dims = synth.Dims(T=T, d=d, E=E, k=k, I=I, I_shared=Is)
        say(f"[case] noalloc call {i} {dims} flags={flags} residual={residual}")
        inp = synth.make_inputs(dims, seed=300 + i)
        w = DeviceWeights.upload(inp)
        x = to_device(inp["x"], "cuda")
        res = (torch.from_numpy(np.random.default_rng(i).standard_normal((T, d)).astype(np.float32)).cuda()
               if residual else None)
        ids, tw, y = _noalloc(dims, x, w, flags, res)
        ref = Workspace(dims, flags)
        layer_call_fused(x, w, ref, residual=res)
        torch.cuda.synchronize()
        assert torch.equal(ids, ref.topk_ids), i
        assert _same(tw, ref.topk_w), i
        assert _same(y, ref.y), i
        if i == 0 and not residual:
            check_parity(inp, ref, label="noalloc reference")


def test_noalloc_rejects_a_shape_beyond_its_array():
    dims = synth.CONFIGS["prefill"].dims
    z = torch.zeros(16, dtype=torch.float32, device="cuda")
    w = {name: z for name in ("w_router", "bias", "w13_qs", "w13_sc", "w2_qs", "w2_sc", "s13_qs", "s13_sc",
                              "s2_qs", "s2_sc")}
    rc = abi.moe_layer_forward_noalloc(dims, z, z, z, w, z, z, z, check=False)
    assert rc == abi.MOE_ENOSPACE
