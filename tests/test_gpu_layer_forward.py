"""GPU: moe_layer_forward (the whole layer in one call; on the small-T path the gate+up workgroups select
their own experts) against moe_route + moe_build_descriptors + moe_q4_forward(_residual) on the same
inputs: the same topk_ids, topk_w and y, bit for bit, and the oracle's parity through the separate calls
(held by the other parity tests) carries over."""
import numpy as np
import pytest
import torch

import synth
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, Workspace, layer_call, layer_call_fused, to_device
from gpu_util import check_parity, say

pytestmark = pytest.mark.gpu

CASES = [  # (T, d, E, k, I, Is, flags): every key-register count of the selection, ragged shapes
    (1, 256, 20, 4, 64, 64, 0),
    (1, 512, 128, 8, 128, 96, 0),
    (3, 256, 256, 10, 128, 128, 0),
    (8, 192, 500, 16, 96, 64, 0),
    (2, 128, 1000, 32, 64, 32, 0),
    (5, 256, 1024, 10, 64, 64, abi.MOE_FLAG_FORCE_GEMV),
    (37, 96, 20, 3, 160, 96, abi.MOE_FLAG_FORCE_GROUPED),
    (64, 256, 256, 10, 128, 128, 0),
    # the decode workload bench.py times (d = 4096, E = 256, top-10, I = I_shared = 1024) at T = 1 and 8
    (1, 4096, 256, 10, 1024, 1024, 0),
    (8, 4096, 256, 10, 1024, 1024, 0),
    # large T: the router's 128-token tiles write the gate+up's fp16 copy of x (ragged last tiles)
    (2000, 1024, 256, 10, 64, 64, 0),
    (4100, 1024, 256, 10, 64, 64, 0),
]


@pytest.mark.parametrize("residual", [False, True], ids=["plain", "residual"])
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}d{c[1]}E{c[2]}k{c[3]}f{c[6]}" for c in CASES])
def test_layer_forward_equals_the_separate_calls(case, residual):
    T, d, E, k, I, Is, flags = case
    dims = synth.Dims(T=T, d=d, E=E, k=k, I=I, I_shared=Is)
    say(f"[case] layer_forward {dims} flags={flags} residual={residual}")
    inp = synth.make_inputs(dims, seed=900 + T + E + k)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    res = torch.from_numpy(np.random.default_rng(T + E).standard_normal((T, d)).astype(np.float32)).cuda()
    a, b = Workspace(dims, flags), Workspace(dims, flags)
    layer_call(x, w, a, residual=res if residual else None)
    layer_call_fused(x, w, b, residual=res if residual else None)
    torch.cuda.synchronize()
    assert torch.equal(a.topk_ids, b.topk_ids)
    assert torch.equal(a.topk_w.view(torch.int32), b.topk_w.view(torch.int32))
    assert torch.equal(a.y.view(torch.int32), b.y.view(torch.int32))
    if d == 4096 and not residual:  # the decode workload's shape: the single call held to the oracle too
        check_parity(inp, b, label=f"layer_forward T={T}")
    # again, with the outputs of the first call still in place: nothing depends on stale contents
    layer_call_fused(x, w, b, residual=res if residual else None)
    torch.cuda.synchronize()
    assert torch.equal(a.y.view(torch.int32), b.y.view(torch.int32))
