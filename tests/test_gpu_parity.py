"""GPU parity of the HIP layer against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, Workspace, layer_call, layer_call_fused, to_device
from gpu_util import check_parity, check_routing_build, run, say

pytestmark = pytest.mark.gpu

GROUPED = abi.MOE_FLAG_FORCE_GROUPED
GEMV = abi.MOE_FLAG_FORCE_GEMV

SMALL = {
    # name: (dims, bias recipe)
    "tiny": (synth.CONFIGS["tiny"].dims, "uniform"),
    "ragged": (synth.Dims(T=37, d=96, E=20, k=3, I=160, I_shared=96), "uniform"),
    "multi_tile": (synth.Dims(T=300, d=512, E=4, k=2, I=256, I_shared=384), "uniform"),
    "single_expert": (synth.Dims(T=5, d=64, E=1, k=1, I=32, I_shared=64), "uniform"),
    "full_mixture": (synth.Dims(T=9, d=128, E=6, k=6, I=64, I_shared=32), "uniform"),
    "one_token": (synth.Dims(T=1, d=256, E=16, k=4, I=128, I_shared=128), "uniform"),
    "skewed": (synth.Dims(T=200, d=256, E=32, k=4, I=96, I_shared=128), "zipf"),
}


@pytest.mark.parametrize("flags", [0, GROUPED, GEMV], ids=["default", "grouped", "gemv"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes(name, flags):
    dims, bias = SMALL[name]
    if flags == GEMV and dims.T > abi.MOE_GEMV_FORCE_MAX_T:
        pytest.skip("the small-T path is limited to T <= 64")
    say(f"[case] small {name} flags={flags} dims={dims}")
    inp = synth.make_inputs(dims, seed=100 + len(name), bias=bias)
    ws, _ = run(inp, flags)
    check_parity(inp, ws, label=f"{name}/{flags}")
    if abi.moe_path(dims, flags) == 1:
        check_routing_build(ws)


def test_tiny_paths_agree_and_are_deterministic():
    inp = synth.make_inputs(synth.CONFIGS["tiny"])
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    a, _ = run(inp, 0, w, x)
    b, _ = run(inp, 0, w, x)
    assert torch.equal(a.y, b.y) and torch.equal(a.topk_ids, b.topk_ids)
    g1, _ = run(inp, GROUPED, w, x)
    g2, _ = run(inp, GROUPED, w, x)
    assert torch.equal(g1.y, g2.y)
    assert torch.equal(a.topk_ids, g1.topk_ids)
    rel = (a.y - g1.y).norm() / g1.y.norm()
    assert rel < 5e-3


@pytest.mark.parametrize("flags", [GROUPED, GEMV], ids=["grouped", "gemv"])
@pytest.mark.parametrize("in_place", [False, True], ids=["separate", "in_place"])
def test_residual_fused_output(flags, in_place):
    """moe_q4_forward_residual: parity with the oracle's (routed + shared) + residual, and bit for bit the
    plain forward's output plus the residual in fp32 (the add comes last); the residual may be y itself."""
    dims, bias = SMALL["ragged"]
    say(f"[case] residual flags={flags} in_place={in_place} dims={dims}")
    inp = synth.make_inputs(dims, seed=121, bias=bias)
    res = (np.random.default_rng(122).standard_normal((dims.T, dims.d)) * 3).astype(np.float32)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    plain, _ = run(inp, flags, w, x)
    ws = Workspace(dims, flags)
    r_dev = torch.from_numpy(res).cuda()
    if in_place:
        ws.y.copy_(r_dev)
    layer_call(x, w, ws, residual=ws.y if in_place else r_dev)
    torch.cuda.synchronize()
    check_parity(inp, ws, label=f"residual/{flags}/{in_place}", residual=res)
    assert torch.equal(ws.y, plain.y + r_dev)


@pytest.mark.parametrize("flags", [GROUPED | abi.MOE_FLAG_ID_ORDER, GROUPED | abi.MOE_FLAG_NO_BANDING,
                                   GROUPED | abi.MOE_FLAG_ID_ORDER | abi.MOE_FLAG_NO_BANDING,
                                   GROUPED | abi.MOE_FLAG_BAND_MAJOR])
def test_schedule_order_does_not_change_bits(flags):
    dims = synth.Dims(T=300, d=512, E=12, k=3, I=256, I_shared=384)
    inp = synth.make_inputs(dims, seed=7, bias="zipf")
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    base, _ = run(inp, GROUPED, w, x)
    other, _ = run(inp, flags, w, x)
    check_routing_build(other)
    assert torch.equal(base.y, other.y)


def test_band_major_order_does_not_change_bits():
    # 8 weight bands in both GEMMs (I = 1024 at 128 columns, d = 2048 at 256), so the band-major walk is
    # the one that runs (it needs a multiple of 8 bands)
    dims = synth.Dims(T=300, d=2048, E=12, k=3, I=1024, I_shared=1024)
    inp = synth.make_inputs(dims, seed=17, bias="zipf")
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    base, _ = run(inp, GROUPED, w, x)
    other, _ = run(inp, GROUPED | abi.MOE_FLAG_BAND_MAJOR, w, x)
    assert torch.equal(base.y, other.y)
    check_parity(inp, other, tokens=np.arange(0, 300, 37), label="band_major")


@pytest.mark.parametrize("flags", [0, GROUPED])
def test_doubling_down_scales_doubles_output(flags):
    dims = synth.Dims(T=24, d=256, E=8, k=2, I=128, I_shared=64)
    inp = synth.make_inputs(dims, seed=9)
    a, w = run(inp, flags)
    inp2 = dict(inp)
    for key in ("w2_sc", "s2_sc"):
        inp2[key] = (inp[key].view(np.float16) * np.float16(2)).view(np.uint16)
    b, _ = run(inp2, flags)
    # Exact doubling, except where an fp16 intermediate (grouped path: per-pair down outputs) falls in
    # the fp16 subnormal range, whose absolute spacing 2^-24 does not scale: at most k such roundings
    # per output element.
    diff = (b.y - 2 * a.y).abs()
    assert float(diff.max()) <= dims.k * 2.0 ** -24 * 2, float(diff.max())
    assert float((diff == 0).float().mean()) > 0.99


@pytest.mark.parametrize("flags", [0, GROUPED])
def test_graph_capture_replays_match_eager(flags):
    dims = synth.Dims(T=6 if flags == 0 else 150, d=256, E=16, k=4, I=128, I_shared=128)
    inp = synth.make_inputs(dims, seed=11)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    eager, _ = run(inp, flags, w, x)
    ref = eager.y.clone()
    ws = Workspace(dims, flags)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer_call(x, w, ws, stream=s)  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer_call(x, w, ws, stream=s)
    for i in range(3):
        ws.y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ws.y, ref), f"replay {i}"
        _ = (ws.y * 2).sum().item()  # eager work between replays


# ----------------------------------------------------------------------------- full-size workloads

def long_prefill_tokens(ws, inp, n_tiles=4):
    """Tokens to compare at T = 8192: every row of n_tiles whole 96-row M-tiles of the largest group
    (its first, last -- ragged -- and two in between), and every outlier row."""
    dims = ws.dims
    counts = ws.routing_view("counts", dims.E).cpu().numpy()
    offsets = ws.routing_view("offsets", dims.E + 1).cpu().numpy()
    sorted_pair = ws.routing_view("sorted_pair", dims.T * dims.k).cpu().numpy()
    g = int(np.argmax(counts))
    nmt = (int(counts[g]) + 95) // 96
    tiles = sorted({0, nmt - 1, nmt // 3, (2 * nmt) // 3})[:n_tiles]
    toks = set()
    for m in tiles:
        lo = int(offsets[g]) + 96 * m
        hi = min(lo + 96, int(offsets[g]) + int(counts[g]))
        toks |= set((sorted_pair[lo:hi] // dims.k).tolist())
    toks |= set(int(t) for t in inp["outlier_rows"])
    say(f"[tokens] long prefill: group {g} ({counts[g]} rows, {nmt} M-tiles), tiles {tiles}, "
        f"{len(inp['outlier_rows'])} outlier rows, {len(toks)} tokens")
    return np.array(sorted(toks))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode", "batched_decode", "prefill", "long_prefill"])
def test_full_size_workloads(name):
    """The four full-size workloads through moe_layer_forward, the call bench.py times, in its default
    launch configuration: every token compared at T = 1, 64 and 2048; at T = 8192 every row of four whole
    M-tiles of the largest group and every outlier row.  Bit-reproducible; the separate calls give the
    same bits; at T = 64 the small-T path too."""
    cfg = synth.CONFIGS[name]
    say(f"[case] full {name} dims={cfg.dims}")
    inp = synth.make_inputs(cfg)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    ws = Workspace(cfg.dims, 0)
    layer_call_fused(x, w, ws)
    torch.cuda.synchronize()
    T = cfg.dims.T
    tokens = long_prefill_tokens(ws, inp) if name == "long_prefill" else np.arange(T)
    check_parity(inp, ws, tokens=tokens, label=name)
    if abi.moe_path(cfg.dims) == 1:
        check_routing_build(ws)
        counts = ws.routing_view("counts", cfg.dims.E).cpu().numpy()
        say(f"[groups] {name}: distinct={int((counts > 0).sum())} max={counts.max()} median={int(np.median(counts))}")
    # bitwise reproducible, and the separate calls give the same bits
    again = Workspace(cfg.dims, 0)
    layer_call_fused(x, w, again)
    sep, _ = run(inp, 0, w, x)
    torch.cuda.synchronize()
    assert torch.equal(again.y, ws.y)
    assert torch.equal(sep.y, ws.y) and torch.equal(sep.topk_ids, ws.topk_ids)
    if T == 64:
        gemv, _ = run(inp, GEMV, w, x)
        assert torch.equal(gemv.topk_ids, ws.topk_ids)
        check_parity(inp, gemv, tokens=tokens, label=name + "/gemv")


@pytest.mark.parametrize("flags", [GEMV, GROUPED], ids=["gemv", "grouped"])
def test_small_t_path_at_its_size_limits(flags):
    """d = 8192 and I = I_shared = 2048, the largest shape the small-T path takes: a wavefront's quarter of
    K in the gate+up GEMV is then exactly 64 Q4 blocks, and the down GEMV stages exactly 64 blocks of h.
    The grouped path on the same shape for comparison."""
    dims = synth.Dims(T=3, d=8192, E=4, k=2, I=2048, I_shared=2048)
    say(f"[case] size limits flags={flags} dims={dims}")
    inp = synth.make_inputs(dims, seed=131)
    ws, _ = run(inp, flags)
    check_parity(inp, ws, label=f"limits/{flags}")


SCALE_RANGES = {
    # the grouped GEMM dequantises in its common form for 2^-10 <= |d| < 2^-4 and in the general form
    # otherwise (chosen per K iteration and wavefront); the small-T path has a single form
    "large": (0.07, 0.5),          # every block past 2^-4
    "tiny": (1.0e-4, 9.0e-4),      # every block below 2^-10
    "mixed": (2.0e-4, 0.2),        # both forms inside one launch, often inside one iteration
}


@pytest.mark.parametrize("flags", [GROUPED, GEMV], ids=["grouped", "gemv"])
@pytest.mark.parametrize("rng_name", list(SCALE_RANGES))
def test_scales_outside_the_common_dequant_range(rng_name, flags):
    """Parity with Q4 scales drawn outside U(0.005, 0.02): the grouped GEMM's general dequantisation form,
    and both forms mixed, held to the oracle like the common one.  Activations are scaled with the
    weights (down for large scales, up for tiny ones) so that every fp16 intermediate of the grouped
    path (h, the per-pair down outputs) stays in the fp16 normal range."""
    lo, hi = SCALE_RANGES[rng_name]
    dims = synth.Dims(T=40, d=256, E=8, k=2, I=128, I_shared=64)
    inp = synth.make_inputs(dims, seed=140 + len(rng_name))
    rng = np.random.default_rng(141)
    for key in ("w13_sc", "w2_sc", "s13_sc", "s2_sc"):
        d = rng.uniform(lo, hi, size=inp[key].shape)
        if rng_name == "mixed":
            d = np.exp(rng.uniform(np.log(lo), np.log(hi), size=inp[key].shape))
        inp[key] = d.astype(np.float16).view(np.uint16)
    x_scale = {"large": 0.05, "tiny": 64.0, "mixed": 1.0}[rng_name]
    x = oracle.bf16_bits_to_f64(inp["x"]) * x_scale
    inp["x"] = synth.bf16_bits_from_f32(x.astype(np.float32))
    say(f"[case] scales {rng_name} flags={flags}")
    ws, _ = run(inp, flags)
    check_parity(inp, ws, label=f"scales/{rng_name}/{flags}")


@pytest.mark.parametrize("flags", [GROUPED, GEMV], ids=["grouped", "gemv"])
def test_zero_experts_give_exact_zero_and_exact_residual(flags):
    """Every code 8 (every routed and shared weight 0): y is exactly 0, and with a residual exactly the
    residual (added after the routed + shared sum), whatever the scales."""
    dims = synth.Dims(T=21, d=96, E=12, k=3, I=64, I_shared=96)
    inp = synth.make_inputs(dims, seed=151)
    for key in ("w13_qs", "w2_qs", "s13_qs", "s2_qs"):
        inp[key][:] = 0x88
    say(f"[case] zero experts flags={flags}")
    ws, w = run(inp, flags)
    assert torch.count_nonzero(ws.y) == 0
    res = torch.randn(dims.T, dims.d, device="cuda")
    ws2 = Workspace(dims, flags)
    layer_call(to_device(inp["x"], "cuda"), w, ws2, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(ws2.y, res)


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.integers(1, 301))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.integers(1, 201))
        d = 32 * int(rng.integers(1, 25))       # 32 .. 768
        I = 32 * int(rng.integers(1, 17))       # 32 .. 512
        Is = 32 * int(rng.integers(1, 17))
        out.append(synth.Dims(T=T, d=d, E=E, k=k, I=I, I_shared=Is))
    return out


SWEEP = _random_shapes(12, 2024)
# many experts: up to 1025 groups (with the shared one) in one grouped launch, most of them tiny
SWEEP += [synth.Dims(T=t, d=d, E=e, k=k, I=i, I_shared=s)
          for t, d, e, k, i, s in [(90, 128, 1024, 32, 64, 96), (33, 96, 777, 5, 160, 32), (64, 64, 640, 17, 96, 64)]]


@pytest.mark.parametrize("dims", SWEEP, ids=[f"T{s.T}d{s.d}E{s.E}k{s.k}I{s.I}Is{s.I_shared}" for s in SWEEP])
def test_random_shape_sweep(dims):
    """Seeded random shapes inside the supported range (any T, E, k <= min(E, 32), d, I, I_shared
    multiples of 32): the default path, the grouped path and, where T <= 64, the small-T path, each held
    to the oracle, with the routing build checked bit for bit on the grouped path."""
    inp = synth.make_inputs(dims, seed=dims.T * 7 + dims.E)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    for flags in (0, GROUPED, GEMV):
        if flags == GEMV and dims.T > abi.MOE_GEMV_FORCE_MAX_T:
            continue
        say(f"[case] sweep {dims} flags={flags}")
        ws, _ = run(inp, flags, w, x)
        check_parity(inp, ws, label=f"sweep/{flags}")
        if abi.moe_path(dims, flags) == 1:
            check_routing_build(ws)


# ----------------------------------------------------------------------------- fp16 range of the activations

def _oracle_h_and_expert_max(inp, X):
    """max |h| and max |expert output| over every expert (routed and shared) on the rows X, from the
    oracle's own dequantisation: shows a case really reaches the values it is meant to."""
    dims = inp["dims"]
    mats = [(inp["w13_qs"][e], inp["w13_sc"][e], inp["w2_qs"][e], inp["w2_sc"][e]) for e in range(dims.E)]
    mats.append((inp["s13_qs"], inp["s13_sc"], inp["s2_qs"], inp["s2_sc"]))
    hmax = ymax = 0.0
    for a, b, c, d in mats:
        w13, w2 = oracle.dequant_q4(a, b), oracle.dequant_q4(c, d)
        I = w13.shape[0] // 2
        g, u = X @ w13[:I].T, X @ w13[I:].T
        h = g * oracle.sigmoid(g) * u
        hmax, ymax = max(hmax, float(np.abs(h).max())), max(ymax, float(np.abs(h @ w2.T).max()))
    return hmax, ymax


@pytest.mark.parametrize("flags", [GROUPED, GEMV], ids=["grouped", "gemv"])
def test_large_activations_inside_the_fp16_range(flags):
    """Activations scaled so that the SwiGLU output h reaches about 1e4 (inside fp16, where both paths
    keep it): parity with the oracle on both paths.  The down scales are divided by 16 so that every
    expert's output stays inside the fp16 range as well."""
    dims = synth.Dims(T=40, d=512, E=8, k=2, I=128, I_shared=128)
    inp = synth.make_inputs(dims, seed=161)
    x = oracle.bf16_bits_to_f64(inp["x"]) * 24.0
    inp["x"] = synth.bf16_bits_from_f32(x.astype(np.float32))
    for key in ("w2_sc", "s2_sc"):
        inp[key] = (inp[key].view(np.float16) / np.float16(16)).view(np.uint16)
    hmax, ymax = _oracle_h_and_expert_max(inp, oracle.bf16_bits_to_f64(inp["x"]))
    assert 5e3 <= hmax < 6e4 and ymax < 6e4, (hmax, ymax)
    say(f"[case] large activations flags={flags}: max|h| {hmax:.3g}, max|expert out| {ymax:.3g}")
    ws, _ = run(inp, flags)
    check_parity(inp, ws, label=f"large_h/{flags}")


def test_x_beyond_the_fp16_range_saturates_alike_on_both_paths():
    """Layer inputs beyond the fp16 range (bf16 holds them) are saturated to +-65504 for the expert
    projections on both paths, while the router sees them unchanged.  Here one input column holds
    +-2^17 and the router ignores that column (its W_r column is zero), so the oracle's selection and
    weights are exact; the expected output is the oracle's layer with that column saturated to
    +-65504, built from the oracle's dequantisation and expert MLP.  The column's gate/up codes are 7
    or 9 (weight -+scale) with scales near 1e-3, so h stays inside fp16; the unsaturated input (2^17)
    would give about twice the output and fail the bound."""
    dims = synth.Dims(T=24, d=256, E=8, k=2, I=64, I_shared=64)
    inp = synth.make_inputs(dims, seed=171)
    rng = np.random.default_rng(172)
    c0 = 77
    inp["w_router"][:, c0] = 0.0
    x = oracle.bf16_bits_to_f64(inp["x"])
    x[:, c0] = rng.choice([-1.0, 1.0], size=dims.T) * 2.0 ** 17
    inp["x"] = synth.bf16_bits_from_f32(x.astype(np.float32))
    for qk, sk in (("w13_qs", "w13_sc"), ("s13_qs", "s13_sc")):
        q = inp[qk]
        code = rng.choice([7, 9], size=q.shape[:-1]).astype(np.uint8)  # weight -scale or +scale
        byte = q[..., c0 // 2]
        q[..., c0 // 2] = (byte & 0xF0) | code if c0 % 2 == 0 else (byte & 0x0F) | (code << 4)
        inp[sk] = rng.uniform(1.0e-3, 1.5e-3, size=inp[sk].shape).astype(np.float16).view(np.uint16)
    x_sat = np.clip(oracle.bf16_bits_to_f64(inp["x"]), -65504.0, 65504.0)
    sel = oracle.forward(inp)  # selection and weights: the router never sees column c0
    ref = np.zeros((dims.T, dims.d))
    for t in range(dims.T):
        for j in range(dims.k):
            e = sel["ids"][t, j]
            ref[t] += sel["w"][t, j] * oracle.swiglu_mlp(
                x_sat[t:t + 1], oracle.dequant_q4(inp["w13_qs"][e], inp["w13_sc"][e]),
                oracle.dequant_q4(inp["w2_qs"][e], inp["w2_sc"][e]))[0]
    ref += oracle.swiglu_mlp(x_sat, oracle.dequant_q4(inp["s13_qs"], inp["s13_sc"]),
                             oracle.dequant_q4(inp["s2_qs"], inp["s2_sc"]))
    hmax, ymax = _oracle_h_and_expert_max(inp, x_sat)
    assert 1e3 <= hmax < 6e4 and ymax < 6e4, (hmax, ymax)
    outs = []
    for flags in (GEMV, GROUPED):
        ws, _ = run(inp, flags)
        ids = ws.topk_ids.cpu().numpy()
        for t in range(dims.T):
            assert sorted(ids[t]) == sorted(sel["ids"][t]), (flags, t)
        y = ws.y.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(y)), flags
        max_rel = np.abs(y - ref).max() / np.abs(ref).max()
        l2_rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
        say(f"[parity] saturated x flags={flags}: max|h| {hmax:.3g} max_rel={max_rel:.3e} l2_rel={l2_rel:.3e}")
        assert max_rel <= 1e-2 and l2_rel <= 5e-3, (flags, max_rel, l2_rel)
        outs.append(y)
    assert np.linalg.norm(outs[0] - outs[1]) <= 5e-3 * np.linalg.norm(ref)
