"""GPU: the fp8-activation variants W4A8 (MXFP4 expert weights) and W8A8 (MXFP8 expert weights) through
the C ABI, against their oracle: the weight requantisations and the activation quantisation bit for bit,
the layers under the parity rule (selection exact outside the margin, max-abs and relative-L2 bounds)."""
import numpy as np
import pytest
import torch

import oracle
import oracle.moe_w4a8 as w4
import synth
from sparse_moe_expert_sigmoid_amd import abi
from sparse_moe_expert_sigmoid_amd.layer import DeviceWeights, Workspace, layer_call, to_device
from gpu_util import check_parity, say
from test_gpu_pack import ref_pack_scales


def ref_pack_blocks(codes: np.ndarray, bb: int) -> np.ndarray:
    """Row-major codes [..., rows, K/32 * bb] -> [..., rows/16, K/32, 16, bb]: block b of row r moves to
    byte ((r/16)*(K/32) + b)*16*bb + (r%16)*bb of its matrix (the header's layout)."""
    *lead, rows, width = codes.shape
    nkb = width // bb
    return np.ascontiguousarray(codes.reshape(*lead, rows // 16, 16, nkb, bb).swapaxes(-3, -2))

pytestmark = pytest.mark.gpu

GROUPED = abi.MOE_FLAG_FORCE_GROUPED


VARIANTS = {
    # name: (requantisation entry, forward entry, scratch query, oracle forward, oracle requantisation,
    #        code bytes per Q4 code byte)
    "w4a8": (abi.moe_q4_to_mxfp4, abi.moe_w4a8_forward, abi.moe_w4a8_scratch_bytes, w4.forward_w4a8,
             w4.mx_requant, 1),
    "w8a8": (abi.moe_q4_to_mxfp8, abi.moe_w8a8_forward, abi.moe_w8a8_scratch_bytes, w4.forward_w8a8,
             w4.mx8_requant, 2),
}


def mx_upload(w: DeviceWeights, variant: str = "w4a8") -> dict:
    """MXFP4 / MXFP8 copies of the packed Q4 stacks, made on the device by moe_q4_to_mxfp4 / _mxfp8."""
    requant, *_, ratio = VARIANTS[variant]
    dims = w.dims
    shapes = {"w13": (dims.E, 2 * dims.I, dims.d), "w2": (dims.E, dims.d, dims.I),
              "s13": (1, 2 * dims.I_shared, dims.d), "s2": (1, dims.d, dims.I_shared)}
    mx = {}
    for name, (n, rows, K) in shapes.items():
        codes = torch.empty(w[name + "_qs"].numel() * ratio, dtype=torch.uint8, device="cuda")
        exps = torch.empty(n * rows * (K // 32), dtype=torch.uint8, device=codes.device)
        requant(n, rows, K, w[name + "_qs"], w[name + "_sc"], codes, exps)
        mx[name + "_codes"], mx[name + "_exps"] = codes, exps
    return mx


def w4a8_call(dims, x, ws: Workspace, mx: dict, flags: int, variant: str = "w4a8") -> torch.Tensor:
    """route + build (the W4A16 calls) then the fp8-activation forward into a fresh output."""
    _, forward, scratch_bytes, *_ = VARIANTS[variant]
    y = torch.full((dims.T, dims.d), float("nan"), dtype=torch.float32, device="cuda")
    scratch = torch.empty(scratch_bytes(dims, flags), dtype=torch.uint8, device="cuda")
    forward(dims, x, ws.topk_ids, ws.topk_w, ws.routing, mx, y, scratch, flags=flags)
    return y


# ----------------------------------------------------------------------------- requantisation, bit for bit

def special_q4(rng, rows, K):
    """Random Q4 codes and scales with hand-placed edge blocks: all-zero values, zero and negative
    scales, subnormal and largest fp16 scales, a single nonzero element, every code equal."""
    qs = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    sc = np.float16(rng.uniform(0.005, 0.02, (rows, K // 32))).view(np.uint16)
    f16 = lambda v: np.float16(v).view(np.uint16)
    qs[0, 0:16] = 0x88                                   # all values zero
    qs[1, 0:16] = rng.integers(0, 256, 16); sc[1, 0] = f16(0.0)
    sc[2, 0] = f16(-0.0113)
    sc[3, 0] = f16(2.0 ** -24)                           # smallest subnormal
    sc[4, 0] = f16(65504.0)
    sc[5, 0] = f16(6.1e-5)                               # around the subnormal edge
    qs[6, 0:16] = 0x88; qs[6, 3] = 0x8F                  # one nonzero element (+7)
    qs[7, 0:16] = 0x00                                   # every value -8
    qs[8, 0:16] = 0xFF                                   # every value +7
    sc[9, :] = f16(-0.25)
    return qs, sc


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("n_mats,rows,K", [(1, 16, 32), (2, 48, 256), (3, 64, 4096), (1, 2048, 1024)])
def test_q4_to_mx_bit_exact(n_mats, rows, K, variant):
    say(f"[case] q4_to_mx {variant} n_mats={n_mats} rows={rows} K={K}")
    requant_gpu, _, _, _, requant_ref, ratio = VARIANTS[variant]
    bb = 16 * ratio  # code bytes per block
    rng = np.random.default_rng(rows + K + n_mats)
    qs = np.empty((n_mats, rows, K // 2), np.uint8)
    sc = np.empty((n_mats, rows, K // 32), np.uint16)
    for m in range(n_mats):
        qs[m], sc[m] = special_q4(rng, rows, K)
    ref = [requant_ref(qs[m], sc[m]) for m in range(n_mats)]
    ref_c = np.stack([r[0] for r in ref])
    ref_e = np.stack([r[1] for r in ref])
    # row-major in, row-major out (block b to block b)
    qi, si = to_device(qs, "cuda"), to_device(sc, "cuda")
    co = torch.full((qi.numel() * ratio,), 0x5A, dtype=torch.uint8, device="cuda")
    eo = torch.full((n_mats * rows * (K // 32),), 0x5A, dtype=torch.uint8, device="cuda")
    requant_gpu(n_mats, rows, K, qi, si, co, eo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(co.cpu().numpy().reshape(-1), ref_c.reshape(-1))
    np.testing.assert_array_equal(eo.cpu().numpy().reshape(-1), ref_e.reshape(-1))
    # the packed 16-row groups in, the same layout out
    qp, sp = torch.empty_like(qi), torch.empty_like(si)
    abi.moe_q4_pack(n_mats, rows, K, qi, si, qp, sp)
    requant_gpu(n_mats, rows, K, qp, sp, co, eo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(co.cpu().numpy().reshape(-1), ref_pack_blocks(ref_c, bb).reshape(-1))
    np.testing.assert_array_equal(eo.cpu().numpy().reshape(-1), ref_pack_scales(ref_e).reshape(-1))


def special_rows(rng, rows, K, fp16: bool):
    X = rng.standard_normal((rows, K)).astype(np.float32)
    X[1] = 0.0                                           # all-zero row: scale 1, zero codes
    X[2] *= 8.0                                          # outlier row
    X[3] = 0.0; X[3, K - 1] = -3.0                       # one nonzero element
    X[4] = np.ldexp(1.0, rng.integers(-30, 0, K)).astype(np.float32) * rng.choice([-1, 1], K)  # wide range:
    X[4, 0] = 1.0                                        # most elements land in the e4m3 subnormals or zero
    X[5, ::2] = -0.0
    if fp16:
        X[6, 0] = 65504.0; X[6, 1] = -65504.0
        bits = np.float16(X).view(np.uint16)
        vals = bits.view(np.float16).astype(np.float32)
    else:
        bits = synth.bf16_bits_from_f32(X)
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, vals


@pytest.mark.parametrize("fp16", [False, True], ids=["bf16", "fp16"])
@pytest.mark.parametrize("rows,K", [(8, 4), (8, 256), (37, 4096), (300, 1024), (7, 520), (9, 8192), (8, 8196)])
def test_rows_to_fp8_bit_exact(rows, K, fp16):
    say(f"[case] rows_to_fp8 rows={rows} K={K} fp16={fp16}")
    rng = np.random.default_rng(rows * 7 + K)
    bits, vals = special_rows(rng, rows, K, fp16)
    codes_ref, s_ref = w4.quant_rows_fp8(vals)
    xi = to_device(bits, "cuda")
    codes = torch.full((rows, K), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    abi.moe_rows_to_fp8(rows, K, xi, codes, s, in_is_fp16=fp16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), codes_ref)


# ----------------------------------------------------------------------------- the layer

SMALL = {
    "tiny": (synth.CONFIGS["tiny"].dims, "uniform"),
    "ragged": (synth.Dims(T=37, d=384, E=20, k=3, I=256, I_shared=128), "uniform"),
    "multi_tile": (synth.Dims(T=300, d=512, E=4, k=2, I=256, I_shared=384), "uniform"),
    "single_expert": (synth.Dims(T=5, d=128, E=1, k=1, I=128, I_shared=128), "uniform"),
    "one_token": (synth.Dims(T=1, d=256, E=16, k=4, I=128, I_shared=128), "uniform"),
    "skewed": (synth.Dims(T=200, d=256, E=32, k=4, I=128, I_shared=256), "zipf"),
    # h rows longer than 1024 (quantised one workgroup per row, routed and shared rows apart)
    "wide_h": (synth.Dims(T=40, d=256, E=8, k=2, I=1280, I_shared=2048), "uniform"),
    # 1024 experts, top-32: most groups empty or of one row
    "many_experts": (synth.Dims(T=64, d=256, E=1024, k=32, I=128, I_shared=128), "uniform"),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", list(SMALL))
def test_fp8act_small_shapes(name, variant):
    dims, bias = SMALL[name]
    say(f"[case] {variant} small {name} dims={dims}")
    inp = synth.make_inputs(dims, seed=300 + len(name), bias=bias)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    ws = Workspace(dims, GROUPED)
    layer_call(x, w, ws)
    mx = mx_upload(w, variant)
    y = w4a8_call(dims, x, ws, mx, GROUPED, variant)
    torch.cuda.synchronize()
    check_parity(inp, ws, label=f"{variant}/{name}", forward=VARIANTS[variant][3], y=y)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_fp8act_schedule_orders_give_the_same_bits(variant):
    dims, bias = SMALL["skewed"]
    inp = synth.make_inputs(dims, seed=9, bias=bias)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    mx = mx_upload(w, variant)
    outs = []
    for flags in (GROUPED, GROUPED | abi.MOE_FLAG_NO_BANDING, GROUPED | abi.MOE_FLAG_BAND_MAJOR,
                  GROUPED | abi.MOE_FLAG_ID_ORDER):
        ws = Workspace(dims, flags)
        layer_call(x, w, ws)
        outs.append(w4a8_call(dims, x, ws, mx, flags, variant))
        outs.append(w4a8_call(dims, x, ws, mx, flags, variant))   # and run to run
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_fp8act_doubling_down_scales_doubles_output(variant):
    """Doubling every Q4 down scale raises each block exponent by one: y doubles exactly."""
    dims, bias = SMALL["ragged"]
    inp = synth.make_inputs(dims, seed=21, bias=bias)
    inp2 = dict(inp)
    for name in ("w2_sc", "s2_sc"):
        inp2[name] = (inp[name].view(np.float16) * np.float16(2)).view(np.uint16)
    x = to_device(inp["x"], "cuda")
    ys = []
    for i in (inp, inp2):
        w = DeviceWeights.upload(i)
        ws = Workspace(dims, GROUPED)
        layer_call(x, w, ws)
        ys.append(w4a8_call(dims, x, ws, mx_upload(w, variant), GROUPED, variant))
    torch.cuda.synchronize()
    # exact, except where a per-pair down output (stored in fp16) falls in the fp16 subnormal range, whose
    # absolute spacing 2^-24 does not scale: at most k + 1 such roundings per output element
    diff = (ys[1] - 2 * ys[0]).abs()
    assert float(diff.max()) <= (dims.k + 1) * 2.0 ** -24 * 2, float(diff.max())
    assert float((diff == 0).float().mean()) > 0.99


_MX_CACHE: dict = {}


def oracle_mx(inp: dict, key: str, experts, variant: str = "w4a8") -> dict:
    """The oracle's requantised matrices for the given experts (and the shared expert), memoised per input
    set so that a full-size check requantises each matrix once."""
    out = {}
    for name in ("w13", "w2"):
        for e in experts:
            k = (key, variant, name, int(e))
            if k not in _MX_CACHE:
                _MX_CACHE[k] = VARIANTS[variant][4](inp[name + "_qs"][e], inp[name + "_sc"][e])
            out[(name, int(e))] = _MX_CACHE[k]
    for name in ("s13", "s2"):
        k = (key, variant, name, None)
        if k not in _MX_CACHE:
            _MX_CACHE[k] = VARIANTS[variant][4](inp[name + "_qs"], inp[name + "_sc"])
        out[(name, None)] = _MX_CACHE[k]
    return out


def few_expert_tokens(ids: np.ndarray, n: int) -> list:
    """n tokens chosen greedily so that together they use as few distinct experts as possible."""
    chosen, used = [], set()
    for _ in range(n):
        best = min((len(used | set(ids[t].tolist())), t) for t in range(len(ids)) if t not in chosen)
        chosen.append(best[1])
        used |= set(ids[best[1]].tolist())
    return sorted(chosen)


@pytest.mark.slow
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name,ntok", [("decode", 1), ("prefill", 3), ("long_prefill", 3)])
def test_fp8act_full_size_sampled_tokens(name, ntok, variant):
    """The full-size workloads (T = 1 on the grouped path), the grouped GEMMs in their default launch
    configuration; the oracle evaluates a few tokens chosen to share experts, with its own requantised
    weights."""
    cfg = synth.CONFIGS[name]
    dims = cfg.dims
    say(f"[case] {variant} full {name} dims={dims}")
    inp = synth.make_inputs(cfg)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    ws = Workspace(dims, GROUPED)
    layer_call(x, w, ws)
    mx = mx_upload(w, variant)
    y = w4a8_call(dims, x, ws, mx, GROUPED, variant)
    y2 = w4a8_call(dims, x, ws, mx_upload(w, variant), GROUPED, variant)
    del mx
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    assert torch.isfinite(y).all()
    ids = ws.topk_ids.cpu().numpy()
    tokens = few_expert_tokens(ids, ntok)
    experts = np.unique(ids[tokens])
    say(f"[sample] {name}: tokens {tokens}, {len(experts)} experts")
    mx = oracle_mx(inp, name, experts, variant)
    ref_forward = VARIANTS[variant][3]
    fwd = lambda i, tokens, ids_override: ref_forward(i, tokens=tokens, ids_override=ids_override, mx=mx)
    check_parity(inp, ws, tokens=np.array(tokens), label=f"{variant}/{name}", forward=fwd, y=y)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_fp8act_prefill_routing_every_token(variant):
    """The prefill workload's token count, expert count, top-k and Zipf-skewed groups (the largest about
    650 rows: several M-tiles, and for MXFP8 weights every tile as two half tiles) with smaller matrices
    (d = 512, I = I_shared = 256), so that the oracle can evaluate every token."""
    dims = synth.Dims(T=2048, d=512, E=256, k=10, I=256, I_shared=256)
    say(f"[case] {variant} prefill routing dims={dims}")
    inp = synth.make_inputs(dims, seed=77, bias="zipf")
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    ws = Workspace(dims, GROUPED)
    layer_call(x, w, ws)
    y = w4a8_call(dims, x, ws, mx_upload(w, variant), GROUPED, variant)
    torch.cuda.synchronize()
    counts = np.bincount(ws.topk_ids.cpu().numpy().ravel(), minlength=dims.E)
    assert counts.max() > 4 * 96  # several M-tiles in the largest group
    check_parity(inp, ws, label=f"{variant}/prefill-routing", forward=VARIANTS[variant][3], y=y)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_fp8act_graph_capture_replays_match_eager(variant):
    """route + build + the fp8-activation forward recorded into a HIP graph: every replay, with eager work
    between replays, gives the eager bits."""
    dims = synth.Dims(T=150, d=256, E=16, k=4, I=128, I_shared=128)
    inp = synth.make_inputs(dims, seed=13)
    w = DeviceWeights.upload(inp)
    x = to_device(inp["x"], "cuda")
    mx = mx_upload(w, variant)
    ws = Workspace(dims, GROUPED)
    layer_call(x, w, ws)
    ref = w4a8_call(dims, x, ws, mx, GROUPED, variant)
    torch.cuda.synchronize()
    _, forward, scratch_bytes, *_ = VARIANTS[variant]
    ws2 = Workspace(dims, GROUPED)
    y = torch.empty((dims.T, dims.d), dtype=torch.float32, device="cuda")
    scratch = torch.empty(scratch_bytes(dims, GROUPED), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def step():
        abi.moe_route(dims, x, w["w_router"], w["bias"], ws2.topk_ids, ws2.topk_w, ws2.routing, flags=GROUPED,
                      stream=s)
        abi.moe_build_descriptors(dims, ws2.topk_ids, ws2.routing, flags=GROUPED, stream=s)
        forward(dims, x, ws2.topk_ids, ws2.topk_w, ws2.routing, mx, y, scratch, flags=GROUPED, stream=s)

    with torch.cuda.stream(s):
        step()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {i}"
        _ = (y * 2).sum().item()  # eager work between replays
