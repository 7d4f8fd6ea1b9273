#!/usr/bin/env python3
"""Throughput of the MI355X Q4 MoE expert layer (route -> build -> forward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|batched_decode|prefill|long_prefill]
    python bench.py --all          (every workload, one JSON line with a list of them)

One step is one call of the whole layer on one batch of synthetic tokens:
moe_layer_forward (with --separate-calls: moe_route + moe_build_descriptors +
moe_q4_forward, the same results).  Steps are captured in
a HIP graph that cycles through L independent layer copies (weights and
tokens), so that successive steps do not find the previous step's weights
in the 256 MB MALL, as in a model with many layers.  W warm-up steps run
first, then exactly K steps are timed with HIP events on the launch stream,
bracketed by device synchronisation.

The primary workload (default: single-token decode, d=4096, E=256, top-10,
I=1024, shared I=1024) gives `value`; the 2048-token prefill chunk is
measured the same way and reported under `secondary`, and again as the W4A8
and W8A8 variants (moe_route + moe_build_descriptors + moe_w4a8_forward /
moe_w8a8_forward on MXFP4 / MXFP8 copies of the weights, fp8 activations)
under `secondary_w4a8` / `secondary_w8a8`, whose gate+up rooflines are priced
against HBM (those GEMMs stream weights: 315 / 166 FLOP per byte, under the
fp8 ridge), with the fraction of the fp8 MFMA peak beside.  Per-kernel average
durations come from graphs that replay only that kernel's nodes, extracted
from the captured layer graph, timed with HIP events on the same stream
(every launch of the layer is idempotent, so replaying one alone is valid).
`cpu_baseline` (primary and secondary line) times the CPU oracle on a
bounded sample of the same workload's tokens.  For an HBM-bound dominant kernel the roofline object also carries the rate
of torch's device copy kernel moving the same number of bytes
(`copy_ceiling`): the practical streaming ceiling beside the nominal peak.

`decode_ctx` times the library's multi-layer decode context on the decode
shape: 8 independent layer copies recorded once into one HIP graph by
moe_decode_ctx_create, a pass taking a residual stream through all of them
(x = bf16(h), h = layer(x) + h); reported per layer, and again with the
pre-MoE RMSNorm in front of every layer (`decode_ctx_norm`).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at T=1 and T=2048; % HBM roofline / % bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
MFMA_F8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (fp8 x fp4 runs at the fp8 rate), TFLOP/s
COPIES = {"decode": 8, "batched_decode": 8, "prefill": 2, "long_prefill": 2}


# ----------------------------------------------------------------------------- HIP graph helpers (ctypes)

class _KernelNodeParams(ctypes.Structure):
    _fields_ = [("blockDim", ctypes.c_uint * 3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p),
                ("gridDim", ctypes.c_uint * 3), ("kernelParams", ctypes.c_void_p),
                ("sharedMemBytes", ctypes.c_uint)]


class Hip:
    """The HIP runtime already loaded in this process (torch's), for graph capture and node surgery."""

    def __init__(self):
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
        self.L = ctypes.CDLL(path or "libamdhip64.so")
        self.live = []

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with hipError {rc}")

    def begin_capture(self, stream: int):
        self._ok(self.L.hipStreamBeginCapture(ctypes.c_void_p(stream), 2), "hipStreamBeginCapture")  # relaxed

    def end_capture(self, stream: int) -> ctypes.c_void_p:
        g = ctypes.c_void_p()
        self._ok(self.L.hipStreamEndCapture(ctypes.c_void_p(stream), ctypes.byref(g)), "hipStreamEndCapture")
        self.live.append(g)
        return g

    def instantiate(self, graph) -> ctypes.c_void_p:
        ex = ctypes.c_void_p()
        self._ok(self.L.hipGraphInstantiate(ctypes.byref(ex), graph, None, None, ctypes.c_size_t(0)),
                 "hipGraphInstantiate")
        return ex

    def launch(self, exec_, stream: int):
        self._ok(self.L.hipGraphLaunch(exec_, ctypes.c_void_p(stream)), "hipGraphLaunch")

    def kernel_nodes(self, graph, stream: int):
        """[(kernel name, params)] of the graph's kernel nodes, in graph order."""
        n = ctypes.c_size_t(0)
        self._ok(self.L.hipGraphGetNodes(graph, None, ctypes.byref(n)), "hipGraphGetNodes")
        nodes = (ctypes.c_void_p * n.value)()
        self._ok(self.L.hipGraphGetNodes(graph, nodes, ctypes.byref(n)), "hipGraphGetNodes")
        self.L.hipKernelNameRefByPtr.restype = ctypes.c_char_p
        out = []
        for node in nodes:
            t = ctypes.c_int(-1)
            self._ok(self.L.hipGraphNodeGetType(ctypes.c_void_p(node), ctypes.byref(t)), "hipGraphNodeGetType")
            if t.value != 0:  # hipGraphNodeTypeKernel
                continue
            p = _KernelNodeParams()
            self._ok(self.L.hipGraphKernelNodeGetParams(ctypes.c_void_p(node), ctypes.byref(p)),
                     "hipGraphKernelNodeGetParams")
            name = self.L.hipKernelNameRefByPtr(ctypes.c_void_p(p.func), ctypes.c_void_p(stream))
            out.append(((name or b"?").decode(), p))
        return out

    def chain_graph(self, params_list):
        """A new graph running the given kernel nodes one after another."""
        g = ctypes.c_void_p()
        self._ok(self.L.hipGraphCreate(ctypes.byref(g), ctypes.c_uint(0)), "hipGraphCreate")
        prev = None
        for p in params_list:
            node = ctypes.c_void_p()
            deps = (ctypes.c_void_p * 1)(prev) if prev is not None else None
            self._ok(self.L.hipGraphAddKernelNode(ctypes.byref(node), g, deps, ctypes.c_size_t(1 if deps else 0),
                                                  ctypes.byref(p)), "hipGraphAddKernelNode")
            prev = node
        self.live.append(g)
        return g


def short_name(mangled: str) -> str:
    for key, nice in (("k_router_gemv", "router_gemv"), ("k_router_mfma", "router_mfma"), ("k_topk", "topk"),
                      ("k_build_count", "build_count"), ("k_build_scatter", "build_scatter"),
                      ("k_gemv_gateup", "gemv_gateup"), ("k_gemv_down_combine", "gemv_down_combine"),
                      ("k_x_to_f16", "x_to_f16"), ("k_groupedILb1", "grouped_gateup"),
                      ("k_groupedILb0", "grouped_down"), ("k_combine", "combine"),
                      ("k_grouped_mxILb1", "grouped_mx_gateup"), ("k_grouped_mxILb0", "grouped_mx_down"),
                      ("k_rows_fp8_waveILb0", "rows_fp8_x"), ("k_rows_fp8_waveILb1", "rows_fp8_h"),
                      ("k_rows_fp8ILb0", "rows_fp8_x"), ("k_rows_fp8ILb1", "rows_fp8_h")):
        if key in mangled:
            return nice
    return mangled


# ----------------------------------------------------------------------------- workload

def device_copy(cfg, seed, torch, device):
    """A further independent layer copy drawn on the GPU with torch's seeded generator, with the
    same distributions as the numpy generator (x ~ N(0,1) -> bf16, W_r ~ N(0, 0.02), Q4 codes uniform,
    scales ~ U(0.005, 0.02) -> fp16, bias per the workload's recipe).  Scales are drawn i.i.d., so
    drawing them directly in the library's 16-row-group layout gives the same distribution."""
    dims = cfg.dims
    T, d, E, I, Is = dims.T, dims.d, dims.E, dims.I, dims.I_shared
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def qs(*shape):
        return torch.randint(0, 256, shape, dtype=torch.uint8, device=device, generator=g)

    def sc(*shape):
        return (torch.rand(shape, device=device, generator=g) * 0.015 + 0.005).half().view(torch.int16)

    x = torch.randn((T, d), device=device, generator=g)
    if cfg.outlier_frac:
        n_out = int(round(cfg.outlier_frac * T))
        rows = torch.randperm(T, device=device, generator=g)[:n_out]
        x[rows] *= 8.0
    w = {
        "w_router": torch.randn((E, d), device=device, generator=g) * 0.02,
        "w13_qs": qs(E, 2 * I, d // 2), "w13_sc": sc(E, 2 * I, d // 32),
        "w2_qs": qs(E, d, I // 2), "w2_sc": sc(E, d, I // 32),
        "s13_qs": qs(2 * Is, d // 2), "s13_sc": sc(2 * Is, d // 32),
        "s2_qs": qs(d, Is // 2), "s2_sc": sc(d, Is // 32),
    }
    if cfg.bias == "zipf":
        pmf = np.arange(1, E + 1, dtype=np.float64) ** -1.2
        pmf /= pmf.sum()
        perm = torch.randperm(E, device=device, generator=g)
        b = torch.empty(E, device=device)
        b[perm] = torch.tensor(pmf, dtype=torch.float32, device=device)
        w["bias"] = b
    else:
        w["bias"] = torch.rand(E, device=device, generator=g) * 0.2 - 0.1
    return x.bfloat16().view(torch.int16), w


# bytes per block of 32 weights: Q4 (16 code bytes + an fp16 scale), MXFP4 (16 + an exponent byte),
# MXFP8 (32 + an exponent byte)
BLOCK_BYTES = {"w4a16": 18, "w4a8": 17, "w8a8": 33}


def expert_bytes(dims, variant="w4a16"):
    bb = BLOCK_BYTES[variant]
    gu = 2 * dims.I * dims.d // 32 * bb
    dn = dims.d * dims.I // 32 * bb
    sgu = 2 * dims.I_shared * dims.d // 32 * bb
    sdn = dims.d * dims.I_shared // 32 * bb
    return gu, dn, sgu, sdn


def layer_flops(dims):
    T, d, E, P, I, Is = dims.T, dims.d, dims.E, dims.T * dims.k, dims.I, dims.I_shared
    router = 2 * T * d * E
    routed = 2 * P * (2 * I * d + d * I)
    shared = 2 * T * (2 * Is * d + d * Is)
    return router, routed, shared


def source_hash(*files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


GEMV_SOURCES = ("sparse_moe_expert_sigmoid_amd/csrc/gemv.hip", "sparse_moe_expert_sigmoid_amd/csrc/moe_device.hpp",
                "sparse_moe_expert_sigmoid_amd/csrc/topk.hpp")
GROUPED_SOURCES = ("sparse_moe_expert_sigmoid_amd/csrc/grouped.hip", "sparse_moe_expert_sigmoid_amd/csrc/moe_device.hpp")
MX_SOURCES = ("sparse_moe_expert_sigmoid_amd/csrc/w4a8.hip", "sparse_moe_expert_sigmoid_amd/csrc/moe_device.hpp")


def recorded_traffic(profile: str, sources) -> int | None:
    """HBM bytes per launch from a committed rocprofv3 FETCH_SIZE/WRITE_SIZE record (copy-calibrated), or
    None when the kernel's sources changed since the counters were taken."""
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "source_sha256_16: ")))
    if fields.get("source_sha256_16") != source_hash(*sources):
        return None
    return int(fields["traffic_bytes_per_launch"])


def mx_weights(abi, torch, dims, w, fp8=False):
    """MXFP4 (moe_q4_to_mxfp4) or MXFP8 (moe_q4_to_mxfp8) copies of one layer copy's packed Q4 stacks."""
    shapes = {"w13": (dims.E, 2 * dims.I, dims.d), "w2": (dims.E, dims.d, dims.I),
              "s13": (1, 2 * dims.I_shared, dims.d), "s2": (1, dims.d, dims.I_shared)}
    mx = {}
    requant = abi.moe_q4_to_mxfp8 if fp8 else abi.moe_q4_to_mxfp4
    for name, (n, rows, K) in shapes.items():
        codes = torch.empty(w[name + "_qs"].numel() * (2 if fp8 else 1), dtype=torch.uint8, device="cuda")
        exps = torch.empty(n * rows * (K // 32), dtype=torch.uint8, device=codes.device)
        requant(n, rows, K, w[name + "_qs"], w[name + "_sc"], codes, exps)
        mx[name + "_codes"], mx[name + "_exps"] = codes, exps
    return mx


def run_workload(name, steps, warmup, torch, hip, abi, layer, synth, oracle_sample=False, residual=False,
                 separate=False, variant="w4a16"):
    cfg = synth.CONFIGS[name]
    dims = cfg.dims
    device = "cuda"
    L = COPIES[name]
    # one layer call: moe_layer_forward, or with `separate` moe_route + moe_build_descriptors + moe_q4_forward;
    # the W4A8 variant: moe_route + moe_build_descriptors + moe_w4a8_forward on MXFP4 copies of the weights
    call = layer.layer_call if separate else layer.layer_call_fused
    inp0 = synth.make_inputs(cfg)
    weights = [layer.DeviceWeights.upload(inp0)]
    xs = [layer.to_device(inp0["x"], device)]
    for c in range(1, L):
        x, w = device_copy(cfg, 7000 + 100 * c + cfg.index, torch, device)
        dw = layer.DeviceWeights()
        dw.update(w)
        dw.dims = dims
        weights.append(dw)
        xs.append(x)
    spaces = [layer.Workspace(dims, 0) for _ in range(L)]
    if variant in ("w4a8", "w8a8"):
        if abi.moe_path(dims, 0) != 1 or residual:
            raise ValueError("the fp8-activation variants run on the grouped path, without a residual")
        fp8w = variant == "w8a8"
        mxs = {id(w): mx_weights(abi, torch, dims, w, fp8w) for w in weights}
        scratch_bytes = abi.moe_w8a8_scratch_bytes if fp8w else abi.moe_w4a8_scratch_bytes
        fwd = abi.moe_w8a8_forward if fp8w else abi.moe_w4a8_forward
        fp8_scratch = {id(ws): torch.empty(scratch_bytes(dims, 0), dtype=torch.uint8, device=device) for ws in spaces}

        def call(x, w, ws, stream=None, residual=None):
            abi.moe_route(dims, x, w["w_router"], w["bias"], ws.topk_ids, ws.topk_w, ws.routing, stream=stream)
            abi.moe_build_descriptors(dims, ws.topk_ids, ws.routing, stream=stream)
            fwd(dims, x, ws.topk_ids, ws.topk_w, ws.routing, mxs[id(w)], ws.y, fp8_scratch[id(ws)], stream=stream)
    # with `residual`, every step goes through moe_q4_forward_residual with its own fp32 [T][d] residual
    res = [torch.randn(dims.T, dims.d, device=device) if residual else None for _ in range(L)]
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for c in range(L):  # eager pass: surfaces launch errors outside capture
            call(xs[c], weights[c], spaces[c], stream=sh, residual=res[c])
    torch.cuda.synchronize()

    def capture(copies):
        hip.begin_capture(sh)
        for c in copies:
            call(xs[c], weights[c], spaces[c], stream=sh, residual=res[c])
        g = hip.end_capture(sh)
        return g, hip.instantiate(g)

    full_graph, full_exec = capture(range(L))
    rem = steps % L
    rem_exec = capture(range(rem))[1] if rem else None

    def run_steps(n):
        for _ in range(n // L):
            hip.launch(full_exec, sh)
        if n % L:
            hip.launch(rem_exec if n % L == rem else capture(range(n % L))[1], sh)

    with torch.cuda.stream(stream):
        run_steps(warmup)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    run_steps(steps)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    ms_per_step = ms / steps

    # per-kernel average durations from graphs of that kernel's nodes alone.  This needs every launch of
    # the layer to be idempotent: replayed alone, a kernel must rewrite the same values (a launch that
    # accumulated into state cleared by an earlier one would corrupt what later replays read).
    nodes = hip.kernel_nodes(full_graph, sh)
    by_kernel = {}
    for kname, p in nodes:
        by_kernel.setdefault(short_name(kname), []).append(p)
    kernel_us = {}
    reps = 50
    for kname, plist in by_kernel.items():
        ex = hip.instantiate(hip.chain_graph(plist))
        with torch.cuda.stream(stream):
            for _ in range(2):
                hip.launch(ex, sh)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            hip.launch(ex, sh)
        b.record(stream)
        torch.cuda.synchronize()
        kernel_us[kname] = a.elapsed_time(b) * 1000.0 / (reps * len(plist))

    # routing statistics of copy 0 (distinct experts decide the bytes a call must read)
    ids = spaces[0].topk_ids.cpu().numpy()
    distinct = int(np.unique(ids).size)
    sizes = np.bincount(ids.ravel(), minlength=dims.E)
    group_stats = {"max": int(sizes.max()), "median": float(np.median(sizes)), "min": int(sizes.min()),
                   "empty": int((sizes == 0).sum())}
    gu, dn, sgu, sdn = expert_bytes(dims, variant)
    T, d, E, P = dims.T, dims.d, dims.E, dims.T * dims.k
    layer_bytes = (E * d * 4 + E * 4 + T * d * 2 + distinct * (gu + dn) + (sgu + sdn) + T * d * 4
                   + P * 8)
    router, routed, shared = layer_flops(dims)
    layer_flop = router + routed + shared
    path = abi.moe_path(dims, 0)
    tokens_per_s = T / (ms_per_step / 1000.0)
    res = {
        "workload": name, "variant": variant, "residual": bool(residual),
        "dims": dict(T=T, d=d, E=E, k=dims.k, I=dims.I, I_shared=dims.I_shared),
        "path": "gemv" if path == 0 else "grouped", "layer_copies": L, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "tokens_per_s": tokens_per_s, "distinct_experts": distinct,
        "group_rows": group_stats,
        "kernel_avg_us": {k: round(v, 3) for k, v in kernel_us.items()},
        "layer_algorithmic_bytes": layer_bytes, "layer_algorithmic_flop": layer_flop,
        "layer_hbm_frac": layer_bytes / (ms_per_step / 1000.0) / (HBM_PEAK_GBS * 1e9),
        "layer_mfma_frac": layer_flop / (ms_per_step / 1000.0) / (MFMA_F16_PEAK_TFLOPS * 1e12),
    }
    if path == 0:
        kname = "gemv_gateup"
        per_launch = T * dims.k * gu + T * sgu + T * d * 2 + (P * dims.I + T * dims.I_shared) * 2
        achieved = per_launch / (kernel_us[kname] * 1e-6) / 1e9
        res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": recorded_traffic("gemv_gateup_decode_T1_traffic.md", GEMV_SOURCES)
                           if name == "decode" else None,
                           "algorithmic_bytes_per_launch": per_launch,
                           "avg_launch_us": round(kernel_us[kname], 3)}
    elif variant in ("w4a8", "w8a8"):
        # At this size the block-scaled fp8 MFMA work (~75 us at the fp8 peak) is well under the weight
        # stream (~140 us at 8 TB/s): the kernel is HBM-bound.  Algorithmic bytes: the codes and block
        # exponents of every expert touched plus the shared expert, x in fp8 once, h written in fp16.
        kname = "grouped_mx_gateup"
        cb = 0.5 if variant == "w4a8" else 1.0  # code bytes per weight
        gu_w = 2 * dims.I * d * (cb + 1 / 32)
        sgu_w = 2 * dims.I_shared * d * (cb + 1 / 32)
        per_launch = int(distinct * gu_w + sgu_w + T * d + T * 4 + (P * dims.I + T * dims.I_shared) * 2)
        flop = 2 * (P * 2 * dims.I + T * 2 * dims.I_shared) * d
        sec_ = kernel_us[kname] * 1e-6
        achieved = per_launch / sec_ / 1e9
        res["roofline"] = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": recorded_traffic(f"grouped_mx_gateup_{variant}_prefill_T2048_traffic.md",
                                                       MX_SOURCES) if name == "prefill" else None,
                           "algorithmic_bytes_per_launch": per_launch, "avg_launch_us": round(kernel_us[kname], 3),
                           "mfma_tflops": round(flop / sec_ / 1e12, 1),
                           "mfma_frac_fp8": round(flop / sec_ / 1e12 / MFMA_F8_PEAK_TFLOPS, 4)}
        res["layer_mfma_frac_fp8"] = layer_flop / (ms_per_step / 1000.0) / (MFMA_F8_PEAK_TFLOPS * 1e12)
    else:
        kname = "grouped_gateup"
        per_launch = 2 * (P * 2 * dims.I + T * 2 * dims.I_shared) * d
        achieved = per_launch / (kernel_us[kname] * 1e-6) / 1e12
        res["roofline"] = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                           "traffic": recorded_traffic("grouped_gateup_prefill_T2048_traffic.md", GROUPED_SOURCES)
                           if name == "prefill" else None,
                           "algorithmic_flop_per_launch": per_launch, "avg_launch_us": round(kernel_us[kname], 3)}
    res["_inp0"] = inp0
    return res


def copy_ceiling(torch, nbytes_list):
    """GB/s (bytes read + bytes written, per second) of torch's device-to-device copy kernel at the given
    total byte counts: the practical streaming ceiling beside the nominal HBM peak.  Buffers rotate through
    1 GiB windows so that repeated copies do not hit the 256 MB MALL."""
    out = {}
    pool = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    for nbytes in nbytes_list:
        half = (nbytes // 2) & ~4095
        nwin = (1 << 30) // half
        reps = 40
        srcs = [pool[i * half:(i + 1) * half] for i in range(nwin)]
        dsts = [pool[(1 << 30) + i * half:(1 << 30) + (i + 1) * half] for i in range(nwin)]
        for i in range(3):
            dsts[i % nwin].copy_(srcs[i % nwin])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            dsts[(i + 3) % nwin].copy_(srcs[(i + 3) % nwin])
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1000.0 / reps
        out[str(2 * half)] = {"us": round(us, 2), "gbs": round(2 * half / (us * 1e-6) / 1e9, 1)}
    del pool
    return out


def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        import threadpoolctl
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpoolctl.threadpool_info()
                if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or blas
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "blas": blas}


def cpu_baseline(inp, budget_s=15.0):
    """The oracle as it stands, on the host, on a bounded sample of the primary workload's tokens."""
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    T = inp["dims"].T
    done, t0 = 0, time.perf_counter()
    calls = 0
    while True:
        tokens = np.arange(T) if T <= 16 else np.arange(16) + (16 * calls) % max(T - 16, 1)
        oracle.forward(inp, tokens=tokens)
        done += len(tokens)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 50:
            break
    return {"value": round(done / el, 4), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} oracle layer calls of {len(tokens)} token(s) each on the workload's layer copy 0, "
                      f"{el:.1f} s wall on the host", **host_info()}


def traffic_run(name, torch, layer, synth, flags=0, variant="w4a16"):
    """Three layer calls and two 256 MiB copies, nothing else: the run that rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE records for the traffic summaries under profiles/ (the copy calibrates the counters).
    `flags` are the layer's MOE_FLAG_* bits (e.g. the grouped GEMMs' work order); `variant` w4a8 runs
    moe_route + moe_build_descriptors + moe_w4a8_forward on MXFP4 copies of the weights instead, w8a8
    moe_w8a8_forward on MXFP8 copies."""
    from sparse_moe_expert_sigmoid_amd import abi
    inp = synth.make_inputs(synth.CONFIGS[name])
    dims = inp["dims"]
    w = layer.DeviceWeights.upload(inp)
    x = layer.to_device(inp["x"], "cuda")
    ws = layer.Workspace(dims, flags)
    if variant != "w4a16":
        fp8w = variant == "w8a8"
        mx = mx_weights(abi, torch, dims, w, fp8w)
        scratch = torch.empty((abi.moe_w8a8_scratch_bytes if fp8w else abi.moe_w4a8_scratch_bytes)(dims, flags),
                              dtype=torch.uint8, device="cuda")
        fwd = abi.moe_w8a8_forward if fp8w else abi.moe_w4a8_forward
    for _ in range(3):
        if variant != "w4a16":
            abi.moe_route(dims, x, w["w_router"], w["bias"], ws.topk_ids, ws.topk_w, ws.routing, flags=flags)
            abi.moe_build_descriptors(dims, ws.topk_ids, ws.routing, flags=flags)
            fwd(dims, x, ws.topk_ids, ws.topk_w, ws.routing, mx, ws.y, scratch, flags=flags)
        else:
            layer.layer_call_fused(x, w, ws)
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": name, "variant": variant, "flags": flags, "layer_calls": 3,
                      "copy_bytes": 256 << 20, "copies": 2}), flush=True)


def run_decode_ctx(passes, torch, abi, layer, synth, n_layers=8, norm=False):
    """The single-token decode layer as a stack of n_layers independent layer copies recorded once by the
    library (moe_decode_ctx_*): a pass takes a residual stream h through every layer (x = bf16(h), or
    with `norm` x = bf16(rmsnorm(h) * gamma), then h = layer(x) + h).  Without the norm nothing keeps the
    stream's scale, so every timed pass starts again from the same small h0 (a 16 KiB device copy, timed
    alone and subtracted; done the same way with the norm)."""
    cfg = synth.CONFIGS["decode"]
    dims = cfg.dims
    weights = [layer.DeviceWeights.upload(synth.make_inputs(cfg))]
    for c in range(1, n_layers):
        _, w = device_copy(cfg, 7000 + 100 * c + cfg.index, torch, "cuda")
        dw = layer.DeviceWeights()
        dw.update(w)
        weights.append(dw)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    if norm:
        for w in weights:
            w["norm_weight"] = torch.rand(dims.d, device="cuda", generator=g) + 0.5
            w["norm_eps"] = 1e-6
    h0 = torch.randn((dims.T, dims.d), device="cuda", generator=g) * 0.1
    h = h0.clone()
    ctx = layer.DecodeContext(dims, weights, h)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        def timed(n, with_ctx):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(n):
                h.copy_(h0)
                if with_ctx:
                    ctx.run(stream)
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1000.0 / n
        timed(max(4, passes // 10), True)
        total = timed(passes, True)
        reset = timed(passes, False)
    finite = bool(torch.isfinite(h).all().item())
    ctx.close()
    per_pass = total - reset
    return {"workload": f"decode stack: {n_layers} layers of T=1 d={dims.d} E={dims.E} top-{dims.k} I={dims.I}"
                        + (", pre-MoE RMSNorm" if norm else ""),
            "layers": n_layers, "passes": passes, "us_per_pass": round(per_pass, 3),
            "us_per_layer": round(per_pass / n_layers, 3), "reset_copy_us": round(reset, 3),
            "tokens_per_s_per_layer": round(1e6 / (per_pass / n_layers), 1), "stream_finite": finite}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--workload", default="decode", choices=["decode", "batched_decode", "prefill", "long_prefill"])
    ap.add_argument("--secondary", default="prefill", help="second workload reported alongside ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-w4a8", action="store_true",
                    help="skip the W4A8 / W8A8 variants (MXFP4 / MXFP8 weights x FP8 activations) of the "
                         "secondary workload")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time each layer as moe_route + moe_build_descriptors + moe_q4_forward instead of "
                         "moe_layer_forward (the same results)")
    ap.add_argument("--residual", action="store_true",
                    help="every step uses moe_q4_forward_residual (adds an fp32 [T][d] residual after the layer)")
    ap.add_argument("--all", action="store_true",
                    help="measure every workload (tiny excluded) and print one JSON line with a list of them")
    ap.add_argument("--traffic-run", metavar="WORKLOAD", default=None,
                    help="for hardware-counter collection only: run WORKLOAD's layer 3 times, then copy a 256 MiB "
                         "device buffer twice (the calibration of FETCH_SIZE / WRITE_SIZE), print one line, exit")
    ap.add_argument("--flags", type=int, default=0,
                    help="MOE_FLAG_* bits for --traffic-run (4 = expert-id group order, 8 = items in launch "
                         "order, 16 = band-major items)")
    ap.add_argument("--variant", default="w4a16", choices=["w4a16", "w4a8", "w8a8"],
                    help="layer variant of --traffic-run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this layer is built and measured on a single MI355X; "
              "multi-GPU (expert-parallel) runs are not part of it. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from sparse_moe_expert_sigmoid_amd import abi, layer
    abi.lib()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    if args.traffic_run:
        traffic_run(args.traffic_run, torch, layer, synth, flags=args.flags, variant=args.variant)
        return
    hip = Hip()
    if args.all:
        rows = []
        for wl, n in (("decode", args.steps), ("batched_decode", max(40, args.steps // 8)),
                      ("prefill", max(20, args.steps // 40)), ("long_prefill", max(10, args.steps // 80))):
            r = run_workload(wl, n, max(4, n // 10), torch, hip, abi, layer, synth, residual=args.residual,
                             separate=args.separate_calls)
            r.pop("_inp0", None)
            rows.append(r)
            print(f"[bench] {wl}: {r['ms_per_step'] * 1000:.1f} us/step, {r['tokens_per_s']:.0f} tokens/s",
                  file=sys.stderr, flush=True)
        ctx = run_decode_ctx(max(50, args.steps // 4), torch, abi, layer, synth)
        ctxn = run_decode_ctx(max(50, args.steps // 4), torch, abi, layer, synth, norm=True)
        print(f"[bench] decode stack context: {ctx['us_per_layer']:.1f} us/layer, with the norm "
              f"{ctxn['us_per_layer']:.1f}", file=sys.stderr, flush=True)
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "workloads": rows, "decode_ctx": ctx, "decode_ctx_norm": ctxn,
                          "copy_ceiling": copy_ceiling(torch, [52 << 20, 1 << 30])}), flush=True)
        return
    prim = run_workload(args.workload, args.steps, args.warmup, torch, hip, abi, layer, synth,
                        residual=args.residual, separate=args.separate_calls)
    sec = None
    if args.secondary and args.secondary != "none" and args.secondary != args.workload:
        n = max(20, args.steps // 40)
        sec = run_workload(args.secondary, n, max(4, n // 10), torch, hip, abi, layer, synth, residual=args.residual,
                           separate=args.separate_calls)
    fp8act = {}
    if sec is not None and not args.no_w4a8 and abi.moe_path(synth.CONFIGS[args.secondary].dims, 0) == 1:
        n = max(20, args.steps // 40)
        for v in ("w4a8", "w8a8"):
            fp8act[v] = run_workload(args.secondary, n, max(4, n // 10), torch, hip, abi, layer, synth, variant=v)
            fp8act[v].pop("_inp0", None)
    ctx = run_decode_ctx(max(50, args.steps // 4), torch, abi, layer, synth) if args.workload == "decode" else None
    ctxn = (run_decode_ctx(max(50, args.steps // 4), torch, abi, layer, synth, norm=True)
            if args.workload == "decode" else None)
    rl = prim["roofline"]
    if rl["unit"] == "GB/s":  # measured right after the GPU work, before the host-only oracle timing
        ceil = copy_ceiling(torch, [rl["algorithmic_bytes_per_launch"]])
        rl["copy_ceiling"] = next(iter(ceil.values())) | {"bytes": int(next(iter(ceil)))}
    cpu = None if args.no_cpu_baseline else cpu_baseline(prim["_inp0"])
    if sec is not None and not args.no_cpu_baseline:  # the oracle on the secondary workload too (one sample)
        sec["cpu_baseline"] = cpu_baseline(sec["_inp0"], budget_s=10.0)
    dims = prim["dims"]
    out = {
        "metric": METRIC,
        "value": round(prim["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; Q4 codes uniform, fp16 scales U(0.005,0.02), x N(0,1) bf16)",
        "config": {"workload": f"{args.workload}: T={dims['T']} d={dims['d']} E={dims['E']} top-{dims['k']} "
                               f"I={dims['I']} shared I={dims['I_shared']} Q4 block-32",
                   "path": prim["path"], "layer_copies": prim["layer_copies"], "parallelism": "single GPU",
                   "residual": bool(args.residual)},
        "roofline": prim["roofline"],
        "cpu_baseline": cpu,
        "layer": {k: prim[k] for k in ("layer_hbm_frac", "layer_mfma_frac", "layer_algorithmic_bytes",
                                       "layer_algorithmic_flop", "distinct_experts", "kernel_avg_us")},
        "kernel_sources": source_hash("sparse_moe_expert_sigmoid_amd/csrc/gemv.hip",
                                      "sparse_moe_expert_sigmoid_amd/csrc/grouped.hip",
                                      "sparse_moe_expert_sigmoid_amd/csrc/w4a8.hip"),
    }
    if sec is not None:
        sec.pop("_inp0", None)
        out["secondary"] = sec
    for v, r in fp8act.items():
        out["secondary_" + v] = r
    if ctx is not None:
        out["decode_ctx"] = ctx
        out["decode_ctx_norm"] = ctxn
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
