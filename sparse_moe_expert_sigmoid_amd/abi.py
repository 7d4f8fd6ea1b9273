"""ctypes binding of libmoe_q4.so: the C ABI of include/moe_q4.h, argument marshalling only.

Array arguments may be torch tensors (their ``data_ptr()`` is passed) or raw
integer device addresses.  ``stream=None`` means torch's current stream on
the current device.  Every call raises MoeError on a non-zero return code
unless ``check=False``, in which case the code is returned.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_size_t, c_uint32, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_Q4_LIB names another build of the same library (the host-sanitized one the CPU tests load)
lib_path = os.environ.get("MOE_Q4_LIB") or os.path.join(HERE, "libmoe_q4.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED, MOE_ENOSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5
MOE_FLAG_DEFAULT = 0
MOE_FLAG_FORCE_GROUPED = 1
MOE_FLAG_FORCE_GEMV = 2
MOE_FLAG_ID_ORDER = 4
MOE_FLAG_NO_BANDING = 8
MOE_FLAG_BAND_MAJOR = 16
MOE_GEMV_MAX_T = 8
MOE_GEMV_FORCE_MAX_T = 64

EXPORTED_SYMBOLS = (
    "moe_supports", "moe_path", "moe_routing_bytes", "moe_routing_layout_of", "moe_scratch_bytes",
    "moe_route", "moe_build_descriptors", "moe_q4_forward", "moe_q4_forward_residual", "moe_layer_forward", "moe_strerror",
    "moe_decode_ctx_workspace_bytes", "moe_decode_ctx_create", "moe_decode_ctx_run", "moe_decode_ctx_destroy",
    "moe_rmsnorm_bf16", "moe_q4_pack", "moe_layer_forward_noalloc",
    "moe_q4_to_mxfp4", "moe_q4_to_mxfp8", "moe_rows_to_fp8", "moe_w4a8_scratch_bytes", "moe_w8a8_scratch_bytes",
    "moe_w4a8_forward", "moe_w8a8_forward",
)
MOE_NOALLOC_MAX_BYTES = 64 << 20


class Dims(Structure):
    _fields_ = [("T", c_int32), ("d", c_int32), ("E", c_int32), ("k", c_int32), ("I", c_int32),
                ("I_shared", c_int32)]

    @classmethod
    def of(cls, dims) -> "Dims":
        if isinstance(dims, Dims):
            return dims
        return cls(dims.T, dims.d, dims.E, dims.k, dims.I, dims.I_shared)


class _Q4(Structure):
    _fields_ = [("qs", c_void_p), ("scales", c_void_p)]


class _Weights(Structure):
    _fields_ = [("w13", _Q4), ("w2", _Q4), ("s13", _Q4), ("s2", _Q4)]


class _Mx(Structure):
    _fields_ = [("codes", c_void_p), ("exps", c_void_p)]


class _MxWeights(Structure):
    _fields_ = [("w13", _Mx), ("w2", _Mx), ("s13", _Mx), ("s2", _Mx)]


class _Layer(Structure):
    _fields_ = [("w_router", c_void_p), ("bias", c_void_p), ("weights", _Weights), ("norm_weight", c_void_p),
                ("norm_eps", c_float)]


_LAYOUT_FIELDS = ("logits", "counts", "offsets", "sorted_pair", "pair_pos", "row_expert", "group_order",
                  "mt_prefix", "chunk_counts", "total")


class RoutingLayout(Structure):
    _fields_ = [(n, c_size_t) for n in _LAYOUT_FIELDS]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n in _LAYOUT_FIELDS}


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {moe_strerror(code)} ({code})" if what else f"{moe_strerror(code)} ({code})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with `python -m sparse_moe_expert_sigmoid_amd.build`")
    L = ctypes.CDLL(lib_path)
    D = POINTER(Dims)
    L.moe_supports.argtypes = [D, c_uint32]
    L.moe_supports.restype = c_int
    L.moe_path.argtypes = [D, c_uint32]
    L.moe_path.restype = c_int
    L.moe_routing_bytes.argtypes = [D, c_uint32]
    L.moe_routing_bytes.restype = c_size_t
    L.moe_routing_layout_of.argtypes = [D, c_uint32, POINTER(RoutingLayout)]
    L.moe_routing_layout_of.restype = c_int
    L.moe_scratch_bytes.argtypes = [D, c_uint32]
    L.moe_scratch_bytes.restype = c_size_t
    L.moe_route.argtypes = [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_uint32,
                            c_void_p]
    L.moe_route.restype = c_int
    L.moe_build_descriptors.argtypes = [D, c_void_p, c_void_p, c_size_t, c_uint32, c_void_p]
    L.moe_build_descriptors.restype = c_int
    L.moe_q4_forward.argtypes = [D, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, POINTER(_Weights), c_void_p,
                                 c_void_p, c_size_t, c_uint32, c_void_p]
    L.moe_q4_forward.restype = c_int
    L.moe_q4_forward_residual.argtypes = [D, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, POINTER(_Weights),
                                          c_void_p, c_void_p, c_void_p, c_size_t, c_uint32, c_void_p]
    L.moe_q4_forward_residual.restype = c_int
    L.moe_layer_forward.argtypes = [D, c_void_p, c_void_p, c_void_p, POINTER(_Weights), c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p, c_size_t, c_uint32, c_void_p]
    L.moe_layer_forward.restype = c_int
    L.moe_decode_ctx_workspace_bytes.argtypes = [D, c_uint32]
    L.moe_decode_ctx_workspace_bytes.restype = c_size_t
    L.moe_decode_ctx_create.argtypes = [D, c_int, POINTER(_Layer), c_void_p, c_void_p, c_size_t, c_uint32,
                                        POINTER(c_void_p)]
    L.moe_decode_ctx_create.restype = c_int
    L.moe_decode_ctx_run.argtypes = [c_void_p, c_void_p]
    L.moe_decode_ctx_run.restype = c_int
    L.moe_decode_ctx_destroy.argtypes = [c_void_p]
    L.moe_decode_ctx_destroy.restype = c_int
    L.moe_rmsnorm_bf16.argtypes = [c_int, c_int, c_void_p, c_void_p, c_float, c_void_p, c_void_p]
    L.moe_rmsnorm_bf16.restype = c_int
    L.moe_layer_forward_noalloc.argtypes = [D, c_void_p, c_void_p, c_void_p, POINTER(_Weights), c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_uint32, c_void_p]
    L.moe_layer_forward_noalloc.restype = c_int
    L.moe_q4_pack.argtypes = [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.moe_q4_pack.restype = c_int
    for name in ("moe_q4_to_mxfp4", "moe_q4_to_mxfp8"):
        getattr(L, name).argtypes = [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        getattr(L, name).restype = c_int
    L.moe_rows_to_fp8.argtypes = [c_int32, c_int32, c_void_p, c_int, c_void_p, c_void_p, c_void_p]
    L.moe_rows_to_fp8.restype = c_int
    for v in ("w4a8", "w8a8"):
        getattr(L, f"moe_{v}_scratch_bytes").argtypes = [D, c_uint32]
        getattr(L, f"moe_{v}_scratch_bytes").restype = c_size_t
        getattr(L, f"moe_{v}_forward").argtypes = [D, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                                   POINTER(_MxWeights), c_void_p, c_void_p, c_size_t, c_uint32,
                                                   c_void_p]
        getattr(L, f"moe_{v}_forward").restype = c_int
    L.moe_strerror.argtypes = [c_int]
    L.moe_strerror.restype = c_char_p
    _lib = L
    return L


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _nbytes(a, given):
    if given is not None:
        return given
    if a is None or isinstance(a, int):
        return 0
    return a.numel() * a.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _done(rc: int, check: bool, what: str) -> int:
    if rc != MOE_OK and check:
        raise MoeError(rc, what)
    return rc


def moe_strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def moe_supports(dims, flags: int = 0) -> int:
    return lib().moe_supports(ctypes.byref(Dims.of(dims)), flags)


def moe_path(dims, flags: int = 0) -> int:
    return lib().moe_path(ctypes.byref(Dims.of(dims)), flags)


def moe_routing_bytes(dims, flags: int = 0) -> int:
    return lib().moe_routing_bytes(ctypes.byref(Dims.of(dims)), flags)


def moe_routing_layout_of(dims, flags: int = 0) -> dict:
    out = RoutingLayout()
    rc = lib().moe_routing_layout_of(ctypes.byref(Dims.of(dims)), flags, ctypes.byref(out))
    _done(rc, True, "moe_routing_layout_of")
    return out.as_dict()


def moe_scratch_bytes(dims, flags: int = 0) -> int:
    return lib().moe_scratch_bytes(ctypes.byref(Dims.of(dims)), flags)


def moe_route(dims, x, w_router, bias, topk_ids, topk_w, routing, routing_bytes=None, flags: int = 0,
              stream=None, check: bool = True) -> int:
    rc = lib().moe_route(ctypes.byref(Dims.of(dims)), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_ids),
                         _ptr(topk_w), _ptr(routing), _nbytes(routing, routing_bytes), flags, _stream(stream))
    return _done(rc, check, "moe_route")


def moe_build_descriptors(dims, topk_ids, routing, routing_bytes=None, flags: int = 0, stream=None,
                          check: bool = True) -> int:
    rc = lib().moe_build_descriptors(ctypes.byref(Dims.of(dims)), _ptr(topk_ids), _ptr(routing),
                                     _nbytes(routing, routing_bytes), flags, _stream(stream))
    return _done(rc, check, "moe_build_descriptors")


def _weights(w) -> _Weights:
    """w: mapping with w13_qs, w13_sc, w2_qs, w2_sc, s13_qs, s13_sc, s2_qs, s2_sc."""
    return _Weights(_Q4(_ptr(w["w13_qs"]), _ptr(w["w13_sc"])), _Q4(_ptr(w["w2_qs"]), _ptr(w["w2_sc"])),
                    _Q4(_ptr(w["s13_qs"]), _ptr(w["s13_sc"])), _Q4(_ptr(w["s2_qs"]), _ptr(w["s2_sc"])))


def moe_q4_forward(dims, x, topk_ids, topk_w, routing, weights, y, scratch, routing_bytes=None,
                   scratch_bytes=None, flags: int = 0, stream=None, check: bool = True) -> int:
    ws = weights if isinstance(weights, _Weights) else _weights(weights)
    rc = lib().moe_q4_forward(ctypes.byref(Dims.of(dims)), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(routing),
                              _nbytes(routing, routing_bytes), ctypes.byref(ws), _ptr(y), _ptr(scratch),
                              _nbytes(scratch, scratch_bytes), flags, _stream(stream))
    return _done(rc, check, "moe_q4_forward")


def moe_q4_forward_residual(dims, x, topk_ids, topk_w, routing, weights, residual, y, scratch, routing_bytes=None,
                            scratch_bytes=None, flags: int = 0, stream=None, check: bool = True) -> int:
    ws = weights if isinstance(weights, _Weights) else _weights(weights)
    rc = lib().moe_q4_forward_residual(ctypes.byref(Dims.of(dims)), _ptr(x), _ptr(topk_ids), _ptr(topk_w),
                                       _ptr(routing), _nbytes(routing, routing_bytes), ctypes.byref(ws),
                                       _ptr(residual), _ptr(y), _ptr(scratch), _nbytes(scratch, scratch_bytes),
                                       flags, _stream(stream))
    return _done(rc, check, "moe_q4_forward_residual")


def moe_layer_forward(dims, x, w_router, bias, weights, y, topk_ids, topk_w, routing, scratch, residual=None,
                      routing_bytes=None, scratch_bytes=None, flags: int = 0, stream=None, check: bool = True) -> int:
    ws = weights if isinstance(weights, _Weights) else _weights(weights)
    rc = lib().moe_layer_forward(ctypes.byref(Dims.of(dims)), _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(ws),
                                 _ptr(residual), _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(routing),
                                 _nbytes(routing, routing_bytes), _ptr(scratch), _nbytes(scratch, scratch_bytes),
                                 flags, _stream(stream))
    return _done(rc, check, "moe_layer_forward")


def moe_decode_ctx_workspace_bytes(dims, flags: int = 0) -> int:
    return lib().moe_decode_ctx_workspace_bytes(ctypes.byref(Dims.of(dims)), flags)


def _layer(layer) -> _Layer:
    """layer: mapping with w_router, bias and the Q4 weight arrays (as for moe_q4_forward), and optionally
    norm_weight (gamma of the pre-MoE norm) with norm_eps."""
    return _Layer(_ptr(layer["w_router"]), _ptr(layer["bias"]), _weights(layer), _ptr(layer.get("norm_weight")),
                  float(layer.get("norm_eps", 0.0)))


def moe_decode_ctx_create(dims, layers, h, workspace, workspace_bytes=None, flags: int = 0,
                          check: bool = True):
    """Returns the context handle (an int), or (when check=False) the return code if creation failed."""
    arr = (_Layer * max(len(layers), 1))(*[_layer(l) for l in layers])
    out = c_void_p()
    rc = lib().moe_decode_ctx_create(ctypes.byref(Dims.of(dims)), len(layers), arr, _ptr(h), _ptr(workspace),
                                     _nbytes(workspace, workspace_bytes), flags, ctypes.byref(out))
    if rc != MOE_OK:
        _done(rc, check, "moe_decode_ctx_create")
        return rc
    return out.value


def moe_decode_ctx_run(ctx: int, stream=None, check: bool = True) -> int:
    return _done(lib().moe_decode_ctx_run(ctx, _stream(stream)), check, "moe_decode_ctx_run")


def moe_decode_ctx_destroy(ctx) -> int:
    return lib().moe_decode_ctx_destroy(ctx)


def moe_rmsnorm_bf16(T: int, d: int, h, gamma, eps: float, x, stream=None, check: bool = True) -> int:
    rc = lib().moe_rmsnorm_bf16(T, d, _ptr(h), _ptr(gamma), float(eps), _ptr(x), _stream(stream))
    return _done(rc, check, "moe_rmsnorm_bf16")


def moe_q4_pack(n_mats: int, rows: int, K: int, qs_in, scales_in, qs_out, scales_out, stream=None,
                check: bool = True) -> int:
    """Row-major Q4 codes [n_mats][rows][K/2] and scales [n_mats][rows][K/32] -> the library's 16-row
    groups, on the device (out of place)."""
    rc = lib().moe_q4_pack(n_mats, rows, K, _ptr(qs_in), _ptr(scales_in), _ptr(qs_out), _ptr(scales_out),
                           _stream(stream))
    return _done(rc, check, "moe_q4_pack")


def moe_layer_forward_noalloc(dims, x, w_router, bias, weights, y, topk_ids, topk_w, residual=None, flags: int = 0,
                              stream=None, check: bool = True) -> int:
    """moe_layer_forward with the routing workspace and scratch in the library's own device array."""
    ws = weights if isinstance(weights, _Weights) else _weights(weights)
    rc = lib().moe_layer_forward_noalloc(ctypes.byref(Dims.of(dims)), _ptr(x), _ptr(w_router), _ptr(bias),
                                         ctypes.byref(ws), _ptr(residual), _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                         flags, _stream(stream))
    return _done(rc, check, "moe_layer_forward_noalloc")


def moe_q4_to_mxfp4(n_mats: int, rows: int, K: int, qs, scales, codes_out, exps_out, stream=None,
                    check: bool = True) -> int:
    """Q4 blocks -> MXFP4 blocks (16 bytes of e2m1 codes, biased block exponents), block for block."""
    rc = lib().moe_q4_to_mxfp4(n_mats, rows, K, _ptr(qs), _ptr(scales), _ptr(codes_out), _ptr(exps_out),
                               _stream(stream))
    return _done(rc, check, "moe_q4_to_mxfp4")


def moe_q4_to_mxfp8(n_mats: int, rows: int, K: int, qs, scales, codes_out, exps_out, stream=None,
                    check: bool = True) -> int:
    """Q4 blocks -> MXFP8 blocks (32 bytes of e4m3 codes, biased block exponents), block for block."""
    rc = lib().moe_q4_to_mxfp8(n_mats, rows, K, _ptr(qs), _ptr(scales), _ptr(codes_out), _ptr(exps_out),
                               _stream(stream))
    return _done(rc, check, "moe_q4_to_mxfp8")


def moe_rows_to_fp8(rows: int, K: int, x, codes_out, scales_out, in_is_fp16: bool = False, stream=None,
                    check: bool = True) -> int:
    """Rows of bf16 (or fp16) bits -> e4m3 codes and fp32 row scales, on the device."""
    rc = lib().moe_rows_to_fp8(rows, K, _ptr(x), 1 if in_is_fp16 else 0, _ptr(codes_out), _ptr(scales_out),
                               _stream(stream))
    return _done(rc, check, "moe_rows_to_fp8")


def moe_w4a8_scratch_bytes(dims, flags: int = 0) -> int:
    return lib().moe_w4a8_scratch_bytes(ctypes.byref(Dims.of(dims)), flags)


def moe_w8a8_scratch_bytes(dims, flags: int = 0) -> int:
    return lib().moe_w8a8_scratch_bytes(ctypes.byref(Dims.of(dims)), flags)


def _mx_weights(w) -> _MxWeights:
    """w: mapping with w13_codes, w13_exps, w2_codes, w2_exps, s13_codes, s13_exps, s2_codes, s2_exps."""
    return _MxWeights(*[_Mx(_ptr(w[n + "_codes"]), _ptr(w[n + "_exps"])) for n in ("w13", "w2", "s13", "s2")])


def _fp8act_forward(variant, dims, x, topk_ids, topk_w, routing, weights, y, scratch, routing_bytes,
                    scratch_bytes, flags, stream, check):
    ws = weights if isinstance(weights, _MxWeights) else _mx_weights(weights)
    fn = getattr(lib(), f"moe_{variant}_forward")
    rc = fn(ctypes.byref(Dims.of(dims)), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(routing),
            _nbytes(routing, routing_bytes), ctypes.byref(ws), _ptr(y), _ptr(scratch), _nbytes(scratch, scratch_bytes),
            flags, _stream(stream))
    return _done(rc, check, f"moe_{variant}_forward")


def moe_w4a8_forward(dims, x, topk_ids, topk_w, routing, weights, y, scratch, routing_bytes=None,
                     scratch_bytes=None, flags: int = 0, stream=None, check: bool = True) -> int:
    """The W4A8 layer (MXFP4 weights from moe_q4_to_mxfp4, fp8 activations)."""
    return _fp8act_forward("w4a8", dims, x, topk_ids, topk_w, routing, weights, y, scratch, routing_bytes,
                           scratch_bytes, flags, stream, check)


def moe_w8a8_forward(dims, x, topk_ids, topk_w, routing, weights, y, scratch, routing_bytes=None,
                     scratch_bytes=None, flags: int = 0, stream=None, check: bool = True) -> int:
    """The W8A8 layer (MXFP8 weights from moe_q4_to_mxfp8, fp8 activations)."""
    return _fp8act_forward("w8a8", dims, x, topk_ids, topk_w, routing, weights, y, scratch, routing_bytes,
                           scratch_bytes, flags, stream, check)
