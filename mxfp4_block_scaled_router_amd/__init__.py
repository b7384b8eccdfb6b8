"""MXFP4 routed-expert MoE layer for MI355X (gfx950): Python binding.

A thin ctypes layer over ``libmxfp4_moe.so`` (C ABI in ``include/mxfp4_moe.h``).
Every function here only marshals arguments: device pointers of torch tensors,
shapes, and the current HIP stream.  All computation runs in the library's
HIP kernels; there is no fallback path.  If the library is missing the calls
raise ``MoEError``.

Build the library with ``python -m mxfp4_block_scaled_router_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxfp4_moe.so")

MXFP4_MOE_A4 = 0x1
MXFP4_MOE_DETERMINISTIC = 0x2
MXFP4_MOE_SHARED_EXPERT = 0x4
MXFP4_MOE_A8 = 0x8
MXFP4_MOE_ROUTE_LAUNCH = 0x10
DTYPE_BF16 = 0
DTYPE_F32 = 1

_lib = None


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = status_string(status) if _lib is not None else str(status)
        extra = ""
        if _lib is not None and name == "MXFP4_MOE_ERR_HIP":
            extra = " (hipError %d)" % _lib.mxfp4_moe_last_hip_error()
        super().__init__("%s failed: %s%s" % (fn, name, extra))
        self.status = status
        self.name = name


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E_global", ctypes.c_int64), ("E_local", ctypes.c_int64),
                ("first_local", ctypes.c_int64), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]

    @classmethod
    def make(cls, T, H, I, E_global, E_local=None, first_local=0, a4=False,
             deterministic=False, shared=False, a8=False, route_launch=False) -> "Dims":
        flags = ((MXFP4_MOE_A4 if a4 else 0) | (MXFP4_MOE_DETERMINISTIC if deterministic else 0)
                 | (MXFP4_MOE_SHARED_EXPERT if shared else 0) | (MXFP4_MOE_A8 if a8 else 0)
                 | (MXFP4_MOE_ROUTE_LAUNCH if route_launch else 0))
        return cls(T, H, I, E_global, E_global if E_local is None else E_local, first_local,
                   flags, 0)

    @property
    def shared(self) -> int:
        """1 when the weights carry the shared expert (one more slot per token)."""
        return 1 if self.flags & MXFP4_MOE_SHARED_EXPERT else 0


class Bf16Experts(ctypes.Structure):
    """mxfp4_moe_bf16_experts: the experts kept in bf16 (device pointers)."""
    _fields_ = [("n", ctypes.c_int64), ("expert_map", ctypes.c_void_p), ("w13", ctypes.c_void_p),
                ("w2", ctypes.c_void_p)]


EXPORTED = ("mxfp4_moe_abi_version", "mxfp4_moe_status_string", "mxfp4_moe_last_hip_error",
            "mxfp4_moe_preshuffled_bytes", "mxfp4_moe_preshuffle", "mxfp4_moe_workspace_bytes",
            "mxfp4_moe_forward", "mxfp4_moe_forward_debug", "mxfp4_moe_forward_timed",
            "mxfp4_moe_route", "mxfp4_moe_quantize", "mxfp4_moe_quantize8", "mxfp4_moe_plan",
            "mxfp4_moe_preshuffle_fused", "mxfp4_moe_forward_mixed", "mxfp4_moe_forward_noalloc",
            "mxfp4_moe_quantize_preshuffle")


def load_library(path: str = LIB_PATH):
    """Load libmxfp4_moe.so and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MoEError("load_library", -10**6)
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    lib.mxfp4_moe_abi_version.restype = ctypes.c_int
    lib.mxfp4_moe_abi_version.argtypes = []
    lib.mxfp4_moe_status_string.restype = ctypes.c_char_p
    lib.mxfp4_moe_status_string.argtypes = [ctypes.c_int]
    lib.mxfp4_moe_last_hip_error.restype = ctypes.c_int
    lib.mxfp4_moe_last_hip_error.argtypes = []
    lib.mxfp4_moe_preshuffled_bytes.restype = ctypes.c_int
    lib.mxfp4_moe_preshuffled_bytes.argtypes = [D, PSZ, PSZ, PSZ, PSZ]
    lib.mxfp4_moe_preshuffle.restype = ctypes.c_int
    lib.mxfp4_moe_preshuffle.argtypes = [D, P, P, P, P, P, P, P, P, P]
    lib.mxfp4_moe_workspace_bytes.restype = ctypes.c_int
    lib.mxfp4_moe_workspace_bytes.argtypes = [D, I32, PSZ]
    PI32 = ctypes.POINTER(ctypes.c_int32)
    lib.mxfp4_moe_plan.restype = ctypes.c_int
    lib.mxfp4_moe_plan.argtypes = [D, I32, PI32, PI32]
    lib.mxfp4_moe_forward.restype = ctypes.c_int
    lib.mxfp4_moe_forward.argtypes = [D, P, P, P, P, P, P, I32, ctypes.c_float, P, P, SZ, P]
    lib.mxfp4_moe_quantize_preshuffle.restype = ctypes.c_int
    lib.mxfp4_moe_quantize_preshuffle.argtypes = [D, P, P, I32, P, P, P, P, P]
    lib.mxfp4_moe_forward_noalloc.restype = ctypes.c_int
    lib.mxfp4_moe_forward_noalloc.argtypes = [D, P, P, P, P, P, P, I32, ctypes.c_float, P, P]
    lib.mxfp4_moe_forward_debug.restype = ctypes.c_int
    lib.mxfp4_moe_forward_debug.argtypes = [D, P, P, P, P, P, P, I32, ctypes.c_float, P, P, SZ,
                                            P, P, P, P, P, P, P]
    lib.mxfp4_moe_forward_timed.restype = ctypes.c_int
    lib.mxfp4_moe_forward_timed.argtypes = [D, P, P, P, P, P, P, I32, ctypes.c_float, P, P, SZ,
                                            P, P]
    lib.mxfp4_moe_route.restype = ctypes.c_int
    lib.mxfp4_moe_route.argtypes = [D, P, I32, P, P, P, P, P, P, P, SZ, P]
    lib.mxfp4_moe_quantize.restype = ctypes.c_int
    lib.mxfp4_moe_quantize.argtypes = [P, I32, I64, I64, P, P, P]
    lib.mxfp4_moe_quantize8.restype = ctypes.c_int
    lib.mxfp4_moe_quantize8.argtypes = [P, I32, I64, I64, P, P, P]
    lib.mxfp4_moe_preshuffle_fused.restype = ctypes.c_int
    lib.mxfp4_moe_preshuffle_fused.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.mxfp4_moe_forward_mixed.restype = ctypes.c_int
    lib.mxfp4_moe_forward_mixed.argtypes = [D, ctypes.POINTER(Bf16Experts), P, P, P, P, P, P, I32,
                                            ctypes.c_float, P, P, SZ, P, P, P, P, P, P, P]
    _lib = lib
    return lib


def _L():
    return load_library()


def status_string(status: int) -> str:
    return _L().mxfp4_moe_status_string(int(status)).decode()


def abi_version() -> int:
    return _L().mxfp4_moe_abi_version()


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, status):
    if status != 0:
        raise MoEError(fn, status)


def _dev_tensor(t, dtype, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError("%s must be a contiguous %s tensor on the GPU" % (name, dtype))
    return t


# ---------------------------------------------------------------- sizes

def mxfp4_moe_workspace_bytes(dims: Dims, top_k: int) -> int:
    out = ctypes.c_size_t()
    _check("mxfp4_moe_workspace_bytes",
           _L().mxfp4_moe_workspace_bytes(ctypes.byref(dims), int(top_k), ctypes.byref(out)))
    return out.value


def mxfp4_moe_plan(dims: Dims, top_k: int) -> dict:
    """How forward runs these dims: token rows per GEMM tile and whether the
    combine is the slot-ordered gather."""
    rows, ordered = ctypes.c_int32(), ctypes.c_int32()
    _check("mxfp4_moe_plan", _L().mxfp4_moe_plan(ctypes.byref(dims), int(top_k), ctypes.byref(rows),
                                                  ctypes.byref(ordered)))
    return {"tile_rows": rows.value, "ordered_combine": bool(ordered.value)}


def mxfp4_moe_preshuffled_bytes(dims: Dims):
    v = [ctypes.c_size_t() for _ in range(4)]
    _check("mxfp4_moe_preshuffled_bytes",
           _L().mxfp4_moe_preshuffled_bytes(ctypes.byref(dims), *[ctypes.byref(x) for x in v]))
    return tuple(x.value for x in v)


# ---------------------------------------------------------------- weights

def mxfp4_moe_preshuffle(dims: Dims, w13, w13s, w2, w2s):
    """Canonical MXFP4 expert weights (uint8 device tensors) -> preshuffled
    (w13, w13s, w2, w2s) uint8 device tensors."""
    for t, n in ((w13, "w13"), (w13s, "w13s"), (w2, "w2"), (w2s, "w2s")):
        _dev_tensor(t, torch.uint8, n)
    sizes = mxfp4_moe_preshuffled_bytes(dims)
    outs = [torch.empty(n, dtype=torch.uint8, device=w13.device) for n in sizes]
    _check("mxfp4_moe_preshuffle",
           _L().mxfp4_moe_preshuffle(ctypes.byref(dims), _p(w13), _p(w13s), _p(w2), _p(w2s),
                                     *[_p(o) for o in outs], _stream()))
    return tuple(outs)


def mxfp4_moe_quantize_preshuffle(dims: Dims, w13, w2):
    """Unquantised expert weights (float32 or bf16 device tensors, w13 [E, 2I, H],
    w2 [E, H, I]) -> preshuffled MXFP4 (w13, w13s, w2, w2s) in one pass."""
    in_dtype = DTYPE_BF16 if w13.dtype == torch.bfloat16 else DTYPE_F32
    want = torch.bfloat16 if in_dtype == DTYPE_BF16 else torch.float32
    _dev_tensor(w13, want, "w13")
    _dev_tensor(w2, want, "w2")
    sizes = mxfp4_moe_preshuffled_bytes(dims)
    outs = [torch.empty(n, dtype=torch.uint8, device=w13.device) for n in sizes]
    _check("mxfp4_moe_quantize_preshuffle",
           _L().mxfp4_moe_quantize_preshuffle(ctypes.byref(dims), _p(w13), _p(w2), int(in_dtype),
                                              *[_p(o) for o in outs], _stream()))
    return tuple(outs)


def mxfp4_moe_quantize(values, in_dtype: int | None = None):
    """OCP MX quantiser on the GPU: [..., K] bf16 or float32 -> (codes [..., K/2],
    scales [..., K/32]) canonical uint8 tensors."""
    if in_dtype is None:
        in_dtype = DTYPE_BF16 if values.dtype == torch.bfloat16 else DTYPE_F32
    want = torch.bfloat16 if in_dtype == DTYPE_BF16 else torch.float32
    _dev_tensor(values, want, "values")
    K = values.shape[-1]
    rows = values.numel() // K if K else 0
    codes = torch.empty(values.shape[:-1] + (K // 2,), dtype=torch.uint8, device=values.device)
    scales = torch.empty(values.shape[:-1] + (K // 32,), dtype=torch.uint8, device=values.device)
    _check("mxfp4_moe_quantize", _L().mxfp4_moe_quantize(_p(values), int(in_dtype), rows, K,
                                                        _p(codes), _p(scales), _stream()))
    return codes, scales


def mxfp4_moe_quantize8(values, in_dtype: int | None = None):
    """OCP MX quantiser with E4M3 elements on the GPU: [..., K] bf16 or float32 ->
    (codes [..., K] one byte each, scales [..., K/32]) uint8 tensors."""
    if in_dtype is None:
        in_dtype = DTYPE_BF16 if values.dtype == torch.bfloat16 else DTYPE_F32
    want = torch.bfloat16 if in_dtype == DTYPE_BF16 else torch.float32
    _dev_tensor(values, want, "values")
    K = values.shape[-1]
    rows = values.numel() // K if K else 0
    codes = torch.empty(values.shape, dtype=torch.uint8, device=values.device)
    scales = torch.empty(values.shape[:-1] + (K // 32,), dtype=torch.uint8, device=values.device)
    _check("mxfp4_moe_quantize8", _L().mxfp4_moe_quantize8(_p(values), int(in_dtype), rows, K,
                                                          _p(codes), _p(scales), _stream()))
    return codes, scales


# ---------------------------------------------------------------- layer

def _workspace(dims, top_k, workspace, device):
    need = mxfp4_moe_workspace_bytes(dims, top_k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def mxfp4_moe_forward(dims: Dims, x, router_logits, w13, w13s, w2, w2s, top_k: int,
                      clamp_limit: float, out=None, workspace=None):
    """The layer: x bf16 [T, H], router_logits float32 [T, E_global], preshuffled
    weights -> out bf16 [T, H]."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(router_logits, torch.float32, "router_logits")
    if out is None:
        out = torch.empty((dims.T, dims.H), dtype=torch.bfloat16, device=x.device)
    workspace, nbytes = _workspace(dims, top_k, workspace, x.device)
    _check("mxfp4_moe_forward",
           _L().mxfp4_moe_forward(ctypes.byref(dims), _p(x), _p(router_logits), _p(w13), _p(w13s),
                                  _p(w2), _p(w2s), int(top_k), float(clamp_limit), _p(out),
                                  _p(workspace), nbytes, _stream()))
    return out


def mxfp4_moe_forward_noalloc(dims: Dims, x, router_logits, w13, w13s, w2, w2s, top_k: int,
                              clamp_limit: float, out):
    """The layer without a workspace argument: the library's static per-GPU
    scratch serves as workspace, and the call allocates nothing (``out`` is
    required).  Calls that overlap on one GPU race on that scratch."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(router_logits, torch.float32, "router_logits")
    _dev_tensor(out, torch.bfloat16, "out")
    _check("mxfp4_moe_forward_noalloc",
           _L().mxfp4_moe_forward_noalloc(ctypes.byref(dims), _p(x), _p(router_logits), _p(w13),
                                          _p(w13s), _p(w2), _p(w2s), int(top_k),
                                          float(clamp_limit), _p(out), _stream()))
    return out


PHASES = ("route", "gate_up", "down", "combine")


def mxfp4_moe_forward_timed(dims: Dims, x, router_logits, w13, w13s, w2, w2s, top_k: int,
                            clamp_limit: float, events, out=None, workspace=None):
    """mxfp4_moe_forward recording five torch.cuda.Event objects (created with
    enable_timing=True) around its phases on the current stream; phase i lasts
    events[i].elapsed_time(events[i+1]) for the names in PHASES."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(router_logits, torch.float32, "router_logits")
    if len(events) != 5:
        raise ValueError("need five events")
    if out is None:
        out = torch.empty((dims.T, dims.H), dtype=torch.bfloat16, device=x.device)
    workspace, nbytes = _workspace(dims, top_k, workspace, x.device)
    handles = (ctypes.c_void_p * 5)(*[ev.cuda_event for ev in events])
    _check("mxfp4_moe_forward_timed",
           _L().mxfp4_moe_forward_timed(ctypes.byref(dims), _p(x), _p(router_logits), _p(w13),
                                        _p(w13s), _p(w2), _p(w2s), int(top_k), float(clamp_limit),
                                        _p(out), _p(workspace), nbytes, handles, _stream()))
    return out


def mxfp4_moe_forward_debug(dims: Dims, x, router_logits, w13, w13s, w2, w2s, top_k: int,
                            clamp_limit: float, out=None, workspace=None):
    """mxfp4_moe_forward plus the intermediates: dict with out, out32 (the fp32 output
    before its bf16 rounding), act (bf16 [T*k, I]) and, in A4 mode, actq/acts/xq/xs."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(router_logits, torch.float32, "router_logits")
    T, H, I, k = dims.T, dims.H, dims.I, int(top_k)
    ks = k + dims.shared  # slots per token
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    act = torch.zeros((T * ks, I), dtype=torch.bfloat16, device=dev)
    a8 = bool(dims.flags & MXFP4_MOE_A8)
    a4 = bool(dims.flags & MXFP4_MOE_A4) or a8   # quantised activations
    q = 1 if a8 else 2                            # elements per code byte
    actq = torch.zeros((T * ks, I // q), dtype=torch.uint8, device=dev) if a4 else None
    acts = torch.zeros((T * ks, I // 32), dtype=torch.uint8, device=dev) if a4 else None
    xq = torch.zeros((T, H // q), dtype=torch.uint8, device=dev) if a4 else None
    xs = torch.zeros((T, H // 32), dtype=torch.uint8, device=dev) if a4 else None
    out32 = torch.zeros((T, H), dtype=torch.float32, device=dev)
    workspace, nbytes = _workspace(dims, top_k, workspace, dev)
    _check("mxfp4_moe_forward_debug",
           _L().mxfp4_moe_forward_debug(ctypes.byref(dims), _p(x), _p(router_logits), _p(w13),
                                        _p(w13s), _p(w2), _p(w2s), k, float(clamp_limit), _p(out),
                                        _p(workspace), nbytes, _p(act), _p(actq), _p(acts),
                                        _p(xq), _p(xs), _p(out32), _stream()))
    return {"out": out, "out32": out32, "act": act, "actq": actq, "acts": acts, "xq": xq,
            "xs": xs}


def mxfp4_moe_route(dims: Dims, router_logits, top_k: int, workspace=None):
    """Routing tables only: dict of ids, weights, counts, offsets, sorted, inv (device
    tensors; the first offsets[-1] entries of sorted are valid)."""
    _dev_tensor(router_logits, torch.float32, "router_logits")
    T, k, El = dims.T, int(top_k), dims.E_local
    ks, Et = k + dims.shared, El + dims.shared  # slots per token, table experts
    dev = router_logits.device
    ids = torch.empty((T, ks), dtype=torch.int32, device=dev)
    w = torch.empty((T, ks), dtype=torch.float32, device=dev)
    counts = torch.empty(Et, dtype=torch.int32, device=dev)
    offsets = torch.empty(Et + 1, dtype=torch.int32, device=dev)
    sorted_ = torch.empty(max(T * ks, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * ks, 1), dtype=torch.int32, device=dev)
    workspace, nbytes = _workspace(dims, top_k, workspace, dev)
    _check("mxfp4_moe_route",
           _L().mxfp4_moe_route(ctypes.byref(dims), _p(router_logits), k, _p(ids), _p(w),
                                _p(counts), _p(offsets), _p(sorted_), _p(inv), _p(workspace),
                                nbytes, _stream()))
    return {"ids": ids, "weights": w, "counts": counts, "offsets": offsets, "sorted": sorted_,
            "inv": inv}


# ---------------------------------------------------------------- bf16 exclusions

def mxfp4_moe_preshuffle_fused(dims: Dims, excluded, w13_fused, w13s_fused, w2_fused, w2s_fused):
    """Fused expert buffers with per-expert dtypes (uint8 device tensors in the
    layout of include/mxfp4_moe.h) and the host exclusion set (one bool per
    expert of the buffers) -> (preshuffled (w13, w13s, w2, w2s), bx) where bx is
    a dict of the bf16 experts: n, expert_map, w13, w2 (device tensors)."""
    for t, n in ((w13_fused, "w13_fused"), (w2_fused, "w2_fused")):
        _dev_tensor(t, torch.uint8, n)
    Ew = dims.E_local + dims.shared
    flags = [1 if v else 0 for v in excluded]
    if len(flags) != Ew:
        raise ValueError("excluded needs %d entries" % Ew)
    n = sum(flags)
    host = (ctypes.c_uint8 * Ew)(*flags)
    dev = w13_fused.device
    sizes = mxfp4_moe_preshuffled_bytes(dims)
    outs = [torch.empty(z, dtype=torch.uint8, device=dev) for z in sizes]
    H, I = dims.H, dims.I
    w13x = torch.empty((n, 2 * I, H), dtype=torch.bfloat16, device=dev)
    w2x = torch.empty((n, H, I), dtype=torch.bfloat16, device=dev)
    xmap = torch.empty(Ew + n, dtype=torch.int32, device=dev)
    _check("mxfp4_moe_preshuffle_fused",
           _L().mxfp4_moe_preshuffle_fused(ctypes.byref(dims), host, _p(w13_fused),
                                           _p(w13s_fused) if w13s_fused.numel() else None,
                                           _p(w2_fused),
                                           _p(w2s_fused) if w2s_fused.numel() else None,
                                           *[_p(o) for o in outs],
                                           _p(w13x) if n else None, _p(w2x) if n else None,
                                           _p(xmap), _stream()))
    return tuple(outs), {"n": n, "expert_map": xmap, "w13": w13x, "w2": w2x}


def mxfp4_moe_forward_mixed(dims: Dims, bx: dict, x, router_logits, w13, w13s, w2, w2s,
                            top_k: int, clamp_limit: float, out=None, workspace=None,
                            debug: bool = False):
    """The layer with experts kept in bf16 (bx from mxfp4_moe_preshuffle_fused).
    Returns out, or with debug the dict of mxfp4_moe_forward_debug."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(router_logits, torch.float32, "router_logits")
    T, H, I, k = dims.T, dims.H, dims.I, int(top_k)
    ks = k + dims.shared
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    st = Bf16Experts(int(bx["n"]), bx["expert_map"].data_ptr() if bx["n"] else None,
                     bx["w13"].data_ptr() if bx["n"] else None,
                     bx["w2"].data_ptr() if bx["n"] else None)
    inter = {"act": None, "actq": None, "acts": None, "xq": None, "xs": None, "out32": None}
    if debug:
        a8 = bool(dims.flags & MXFP4_MOE_A8)
        mxa = bool(dims.flags & MXFP4_MOE_A4) or a8
        q = 1 if a8 else 2
        inter["act"] = torch.zeros((T * ks, I), dtype=torch.bfloat16, device=dev)
        if mxa:
            inter["actq"] = torch.zeros((T * ks, I // q), dtype=torch.uint8, device=dev)
            inter["acts"] = torch.zeros((T * ks, I // 32), dtype=torch.uint8, device=dev)
            inter["xq"] = torch.zeros((T, H // q), dtype=torch.uint8, device=dev)
            inter["xs"] = torch.zeros((T, H // 32), dtype=torch.uint8, device=dev)
        inter["out32"] = torch.zeros((T, H), dtype=torch.float32, device=dev)
    workspace, nbytes = _workspace(dims, top_k, workspace, dev)
    _check("mxfp4_moe_forward_mixed",
           _L().mxfp4_moe_forward_mixed(ctypes.byref(dims), ctypes.byref(st), _p(x),
                                        _p(router_logits), _p(w13), _p(w13s), _p(w2), _p(w2s), k,
                                        float(clamp_limit), _p(out), _p(workspace), nbytes,
                                        *[_p(inter[n]) for n in ("act", "actq", "acts", "xq",
                                                                  "xs", "out32")], _stream()))
    if not debug:
        return out
    return dict(inter, out=out)
