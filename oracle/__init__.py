"""CPU oracle for the MXFP4 routed-expert MoE layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the two
share no code: the oracle is plain C (``moe_oracle.c``) built with gcc,
``-O2 -ffp-contract=off`` and no fast-math, loaded here through ctypes with
NumPy arrays.

What it computes, and the page passages each step follows, is stated in
``moe_oracle.c``.  Parity pins for every function live in
``tests/test_oracle_*.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libmoe_oracle.so``."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_e2m1_value.argtypes = [i32]
    lib.orc_ue8m0_value.restype = ctypes.c_double
    lib.orc_ue8m0_value.argtypes = [i32]
    lib.orc_dequant.argtypes = [P, P, i64, i64, P]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [i32]
    lib.orc_dequant8.argtypes = [P, P, i64, i64, P]
    for name in ("orc_quantize8_f64", "orc_quantize8_bf16"):
        getattr(lib, name).argtypes = [P, i64, i64, P, P]
    for name in ("orc_quantize_f64", "orc_quantize_f32", "orc_quantize_bf16"):
        getattr(lib, name).argtypes = [P, i64, i64, P, P]
    lib.orc_bf16_from_f32.restype = ctypes.c_uint16
    lib.orc_bf16_from_f32.argtypes = [ctypes.c_float]
    lib.orc_bf16_round_array.argtypes = [P, i64, P]
    lib.orc_route.restype = ctypes.c_int
    lib.orc_route.argtypes = [P, i64, i64, i32, P, P]
    lib.orc_permute.restype = i64
    lib.orc_permute.argtypes = [P, i64, i32, i64, i64, i64, P, P, P, P]
    lib.orc_swiglu.restype = ctypes.c_float
    lib.orc_swiglu.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
    lib.orc_moe_forward.restype = i64
    lib.orc_moe_forward.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P,
                                    P, P, P, P, P, P, P, P, P, P, P, P, P, i32]
    _lib = lib
    return lib


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E_global", ctypes.c_int64), ("E_local", ctypes.c_int64),
                ("first_local", ctypes.c_int64), ("top_k", ctypes.c_int32),
                ("clamp_limit", ctypes.c_float), ("a4", ctypes.c_int32),
                ("shared", ctypes.c_int32), ("given_actq", ctypes.c_int32),
                ("a8", ctypes.c_int32), ("bf16_expert", ctypes.c_void_p),
                ("w13_bf16", ctypes.c_void_p), ("w2_bf16", ctypes.c_void_p)]


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


# ------------------------------------------------------------------ codec

def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def ue8m0_value(s: int) -> float:
    return _load().orc_ue8m0_value(int(s))


def dequant(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Canonical packed codes [..., K/2] + scales [..., K/32] -> float32 [..., K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.size // (K // 2)
    assert scales.size == rows * (K // 32)
    out = np.empty(codes.shape[:-1] + (K,), dtype=np.float32)
    _load().orc_dequant(_ptr(codes), _ptr(scales), rows, K, _ptr(out))
    return out


def quantize(v: np.ndarray):
    """OCP MX quantiser along the last axis.  ``v`` may be float64, float32, or
    uint16 holding bf16 bits.  Returns (codes [..., K/2], scales [..., K/32])."""
    v = np.ascontiguousarray(v)
    K = v.shape[-1]
    assert K % 32 == 0
    rows = v.size // K
    codes = np.empty(v.shape[:-1] + (K // 2,), dtype=np.uint8)
    scales = np.empty(v.shape[:-1] + (K // 32,), dtype=np.uint8)
    lib = _load()
    fn = {np.dtype(np.float64): lib.orc_quantize_f64, np.dtype(np.float32): lib.orc_quantize_f32,
          np.dtype(np.uint16): lib.orc_quantize_bf16}[v.dtype]
    fn(_ptr(v), rows, K, _ptr(codes), _ptr(scales))
    return codes, scales


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def dequant8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 codes [..., K] (one E4M3 byte each) + scales [..., K/32] -> float32."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K = codes.shape[-1]
    rows = codes.size // K
    assert scales.size == rows * (K // 32)
    out = np.empty(codes.shape, dtype=np.float32)
    _load().orc_dequant8(_ptr(codes), _ptr(scales), rows, K, _ptr(out))
    return out


def quantize8(v: np.ndarray):
    """OCP MX quantiser with E4M3 elements along the last axis.  ``v``: float64
    or uint16 bf16 bits.  Returns (codes [..., K], scales [..., K/32])."""
    v = np.ascontiguousarray(v)
    K = v.shape[-1]
    assert K % 32 == 0
    rows = v.size // K
    codes = np.empty(v.shape, dtype=np.uint8)
    scales = np.empty(v.shape[:-1] + (K // 32,), dtype=np.uint8)
    lib = _load()
    fn = {np.dtype(np.float64): lib.orc_quantize8_f64, np.dtype(np.uint16): lib.orc_quantize8_bf16}[v.dtype]
    fn(_ptr(v), rows, K, _ptr(codes), _ptr(scales))
    return codes, scales


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE); returns the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_bf16_round_array(_ptr(a), a.size, _ptr(out))
    return out


def swiglu(g: float, u: float, limit: float) -> float:
    return _load().orc_swiglu(float(g), float(u), float(limit))


# ------------------------------------------------------------------ routing

def route(logits: np.ndarray, top_k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float32)
    rc = _load().orc_route(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle route: NaN router logit")
    return ids, w


def permute(ids: np.ndarray, first_local: int, E_local: int, shared_id: int = -1):
    """Counting sort of the slots by local expert; with shared_id >= 0 the slots
    holding that id form one more expert, table entry E_local."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    n_exp = E_local + (1 if shared_id >= 0 else 0)
    counts = np.empty(n_exp, dtype=np.int32)
    offsets = np.empty(n_exp + 1, dtype=np.int32)
    sorted_ = np.empty(T * k, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    n = _load().orc_permute(_ptr(ids), T, k, first_local, E_local, shared_id, _ptr(counts),
                            _ptr(offsets), _ptr(sorted_), _ptr(inv))
    return counts, offsets, sorted_[:n].copy(), inv


# ------------------------------------------------------------------ layer

@dataclass
class OracleResult:
    ids: np.ndarray
    w: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    sorted: np.ndarray
    inv: np.ndarray
    act: np.ndarray | None       # bf16 bits [N_assign, I]
    out32: np.ndarray            # float32 [T, H]
    out: np.ndarray              # bf16 bits [T, H]
    xq: np.ndarray | None = None
    xs: np.ndarray | None = None
    actq: np.ndarray | None = None
    acts: np.ndarray | None = None
    n_assign: int = 0


def unfuse(fused, fused_scales, excluded, R: int, K: int):
    """Split a fused expert buffer whose experts have their own dtype (campaign
    page, section "A fused tensor with two dtypes in it": a packed expert's rows
    are half the logical width in bytes, an excluded bf16 expert keeps the full
    width, so one stride cannot slice both and the exclusion set has to be
    carried per expert).  Expert e of the buffer takes R*K/2 bytes of packed
    E2M1 codes, or R*K*2 bytes of bf16 when excluded, back to back in expert
    order; the scale tensor holds R*K/32 bytes per packed expert, in order.
    Returns (codes [E, R, K/2], scales [E, R, K/32], bf16 bits [n, R, K]), the
    MXFP4 slots of excluded experts zero."""
    ex = np.asarray(excluded, dtype=bool)
    fused = np.ascontiguousarray(fused, dtype=np.uint8).reshape(-1)
    fs = np.ascontiguousarray(fused_scales, dtype=np.uint8).reshape(-1)
    E = ex.size
    codes = np.zeros((E, R, K // 2), np.uint8)
    scales = np.zeros((E, R, K // 32), np.uint8)
    bf = np.zeros((int(ex.sum()), R, K), np.uint16)
    off = soff = j = 0
    for e in range(E):
        if ex[e]:
            nb = R * K * 2
            bf[j] = fused[off:off + nb].view(np.uint16).reshape(R, K)
            j += 1
        else:
            nb = R * K // 2
            codes[e] = fused[off:off + nb].reshape(R, K // 2)
            scales[e] = fs[soff:soff + R * K // 32].reshape(R, K // 32)
            soff += R * K // 32
        off += nb
    if off != fused.size or soff != fs.size:
        raise ValueError("fused buffer is %d bytes (scales %d), the exclusion set needs %d (%d)"
                         % (fused.size, fs.size, off, soff))
    return codes, scales, bf


def moe_forward(x_bits, logits, w13, w13s, w2, w2s, *, top_k, clamp_limit, E_global=None,
                first_local=0, a4=False, shared=False, token_mask=None, want_act=True, nthreads=0,
                actq_in=None, acts_in=None, a8=False, bf16_experts=None, w13_bf16=None,
                w2_bf16=None):
    """The whole layer on canonical-layout inputs (see ``moe_oracle.h``).

    ``x_bits``: uint16 bf16 bits [T, H]; ``logits``: float32 [T, E_global];
    ``w13``: uint8 [E, 2I, H/2]; ``w13s``: uint8 [E, 2I, H/32];
    ``w2``: uint8 [E, H, I/2]; ``w2s``: uint8 [E, H, I/32], where E = E_local
    routed experts, plus one shared expert (the last) when ``shared``.  The
    tables then have top_k + 1 slots per token (slot top_k: id E_global, weight
    1) and E_local + 1 experts.
    ``token_mask`` (bool [T]) restricts expert work and the combine to the
    marked tokens; rows of ``out``/``out32`` for other tokens are left zero.
    ``actq_in``/``acts_in`` (A4/A8 only; [N_assign, I/2] or [N_assign, I],
    and [N_assign, I/32], in sorted order): down reads these quantised SwiGLU
    outputs instead of quantising its own, so a comparison downstream of that
    quantisation starts from the same codes on both sides.
    ``a8``: as ``a4`` with MXFP8 (E4M3) codes, one byte per element.
    ``bf16_experts`` (bool [E]): experts stored in bf16 instead of MXFP4 (their
    slots of the MXFP4 arrays are ignored); ``w13_bf16`` uint16 [n, 2I, H] and
    ``w2_bf16`` uint16 [n, H, I] hold their weights, the j-th excluded expert in
    slot j.  They compute on bf16 activations in every mode.
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    w13 = np.ascontiguousarray(w13, dtype=np.uint8)
    w13s = np.ascontiguousarray(w13s, dtype=np.uint8)
    w2 = np.ascontiguousarray(w2, dtype=np.uint8)
    w2s = np.ascontiguousarray(w2s, dtype=np.uint8)
    T, H = x_bits.shape
    Ew, two_i, _ = w13.shape
    I = two_i // 2
    sh = 1 if shared else 0
    E_local = Ew - sh
    Eg = logits.shape[1] if E_global is None else E_global
    assert logits.shape == (T, Eg) and E_local >= 1
    assert w13.shape == (Ew, 2 * I, H // 2) and w13s.shape == (Ew, 2 * I, H // 32)
    assert w2.shape == (Ew, H, I // 2) and w2s.shape == (Ew, H, I // 32)
    given = actq_in is not None
    assert given == (acts_in is not None) and (a4 or a8 or not given) and not (a4 and a8)
    xmask = b13 = b2 = None
    if bf16_experts is not None:
        xmask = np.ascontiguousarray(np.asarray(bf16_experts, dtype=bool).astype(np.uint8))
        assert xmask.shape == (Ew,)
        n_x = int(xmask.sum())
        b13 = np.ascontiguousarray(w13_bf16, dtype=np.uint16)
        b2 = np.ascontiguousarray(w2_bf16, dtype=np.uint16)
        assert b13.shape == (n_x, 2 * I, H) and b2.shape == (n_x, H, I)
    d = _Dims(T, H, I, Eg, E_local, first_local, top_k, clamp_limit, 1 if a4 else 0, sh,
              1 if given else 0, 1 if a8 else 0, None if xmask is None else xmask.ctypes.data,
              None if b13 is None else b13.ctypes.data, None if b2 is None else b2.ctypes.data)
    k = top_k + sh
    S = T * k
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    counts = np.empty(Ew, np.int32)
    offsets = np.empty(Ew + 1, np.int32)
    sorted_ = np.zeros(max(S, 1), np.int32)
    inv = np.empty(max(S, 1), np.int32)
    act = np.zeros((max(S, 1), I), np.uint16) if want_act else None
    out32 = np.zeros((T, H), np.float32)
    out = np.zeros((T, H), np.uint16)
    aq = a4 or a8
    cpe = 1 if a8 else 2   # codes per byte
    xq = np.zeros((T, H // cpe), np.uint8) if aq else None
    xs = np.zeros((T, H // 32), np.uint8) if aq else None
    actq = np.zeros((max(S, 1), I // cpe), np.uint8) if aq else None
    acts = np.zeros((max(S, 1), I // 32), np.uint8) if aq else None
    if given:
        n_in = np.asarray(actq_in).shape[0]
        actq[:n_in] = actq_in
        acts[:n_in] = acts_in
    mask = None
    if token_mask is not None:
        mask = np.ascontiguousarray(np.asarray(token_mask, dtype=bool).astype(np.uint8))
        assert mask.shape == (T,)
    n = _load().orc_moe_forward(ctypes.byref(d), _ptr(x_bits), _ptr(logits), _ptr(w13),
                                _ptr(w13s), _ptr(w2), _ptr(w2s), _ptr(mask), _ptr(ids), _ptr(w),
                                _ptr(counts), _ptr(offsets), _ptr(sorted_), _ptr(inv),
                                _ptr(act), _ptr(xq), _ptr(xs), _ptr(actq), _ptr(acts),
                                _ptr(out32), _ptr(out), int(nthreads))
    if n < 0:
        raise ValueError("oracle moe_forward failed with status %d" % n)
    return OracleResult(ids=ids, w=w, counts=counts, offsets=offsets, sorted=sorted_[:n].copy(),
                        inv=inv[:S].copy(), act=None if act is None else act[:n].copy(),
                        out32=out32, out=out, xq=xq, xs=xs,
                        actq=None if actq is None else actq[:n].copy(),
                        acts=None if acts is None else acts[:n].copy(), n_assign=int(n))
