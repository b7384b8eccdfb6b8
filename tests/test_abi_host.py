"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and refuses each bad argument by name before touching a GPU.

Pointers passed here are fake, suitably aligned integers: every refusal under
test happens in host validation, before any device work."""
import ctypes
import os
import re

import pytest

import mxfp4_block_scaled_router_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4_moe.h")

OK = 0
NULL_POINTER, EMPTY_SHAPE, SHAPE_OVERFLOW, UNSUPPORTED_SHAPE = -1, -2, -3, -4
BAD_TOP_K, BAD_CLAMP, WORKSPACE_TOO_SMALL, MISALIGNED = -5, -6, -7, -8
UNSUPPORTED_DEVICE, HIP_ERR, BAD_FLAGS, BAD_ARGUMENT = -9, -10, -11, -12


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        from mxfp4_block_scaled_router_amd import build
        build.build(verbose=False)
    return mx.load_library()


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(mxfp4_moe_\w+)\(", src, re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mx.EXPORTED)


def test_version_and_status_strings(lib):
    assert mx.abi_version() == 1
    src = open(HEADER).read()
    for name, val in re.findall(r"#define (MXFP4_MOE_(?:OK|ERR_\w+)) \(?(-?\d+)\)?", src):
        assert mx.status_string(int(val)) == name
    assert mx.status_string(-999) == "MXFP4_MOE_ERR_UNKNOWN"


def dims(**kw):
    base = dict(T=16, H=512, I=256, E_global=8, E_local=8, first_local=0)
    base.update(kw)
    flags = kw.pop("flags", 0)
    d = mx.Dims(base["T"], base["H"], base["I"], base["E_global"], base["E_local"],
                base["first_local"], flags, 0)
    return d


def ws_status(d, k=2):
    out = ctypes.c_size_t()
    return mx.load_library().mxfp4_moe_workspace_bytes(ctypes.byref(d), k, ctypes.byref(out)), \
        out.value


@pytest.mark.parametrize("kw,k,expect", [
    ({}, 2, OK),
    ({"H": 0}, 2, EMPTY_SHAPE), ({"I": 0}, 2, EMPTY_SHAPE), ({"E_global": 0}, 2, EMPTY_SHAPE),
    ({"E_local": 0}, 2, EMPTY_SHAPE), ({}, 0, EMPTY_SHAPE),
    ({"H": 500}, 2, UNSUPPORTED_SHAPE), ({"I": 200}, 2, UNSUPPORTED_SHAPE),
    ({"T": -1}, 2, UNSUPPORTED_SHAPE), ({"first_local": 4}, 2, UNSUPPORTED_SHAPE),
    ({"first_local": -1}, 2, UNSUPPORTED_SHAPE), ({"E_global": 2048, "E_local": 8}, 2, UNSUPPORTED_SHAPE),
    ({"E_global": 513, "E_local": 8}, 2, UNSUPPORTED_SHAPE), ({"E_global": 512, "E_local": 8}, 2, OK),
    ({}, -1, BAD_TOP_K), ({}, 9, BAD_TOP_K), ({"E_global": 64, "E_local": 64}, 33, BAD_TOP_K),
    ({"T": 1 << 40}, 8, SHAPE_OVERFLOW), ({"T": 1 << 60, "H": 1 << 10}, 2, SHAPE_OVERFLOW),
    ({"first_local": (1 << 63) - 4}, 2, SHAPE_OVERFLOW),
    ({"flags": 0x20}, 2, BAD_FLAGS),
    ({"flags": 0x1 | 0x8}, 2, BAD_FLAGS),     # A4 and A8 exclude each other
])
def test_dims_refusals(lib, kw, k, expect):
    st, _ = ws_status(dims(**kw), k)
    assert st == expect, (mx.status_string(st), kw, k)


def test_reserved_field_must_be_zero(lib):
    d = dims()
    d.reserved = 1
    assert ws_status(d)[0] == BAD_ARGUMENT


def test_workspace_grows_with_flags(lib):
    _, base = ws_status(dims())
    _, det = ws_status(dims(flags=mx.MXFP4_MOE_DETERMINISTIC))
    _, a4 = ws_status(dims(flags=mx.MXFP4_MOE_A4))
    assert base > 0 and det > 0 and a4 > base


def test_shared_expert_sizes(lib):
    """The shared expert is one more expert in the weight buffers and one more
    slot per token in the workspace."""
    plain = mx.mxfp4_moe_preshuffled_bytes(dims(H=512, I=256, E_local=8))
    shared = mx.mxfp4_moe_preshuffled_bytes(dims(H=512, I=256, E_local=8,
                                                 flags=mx.MXFP4_MOE_SHARED_EXPERT))
    for a, b in zip(plain, shared):
        assert b == a // 8 * 9
    _, base = ws_status(dims())
    st, sh = ws_status(dims(flags=mx.MXFP4_MOE_SHARED_EXPERT))
    assert st == 0 and sh > base
    d = dims(flags=mx.MXFP4_MOE_SHARED_EXPERT)
    assert mx.mxfp4_moe_plan(d, 2)["tile_rows"] in (16, 64, 128)


def test_a8_workspace_holds_byte_codes(lib):
    """A8 keeps one code byte per element: its workspace exceeds A4's by the
    x and act code bytes (T*H/2 + T*k*I/2, each region 256-byte aligned)."""
    _, a4 = ws_status(dims(flags=mx.MXFP4_MOE_A4))
    st, a8 = ws_status(dims(flags=mx.MXFP4_MOE_A8))
    assert st == 0
    T, H, I, k = 16, 512, 256, 2
    assert a8 - a4 >= T * H // 2 + T * k * I // 2
    assert mx.mxfp4_moe_plan(dims(flags=mx.MXFP4_MOE_A8), 2)["tile_rows"] in (16, 128)


def test_null_dims(lib):
    out = ctypes.c_size_t()
    assert lib.mxfp4_moe_workspace_bytes(None, 2, ctypes.byref(out)) == NULL_POINTER
    assert lib.mxfp4_moe_workspace_bytes(ctypes.byref(dims()), 2, None) == NULL_POINTER


def test_plan_query(lib):
    # decode-sized call: 16-row K-split tiles, atomic combine unless deterministic
    assert mx.mxfp4_moe_plan(dims(), 2) == {"tile_rows": 16, "ordered_combine": False}
    det = mx.mxfp4_moe_plan(dims(flags=mx.MXFP4_MOE_DETERMINISTIC), 2)
    assert det == {"tile_rows": 16, "ordered_combine": True}
    # many rows per expert: large tiles, always the slot-ordered gather
    big = mx.mxfp4_moe_plan(dims(T=4096, E_global=8, E_local=8), 2)
    assert big == {"tile_rows": 128, "ordered_combine": True}
    # MXFP4 activations: 320-row gate_up tiles while they hold a whole expert
    # and its scale rows fit LDS (K <= 4352), else 128
    assert mx.mxfp4_moe_plan(dims(T=1024, H=4352, flags=mx.MXFP4_MOE_A4), 2)["tile_rows"] == 320
    assert mx.mxfp4_moe_plan(dims(T=1024, H=4480, flags=mx.MXFP4_MOE_A4), 2)["tile_rows"] == 128
    assert mx.mxfp4_moe_plan(dims(T=4096, flags=mx.MXFP4_MOE_A4), 2)["tile_rows"] == 128
    # speculative-verify shapes of the decode layer (T = 6 per sequence): the
    # tile height follows the expected rows per expert T*k/E_global (K-split
    # tiles of 32 rows from 64 tokens on where two row blocks fit the registers:
    # not with the bf16 rows of the 5120-wide EP share)
    from mxfp4_block_scaled_router_amd import workloads as W
    want = {"verify_b1": 16, "verify_b8": 16, "verify_b16": 32, "verify_b32": 32, "verify_b48": 64,
            "decode": 16, "ep_share": 16, "prefill": 128, "a4": 320, "a8": 128}
    for name, rows in want.items():
        wl = W.WORKLOADS[name]
        d = mx.Dims.make(wl.T, wl.H, wl.I, wl.E_global, wl.E_local, wl.first_local, a4=wl.a4,
                         a8=wl.a8)
        assert mx.mxfp4_moe_plan(d, wl.top_k)["tile_rows"] == rows, name
    out = ctypes.c_int32()
    assert lib.mxfp4_moe_plan(ctypes.byref(dims()), 2, None, ctypes.byref(out)) == NULL_POINTER
    assert lib.mxfp4_moe_plan(ctypes.byref(dims(H=0)), 2, ctypes.byref(out), ctypes.byref(out)) == EMPTY_SHAPE


def test_preshuffled_bytes(lib):
    d = dims(H=512, I=256, E_local=8)
    w13, w13s, w2, w2s = mx.mxfp4_moe_preshuffled_bytes(d)
    assert w13 == 8 * 512 * 256 and w2 == 8 * 512 * 128
    # scales padded to whole 512-element K groups: one group of 256 bytes per 16 rows
    assert w13s == 8 * (512 // 16) * 1 * 256
    assert w2s == 8 * (512 // 16) * 1 * 256


A = 1 << 20  # fake, 256-byte aligned "device" addresses


def fwd(lib, d, k=2, clamp=7.0, ptrs=None, ws_bytes=None):
    p = dict(x=A, logits=A, w13=A, w13s=A, w2=A, w2s=A, out=A, ws=A)
    if ptrs:
        p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = ws_status(d, k)[1] if ws_status(d, k)[0] == 0 else 0
    V = ctypes.c_void_p
    return lib.mxfp4_moe_forward(ctypes.byref(d), V(p["x"]), V(p["logits"]), V(p["w13"]),
                                 V(p["w13s"]), V(p["w2"]), V(p["w2s"]), k, clamp, V(p["out"]),
                                 V(p["ws"]), ws_bytes, None)


@pytest.mark.parametrize("name", ["x", "logits", "w13", "w13s", "w2", "w2s", "out", "ws"])
def test_forward_null_pointers(lib, name):
    assert fwd(lib, dims(), ptrs={name: 0}) == NULL_POINTER


@pytest.mark.parametrize("name,off", [("x", 8), ("w13", 4), ("w2s", 2), ("out", 1), ("ws", 16),
                                      ("logits", 2)])
def test_forward_misaligned(lib, name, off):
    assert fwd(lib, dims(), ptrs={name: A + off}) == MISALIGNED


@pytest.mark.parametrize("clamp", [float("nan"), 0.0, -1.0])
def test_forward_bad_clamp(lib, clamp):
    assert fwd(lib, dims(), clamp=clamp) == BAD_CLAMP


def test_forward_inf_clamp_passes_validation(lib):
    st = fwd(lib, dims(), clamp=float("inf"))
    assert st in (OK, UNSUPPORTED_DEVICE)  # no GPU here: the device check is last


def test_forward_workspace_too_small(lib):
    d = dims()
    need = ws_status(d)[1]
    assert fwd(lib, d, ws_bytes=need - 1) == WORKSPACE_TOO_SMALL


def test_forward_shape_refusals_come_first(lib):
    assert fwd(lib, dims(H=0)) == EMPTY_SHAPE
    assert fwd(lib, dims(), k=9) == BAD_TOP_K


def test_quantize_refusals(lib):
    V = ctypes.c_void_p
    q = lib.mxfp4_moe_quantize
    assert q(V(A), 2, 4, 64, V(A), V(A), None) == BAD_ARGUMENT
    assert q(V(A), 0, 4, 0, V(A), V(A), None) == EMPTY_SHAPE
    assert q(V(A), 0, 4, 48, V(A), V(A), None) == UNSUPPORTED_SHAPE
    assert q(V(A), 0, -1, 64, V(A), V(A), None) == UNSUPPORTED_SHAPE
    assert q(V(A), 0, 1 << 62, 64, V(A), V(A), None) == SHAPE_OVERFLOW
    assert q(None, 0, 4, 64, V(A), V(A), None) == NULL_POINTER
    assert q(V(A + 2), 0, 4, 64, V(A), V(A), None) == MISALIGNED


def test_route_refusals(lib):
    V = ctypes.c_void_p
    d = dims()
    r = lib.mxfp4_moe_route
    args = [V(A)] * 7
    assert r(ctypes.byref(d), V(A), 2, *args[:6], V(A), 0, None) == WORKSPACE_TOO_SMALL
    assert r(ctypes.byref(d), None, 2, *args[:6], V(A), 1 << 30, None) == NULL_POINTER
    assert r(ctypes.byref(d), V(A), 0, *args[:6], V(A), 1 << 30, None) == EMPTY_SHAPE


def test_no_gpu_gives_device_refusal_not_a_crash(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert fwd(lib, dims()) == UNSUPPORTED_DEVICE


def mixed(lib, d, bx, k=2, ptrs=None):
    p = dict(x=A, logits=A, w13=A, w13s=A, w2=A, w2s=A, out=A, ws=A)
    if ptrs:
        p.update(ptrs)
    ws = ws_status(d, k)[1]
    V = ctypes.c_void_p
    return lib.mxfp4_moe_forward_mixed(ctypes.byref(d), None if bx is None else ctypes.byref(bx),
                                       V(p["x"]), V(p["logits"]), V(p["w13"]), V(p["w13s"]),
                                       V(p["w2"]), V(p["w2s"]), k, 7.0, V(p["out"]), V(p["ws"]),
                                       ws, None, None, None, None, None, None, None)


def test_forward_mixed_refusals(lib):
    d = dims()
    assert mixed(lib, d, None) == NULL_POINTER
    assert mixed(lib, d, mx.Bf16Experts(-1, A, A, A)) == BAD_ARGUMENT
    assert mixed(lib, d, mx.Bf16Experts(9, A, A, A)) == BAD_ARGUMENT      # > E_local
    assert mixed(lib, d, mx.Bf16Experts(2, None, A, A)) == NULL_POINTER
    assert mixed(lib, d, mx.Bf16Experts(2, A, None, A)) == NULL_POINTER
    assert mixed(lib, d, mx.Bf16Experts(2, A, A + 8, A)) == MISALIGNED
    assert mixed(lib, d, mx.Bf16Experts(2, A + 2, A, A)) == MISALIGNED
    # with the shared expert the buffers hold E_local + 1 experts
    ds = dims(flags=mx.MXFP4_MOE_SHARED_EXPERT)
    assert mixed(lib, ds, mx.Bf16Experts(9, A, A, A)) in (OK, UNSUPPORTED_DEVICE)
    assert mixed(lib, ds, mx.Bf16Experts(10, A, A, A)) == BAD_ARGUMENT
    # n = 0 needs no map or weights; the usual forward checks come first
    assert mixed(lib, d, mx.Bf16Experts(0, None, None, None)) in (OK, UNSUPPORTED_DEVICE)
    assert mixed(lib, d, mx.Bf16Experts(0, None, None, None), ptrs={"w13": 0}) == NULL_POINTER
    assert mixed(lib, dims(H=0), mx.Bf16Experts(0, None, None, None)) == EMPTY_SHAPE


def test_preshuffle_fused_refusals(lib):
    V = ctypes.c_void_p
    d = dims()
    f = lib.mxfp4_moe_preshuffle_fused

    def call(flags, **kw):
        p = dict(w13f=A, w13sf=A, w2f=A, w2sf=A, w13=A, w13s=A, w2=A, w2s=A, b13=A, b2=A, map=A)
        p.update(kw)
        ex = None if flags is None else (ctypes.c_uint8 * len(flags))(*flags)
        return f(ctypes.byref(d), ex, *[V(p[n]) for n in ("w13f", "w13sf", "w2f", "w2sf", "w13",
                                                          "w13s", "w2", "w2s", "b13", "b2", "map")],
                 None)
    ok = (OK, UNSUPPORTED_DEVICE)
    assert call(None) == NULL_POINTER
    assert call([0, 2, 0, 0, 0, 0, 0, 0]) == BAD_ARGUMENT
    assert call([0, 1, 0, 0, 0, 0, 0, 0], b13=0) == NULL_POINTER
    assert call([0] * 8, b13=0, b2=0) in ok                     # nothing excluded: no bf16 outputs
    assert call([1] * 8, w13sf=0, w2sf=0) in ok                 # all excluded: no scale tensors
    assert call([0, 1, 0, 0, 0, 0, 0, 0], w13sf=0) == NULL_POINTER
    assert call([0] * 8, map=0) == NULL_POINTER
    assert call([0] * 8, w2f=A + 8) == MISALIGNED
    assert call([0, 1, 0, 0, 0, 0, 0, 0], map=A + 2) == MISALIGNED


def test_noalloc_refusals(lib):
    """mxfp4_moe_forward_noalloc: a call whose workspace exceeds the static
    scratch is refused by name before anything else; other refusals as
    mxfp4_moe_forward; in range, without a GPU, the device refusal."""
    f = lib.mxfp4_moe_forward_noalloc
    P = 1 << 20
    big = dims(T=8192, H=4096, I=1536, E_global=128, E_local=128)
    assert f(ctypes.byref(big), P, P, P, P, P, P, 8, 7.0, P, None) == -13
    assert mx.status_string(-13) == "MXFP4_MOE_ERR_SCRATCH_LIMIT"
    d = dims()
    assert f(ctypes.byref(d), P, P, P, P, P, P, 9, 7.0, P, None) == BAD_TOP_K
    assert f(None, P, P, P, P, P, P, 2, 7.0, P, None) == NULL_POINTER
    assert f(ctypes.byref(d), P, P, P, P, P, P, 2, float("nan"), P, None) in (BAD_CLAMP, UNSUPPORTED_DEVICE)
    st = f(ctypes.byref(d), P, P, P, P, P, P, 2, 7.0, P, None)
    assert st == UNSUPPORTED_DEVICE
    # the limit admits the decode, verify and expert-parallel-share workloads
    for kw, k in ((dict(T=16, H=2048, I=1536, E_global=64, E_local=64), 8),
                  (dict(T=288, H=2048, I=1536, E_global=64, E_local=64), 8),
                  (dict(T=256, H=5120, I=1536, E_global=256, E_local=64), 8),
                  (dict(T=256, H=5120, I=1536, E_global=256, E_local=64, flags=0x2), 8)):
        st, n = ws_status(dims(**kw), k)
        assert st == OK and n <= 64 << 20, (kw, n)


def test_quantize_preshuffle_refusals(lib):
    f = lib.mxfp4_moe_quantize_preshuffle
    P = 1 << 20
    d = dims()
    assert f(None, P, P, 1, P, P, P, P, None) == NULL_POINTER
    assert f(ctypes.byref(d), P, P, 2, P, P, P, P, None) == BAD_ARGUMENT
    assert f(ctypes.byref(d), None, P, 1, P, P, P, P, None) == NULL_POINTER
    assert f(ctypes.byref(d), P + 4, P, 1, P, P, P, P, None) == MISALIGNED
    assert f(ctypes.byref(dims(H=500)), P, P, 1, P, P, P, P, None) == UNSUPPORTED_SHAPE
    assert f(ctypes.byref(d), P, P, 1, P, P, P, P, None) == UNSUPPORTED_DEVICE
