"""The A4/A8 output bound of the GPU parity tests (quant_step_bound), checked on
the CPU with the oracle alone: act elements moved by one bf16 ulp (as the
SwiGLU output of another summation order may be) are quantised and run through
the oracle's down and combine; the resulting output must stay within the
bound, and a planted error beyond a quantisation step must not."""
import types

import numpy as np
import pytest

import oracle
from mxfp4_block_scaled_router_amd import workloads as W
from tests.gpu_helpers import TOL_REL_RMS, quant_step_bound


def _case(a8: bool):
    wl = W.WORKLOADS["a8" if a8 else "a4"].replace(T=48, H=512, I=256, E_global=8, E_local=8,
                                                   top_k=2)
    inp = W.make_inputs(wl)
    for which, (c, s) in (("w13", ("w13", "w13s")), ("w2", ("w2", "w2s"))):
        q = [oracle.quantize(W.student_t_expert(wl, e, which).numpy()) for e in range(8)]
        inp[c] = np.stack([a for a, _ in q])
        inp[s] = np.stack([b for _, b in q])
    case = types.SimpleNamespace(wl=wl, a8=a8, a4=not a8, bx=None, inp=inp,
                                 excluded_rows=lambda o: np.zeros(o.n_assign, bool))
    return case


def _run(case, **kw):
    wl, inp = case.wl, case.inp
    return oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"],
                              inp["w2s"], top_k=wl.top_k, clamp_limit=wl.clamp_limit,
                              a4=case.a4, a8=case.a8, **kw)


def _moved_act(o, frac, seed):
    """The oracle's act with a fraction of its elements moved by one bf16 ulp
    (either way, including the block maxima)."""
    rng = np.random.default_rng(seed)
    act = o.act.copy()
    m = rng.random(act.shape) < frac
    # the largest element of a few blocks too: a scale change
    blk = act.reshape(act.shape[0], -1, 32)
    mag = blk & 0x7FFF
    top = np.argmax(mag, axis=2)
    pick = rng.random(top.shape) < 0.05
    r, b = np.nonzero(pick)
    m.reshape(blk.shape)[r, b, top[r, b]] = True
    step = np.where(rng.random(act.shape) < 0.5, 1, -1).astype(np.int32)
    moved = act.astype(np.int32) + np.where(m & ((act & 0x7FFF) > 0), step, 0)
    return moved.astype(np.uint16), m


@pytest.mark.parametrize("a8", [False, True])
def test_bound_covers_one_ulp_moves(a8):
    case = _case(a8)
    o = _run(case)
    moved, _ = _moved_act(o, 0.01, 3)
    quant = oracle.quantize8 if a8 else oracle.quantize
    q, s = quant(moved)
    o2 = _run(case, actq_in=q, acts_in=s)
    B = quant_step_bound(case, o, moved, np.ones(o.n_assign, bool))
    rms = np.sqrt(np.mean(o.out32.astype(np.float64) ** 2))
    d = np.abs(o2.out32.astype(np.float64) - o.out32)
    # the codes moved somewhere, and the move is not within the plain bar alone
    assert ((q != o.actq).any(axis=1)).sum() > 0
    assert (d <= TOL_REL_RMS * rms + B).all(), float((d - B).max() / rms)
    assert B.max() > 0
    # tokens whose act did not move get no slack
    tok = o.sorted // o.ids.shape[1]
    moved_tok = np.zeros(case.wl.T, bool)
    moved_tok[np.unique(tok[(moved != o.act).any(axis=1)])] = True
    assert not (B[~moved_tok] > 0).any()


@pytest.mark.parametrize("a8", [False, True])
def test_bound_rejects_larger_error(a8):
    """Codes moved by two steps in every block of one row (beyond what a 1-ulp
    act move can do): the bound computed for 1-ulp moves does not cover it."""
    case = _case(a8)
    o = _run(case)
    moved, _ = _moved_act(o, 0.01, 4)
    quant = oracle.quantize8 if a8 else oracle.quantize
    q, s = quant(moved)
    q = q.copy()
    row = int(np.argmax((moved != o.act).sum(axis=1)))
    if a8:
        q[row] = np.where((q[row] & 0x7F) < 0x70, q[row] + 16, q[row])
    else:
        q[row] ^= 0x44           # every magnitude code moved by four grid points
    o2 = _run(case, actq_in=q, acts_in=s)
    B = quant_step_bound(case, o, moved, np.ones(o.n_assign, bool))
    rms = np.sqrt(np.mean(o.out32.astype(np.float64) ** 2))
    d = np.abs(o2.out32.astype(np.float64) - o.out32)
    assert not (d <= TOL_REL_RMS * rms + B).all()
