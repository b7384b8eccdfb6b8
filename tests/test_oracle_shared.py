"""Pins for the oracle's shared expert: an always-active MXFP4 MLP that every
token reads with weight 1, as one more slot after its k routed picks.  Checked
against the routing tables' definition, a NumPy fp64 dense MLP (the shared
expert alone is a dense layer), the routed layer without it, and a zero
expert."""
import numpy as np

import oracle
from mxfp4_block_scaled_router_amd import workloads as wlmod

from .test_oracle_moe import _bf16_to_f64, _decode_np


def _inputs(T=24, H=256, I=128, E=6, Eg=None, k=2, seed=91):
    """Routed experts' weights plus one more expert (the shared one) appended."""
    Eg = Eg or E
    wl = wlmod.Workload("shared", T, H, I, Eg, E + 1, 0, k, seed=seed)
    inp = wlmod.make_inputs(wl)
    inp["logits"] = np.ascontiguousarray(inp["logits"][:, :Eg])
    return inp


def _run(inp, k, shared, **kw):
    return oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"],
                              inp["w2s"], top_k=k, clamp_limit=7.0, shared=shared, **kw)


def _routed_only(inp):
    return {n: np.ascontiguousarray(inp[n][:-1]) for n in ("w13", "w13s", "w2", "w2s")}


def _dense_mlp_fp64(x_bits, w13, w13s, w2, w2s, I, L=7.0):
    x = _bf16_to_f64(x_bits)
    h = x @ _decode_np(w13, w13s).T
    g = np.minimum(h[:, :I], L)
    u = np.clip(h[:, I:], -L, L)
    return g / (1 + np.exp(-g)) * u, _decode_np(w2, w2s)


def test_shared_slot_tables():
    inp = _inputs()
    T, k, E = 24, 2, 6
    r = _run(inp, k, True)
    base = _run(dict(inp, **_routed_only(inp)), k, False)
    assert r.ids.shape == (T, k + 1)
    np.testing.assert_array_equal(r.ids[:, :k], base.ids)
    assert (r.ids[:, k] == E).all() and (r.w[:, k] == 1.0).all()
    np.testing.assert_array_equal(r.w[:, :k], base.w)
    np.testing.assert_array_equal(r.counts[:E], base.counts)
    assert r.counts[E] == T and r.n_assign == base.n_assign + T
    o = r.offsets[E]
    np.testing.assert_array_equal(r.sorted[o:o + T], np.arange(T) * (k + 1) + k)
    np.testing.assert_array_equal(r.inv.reshape(T, k + 1)[:, k], o + np.arange(T))


def test_shared_alone_is_a_dense_mlp():
    """No routed pick is local (E_local = 1 holds expert 7, which the logits
    never pick), so the output is the shared MLP alone, against NumPy fp64."""
    T, H, I = 32, 256, 128
    wl = wlmod.Workload("s1", T, H, I, 8, 2, 7, 2, seed=92)
    inp = wlmod.make_inputs(wl)
    inp["logits"][:, 7] = -50.0
    r = oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"],
                           inp["w2s"], top_k=2, clamp_limit=7.0, first_local=7, shared=True)
    assert r.n_assign == T and r.counts[0] == 0 and r.counts[1] == T
    a64, W2 = _dense_mlp_fp64(inp["x"], inp["w13"][1], inp["w13s"][1], inp["w2"][1],
                              inp["w2s"][1], I)
    act = _bf16_to_f64(r.act)                    # the shared segment, tokens in order
    assert np.abs(act - a64).max() <= np.abs(a64).max() * 2.0 ** -7
    y = act @ W2.T
    rms = np.sqrt((y ** 2).mean())
    assert np.abs(r.out32 - y).max() < 1e-5 * rms * np.sqrt(I)


def test_shared_adds_its_mlp_to_the_routed_layer():
    inp = _inputs(T=20, H=256, I=128, E=6, k=3)
    I = 128
    r = _run(inp, 3, True)
    base = _run(dict(inp, **_routed_only(inp)), 3, False)
    n = base.n_assign
    # routed rows of act are bit-identical; the shared segment comes last
    np.testing.assert_array_equal(r.act[:n], base.act)
    _, W2 = _dense_mlp_fp64(inp["x"], inp["w13"][-1], inp["w13s"][-1], inp["w2"][-1],
                            inp["w2s"][-1], I)
    y = _bf16_to_f64(r.act[n:]) @ W2.T           # fp64 down of the oracle's shared act
    diff = r.out32.astype(np.float64) - base.out32.astype(np.float64) - y
    scale = np.abs(base.out32).max() + np.abs(y).max()
    assert np.abs(diff).max() <= 4 * 2.0 ** -24 * scale + 1e-5 * np.sqrt((y ** 2).mean()) * np.sqrt(I)


def test_zero_shared_expert_changes_nothing():
    inp = _inputs(T=16, k=2)
    inp["w2"] = inp["w2"].copy()
    inp["w2"][-1] = 0                             # E2M1 code 0 = +0: y_shared = +0
    r = _run(inp, 2, True)
    base = _run(dict(inp, **_routed_only(inp)), 2, False)
    assert (r.out32 == base.out32).all()
    np.testing.assert_array_equal(r.out, base.out)
