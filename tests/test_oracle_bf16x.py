"""Pins for the oracle's per-expert bf16 exclusions: the fused-buffer split
(hand-computed offsets, the single-stride misread, round trips), an excluded
expert whose bf16 weights equal its decoded MXFP4 weights (bit-identical layer),
the A4/A8 modes leaving excluded rows unquantised, and an all-excluded layer
against a NumPy fp64 dense MLP."""
import numpy as np
import pytest

import oracle
from mxfp4_block_scaled_router_amd import workloads as wlmod

from .test_oracle_moe import _bf16_to_f64, _decode_np


def test_unfuse_offsets_follow_each_experts_dtype():
    """E = 3, expert 1 in bf16, R = 2 rows of K = 64: packed experts take
    2*64/2 = 64 bytes, the bf16 one 2*64*2 = 256, so the experts start at bytes
    0, 64 and 320; the scale tensor has 4 bytes for each packed expert only."""
    R, K = 2, 64
    fused = np.concatenate([np.full(64, 0x11, np.uint8), np.full(256, 0x22, np.uint8),
                            np.full(64, 0x33, np.uint8)])
    fs = np.concatenate([np.full(4, 0x70, np.uint8), np.full(4, 0x71, np.uint8)])
    codes, scales, bf = oracle.unfuse(fused, fs, [False, True, False], R, K)
    assert (codes[0] == 0x11).all() and (codes[2] == 0x33).all() and (codes[1] == 0).all()
    assert (scales[0] == 0x70).all() and (scales[2] == 0x71).all()
    assert bf.shape == (1, R, K) and (bf[0] == 0x2222).all()
    # one stride for the whole buffer (the packed one) misreads every expert
    # after the bf16 one: expert 2 would start inside expert 1
    single = fused.reshape(-1)[2 * 64:3 * 64]
    assert (single == 0x22).all()
    with pytest.raises(ValueError):
        oracle.unfuse(fused[:-1], fs, [False, True, False], R, K)
    with pytest.raises(ValueError):
        oracle.unfuse(fused, fs, [False, False, False], R, K)


@pytest.mark.parametrize("excluded", [[0, 1, 0, 0, 1, 0], [1, 0, 0, 0, 0, 0], [0] * 6, [1] * 6])
def test_fuse_unfuse_round_trip(excluded):
    rng = np.random.default_rng(sum(excluded) + 3)
    E, R, K = 6, 48, 128
    ex = np.array(excluded, bool)
    codes = rng.integers(0, 256, (E, R, K // 2), dtype=np.uint8)
    scales = rng.integers(100, 130, (E, R, K // 32), dtype=np.uint8)
    codes[ex] = 0
    scales[ex] = 0
    bf = rng.integers(0, 1 << 16, (int(ex.sum()), R, K), dtype=np.uint16)
    fused, fs = wlmod.fuse(codes, scales, bf, ex)
    assert fused.size == (E - ex.sum()) * R * K // 2 + ex.sum() * R * K * 2
    c2, s2, b2 = oracle.unfuse(fused, fs, ex, R, K)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(b2, bf)


def _decoded_as_bf16(codes, scales):
    """The expert's MXFP4 values as bf16 bits (exact: E2M1 values times a power
    of two in bf16's range are bf16 values)."""
    v = _decode_np(codes, scales).astype(np.float32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert ((bits.astype(np.uint32) << 16) == v.view(np.uint32)).all()
    return bits


def _layer(inp, k, **kw):
    return oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"],
                              inp["w2s"], top_k=k, clamp_limit=7.0, **kw)


def _exclusions(inp, excluded):
    ex = np.array(excluded, bool)
    idx = np.nonzero(ex)[0]
    b13 = np.stack([_decoded_as_bf16(inp["w13"][e], inp["w13s"][e]) for e in idx]) if idx.size \
        else np.zeros((0,) + inp["w13"].shape[1:-1] + (inp["w13"].shape[-1] * 2,), np.uint16)
    b2 = np.stack([_decoded_as_bf16(inp["w2"][e], inp["w2s"][e]) for e in idx]) if idx.size \
        else np.zeros((0,) + inp["w2"].shape[1:-1] + (inp["w2"].shape[-1] * 2,), np.uint16)
    return dict(bf16_experts=ex, w13_bf16=b13, w2_bf16=b2)


@pytest.mark.parametrize("shared", [False, True])
def test_excluded_expert_with_its_decoded_weights_changes_nothing(shared):
    """W4A16: an expert read from bf16 weights equal to its decoded MXFP4 values
    gives the same layer bit for bit (a transposed or misaligned bf16 read, or a
    dropped expert, would not); its MXFP4 slots are ignored (garbage there)."""
    wl = wlmod.Workload("x", 24, 256, 128, 6, 6 + (1 if shared else 0), 0, 2, seed=41)
    inp = wlmod.make_inputs(wl)
    inp["logits"] = np.ascontiguousarray(inp["logits"][:, :6])
    base = _layer(inp, 2, E_global=6, shared=shared)
    excluded = [0, 1, 0, 0, 1, 0] + ([1] if shared else [])
    kw = _exclusions(inp, excluded)
    garbage = dict(inp)
    for n in ("w13", "w2"):
        garbage[n] = inp[n].copy()
        garbage[n][np.array(excluded, bool)] = 0xFF
    r = _layer(garbage, 2, E_global=6, shared=shared, **kw)
    assert (np.array(excluded) == 1).any() and base.n_assign == r.n_assign
    np.testing.assert_array_equal(r.act, base.act)
    np.testing.assert_array_equal(r.out32.view(np.uint32), base.out32.view(np.uint32))


@pytest.mark.parametrize("mode", ["a4", "a8"])
def test_excluded_experts_skip_activation_quantisation(mode):
    """A4/A8: rows of excluded experts are computed from the bf16 x and the bf16
    SwiGLU output, so they equal the W4A16 layer's rows and leave actq/acts
    untouched; a token whose one pick is excluded gets the W4A16 output."""
    wl = wlmod.Workload("x", 32, 256, 128, 4, 4, 0, 1, seed=43)
    inp = wlmod.make_inputs(wl)
    excluded = [1, 0, 1, 0]
    kw = _exclusions(inp, excluded)
    q = _layer(inp, 1, **{mode: True}, **kw)
    plain = _layer(inp, 1, **kw)
    full_q = _layer(inp, 1, **{mode: True})
    ex_pos = np.zeros(q.n_assign, bool)
    for e in (0, 2):
        ex_pos[q.offsets[e]:q.offsets[e + 1]] = True
    assert ex_pos.any() and (~ex_pos).any()
    np.testing.assert_array_equal(q.act[ex_pos], plain.act[ex_pos])
    assert (q.actq[ex_pos] == 0).all() and (q.acts[ex_pos] == 0).all()
    # packed experts' rows are those of the all-packed quantised layer
    np.testing.assert_array_equal(q.act[~ex_pos], full_q.act[~ex_pos])
    np.testing.assert_array_equal(q.actq[~ex_pos], full_q.actq[~ex_pos])
    tok_ex = np.isin(q.ids[:, 0], [0, 2])
    np.testing.assert_array_equal(q.out32[tok_ex], plain.out32[tok_ex])
    np.testing.assert_array_equal(q.out32[~tok_ex], full_q.out32[~tok_ex])


def test_all_excluded_layer_is_a_dense_bf16_mlp():
    """One expert, kept in bf16, every token on it with weight 1: the layer is a
    dense MLP; against NumPy fp64 on the same bf16 weights (act within its bf16
    rounding, out32 within fp32 accumulation of the oracle's own act)."""
    T, H, I = 20, 256, 128
    wl = wlmod.Workload("x", T, H, I, 1, 1, 0, 1, seed=45)
    inp = wlmod.make_inputs(wl)
    b13 = wlmod.bf16_expert(wl, 0, "w13")[None]
    b2 = wlmod.bf16_expert(wl, 0, "w2")[None]
    r = _layer(inp, 1, bf16_experts=[True], w13_bf16=b13, w2_bf16=b2)
    assert r.n_assign == T and (r.w == 1.0).all()
    x = _bf16_to_f64(inp["x"])
    h = x @ _bf16_to_f64(b13[0]).T
    g = np.minimum(h[:, :I], 7.0)
    u = np.clip(h[:, I:], -7.0, 7.0)
    a64 = g / (1 + np.exp(-g)) * u
    act = _bf16_to_f64(r.act)[np.argsort(r.sorted)]      # sorted position -> token order
    assert np.abs(act - a64).max() <= np.abs(a64).max() * 2.0 ** -7
    W2 = _bf16_to_f64(b2[0])
    y = act @ W2.T
    bound = 2.0 ** -22 * I * (np.abs(act) @ np.abs(W2).T)
    assert (np.abs(r.out32 - y) <= bound + 1e-30).all()
