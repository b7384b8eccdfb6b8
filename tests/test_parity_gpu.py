"""Parity of the HIP path (called through the C ABI) with the CPU oracle.

Bars: routing tables bit-exact (router weights within 2^-22); the x and SwiGLU
quantisations of the A4 path bit-exact; the bf16 SwiGLU intermediate >= 99.9%
bit-equal with every other element within 1 bf16 ulp; the output within
max|gpu - oracle out32| <= 2e-2 * rms(oracle out32).

Sizes: the five workloads at full size (the tiny and decode ones compared
whole; the larger ones on sampled tokens, which the oracle computes one by one)
plus scaled-down shapes that span several tiles and ragged tails in both
kernel variants, and the degenerate cases of the method.
"""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_router_amd as mx
from mxfp4_block_scaled_router_amd import workloads as W
from tests.gpu_helpers import (ACT_EQUAL_MIN, Case, bits_of, compare_act, compare_out,
                               compare_route, log, quant_step_bound, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.load_library()   # fails loudly if the HIP library is missing
    yield


def scaled(name, **kw):
    return W.WORKLOADS[name].replace(**kw)


SMALL_CASES = {
    "tiny": W.WORKLOADS["tiny"],
    "decode_T1": scaled("decode", T=1),
    "decode_T5_H256": scaled("decode", T=5, H=256, I=128, E_global=16, E_local=16, top_k=3),
    "ep_share_small": scaled("ep_share", T=64, H=512, I=256, E_global=64, E_local=16,
                             first_local=16),
    "mid_lds": W.Workload("mid_lds", 256, 1024, 512, 32, 16, 8, 4, seed=77),
    "prefill_small": scaled("prefill", T=1024, H=1024, I=384, E_global=16, E_local=16, top_k=4),
    "dense_E1": W.Workload("dense_E1", 40, 256, 128, 1, 1, 0, 1, seed=5),
    "all_experts": W.Workload("all_experts", 24, 256, 256, 6, 6, 0, 6, seed=6),
    "topk32": W.Workload("topk32", 8, 128, 128, 64, 64, 0, 32, seed=7),
    "no_clamp": W.Workload("no_clamp", 32, 512, 256, 8, 8, 0, 2, clamp_limit=float("inf"),
                           seed=8),
    # K of 56 and 48 k-tiles: the 16-row kernels' 7- and 6-k-tiles-per-wave
    # variants; 256 global experts: the routing kernel path (too many for the
    # fused one)
    "wide_h_e256": W.Workload("wide_h_e256", 4, 7168, 256, 256, 32, 64, 8, scale_lo=118,
                              scale_hi=124, seed=9),
    "wide_i": W.Workload("wide_i", 8, 256, 6144, 16, 16, 0, 2, scale_lo=118, scale_hi=124,
                         seed=10),
    # the fused routing's token masks at their limits: 32 tokens (mask bit 31)
    # on 64 local experts, 64 of 128 experts local from expert 32, and 33
    # tokens (past the fused routing)
    "masks_T32": W.Workload("masks_T32", 32, 256, 128, 64, 64, 0, 8, seed=11),
    "masks_ep_T24": W.Workload("masks_ep_T24", 24, 256, 128, 128, 64, 32, 4, seed=12),
    "T33": W.Workload("T33", 33, 256, 128, 64, 64, 0, 8, seed=13),
    # 32-row K-split tiles (64 tokens or more) under a skewed routing: hot
    # experts span several tiles, the last ones partial
    "skew_rows32": scaled("ep_share", T=128, H=512, I=256, E_global=64, E_local=64, first_local=0),
    # 64 tokens whose bf16 rows are too wide for two row blocks (K of 36
    # k-tiles): 16-row tiles with cached weight loads
    "wide_h_t64": W.Workload("wide_h_t64", 64, 4608, 256, 32, 32, 0, 4, seed=14),
}
A4_CASES = {
    "a4_tiny": W.WORKLOADS["a4"].replace(T=64, H=512, I=256, E_global=8, E_local=8, top_k=2),
    "a4_mid": W.WORKLOADS["a4"].replace(T=512, H=1024, I=512, E_global=16, E_local=16, top_k=4),
    # 32 rows per expert: the 64-row tiles
    "a4_rows32": W.WORKLOADS["a4"].replace(T=64, H=512, I=256, E_global=8, E_local=8, top_k=4),
    # 16-row kernels with 6 (gate_up, 48 k-tiles) and 7 (down, 56 k-tiles)
    # k-tiles per wave: a wave's scale bytes span up to three dwords
    "a4_wide": W.WORKLOADS["a4"].replace(T=4, H=6144, I=7168, E_global=4, E_local=4, top_k=2),
    # 320-row tiles with skewed routing: the hottest experts take several
    # tiles, a cold one a partial tile
    "a4_skew": W.WORKLOADS["a4"].replace(T=1024, H=512, I=256, E_global=16, E_local=16, top_k=4,
                                         logits_kind="zipf_bias"),
    # 320-row tiles at the widest K whose scale rows fit LDS: gate_up's rows of
    # 136 scale bytes (not a multiple of 16) take the 4-byte copies
    "a4_k4352": W.WORKLOADS["a4"].replace(T=128, H=4352, I=256, E_global=8, E_local=8, top_k=4),
    # down on the direct-weight 320 x 256 tiles (I a multiple of 512) with a
    # half last tile (H = 640: 2.5 tiles of 256 weight rows); gate_up (K = 640)
    # on the 320 x 128 tiles
    "a4_dw_partial": W.WORKLOADS["a4"].replace(T=512, H=640, I=512, E_global=16, E_local=16, top_k=4),
}
A8_CASES = {
    "a8_tiny": W.WORKLOADS["a8"].replace(T=64, H=512, I=256, E_global=8, E_local=8, top_k=2),
    "a8_mid": W.WORKLOADS["a8"].replace(T=512, H=1024, I=512, E_global=16, E_local=16, top_k=4),
    # 32 rows per expert: 128-row tiles (A8 has no 64-row kernels)
    "a8_rows32": W.WORKLOADS["a8"].replace(T=64, H=512, I=256, E_global=8, E_local=8, top_k=4),
    # decode dims, routing inside gate_up
    "a8_decode": W.WORKLOADS["a8"].replace(T=16, H=2048, I=1536, E_global=64, E_local=64, top_k=8),
    # 16-row kernels with 7 (gate_up) and 5 (down) k-tiles per wave
    "a8_wide": W.WORKLOADS["a8"].replace(T=4, H=7168, I=5120, E_global=4, E_local=4, top_k=2),
    "a8_skew": W.WORKLOADS["a8"].replace(T=1024, H=512, I=256, E_global=16, E_local=16, top_k=4,
                                         logits_kind="zipf_bias"),
}


def _check_case(case: Case, token_mask=None):
    log("case %s T=%d H=%d I=%d E=%d/%d k=%d a4=%d a8=%d det=%d shared=%d" % (
        case.wl.name, case.wl.T, case.wl.H, case.wl.I, case.wl.E_local, case.wl.E_global,
        case.wl.top_k, case.a4, case.a8, case.deterministic, case.shared))
    g = case.run_gpu(debug=True)
    o = case.run_oracle(token_mask=token_mask)
    rt = case.run_route()
    compare_route(rt, o)
    stats = {}
    mode = "a8" if case.a8 else "a4" if case.a4 else "bf16"
    if token_mask is None:
        stats.update(compare_act(bits_of(g["act"]), o.act, min_equal=ACT_EQUAL_MIN[mode]))
    if case.a4 or case.a8:
        # sorted positions of the compared tokens
        n = o.n_assign
        rows = (np.arange(n) if token_mask is None else
                np.nonzero(np.asarray(token_mask)[o.sorted // o.ids.shape[1]])[0])
        if token_mask is not None:
            stats.update(compare_act(bits_of(g["act"]), o.act, rows=rows,
                                     min_equal=ACT_EQUAL_MIN[mode]))
        tok = np.nonzero(token_mask)[0] if token_mask is not None else slice(None)
        np.testing.assert_array_equal(g["xq"].cpu().numpy()[tok], o.xq[tok])
        np.testing.assert_array_equal(g["xs"].cpu().numpy()[tok], o.xs[tok])
        # the GPU's act re-quantised by the oracle must equal the GPU's actq/acts
        gact = bits_of(g["act"])[:n][rows]
        quant = oracle.quantize8 if case.a8 else oracle.quantize
        q, s = quant(np.ascontiguousarray(gact))
        np.testing.assert_array_equal(g["actq"].cpu().numpy()[:n][rows], q)
        np.testing.assert_array_equal(g["acts"].cpu().numpy()[:n][rows], s)
        _a4_output_checks(case, g, o, token_mask, stats)
    elif token_mask is None:
        stats.update(compare_out(g, o))
    else:
        stats.update(compare_out(g, o, rows=np.nonzero(token_mask)[0]))
    log("  ok %s" % stats)
    return g, o


def _a4_output_checks(case, g, o, token_mask, stats):
    """A4 / A8 output parity, end to end against the oracle's own quantisation
    for every compared token.  Each side quantises its own SwiGLU output along
    I; the act comparison holds the GPU's act within a rounding of the
    oracle's, and an element that moved by a rounding can land on the other
    side of a quantisation boundary (or move its block's scale), after which
    the down inputs differ by a whole quantisation step.  The bar is therefore
    max |gpu32 - oracle out32| <= 2e-2 rms + B, where B (quant_step_bound) is
    the largest effect those moved elements can have, computed from the
    oracle's act, quantiser and w2 alone; B is zero for every token none of
    whose act elements moved.  Also: only rows whose act differs may get other
    codes, and with E2M1 (a step of a quarter of the block maximum, so a 1-ulp
    move rarely crosses it) such rows are rare.  The oracle's down and combine
    run on the GPU's own codes (given_actq) is reported as a diagnostic, not
    gated on."""
    n = o.n_assign
    gq = np.ascontiguousarray(g["actq"].cpu().numpy()[:n])
    gs = np.ascontiguousarray(g["acts"].cpu().numpy()[:n])
    slots = o.ids.shape[1]
    tok = o.sorted // slots                      # token of each sorted position
    checked = np.ones(n, bool) if token_mask is None else np.asarray(token_mask)[tok]
    # rows of experts kept in bf16 have no codes on the oracle's side
    div = ((gq != o.actq[:n]).any(axis=1) | (gs != o.acts[:n]).any(axis=1)) & checked & \
        ~case.excluded_rows(o)
    stats["actq_rows_diverging"] = int(div.sum())
    gact = bits_of(g["act"])[:n]
    act_differs = (gact != o.act[:n]).any(axis=1)
    assert not (div & ~act_differs).any(), stats
    if not case.a8:
        assert div.sum() <= max(2, n // 1000), stats
    slack = quant_step_bound(case, o, gact, checked)
    rows = None if token_mask is None else np.nonzero(token_mask)[0]
    e2e = compare_out(g, o, rows=rows, slack=slack)
    sel_tok = np.ones(case.wl.T, bool) if token_mask is None else np.asarray(token_mask, bool)
    stats["end_to_end_tokens"] = int(sel_tok.sum())
    stats["tokens_with_zero_slack"] = int((sel_tok & ~(slack > 0).any(axis=1)).sum())
    stats.update({"e2e_" + k: v for k, v in e2e.items()})
    # diagnostic: the oracle's down + combine on the GPU's codes
    o2 = case.run_oracle(token_mask=token_mask, actq_in=gq, acts_in=gs)
    d = compare_out(g, o2, rows=rows, slack=np.full((case.wl.T, case.wl.H), np.inf))
    stats["diag_given_actq_max_err_over_rms"] = d["max_raw_err_over_rms"]


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_forward_small(name):
    _check_case(Case(SMALL_CASES[name]))


@pytest.mark.parametrize("name", ["tiny", "decode_T5_H256", "mid_lds", "prefill_small", "skew_rows32"])
def test_forward_deterministic(name):
    case = Case(SMALL_CASES[name], deterministic=True)
    g1, o = _check_case(case)
    g2 = case.run_gpu()
    np.testing.assert_array_equal(bits_of(g1["out"]), bits_of(g2["out"]))


@pytest.mark.parametrize("name", ["decode", "verify_b1", "tiny"])
def test_fused_routing_matches_routing_kernel(name):
    """Decode shapes route inside gate_up, whose first workgroup also writes the
    down kernel's shares and first tiles; with the separate routing kernel
    (MXFP4_MOE_ROUTE_LAUNCH: down then reads the tile table itself) the ordered
    layer gives the same bits, act and out."""
    case = Case(W.WORKLOADS[name], deterministic=True)
    fused = case.run_gpu(debug=True)
    case.dims.flags |= mx.MXFP4_MOE_ROUTE_LAUNCH
    separate = case.run_gpu(debug=True)
    for k in ("act", "out"):
        np.testing.assert_array_equal(bits_of(fused[k]), bits_of(separate[k]))


@pytest.mark.parametrize("name", list(A4_CASES))
def test_forward_a4(name):
    case = Case(A4_CASES[name])
    assert case.quant_mismatch == 0
    _check_case(case)


def test_forward_tiny_full_and_decode_full():
    _check_case(Case(W.WORKLOADS["tiny"]))
    _check_case(Case(W.WORKLOADS["decode"]))


def _sample_mask(T, n, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros(T, bool)
    m[rng.choice(T, size=min(n, T), replace=False)] = True
    m[0] = m[T - 1] = True
    return m


@pytest.mark.parametrize("name", ["verify_b1", "verify_b8", "verify_b32", "verify_b48"])
def test_forward_verify_shapes(name):
    """Speculative-verify batches at full size, through the tile height each
    one is dispatched to (16-row tiles up to batch 32, 64-row at batch 48)."""
    case = Case(W.WORKLOADS[name])
    T = case.wl.T
    _check_case(case, token_mask=None if T <= 16 else _sample_mask(T, 24, 2))


SHARED_CASES = {
    "tiny": (W.WORKLOADS["tiny"], {}),
    "decode": (W.WORKLOADS["decode"], {}),                        # 16-row tiles, routing in gate_up
    "decode_det": (W.WORKLOADS["decode"], {"deterministic": True}),  # ordered gather, 9 slots
    "ep_share_small": (SMALL_CASES["ep_share_small"], {}),
    "mid_lds": (SMALL_CASES["mid_lds"], {}),                      # 64-row tiles
    "prefill_small": (SMALL_CASES["prefill_small"], {}),          # 128-row tiles
    "a4_tiny": (A4_CASES["a4_tiny"], {}),
    "a4_mid": (A4_CASES["a4_mid"], {}),
    # few tokens: the fused routing's token masks with the shared slot, A4 / A8
    "a4_wide": (A4_CASES["a4_wide"], {}),
    "a8_decode_det": (A8_CASES["a8_decode"], {"deterministic": True}),
}


@pytest.mark.parametrize("name", list(A8_CASES))
def test_forward_a8(name):
    """MXFP8 (E4M3) activations against MXFP4 weights, through 16- and 128-row
    tiles and the routing inside gate_up."""
    case = Case(A8_CASES[name])
    assert case.quant_mismatch == 0
    _check_case(case)


def test_forward_a8_shared_expert():
    _check_case(Case(A8_CASES["a8_mid"], shared=True))


def test_forward_a8_full_sampled():
    case = Case(W.WORKLOADS["a8"])
    assert case.quant_mismatch == 0
    _check_case(case, token_mask=_sample_mask(case.wl.T, 16, 4))


EXCLUSION_CASES = {
    # (workload, excluded experts of the weight buffers, Case options)
    "tiny": (W.WORKLOADS["tiny"], [1, 5], {}),
    "tiny_all": (W.WORKLOADS["tiny"], list(range(8)), {}),
    "decode": (W.WORKLOADS["decode"], [3, 17, 40, 63], {}),           # routing in gate_up
    "decode_det": (W.WORKLOADS["decode"], [0, 33], {"deterministic": True}),
    "decode_shared": (W.WORKLOADS["decode"], [5, 64], {"shared": True}),  # the shared one too
    "ep_share_small": (SMALL_CASES["ep_share_small"], [2, 9], {}),
    "mid_lds": (SMALL_CASES["mid_lds"], [0, 7, 12], {}),             # 64-row tiles
    "prefill_small": (SMALL_CASES["prefill_small"], [4, 11], {}),    # 128-row tiles
    "a4_mid": (A4_CASES["a4_mid"], [2, 9], {}),
    "a8_mid": (A8_CASES["a8_mid"], [6], {}),
    "a8_decode": (A8_CASES["a8_decode"], [1, 30], {}),
}


@pytest.mark.parametrize("name", list(EXCLUSION_CASES))
def test_forward_bf16_exclusions(name):
    """Experts kept in bf16 inside fused expert buffers: the fused loader, the
    routing without their tiles and the bf16 expert kernels, through each tile
    height, both combines, A4/A8 and the shared expert."""
    wl, ex, kw = EXCLUSION_CASES[name]
    case = Case(wl, excluded=ex, **kw)
    log("excluded %s" % (list(np.nonzero(case.excluded)[0]),))
    _check_case(case)


def test_forward_bf16_exclusions_prefill_sampled():
    case = Case(W.WORKLOADS["prefill"], excluded=[0, 64, 127])
    _check_case(case, token_mask=_sample_mask(case.wl.T, 24, 5))


def test_preshuffle_fused_matches_preshuffle():
    """The fused loader: packed experts' preshuffled slots equal
    mxfp4_moe_preshuffle's, the bf16 buffers hold the excluded experts in order,
    and the expert map lists both directions."""
    wl = W.WORKLOADS["tiny"]
    excluded = [0, 3, 4, 7]
    plain = Case(wl)
    fused = Case(wl, inp=plain.inp, excluded=excluded)
    sizes = mx.mxfp4_moe_preshuffled_bytes(plain.dims)
    for i, n in enumerate(("w13", "w13s", "w2", "w2s")):
        per = sizes[i] // wl.E_local
        a = plain.pw[i].view(wl.E_local, per).cpu().numpy()
        b = fused.pw[i].view(wl.E_local, per).cpu().numpy()
        keep = ~fused.excluded
        np.testing.assert_array_equal(a[keep], b[keep], err_msg=n)
    ow = fused.oracle_w
    np.testing.assert_array_equal(bits_of(fused.bx["w13"]).reshape(ow["w13_bf16"].shape),
                                  ow["w13_bf16"])
    np.testing.assert_array_equal(bits_of(fused.bx["w2"]).reshape(ow["w2_bf16"].shape),
                                  ow["w2_bf16"])
    m = fused.bx["expert_map"].cpu().numpy()
    expect = [-1] * 8
    for j, e in enumerate(excluded):
        expect[e] = j
    np.testing.assert_array_equal(m, expect + excluded)


@pytest.mark.parametrize("name", list(SHARED_CASES))
def test_forward_shared_expert(name):
    """The shared expert: one more MXFP4 expert that every token reads with
    weight 1, through each tile height, the A4 path and both combines."""
    wl, kw = SHARED_CASES[name]
    case = Case(wl, shared=True, **kw)
    _check_case(case)


def test_forward_ep_share_full_sampled():
    case = Case(W.WORKLOADS["ep_share"])
    _check_case(case, token_mask=_sample_mask(case.wl.T, 48, 1))


def test_ep_shares_sum_to_full_layer():
    """Four expert-parallel shares (first_local = 0, 16, 32, 48 of 64) summed
    equal the whole layer within the tolerance."""
    full_wl = W.Workload("ep4", 48, 512, 256, 64, 64, 0, 8, seed=31)
    inp = W.make_inputs(full_wl)
    full = Case(full_wl, inp=inp)
    o = full.run_oracle()
    acc = np.zeros((full_wl.T, full_wl.H), np.float64)
    for f in range(0, 64, 16):
        sub = dict(inp)
        for k in ("w13", "w13s", "w2", "w2s"):
            sub[k] = inp[k][f:f + 16]
        wl = full_wl.replace(E_local=16, first_local=f)
        c = Case(wl, inp=sub)
        log("share first_local=%d" % f)
        g = c.run_gpu(debug=False)
        acc += (g["out"].float().cpu().numpy()).astype(np.float64)
    rms = np.sqrt(np.mean(o.out32.astype(np.float64) ** 2))
    assert np.abs(acc - o.out32).max() <= 4 * 2e-2 * rms


def test_ep_shares_sum_to_full_layer_full_shape():
    """Expert parallelism at the expert-parallel share's real shape: the four
    shares (first_local = 0, 64, 128, 192) of 256 global experts at T = 256,
    H = 5120, I = 1536, each run through the C ABI on its own 64 experts,
    summed; compared on sampled tokens with the oracle's whole 256-expert
    layer.  The fp32 partial outputs sum to the layer within the bar; the sum
    of the four bf16 partial outputs within four roundings more."""
    base = W.WORKLOADS["ep_share"]
    full_wl = base.replace(name="ep_full", E_local=256)
    inp = W.make_inputs(full_wl)
    mask = _sample_mask(full_wl.T, 12, 7)
    log("oracle: whole layer, 256 experts, %d sampled tokens" % mask.sum())
    o = oracle.moe_forward(inp["x"], inp["logits"], inp["w13"], inp["w13s"], inp["w2"], inp["w2s"],
                           top_k=full_wl.top_k, clamp_limit=full_wl.clamp_limit, E_global=256,
                           first_local=0, token_mask=mask, want_act=False)
    acc32 = np.zeros((full_wl.T, full_wl.H), np.float64)
    acc16 = np.zeros((full_wl.T, full_wl.H), np.float64)
    for f in range(0, 256, 64):
        sub = {"x": inp["x"], "logits": inp["logits"]}
        for k in ("w13", "w13s", "w2", "w2s"):
            sub[k] = inp[k][f:f + 64]
        wl = base.replace(first_local=f)
        log("share first_local=%d" % f)
        c = Case(wl, inp=sub)
        g = c.run_gpu(debug=True)
        acc32 += g["out32"].cpu().numpy().astype(np.float64)
        acc16 += g["out"].float().cpu().numpy().astype(np.float64)
        del c, g
        torch.cuda.empty_cache()
    rows = np.nonzero(mask)[0]
    ref = o.out32[rows].astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err32 = np.abs(acc32[rows] - ref).max()
    err16 = np.abs(acc16[rows] - ref).max()
    log("  fp32 partials max err / rms %.3e, bf16 partials %.3e" % (err32 / rms, err16 / rms))
    assert err32 <= 2e-2 * rms
    assert err16 <= 4 * 2e-2 * rms


def test_forward_prefill_full_sampled():
    case = Case(W.WORKLOADS["prefill"])
    _check_case(case, token_mask=_sample_mask(case.wl.T, 24, 2))


def test_forward_a4_full_sampled():
    case = Case(W.WORKLOADS["a4"])
    assert case.quant_mismatch == 0
    _check_case(case, token_mask=_sample_mask(case.wl.T, 16, 3))


def test_route_tables_full_sizes():
    """Routing tables at full sizes against the oracle: the one-workgroup
    routing (decode), the three routing kernels at mid sizes (ep_share, verify
    batches 16 and 48) and at prefill sizes."""
    extra = {
        # the chunked kernels with a wave per token: 24 picks of 128 experts
        # (two logits per lane, picks past 16), and 512 experts (eight per lane)
        "e128_k24": W.Workload("e128_k24", 64, 256, 128, 128, 32, 96, 24, seed=61),
        "e512_k4": W.Workload("e512_k4", 48, 256, 128, 512, 64, 0, 4, seed=62),
    }
    for name in ("decode", "ep_share", "verify_b16", "verify_b48", "prefill", "a4", "e128_k24",
                 "e512_k4"):
        wl = extra[name] if name in extra else W.WORKLOADS[name]
        inp = W.make_inputs(wl, weights=False)
        dims = mx.Dims.make(wl.T, wl.H, wl.I, wl.E_global, wl.E_local, wl.first_local)
        log("route %s" % name)
        r = mx.mxfp4_moe_route(dims, to_dev(inp["logits"]), wl.top_k)
        torch.cuda.synchronize()
        r = {k: v.cpu().numpy() for k, v in r.items()}
        ids, w = oracle.route(inp["logits"], wl.top_k)
        counts, offsets, sorted_, inv = oracle.permute(ids, wl.first_local, wl.E_local)

        class O:
            pass
        o = O()
        o.ids, o.w, o.counts, o.offsets, o.sorted, o.inv = ids, w, counts, offsets, sorted_, inv
        compare_route(r, o)


def test_quantize_bit_exact():
    rng = np.random.default_rng(17)
    v = (rng.standard_normal((257, 512)) * np.exp2(rng.integers(-30, 30, size=(257, 1)))).astype(
        np.float32)
    v[3, 5] = np.nan
    v[4, 70] = np.inf
    v[5, :32] = 0.0
    v[5, 3] = -0.0
    v[6, :] = np.float32(2.0 ** -130)      # subnormal block
    v[7, 40] = 3.0e38
    # grid midpoints times powers of two
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], np.float32)
    v[8, :32] = np.tile(mids, 4) * 2.0 ** -3
    for dt in ("f32", "bf16"):
        if dt == "f32":
            vin = v
            gc, gs = mx.mxfp4_moe_quantize(torch.from_numpy(vin).cuda())
            oc, os_ = oracle.quantize(vin)
        else:
            bits = (v.view(np.uint32) >> 16).astype(np.uint16)
            gc, gs = mx.mxfp4_moe_quantize(
                torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
            oc, os_ = oracle.quantize(bits)
        np.testing.assert_array_equal(gc.cpu().numpy(), oc)
        np.testing.assert_array_equal(gs.cpu().numpy(), os_)


def test_quantize_every_bf16_value():
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    rows = allb.reshape(-1, 32)           # 2048 blocks, each a run of consecutive codes
    gc, gs = mx.mxfp4_moe_quantize(torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).cuda())
    oc, os_ = oracle.quantize(np.ascontiguousarray(rows))
    np.testing.assert_array_equal(gc.cpu().numpy(), oc)
    np.testing.assert_array_equal(gs.cpu().numpy(), os_)


def test_quantize8_bit_exact():
    """The GPU's MXFP8 quantiser equals the oracle's: random rows over a wide
    range of scales, special blocks, and every bf16 value in blocks whose
    largest element sits 0, 4 or 9 binades above it."""
    rng = np.random.default_rng(19)
    v = (rng.standard_normal((257, 512)) * np.exp2(rng.integers(-30, 30, size=(257, 1)))).astype(
        np.float32)
    v[3, 5] = np.nan
    v[4, 70] = np.inf
    v[5, :32] = 0.0
    v[5, 3] = -0.0
    v[6, :] = np.float32(2.0 ** -130)
    v[7, 40] = 3.0e38
    gc, gs = mx.mxfp4_moe_quantize8(torch.from_numpy(v).cuda())
    oc, os_ = oracle.quantize8(v.astype(np.float64))
    np.testing.assert_array_equal(gc.cpu().numpy(), oc)
    np.testing.assert_array_equal(gs.cpu().numpy(), os_)
    allb = np.arange(1 << 16, dtype=np.uint32)
    f = (allb << 16).view(np.float32)
    fin = np.isfinite(f) & (np.abs(f) < 2.0 ** 118)     # anchors stay finite
    for shift in (0, 4, 9):
        vals = f[fin]
        e = np.floor(np.log2(np.maximum(np.abs(vals), np.float32(1e-45))))
        anchor = np.ldexp(np.float32(1.0), (e + shift).astype(np.int64)).astype(np.float32)
        blocks = np.repeat(vals[:, None], 32, axis=1)
        blocks[:, 0] = np.where(vals != 0, anchor, 0.0)
        bits = (blocks.view(np.uint32) >> 16).astype(np.uint16)
        gc, gs = mx.mxfp4_moe_quantize8(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
        oc, os_ = oracle.quantize8(np.ascontiguousarray(bits))
        np.testing.assert_array_equal(gc.cpu().numpy(), oc)
        np.testing.assert_array_equal(gs.cpu().numpy(), os_)


def test_t_zero_is_a_noop():
    wl = W.Workload("t1", 1, 256, 128, 8, 8, 0, 2, seed=3)
    case = Case(wl)
    dims = mx.Dims.make(0, 256, 128, 8, 8)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    out = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_moe_forward(dims, x, lg, *case.pw, 2, 7.0, out=out)
    torch.cuda.synchronize()


def test_all_nonlocal_share_gives_zero_output():
    wl = W.Workload("nonlocal", 20, 256, 128, 16, 4, 12, 2, seed=9)
    inp = W.make_inputs(wl)
    inp["logits"][:, 12:] -= 100.0          # nobody picks experts 12..15
    case = Case(wl, inp=inp)
    g, o = _check_case_zero(case)


def _check_case_zero(case):
    g = case.run_gpu()
    o = case.run_oracle()
    assert o.n_assign == 0
    assert (bits_of(g["out"]) & 0x7FFF == 0).all()
    return g, o


def test_nan_scale_poisons_routed_rows():
    wl = W.Workload("nan", 40, 256, 128, 8, 8, 0, 2, seed=31)
    inp = W.make_inputs(wl)
    inp["w13s"][3, 17, 2] = 255
    case = Case(wl, inp=inp)
    g = case.run_gpu()
    o = case.run_oracle()
    out = bits_of(g["out"])
    outf = (out.astype(np.uint32) << 16).view(np.float32)
    routed = (o.ids == 3).any(axis=1)
    assert routed.any() and (~routed).any()
    assert np.isnan(outf[routed]).all()
    assert np.isfinite(outf[~routed]).all()


def test_tamper_control_fails_parity():
    """A flipped code byte of a routed expert must make the output check fail."""
    wl = W.Workload("tamper", 32, 512, 256, 8, 8, 0, 2, seed=41)
    inp = W.make_inputs(wl)
    o = Case(wl, inp=inp).run_oracle()
    e = int(o.ids[0, 0])
    bad = dict(inp)
    bad["w2"] = inp["w2"].copy()
    bad["w2"][e, :, :] ^= 0x77
    g = Case(wl, inp=bad).run_gpu(debug=True)
    with pytest.raises(AssertionError):
        compare_out(g, o)
