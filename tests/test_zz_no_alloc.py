"""mxfp4_moe_forward_noalloc (workspace = the library's static per-GPU scratch)
against mxfp4_moe_forward with a caller workspace, called through the C ABI:
two calls in a row, the second on a smaller input, in both combine modes."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_router_amd as mx
from mxfp4_block_scaled_router_amd import workloads as W
from tests.gpu_helpers import TOL_REL_RMS, Case, bits_of, bf16_to_f32, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.load_library()
    yield


def _both(case: Case, T: int):
    """Both entry points on the first T tokens of the case."""
    wl = case.wl
    dims = mx.Dims.make(T, wl.H, wl.I, wl.E_global, wl.E_local, wl.first_local,
                        deterministic=case.deterministic)
    x, lg = case.x[:T].contiguous(), case.logits[:T].contiguous()
    ref = mx.mxfp4_moe_forward(dims, x, lg, *case.pw, wl.top_k, wl.clamp_limit)
    out = torch.full((T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
    mx.mxfp4_moe_forward_noalloc(dims, x, lg, *case.pw, wl.top_k, wl.clamp_limit, out)
    torch.cuda.synchronize()
    return bits_of(out), bits_of(ref)


@pytest.mark.parametrize("name,deterministic", [("decode", True), ("decode", False),
                                                ("verify_b8", True), ("ep_share", False)])
def test_noalloc_matches_forward(name, deterministic):
    case = Case(W.WORKLOADS[name], deterministic=deterministic)
    T = case.wl.T
    for t in (T, max(1, T // 3)):             # the second call is smaller
        log("noalloc %s T=%d deterministic=%d" % (name, t, deterministic))
        got, ref = _both(case, t)
        if deterministic:
            np.testing.assert_array_equal(got, ref)
        else:
            g, r = bf16_to_f32(got).astype(np.float64), bf16_to_f32(ref).astype(np.float64)
            assert np.isfinite(g).all()
            rms = np.sqrt(np.mean(r ** 2))
            assert np.abs(g - r).max() <= TOL_REL_RMS * rms


def test_noalloc_refuses_beyond_scratch():
    wl = W.WORKLOADS["prefill"]
    dims = mx.Dims.make(wl.T, wl.H, wl.I, wl.E_global, wl.E_local)
    with pytest.raises(mx.MoEError) as ei:
        mx.mxfp4_moe_forward_noalloc(dims, torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda"),
                                     torch.zeros((wl.T, wl.E_global), device="cuda"), 0, 0, 0, 0,
                                     wl.top_k, wl.clamp_limit,
                                     torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda"))
    assert "SCRATCH_LIMIT" in str(ei.value)
