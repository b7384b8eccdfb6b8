"""The one-pass load-time conversion (mxfp4_moe_quantize_preshuffle): its output
equals mxfp4_moe_preshuffle applied to the oracle's canonical MXFP4 codes of
the same weights, byte for byte, from fp32 and from bf16; and a layer on the
converted weights passes parity with the oracle on those codes."""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_router_amd as mx
from mxfp4_block_scaled_router_amd import workloads as W
from tests.gpu_helpers import Case, compare_out, compare_route, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.load_library()
    yield


def _weights(wl, E):
    w13 = torch.stack([W.student_t_expert(wl, e, "w13", device="cuda") for e in range(E)])
    w2 = torch.stack([W.student_t_expert(wl, e, "w2", device="cuda") for e in range(E)])
    return w13, w2


# K of 512 (one scale group), 640 (a padded second group) and 1536 with 128 rows
@pytest.mark.parametrize("H,I,E,shared", [(512, 256, 4, False), (640, 384, 3, True), (1536, 128, 2, False)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_preshuffle_bytes(H, I, E, shared, dtype):
    wl = W.WORKLOADS["a4"].replace(T=8, H=H, I=I, E_global=E, E_local=E, top_k=1)
    dims = mx.Dims.make(8, H, I, E, E, 0, shared=shared)
    Ew = E + (1 if shared else 0)
    w13, w2 = _weights(wl, Ew)
    if dtype == "bf16":
        w13, w2 = w13.to(torch.bfloat16), w2.to(torch.bfloat16)
        host = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        host = lambda t: t.cpu().numpy()
    log("quantize_preshuffle H=%d I=%d E=%d shared=%d %s" % (H, I, E, shared, dtype))
    got = mx.mxfp4_moe_quantize_preshuffle(dims, w13, w2)
    c13, s13 = oracle.quantize(host(w13))
    c2, s2 = oracle.quantize(host(w2))
    ref = mx.mxfp4_moe_preshuffle(dims, *[torch.from_numpy(a).cuda() for a in (c13, s13, c2, s2)])
    torch.cuda.synchronize()
    for g, r, n in zip(got, ref, ("w13", "w13s", "w2", "w2s")):
        np.testing.assert_array_equal(g.cpu().numpy(), r.cpu().numpy(), err_msg=n)


def test_forward_on_converted_weights():
    """A4 layer on weights converted in one pass, against the oracle run on its
    own quantisation of the same fp32 weights."""
    wl = W.WORKLOADS["a4"].replace(T=64, H=512, I=256, E_global=8, E_local=8, top_k=2)
    case = Case(wl)                            # oracle codes of the same Student-t draws
    w13, w2 = _weights(wl, wl.E_local)
    case.pw = mx.mxfp4_moe_quantize_preshuffle(case.dims, w13, w2)
    g = case.run_gpu(debug=True)
    o = case.run_oracle()
    compare_route(case.run_route(), o)
    # the GPU's act codes equal the oracle's quantiser on the GPU's act, and
    # the output is checked end to end as in the other A4 cases
    from tests.test_parity_gpu import _a4_output_checks
    stats = {}
    _a4_output_checks(case, g, o, None, stats)
    log("  ok %s" % stats)
