"""Execution contract of the C ABI on the GPU: calls on two streams with their
own workspaces run concurrently and give the results of sequential calls, and
a forward recorded into a HIP graph gives the eager result on every replay.
Deterministic (slot-ordered) combine, so results compare bit for bit."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_router_amd as mx
from mxfp4_block_scaled_router_amd import workloads as W
from tests.gpu_helpers import Case, bits_of, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.load_library()
    yield


def _forward(case, logits, out, ws):
    wl = case.wl
    mx.mxfp4_moe_forward(case.dims, case.x, logits, *case.pw, wl.top_k, wl.clamp_limit, out=out,
                         workspace=ws)


# MXFP4 activations on the direct-weight 320 x 256 tiles (x and SwiGLU-output
# quantisation, chunked routing, both tile GEMMs and the ordered gather)
EXTRA = {"a4_dw": W.WORKLOADS["a4"].replace(T=512, H=1024, I=512, E_global=16, E_local=16, top_k=4)}


def _setup(name):
    case = Case(EXTRA[name] if name in EXTRA else W.WORKLOADS[name], deterministic=True)
    wl = case.wl
    ws = torch.empty(mx.mxfp4_moe_workspace_bytes(case.dims, wl.top_k), dtype=torch.uint8,
                     device="cuda")
    # three batches of router logits: the case's own and two permutations of its tokens
    gen = torch.Generator(device="cpu").manual_seed(7)
    lgs = [case.logits] + [case.logits[torch.randperm(wl.T, generator=gen).cuda()].contiguous()
                           for _ in range(2)]
    outs = [torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device="cuda") for _ in lgs]
    return case, ws, lgs, outs


def test_two_streams_run_concurrently():
    """decode (routing inside gate_up) and verify_b8 (separate routing kernels)
    enqueued alternately on two streams, each with its own workspace."""
    a = _setup("decode")
    b = _setup("verify_b8")
    ref = []
    for case, ws, lgs, outs in (a, b):
        for lg, o in zip(lgs, outs):
            _forward(case, lg, o, ws)
        torch.cuda.synchronize()
        ref.append([bits_of(o) for o in outs])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for o in a[3] + b[3]:
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    for i in range(3):
        for (case, ws, lgs, outs), st in zip((a, b), streams):
            with torch.cuda.stream(st):
                _forward(case, lgs[i], outs[i], ws)
    torch.cuda.synchronize()
    for (case, ws, lgs, outs), r in zip((a, b), ref):
        for o, want in zip(outs, r):
            np.testing.assert_array_equal(bits_of(o), want)


@pytest.mark.parametrize("name", ["decode", "ep_share", "verify_b32", "a4_dw"])
def test_graph_replays_match_eager(name):
    """Three forwards recorded into one graph (each plan's kernels, no memset
    nodes: buffers are cleared by kernels), replayed three times with eager
    work and synchronisations between the replays; every replay's outputs
    equal the eager ones bit for bit."""
    case, ws, lgs, outs = _setup(name)
    for lg, o in zip(lgs, outs):
        _forward(case, lg, o, ws)
    torch.cuda.synchronize()
    eager = [bits_of(o) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _forward(case, lgs[0], outs[0], ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for lg, o in zip(lgs, outs):
            _forward(case, lg, o, ws)
    torch.cuda.synchronize()
    for rep in range(3):
        log("graph %s replay %d" % (name, rep))
        for o in outs:
            o.fill_(float("nan"))
        # eager work of the program between replays, through the same workspace
        scratch = torch.empty_like(outs[0])
        _forward(case, lgs[(rep + 1) % 3], scratch, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outs, eager):
            np.testing.assert_array_equal(bits_of(o), want)
