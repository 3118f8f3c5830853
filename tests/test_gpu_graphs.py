"""Every entry point under HIP graph capture (torch.cuda.graph, which records
on a stream of its own: a call without an explicit stream must follow it).
Each graph is replayed several times, with eager work and synchronizations
between the replays and the output refilled with NaN before each, and every
replay must equal the eager call bit for bit (same plan, fixed summation
order).  The calls are planned eagerly once before capture, so the capture
records launches only; the library records no memset and allocates nothing.
"""
import numpy as np
import pytest

import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import (CONFIGS, ConvShape, MhaShape,
                                                    RmsShape, draw, draw_forward, draw_mha,
                                                    draw_rms)
from tests.gpu_helpers import params_of

pytestmark = pytest.mark.gpu
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _replays_match(call, out):
    """Eager result of call() into `out`, then the captured call replayed."""
    import torch
    out.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        noise = torch.randn(1 << 16, device=out.device)     # eager work between replays
        noise.mul_(2.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), ("replay", r)
    del graph


def _reduced(sh: ConvShape, batch: int) -> ConvShape:
    d = sh.as_dict()
    d["batch"] = batch
    d["name"] = sh.name + "_b%d" % batch
    return ConvShape(**d)


@pytest.mark.parametrize("idx", [1, 2, 3, 4], ids=[CONFIGS[i].name for i in [1, 2, 3, 4]])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_conv_entry_points_under_graph_capture(idx, f16):
    import torch
    sh = _reduced(CONFIGS[idx], 2)
    print("case graph", sh.name, "f16" if f16 else "fp32", flush=True)
    dev = torch.device("cuda", 0)
    p = params_of(sh)
    go, w = draw(sh, idx)
    x, _ = draw_forward(sh, idx)
    tgo, tw, tx = (torch.from_numpy(a).to(dev) for a in (go, w, x))
    gi = torch.empty(sh.gi_shape, device=dev)
    y = torch.empty(sh.go_shape, device=dev)
    _replays_match(lambda: c2b.grad_input_into(gi, tgo, tw, p, f16=f16), gi)
    _replays_match(lambda: c2b.forward_into(y, tx, tw, p, f16=f16), y)
    if not f16:
        gw = torch.empty(sh.w_shape, device=dev)
        ws = torch.empty(max(c2b.grad_weight_workspace_size(p), 1), dtype=torch.uint8,
                         device=dev)
        _replays_match(lambda: c2b.grad_weight_into(gw, tgo, tx, p, workspace=ws), gw)


def test_rms_norm_matmul_under_graph_capture():
    import torch
    dev = torch.device("cuda", 0)
    for sh in (RmsShape("g_dma", 300, 256, 260), RmsShape("g_reg", 129, 95, 131)):
        print("case graph", sh.name, flush=True)
        x, g, w = draw_rms(sh, 9)
        tx, tg, tw = (torch.from_numpy(a).to(dev) for a in (x, g, w))
        out = torch.empty(sh.m, sh.n, device=dev)
        _replays_match(lambda: c2b.rms_norm_matmul_into(out, tx, tg, tw, sh.eps), out)


def test_mha_grad_v_under_graph_capture():
    """The causal split zeroes dv with a fill kernel and adds two partial sums
    atomically; both are captured, and the replays stay bitwise equal."""
    import torch
    import oracle
    dev = torch.device("cuda", 0)
    for sh in (MhaShape("g_causal", 256, 256, 8, 2), MhaShape("g_window", 200, 200, 4, 2,
                                                               window=64)):
        print("case graph", sh.name, flush=True)
        q, k, g = draw_mha(sh, 11)
        lse = oracle.attention_lse(q, k, sh.kv_heads, sh.window, sh.causal).astype(np.float32)
        tq, tk, tg, tl = (torch.from_numpy(np.ascontiguousarray(a)).to(dev)
                          for a in (q, k, g, lse))
        dv = torch.empty(k.shape, device=dev)
        _replays_match(lambda: c2b.mha_grad_v_into(dv, tg, tq, tk, tl, sh.window, sh.causal),
                       dv)
