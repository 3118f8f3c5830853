"""Parity of the RMSNorm-fused matrix product (rms_norm_matmul) with the CPU
oracle's, through the C ABI.

Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32 operands and
accumulation, as the conv paths); every output element written (NaN
pre-fill) and nothing around it touched (guard bands); exact zeros for zero
rows.  At the full sizes the oracle computes sampled rows (first, last,
tile edges, random).
"""
import sys

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import RMS_CONFIGS, RmsShape, draw_rms
from tests.gpu_helpers import CANARY, GUARD

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def run_rms(x, g, w, eps):
    """C of the HIP path (NaN-filled, guarded output) as numpy."""
    import torch
    dev = torch.device("cuda", 0)
    m, k = x.shape
    n = w.shape[1]
    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    tg = torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to(dev)
    tw = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev)
    total = m * n
    buf = torch.full((total + 2 * GUARD,), float("nan"), dtype=torch.float32, device=dev)
    buf[:GUARD] = CANARY
    buf[GUARD + total:] = CANARY
    out = buf[GUARD:GUARD + total].view(m, n)
    c2b.rms_norm_matmul_into(out, tx, tg, tw, eps)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == np.float32(CANARY)), "write before out"
    assert np.all(host[GUARD + total:] == np.float32(CANARY)), "write after out"
    got = host[GUARD:GUARD + total].reshape(m, n)
    assert not np.any(np.isnan(got)), "unwritten output elements"
    return got


def rel_err(a, b):
    scale = max(float(np.max(np.abs(b))), 1e-30)
    return float(np.max(np.abs(a.astype(np.float64) - b)) / scale) if a.size else 0.0


def _check(sh: RmsShape, seed: int, rows=None):
    x, g, w = draw_rms(sh, seed)
    got = run_rms(x, g, w, sh.eps)
    ref = oracle.rms_norm_matmul(x, g, w, sh.eps, rows=rows)
    err = rel_err(got if rows is None else got[rows], ref)
    _say("  %s rel err %.3e" % (sh.name, err))
    assert err <= TOL, (sh.name, err)


def test_rms_small_configs():
    for i, sh in enumerate(RMS_CONFIGS):
        if sh.m * sh.n * sh.k <= 5e9:
            _say("case rms", sh.name)
            _check(sh, 50 + i)


@pytest.mark.parametrize("idx", range(len(RMS_CONFIGS)), ids=[c.name for c in RMS_CONFIGS])
def test_rms_full_size_sampled_rows(idx):
    """At the full size, rows sampled across tiles: first, last, tile edges
    and random ones, each compared in full against the oracle."""
    sh = RMS_CONFIGS[idx]
    rng = np.random.default_rng(idx)
    edges = [0, sh.m - 1] + [r for t in range(128, sh.m, 128) for r in (t - 1, t)][:16]
    rows = sorted(set(edges) | set(rng.integers(0, sh.m, 24).tolist()))
    _say("case rms full", sh.name, "rows", len(rows))
    _check(sh, 60 + idx, rows=rows)


EDGE = [
    RmsShape("one", 1, 1, 1),
    RmsShape("k1", 130, 1, 129),
    RmsShape("n1_k33", 257, 33, 1),
    RmsShape("m1", 1, 31, 300),
    RmsShape("k_tail", 129, 95, 131),
    RmsShape("big_eps", 64, 40, 70, eps=0.5),
    RmsShape("zero_eps", 64, 40, 70, eps=0.0),
    RmsShape("tiles_exact", 256, 64, 256),
    RmsShape("long_k", 40, 2500, 50),
]


# k and n multiples of 4 take the direct-to-LDS kernel: partial tiles, a
# single k quad, stage tails, one row, zero-padding k quads
EDGE_DMA = [
    RmsShape("dma_min", 1, 4, 4),
    RmsShape("dma_partial_tiles", 129, 36, 132),
    RmsShape("dma_one_stage", 300, 32, 260),
    RmsShape("dma_k_tail", 77, 100, 388),
    RmsShape("dma_tiles_exact", 256, 128, 256, eps=0.1),
    RmsShape("dma_long_k", 40, 2504, 52),
]
EDGE = EDGE + EDGE_DMA


@pytest.mark.parametrize("sh", EDGE, ids=[s.name for s in EDGE])
def test_rms_edge_shapes(sh):
    _say("case rms", sh.name)
    _check(sh, 7)


def test_rms_zero_and_constant_rows():
    """Zero rows give exact zeros (eps > 0); rows scaled by a positive factor
    give the same output at eps = 0."""
    sh = RmsShape("rows", 200, 70, 90, eps=1e-6)
    x, g, w = draw_rms(sh, 3)
    x[5] = 0.0
    x[130] = 0.0
    got = run_rms(x, g, w, sh.eps)
    assert np.all(got[5] == 0.0) and np.all(got[130] == 0.0)
    ref = oracle.rms_norm_matmul(x, g, w, sh.eps)
    assert rel_err(got, ref) <= TOL
    # the same on the direct-to-LDS kernel (k and n multiples of 4)
    got4 = run_rms(x[:, :68], g[:68], w[:68, :88], sh.eps)
    assert np.all(got4[5] == 0.0) and np.all(got4[130] == 0.0)
    assert rel_err(got4, oracle.rms_norm_matmul(x[:, :68], g[:68], w[:68, :88], sh.eps)) <= TOL
    # eps = 0 (no zero rows here: 0 * rsqrt(0) has no value)
    x, _, _ = draw_rms(sh, 4)
    scale = np.linspace(0.01, 50.0, sh.m, dtype=np.float32)[:, None]
    a = run_rms(x * scale, g, w, 0.0)
    b = run_rms(x, g, w, 0.0)
    b_ref = oracle.rms_norm_matmul(x, g, w, 0.0)
    assert rel_err(a, b_ref) <= TOL and rel_err(b, b_ref) <= TOL


def test_rms_empty_and_errors():
    import torch
    dev = torch.device("cuda", 0)
    x = torch.zeros(0, 5, device=dev)
    g = torch.ones(5, device=dev)
    w = torch.zeros(5, 3, device=dev)
    assert c2b.rms_norm_matmul(x, g, w).shape == (0, 3)
    x = torch.ones(4, 5, device=dev)
    out = torch.empty(4, 3, device=dev)
    p = c2b.make_rms_params(4, 3, 5)
    # out aliasing x
    assert c2b.conv2d_rms_norm_matmul_raw(x.data_ptr(), g.data_ptr(), w.data_ptr(),
                                          x.data_ptr(), p) == -3
    assert c2b.conv2d_rms_norm_matmul_raw(x.data_ptr(), g.data_ptr(), w.data_ptr(),
                                          out.data_ptr(), c2b.make_rms_params(4, 3, 0)) == -2
