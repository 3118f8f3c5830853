"""Parity of the weight gradient (conv2d_grad_weight) with the CPU oracle's,
and its adjoint identity with the forward convolution at full size.

Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32); integer-valued inputs
bit-exact (every partial sum stays below 2^24); every grad_weight element
written (NaN pre-fill); the result does not depend on what a reused
workspace held.
"""
import sys

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import CONFIGS, ConvShape, draw, draw_forward
from tests.gpu_helpers import GUARD, CANARY, VARIANT_SHAPES, params_of, rel_err
from tests.test_gpu_parity import EDGE, RANDOM

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _oracle_gw(sh, go, x):
    return oracle.grad_weight(go, x, sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h,
                              sh.padding_w)


def run_gw(sh, go, x, workspace=None, variant=-1):
    """grad_weight of the HIP path (NaN-filled, guarded output) as numpy."""
    import torch
    dev = torch.device("cuda", 0)
    tgo = torch.from_numpy(np.ascontiguousarray(go, dtype=np.float32)).to(dev)
    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    n = int(np.prod(sh.w_shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch.float32, device=dev)
    buf[:GUARD] = CANARY
    buf[GUARD + n:] = CANARY
    gw = buf[GUARD:GUARD + n].view(sh.w_shape)
    c2b.grad_weight_into(gw, tgo, tx, params_of(sh), workspace=workspace, variant=variant)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == np.float32(CANARY)), "write before grad_weight"
    assert np.all(host[GUARD + n:] == np.float32(CANARY)), "write after grad_weight"
    return host[GUARD:GUARD + n].reshape(sh.w_shape)


def _reduced(sh: ConvShape, batch: int) -> ConvShape:
    d = sh.as_dict()
    d["batch"] = batch
    d["name"] = sh.name + "_b%d" % batch
    return ConvShape(**d)


def _check(sh, seed, variants=(-1,)):
    go, _ = draw(sh, seed)
    x, _ = draw_forward(sh, seed + 1)
    ref = _oracle_gw(sh, go, x)
    worst = 0.0
    for v in variants:
        got = run_gw(sh, go, x, variant=v)
        assert not np.any(np.isnan(got)), ("unwritten grad_weight elements", v)
        err = rel_err(got, ref)
        assert err <= TOL, (sh.name, v, err)
        worst = max(worst, err)
    return worst


ALL_VARIANTS = (-1,) + tuple(range(c2b.GRAD_WEIGHT_VARIANTS))


@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
def test_grad_weight_config_reduced_batch(idx):
    cfg = CONFIGS[idx]
    sh = cfg if cfg.batch <= 2 else _reduced(cfg, 2 if idx != 2 else 1)
    _say("case grad_weight", sh.name)
    _say("  rel err", _check(sh, 600 + idx, ALL_VARIANTS))


@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
def test_grad_weight_integer_inputs_bit_exact(idx):
    cfg = CONFIGS[idx]
    sh = cfg if cfg.batch <= 2 else _reduced(cfg, 1)
    _say("case grad_weight int", sh.name)
    rng = np.random.default_rng(700 + idx)
    go = rng.integers(-4, 5, size=sh.go_shape).astype(np.float32)
    x = rng.integers(-4, 5, size=sh.gi_shape).astype(np.float32)
    ref = _oracle_gw(sh, go, x)
    for v in ALL_VARIANTS:
        got = run_gw(sh, go, x, variant=v)
        assert np.array_equal(got.astype(np.float64), ref), v


GW_EXTRA = [
    # no image: grad_weight is all zeros
    ConvShape("n0", 0, 3, 7, 7, 5, 3, 3, 1, 1, 1, 7, 7, dist="uniform"),
    # many chunks crossing image boundaries, columns past a 64-column tile
    ConvShape("chunks", 5, 9, 21, 17, 70, 3, 3, 1, 1, 1, 21, 17, dist="uniform"),
    # planes of fewer than 64 pixels (a stage spans several images; the pixel
    # walk carries into the image index), one-row and one-column images
    ConvShape("tiny_planes", 9, 20, 4, 5, 33, 3, 3, 1, 1, 1, 4, 5, dist="uniform"),
    ConvShape("one_pixel", 70, 17, 1, 1, 9, 1, 1, 1, 0, 0, 1, 1, dist="uniform"),
    ConvShape("row", 3, 40, 1, 90, 20, 1, 5, 2, 0, 2, 1, 45, dist="uniform"),
    ConvShape("column", 3, 24, 77, 1, 12, 4, 1, 3, 2, 0, 26, 1, dist="uniform"),
]


@pytest.mark.parametrize("sh", EDGE + list(VARIANT_SHAPES) + GW_EXTRA,
                         ids=[s.name for s in EDGE + list(VARIANT_SHAPES) + GW_EXTRA])
def test_grad_weight_shapes(sh):
    _say("case grad_weight", sh.name)
    _check(sh, 31, ALL_VARIANTS)
    if sh.batch == 0:
        assert np.all(run_gw(sh, np.zeros(sh.go_shape), np.zeros(sh.gi_shape)) == 0.0)


def test_grad_weight_random_small_shapes():
    for i, sh in enumerate(RANDOM):
        _say("case grad_weight", sh)
        _check(sh, 800 + i, (-1, i % c2b.GRAD_WEIGHT_VARIANTS))


def test_grad_weight_workspace_reuse():
    """Two shapes in a row on one workspace, the second smaller: the second
    result is that of a fresh workspace."""
    import torch
    big = ConvShape("ws_big", 3, 20, 30, 30, 40, 3, 3, 1, 1, 1, 30, 30, dist="uniform")
    small = ConvShape("ws_small", 1, 7, 9, 11, 5, 3, 3, 2, 1, 1, 5, 6, dist="uniform")
    need = c2b.grad_weight_workspace_size(params_of(big))
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    for sh in (big, small):
        go, _ = draw(sh, 5)
        x, _ = draw_forward(sh, 6)
        a = run_gw(sh, go, x, workspace=ws)
        b = run_gw(sh, go, x)
        assert np.array_equal(a, b), sh.name
        assert rel_err(a, _oracle_gw(sh, go, x)) <= TOL


@pytest.mark.parametrize("idx", range(1, len(CONFIGS)), ids=[c.name for c in CONFIGS[1:]])
def test_grad_weight_adjoint_full_size(idx):
    """<grad_weight(go, x), V> = <go, forward(x, V)> on the GPU at the
    workload's full size, normalised by |gw| |V| (fp32 rounding stays far
    below 1e-5 of it; a wrong pixel, tap or channel moves it by ~1/sqrt)."""
    import torch
    sh = CONFIGS[idx]
    _say("case grad_weight adjoint", sh.name)
    go, v = draw(sh, idx)
    x, _ = draw_forward(sh, 900 + idx)
    gw = run_gw(sh, go, x).astype(np.float64)
    assert not np.any(np.isnan(gw))
    dev = torch.device("cuda", 0)
    y = c2b.forward(torch.from_numpy(x).to(dev), torch.from_numpy(v).to(dev), sh.stride,
                    sh.padding_h, sh.padding_w)
    torch.cuda.synchronize()
    lhs = float(np.dot(gw.ravel(), v.astype(np.float64).ravel()))
    rhs = float(np.dot(go.astype(np.float64).ravel(), y.cpu().numpy().astype(np.float64).ravel()))
    bound = float(np.linalg.norm(gw)) * float(np.linalg.norm(v.astype(np.float64)))
    _say("  <gw,V> %.6e  <go,y> %.6e  diff/bound %.3e" % (lhs, rhs, abs(lhs - rhs) / bound))
    assert abs(lhs - rhs) <= 1e-5 * bound
