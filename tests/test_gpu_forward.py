"""Parity of the forward convolution (conv2d_forward, the adjoint operator
of the input gradient, on the same kernels) with the CPU oracle's forward
convolution, and the adjoint identity of the two GPU entry points at the
workloads' full sizes.

Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32 path) and <= 2e-2
(f16-staged path); integer-valued inputs bit-exact on both paths; every y
element written (NaN pre-fill), nothing outside y (guard canaries).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import (CONFIGS, ConvShape, draw, draw_forward,
                                                    draw_integers)
from tests.gpu_helpers import (PW_RANDOM, TOL, VARIANT_SHAPES, params_of, rel_err,
                               round_f16, run_gpu, run_gpu_forward)
from tests.test_gpu_parity import EDGE, PW_SHAPES, RANDOM

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _oracle_fwd(sh, x, w):
    return oracle.conv2d_forward(x, w, sh.out_h, sh.out_w, sh.stride, sh.padding_h,
                                 sh.padding_w)


def _reduced(sh: ConvShape, batch: int) -> ConvShape:
    d = sh.as_dict()
    d["batch"] = batch
    d["name"] = sh.name + "_b%d" % batch
    return ConvShape(**d)


def _check(sh, x, w, f16, variant=None):
    ref = _oracle_fwd(sh, x, w)
    got = run_gpu_forward(sh, x, w, f16=f16, variant=variant)
    assert not np.any(np.isnan(got)), "unwritten y elements"
    err = rel_err(got, ref)
    assert err <= TOL[f16], (sh.name, f16, variant, err)
    if f16:
        # exact sum of f16-rounded operands up to fp32 accumulation rounding
        err16 = rel_err(got, _oracle_fwd(sh, round_f16(x), round_f16(w)))
        assert err16 <= 1e-5, (sh.name, variant, err16)
    return err


@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_config_reduced_batch(idx, f16):
    cfg = CONFIGS[idx]
    sh = cfg if cfg.batch <= 2 else _reduced(cfg, 2 if idx != 2 else 1)
    _say("case forward", sh.name, "f16" if f16 else "fp32")
    x, w = draw_forward(sh, 200 + idx)
    _say("  rel err", _check(sh, x, w, f16))


@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_integer_inputs_bit_exact(idx, f16):
    cfg = CONFIGS[idx]
    sh = cfg if cfg.batch <= 2 else _reduced(cfg, 1)
    _say("case forward int", sh.name, "f16" if f16 else "fp32")
    # integers in [-4, 4] (x drawn like grad_out, with x's shape)
    rng = np.random.default_rng(300 + idx)
    x = rng.integers(-4, 5, size=sh.gi_shape).astype(np.float32)
    _, w = draw_integers(sh, 400 + idx)
    got = run_gpu_forward(sh, x, w, f16=f16)
    assert np.array_equal(got.astype(np.float64), _oracle_fwd(sh, x, w))


@pytest.mark.parametrize("variant", range(c2b.num_variants()))
def test_forward_every_variant(variant):
    if c2b.variant_uses_column_taps(variant) == 1:
        pytest.skip("variants with column taps have no forward instance")
    if c2b.variant_is_multi_class(variant) == 1:
        pytest.skip("multi-class variants have no forward instance")
    f16 = bool(c2b.variant_is_f16(variant))
    for sh in VARIANT_SHAPES:
        _say("case forward variant", variant, sh.name)
        x, w = draw_forward(sh, 11)
        _check(sh, x, w, f16, variant=variant)


FWD_EXTRA = [
    # no input channel: y must be all zeros
    ConvShape("ci0", 2, 0, 7, 7, 5, 3, 3, 1, 1, 1, 7, 7, dist="uniform"),
    # input channels not a multiple of a stage's 16-channel groups
    ConvShape("ci37_s2", 1, 37, 12, 11, 20, 3, 3, 2, 1, 1, 6, 6, dist="uniform"),
]


@pytest.mark.parametrize("sh", EDGE + FWD_EXTRA, ids=[s.name for s in EDGE + FWD_EXTRA])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_edge_shapes(sh, f16):
    _say("case forward edge", sh.name, "f16" if f16 else "fp32")
    x, w = draw_forward(sh, 7)
    _check(sh, x, w, f16)
    if sh.in_channels == 0:
        got = run_gpu_forward(sh, x, w, f16=f16)
        assert np.all(got == 0.0)


def test_forward_random_small_shapes():
    for sh in RANDOM:
        _say("case forward", sh)
        x, w = draw_forward(sh, zlib.crc32(sh.name.encode()))
        for f16 in (False, True):
            _check(sh, x, w, f16)


# ---- 1x1, stride 1, unpadded: the forward on the 1x1 GEMM --------------------
@pytest.mark.parametrize("sh", PW_SHAPES, ids=[s.name for s in PW_SHAPES])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_pointwise_gemm_shapes(sh, f16):
    """Ragged 128-row output-channel tiles, pixel tiles across images, a
    contraction that is not a multiple of the 32-deep stage; integer inputs
    bit-exact."""
    _say("case forward pointwise", sh.name, "f16" if f16 else "fp32")
    p = c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w, sh.out_channels, 1, 1,
                        1, 0, 0)
    few = sh.in_channels < 16 and not f16           # the im2col GEMM takes these
    assert c2b.planned_forward_variant(p, f16) == -1
    x, w = draw_forward(sh, zlib.crc32(sh.name.encode()))
    _say("  rel err", _check(sh, x, w, f16), "(im2col GEMM)" if few else "")
    rng = np.random.default_rng(zlib.crc32(sh.name.encode()) + 1)
    xi = rng.integers(-4, 5, size=sh.gi_shape).astype(np.float32)
    wi = rng.integers(-4, 5, size=sh.w_shape).astype(np.float32)
    got = run_gpu_forward(sh, xi, wi, f16=f16)
    assert np.array_equal(got.astype(np.float64), _oracle_fwd(sh, xi, wi))


@pytest.mark.parametrize("sh", PW_RANDOM, ids=[s.name for s in PW_RANDOM])
def test_forward_pointwise_random_shapes(sh):
    """Random 1x1 shapes (the ones the host replay walks) as forward
    convolutions, on both paths, against the oracle."""
    _say("case forward pointwise random", sh)
    x, w = draw_forward(sh, zlib.crc32(sh.name.encode()) + 2)
    for f16 in (False, True):
        assert c2b.planned_forward_variant(params_of(sh), f16) == -1
        _check(sh, x, w, f16)


def test_forward_pointwise_misaligned_input_takes_the_variant_kernels():
    """An x that is not 16-byte aligned cannot use the 16-byte loads: the
    call must still be right (it runs on the variant kernels)."""
    import torch
    sh = PW_SHAPES[2]
    x, w = draw_forward(sh, 5)
    dev = torch.device("cuda", 0)
    store = torch.zeros(x.size + 1, dtype=torch.float32, device=dev)
    store[1:] = torch.from_numpy(x.ravel()).to(dev)
    tx = store[1:].view(sh.gi_shape)
    assert tx.data_ptr() % 16 == 4
    y = torch.full(sh.go_shape, float("nan"), device=dev)
    p = c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w, sh.out_channels, 1, 1,
                        1, 0, 0)
    c2b.forward_into(y, tx, torch.from_numpy(w).to(dev), p)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), _oracle_fwd(sh, x, w)) <= TOL[False]


@pytest.mark.parametrize("idx", range(1, len(CONFIGS)), ids=[c.name for c in CONFIGS[1:]])
def test_adjoint_identity_full_size(idx):
    """<grad_input(go), x> = <go, forward(x)> on the GPU at the workload's full
    size (fp32 path, both launch plans the default entry points choose).
    Normalised by |gi| |x|: fp32 rounding stays below about 1e-6 of it, a
    wrong tap, channel or pixel anywhere moves it by about 1/sqrt(size)."""
    sh = CONFIGS[idx]
    _say("case adjoint", sh.name)
    go, w = draw(sh, idx)
    x, _ = draw_forward(sh, 500 + idx)
    gi = run_gpu(sh, go, w, f16=False).astype(np.float64)
    y = run_gpu_forward(sh, x, w, f16=False).astype(np.float64)
    assert not np.any(np.isnan(gi)) and not np.any(np.isnan(y))
    lhs = float(np.dot(gi.ravel(), x.astype(np.float64).ravel()))
    rhs = float(np.dot(go.astype(np.float64).ravel(), y.ravel()))
    bound = float(np.linalg.norm(gi)) * float(np.linalg.norm(x.astype(np.float64)))
    _say("  <gi,x> %.6e  <go,y> %.6e  diff/bound %.3e  1/sqrt(n) %.3e"
         % (lhs, rhs, abs(lhs - rhs) / bound, 1 / np.sqrt(x.size)))
    assert abs(lhs - rhs) <= 1e-5 * bound
