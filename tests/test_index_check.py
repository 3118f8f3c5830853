"""Host replay of the kernels' addressing (conv2d_check_indexing), CPU only.

For each shape the library walks every workgroup and thread it would launch
and checks bounds of every global/LDS access, that every tap reads the
grad_out and weight element of the gather rule, and that each grad_input
element is written exactly once.  Runs on the shapes the GPU tests and the
benchmark use, before any of them touches a GPU.
"""
import numpy as np
import pytest

import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import CONFIGS, ConvShape, random_shape
from tests.gpu_helpers import (MC_SHAPES, PW_RANDOM, SMALL_CI_SHAPES, VARIANT_SHAPES,
                               params_of)
from tests.test_gpu_parity import EDGE, PW_SHAPES, RANDOM


def _check(sh, f16):
    rc, msg = c2b.check_indexing(params_of(sh), f16)
    assert rc == 0, (sh, f16, rc, msg)


@pytest.mark.parametrize("sh", CONFIGS, ids=[c.name for c in CONFIGS])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_workloads(sh, f16):
    _check(sh, f16)


@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_gpu_test_shapes(f16):
    for sh in EDGE + RANDOM:
        _check(sh, f16)


@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_random_stress(f16):
    rng = np.random.default_rng(99)
    for i in range(150):
        sh = random_shape(rng, max_n=3, max_c=140, max_hw=70, max_k=9, max_s=5,
                          name="s%d" % i)
        _check(sh, f16)


def _mc_tiles(sh):
    """Multi-class variants tile stride-2 shapes whose four classes have
    pixels and taps, with at most 9 kernel taps."""
    return (sh.stride == 2 and sh.kernel_h >= 2 and sh.kernel_w >= 2 and sh.in_h >= 2
            and sh.in_w >= 2 and sh.kernel_h * sh.kernel_w <= 9)


@pytest.mark.parametrize("variant", range(c2b.num_variants()))
def test_every_variant_replay(variant):
    shapes = list(VARIANT_SHAPES) + [CONFIGS[0]]
    mc = c2b.variant_is_multi_class(variant) == 1
    if mc:
        shapes += MC_SHAPES + [CONFIGS[2]]
    ran = 0
    for sh in shapes:
        rc, msg = c2b.check_indexing_variant(params_of(sh), variant)
        if mc and not _mc_tiles(sh):
            assert rc == -5, (variant, sh.name, rc)   # not a multi-class shape
            continue
        assert rc == 0, (variant, sh.name, rc, msg)
        ran += 1
    assert ran >= 1


def test_variant_queries():
    n = c2b.num_variants()
    kinds = [c2b.variant_is_f16(v) for v in range(n)]
    assert set(kinds) == {0, 1}
    assert c2b.variant_is_f16(-1) == -5 and c2b.variant_is_f16(n) == -5
    p = params_of(VARIANT_SHAPES[0])
    assert c2b.check_indexing_variant(p, n)[0] == -5


def test_checker_rejects_bad_shape():
    p = c2b.make_params(1, 3, 8, 8, 4, 3, 3, 1, 1, 1, 7, 8)
    rc, _ = c2b.check_indexing(p)
    assert rc == -2


def test_column_tap_variants_replay():
    cm = [v for v in range(c2b.num_variants()) if c2b.variant_uses_column_taps(v) == 1]
    assert cm, "no variant puts column taps in the matrix rows"
    for v in cm:
        for sh in SMALL_CI_SHAPES + [CONFIGS[4]]:
            rc, msg = c2b.check_indexing_variant(params_of(sh), v)
            assert rc == 0, (v, sh.name, rc, msg)


# ---- forward convolution launches (the same kernels, roles exchanged) ------
# conv2d_check_indexing_forward checks every tap of every output pixel
# against the forward definition (x[n, ci, s*oh - padding_h + kh, ...]
# times w[co, ci, kh, kw]) with the caller's stride and paddings, and that
# each y element is written exactly once.

def _check_fwd(sh, f16):
    rc, msg = c2b.check_indexing_forward(params_of(sh), f16)
    assert rc == 0, (sh, f16, rc, msg)


@pytest.mark.parametrize("sh", CONFIGS, ids=[c.name for c in CONFIGS])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_workloads(sh, f16):
    _check_fwd(sh, f16)


@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_test_shapes(f16):
    for sh in EDGE + RANDOM + list(VARIANT_SHAPES) + list(SMALL_CI_SHAPES):
        _check_fwd(sh, f16)


@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_random_stress(f16):
    rng = np.random.default_rng(98)
    for i in range(100):
        sh = random_shape(rng, max_n=3, max_c=140, max_hw=70, max_k=9, max_s=5,
                          name="f%d" % i)
        _check_fwd(sh, f16)


@pytest.mark.parametrize("variant", range(c2b.num_variants()))
def test_forward_every_variant_replay(variant):
    shapes = list(VARIANT_SHAPES) + [CONFIGS[0]]
    for sh in shapes:
        rc, msg = c2b.check_indexing_forward_variant(params_of(sh), variant)
        if c2b.variant_uses_column_taps(variant) == 1 or c2b.variant_is_multi_class(variant) == 1:
            assert rc == -5, (variant, sh.name, rc)   # no forward instance
        else:
            assert rc == 0, (variant, sh.name, rc, msg)


# ---- the 1x1 GEMM, both directions ------------------------------------------
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_pointwise_replay_both_directions(f16):
    """Every stage load, LDS cell, read and store of the 1x1 GEMM, as the
    input gradient and as the forward convolution, on channel counts that
    leave ragged 128-row tiles and 32-deep stages."""
    shapes = PW_SHAPES + PW_RANDOM
    for sh in shapes:
        assert (sh.in_h * sh.in_w) % 4 == 0, sh
        _check(sh, f16)
        if sh.in_channels >= 16 or f16:   # fewer: the im2col forward GEMM
            _check_fwd(sh, f16)


def test_forward_checker_rejects_bad_shape():
    p = c2b.make_params(1, 3, 8, 8, 4, 3, 3, 1, 1, 1, 7, 8)
    assert c2b.check_indexing_forward(p)[0] == -2


# ---- weight gradient (conv2d_grad_weight) -------------------------------------

@pytest.mark.parametrize("sh", CONFIGS, ids=[c.name for c in CONFIGS])
def test_grad_weight_workloads(sh):
    rc, msg = c2b.check_indexing_grad_weight(params_of(sh))
    assert rc == 0, (sh.name, rc, msg)


@pytest.mark.parametrize("variant", range(c2b.GRAD_WEIGHT_VARIANTS))
def test_grad_weight_workloads_every_variant(variant):
    for sh in CONFIGS[:3]:
        rc, msg = c2b.check_indexing_grad_weight_variant(params_of(sh), variant)
        assert rc == 0, (sh.name, variant, rc, msg)


def test_grad_weight_test_shapes():
    for sh in EDGE + RANDOM + list(VARIANT_SHAPES) + list(SMALL_CI_SHAPES):
        for v in [-1] + list(range(c2b.GRAD_WEIGHT_VARIANTS)):
            rc, msg = (c2b.check_indexing_grad_weight(params_of(sh)) if v < 0 else
                       c2b.check_indexing_grad_weight_variant(params_of(sh), v))
            assert rc == 0, (sh.name, v, rc, msg)


def test_grad_weight_random_stress():
    rng = np.random.default_rng(97)
    for i in range(60):
        sh = random_shape(rng, max_n=3, max_c=90, max_hw=40, max_k=7, max_s=4, name="w%d" % i)
        rc, msg = c2b.check_indexing_grad_weight(params_of(sh))
        assert rc == 0, (sh, rc, msg)
        v = i % c2b.GRAD_WEIGHT_VARIANTS
        rc, msg = c2b.check_indexing_grad_weight_variant(params_of(sh), v)
        assert rc == 0, (sh, v, rc, msg)


# ---- RMSNorm-fused matrix product (rms_norm_matmul) ----------------------------

# (m, n, k); k and n multiples of 4 also replay the direct-to-LDS kernel
RMS_REPLAY = [(1, 1, 1), (7, 19, 45), (128, 128, 32), (129, 127, 33), (300, 257, 100),
              (5, 300, 64), (256, 130, 31), (40, 50, 2500), (3000, 1500, 1000),
              (1, 4, 4), (129, 132, 36), (300, 260, 32), (77, 388, 100), (40, 52, 2504)]


@pytest.mark.parametrize("mnk", RMS_REPLAY, ids=lambda t: "m%d_n%d_k%d" % t)
def test_rms_norm_matmul_replay(mnk):
    rc, msg = c2b.check_indexing_rms_norm_matmul(c2b.make_rms_params(*mnk))
    assert rc == 0, (mnk, rc, msg)


def test_rms_norm_matmul_replay_rejects_bad_params():
    for m, n, k, eps in [(4, 4, 0, 1e-6), (4, 4, 4, -1.0), (4, 4, 4, float("inf")),
                         (4, 4, 4, float("nan"))]:
        assert c2b.check_indexing_rms_norm_matmul(c2b.make_rms_params(m, n, k, eps))[0] == -2
    # a tensor of 2^31 bytes
    assert c2b.check_indexing_rms_norm_matmul(c2b.make_rms_params(1 << 16, 8, 1 << 13))[0] == -4


# ---- attention dV (mha_grad_v) ----------------------------------------------------

MHA_REPLAY = [(37, 37, 4, 2, 0, 1), (1, 1, 1, 1, 0, 1), (64, 64, 2, 1, 0, 1),
              (65, 65, 3, 3, 5, 1), (100, 70, 4, 2, 0, 0), (100, 70, 4, 2, 9, 0),
              (130, 130, 8, 2, 64, 1), (7, 200, 2, 1, 3, 0), (4096, 4096, 32, 8, 512, 1),
              (4096, 4096, 32, 8, 0, 1), (130, 130, 4, 2, 0, 1), (100, 100, 3, 1, 0, 1),
              (200, 200, 6, 1, 0, 1), (8, 8, 0, 1, 0, 1)]


@pytest.mark.parametrize("case", MHA_REPLAY, ids=lambda c: "q%d_kv%d_h%d_kv%d_w%d_c%d" % c)
def test_mha_grad_v_replay(case):
    qs, ks, h, hkv, w, c = case
    rc, msg = c2b.check_indexing_mha_grad_v(c2b.make_mha_params(qs, ks, h, hkv, 64, w, c))
    assert rc == 0, (case, rc, msg)


def test_mha_grad_v_replay_rejects_bad_params():
    for bad in [(8, 8, 2, 1, 32, 0, 1), (8, 8, 3, 2, 64, 0, 1), (8, 9, 2, 1, 64, 0, 1),
                (8, 8, 2, 0, 64, 0, 1)]:
        assert c2b.check_indexing_mha_grad_v(c2b.make_mha_params(*bad))[0] == -2
