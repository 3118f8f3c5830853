"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: max|gpu - oracle| / max|oracle| <= 1e-4 for the fp32 path and <= 2e-2
for the f16-staged path; integer-valued inputs must match bit for bit on both
paths; every grad_input element is written (NaN pre-fill) and nothing outside
it is (guard canaries).
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import (CONFIGS, ConvShape, draw,
                                                    draw_integers, random_shape)
from tests.gpu_helpers import (MC_SHAPES, PW_RANDOM, SMALL_CI_SHAPES, TOL, VARIANT_SHAPES,
                               params_of, rel_err, round_f16, run_gpu)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _oracle(sh, go, w):
    return oracle.grad_input_gather(go, w, sh.in_h, sh.in_w, sh.stride,
                                    sh.padding_h, sh.padding_w)


def _reduced(sh: ConvShape, batch: int) -> ConvShape:
    d = sh.as_dict()
    d["batch"] = batch
    d["name"] = sh.name + "_b%d" % batch
    return ConvShape(**d)


# ---- the five workloads, full oracle at reduced batch -----------------------
@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_config_reduced_batch(idx, f16):
    cfg = CONFIGS[idx]
    sh = cfg if cfg.batch <= 2 else _reduced(cfg, 2 if idx != 2 else 1)
    _say("case", sh.name, "f16" if f16 else "fp32")
    go, w = draw(sh, idx)
    ref = _oracle(sh, go, w)
    got = run_gpu(sh, go, w, f16=f16)
    assert not np.any(np.isnan(got)), "unwritten grad_input elements"
    err = rel_err(got, ref)
    _say("  rel err", err)
    assert err <= TOL[f16], err
    if f16:
        # the f16-staged path is the exact sum of f16-rounded operands, up to
        # fp32 accumulation rounding
        ref16 = _oracle(sh, round_f16(go), round_f16(w))
        assert rel_err(got, ref16) <= 1e-5, rel_err(got, ref16)


@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=[c.name for c in CONFIGS])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_config_integer_inputs_bit_exact(idx, f16):
    cfg = CONFIGS[idx]
    sh = cfg if cfg.batch <= 2 else _reduced(cfg, 1)
    _say("case int", sh.name, "f16" if f16 else "fp32")
    go, w = draw_integers(sh, 100 + idx)
    ref = _oracle(sh, go, w)
    got = run_gpu(sh, go, w, f16=f16)
    assert np.array_equal(got.astype(np.float64), ref)


# ---- random small shapes: strides 1-3, asymmetric padding, ragged tiles ----
RANDOM = [random_shape(np.random.default_rng(500 + i), max_n=3, max_c=9, max_hw=23,
                       max_k=7, max_s=4, name="r%d" % i) for i in range(60)]


@pytest.mark.parametrize("sh", RANDOM, ids=[s.name for s in RANDOM])
def test_random_small_shapes(sh):
    _say("case", sh)
    rng = np.random.default_rng(zlib.crc32(sh.name.encode()))
    go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
    w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
    ref = _oracle(sh, go, w)
    for f16 in (False, True):
        got = run_gpu(sh, go, w, f16=f16)
        assert not np.any(np.isnan(got))
        assert rel_err(got, ref) <= TOL[f16], (f16, rel_err(got, ref))


# ---- edge cases --------------------------------------------------------------
EDGE = [
    # channels not a multiple of the 64-channel tile; pixel tails
    ConvShape("ci65_co3", 2, 65, 9, 11, 3, 3, 3, 1, 1, 1, 9, 11, dist="uniform"),
    ConvShape("ci130_s2", 1, 130, 10, 9, 17, 3, 3, 2, 1, 1, 5, 5, dist="uniform"),
    ConvShape("ci3_stem_small", 2, 3, 30, 30, 8, 7, 7, 2, 3, 3, 15, 15, dist="uniform"),
    # very wide rows (band split) and a one-column image (tall halo)
    ConvShape("wide", 1, 4, 5, 700, 5, 3, 7, 1, 1, 3, 5, 700, dist="uniform"),
    ConvShape("one_col", 1, 3, 300, 1, 4, 3, 3, 1, 1, 1, 300, 1, dist="uniform"),
    ConvShape("one_px", 3, 5, 1, 1, 6, 1, 1, 1, 0, 0, 1, 1, dist="uniform"),
    # padding larger than the kernel; stride larger than the kernel
    ConvShape("pad_gt_k", 1, 3, 6, 6, 4, 2, 3, 1, 3, 4, 11, 12, dist="uniform"),
    ConvShape("s3_k2", 2, 4, 13, 11, 5, 2, 2, 3, 1, 0, 5, 4, dist="uniform"),
    ConvShape("s4_k1", 1, 6, 15, 17, 7, 1, 1, 4, 0, 0, 4, 5, dist="uniform"),
    # large kernel at stride 1 (several tap groups per stage)
    ConvShape("k11", 1, 5, 20, 20, 9, 11, 11, 1, 5, 5, 20, 20, dist="uniform"),
    # output channels not a multiple of the stage depth
    ConvShape("co13", 1, 7, 12, 12, 13, 3, 3, 1, 1, 1, 12, 12, dist="uniform"),
    # zero output channels: grad_input must be all zeros (a 3x3 layer, and a
    # 1x1 one on the 1x1 GEMM, whose forward then has no tile to launch)
    ConvShape("co0", 2, 5, 7, 7, 0, 3, 3, 1, 1, 1, 7, 7, dist="uniform"),
    ConvShape("pw_co0", 2, 20, 6, 6, 0, 1, 1, 1, 0, 0, 6, 6, dist="uniform"),
    # stride 5: 25 classes in two launches; one tap each (classes of equal
    # stage counts, dealt image by image), and 7x7 taps (unequal classes)
    ConvShape("s5_k5", 2, 5, 23, 23, 6, 5, 5, 5, 2, 2, 5, 5, dist="uniform"),
    ConvShape("s5_k7", 3, 4, 21, 19, 3, 7, 7, 5, 3, 3, 5, 4, dist="uniform"),
]


@pytest.mark.parametrize("sh", EDGE, ids=[s.name for s in EDGE])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_edge_shapes(sh, f16):
    _say("case", sh.name, "f16" if f16 else "fp32")
    rng = np.random.default_rng(7)
    go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
    w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
    ref = _oracle(sh, go, w)
    got = run_gpu(sh, go, w, f16=f16)
    assert not np.any(np.isnan(got))
    if sh.out_channels == 0:
        assert np.all(got == 0.0)
    assert rel_err(got, ref) <= TOL[f16], rel_err(got, ref)


def test_empty_batch_is_noop():
    import torch
    import conv2d_backward_implicit_amd as c2b
    dev = torch.device("cuda", 0)
    go = torch.zeros((0, 4, 5, 5), device=dev)
    w = torch.zeros((4, 3, 3, 3), device=dev)
    gi = c2b.grad_input(go, w, 5, 5, 1, 1, 1)
    torch.cuda.synchronize()
    assert gi.shape == (0, 3, 5, 5)


def test_deterministic_and_on_side_stream():
    import torch
    sh = _reduced(CONFIGS[2], 1)
    go, w = draw(sh, 2)
    a = run_gpu(sh, go, w)
    s = torch.cuda.Stream()
    b = run_gpu(sh, go, w, stream=s)
    assert np.array_equal(a, b)


def test_call_without_stream_runs_on_torchs_current_stream():
    """With no stream given, a call goes to torch's current stream, also
    inside a ``torch.cuda.stream`` context, and gives the same result."""
    import torch
    sh = _reduced(CONFIGS[2], 1)
    go, w = draw(sh, 2)
    ref = run_gpu(sh, go, w)
    assert c2b._stream_id(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert c2b._stream_id(None) == side.cuda_stream
        got = run_gpu(sh, go, w)
    assert np.array_equal(ref, got)


def test_bad_status_raises():
    import torch
    import conv2d_backward_implicit_amd as c2b
    dev = torch.device("cuda", 0)
    go = torch.zeros((1, 4, 5, 5), device=dev)
    w = torch.zeros((4, 3, 3, 3), device=dev)
    p = c2b.make_params(1, 3, 5, 5, 4, 3, 3, 1, 1, 1, 5, 5)
    with pytest.raises(c2b.Conv2dError):
        c2b.grad_input_into(go.view(1, 4, 5, 5)[:, :3], go, w, p)  # alias


# ---- every kernel variant, forced through conv2d_grad_input_variant ---------
def _num_variants():
    import conv2d_backward_implicit_amd as c2b
    return c2b.num_variants()


@pytest.mark.parametrize("variant", range(c2b.num_variants()))
def test_every_variant(variant):
    import conv2d_backward_implicit_amd as c2b
    f16 = bool(c2b.variant_is_f16(variant))
    mc = c2b.variant_is_multi_class(variant) == 1
    ran = 0
    for sh in VARIANT_SHAPES + (MC_SHAPES if mc else []):
        if mc:
            try:
                c2b.describe_plan_variant(params_of(sh), variant)
            except c2b.Conv2dError:
                continue   # not a stride-2 shape the multi-class tiles cover
        ran += 1
        _say("case variant", variant, sh.name)
        rng = np.random.default_rng(11)
        go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
        w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
        ref = _oracle(sh, go, w)
        got = run_gpu(sh, go, w, variant=variant)
        assert not np.any(np.isnan(got)), "unwritten grad_input elements"
        err = rel_err(got, ref)
        assert err <= TOL[f16], (sh.name, err)
        if f16:
            err16 = rel_err(got, _oracle(sh, round_f16(go), round_f16(w)))
            assert err16 <= 1e-5, (sh.name, err16)
        # integer inputs: exact on every path and in any summation order
        gi_, wi_ = draw_integers(sh, 3)
        got_i = run_gpu(sh, gi_, wi_, variant=variant)
        assert np.array_equal(got_i.astype(np.float64), _oracle(sh, gi_, wi_)), sh.name
    assert ran >= 1


# ---- variants with column taps in the matrix rows, on few-channel shapes ----
def _cm_variants():
    return [v for v in range(c2b.num_variants()) if c2b.variant_uses_column_taps(v) == 1]


@pytest.mark.parametrize("variant", _cm_variants())
def test_column_tap_variants_small_ci(variant):
    f16 = bool(c2b.variant_is_f16(variant))
    for sh in SMALL_CI_SHAPES:
        _say("case variant", variant, sh.name)
        rng = np.random.default_rng(17)
        go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
        w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
        got = run_gpu(sh, go, w, variant=variant)
        assert not np.any(np.isnan(got)), "unwritten grad_input elements"
        err = rel_err(got, _oracle(sh, go, w))
        _say("  rel err", err)
        assert err <= TOL[f16], (sh.name, err)
        if f16:
            err16 = rel_err(got, _oracle(sh, round_f16(go), round_f16(w)))
            assert err16 <= 1e-5, (sh.name, err16)
        gi_, wi_ = draw_integers(sh, 5)
        got_i = run_gpu(sh, gi_, wi_, variant=variant)
        assert np.array_equal(got_i.astype(np.float64), _oracle(sh, gi_, wi_)), sh.name


# ---- measured plan choice ----------------------------------------------------
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_tune_picks_a_variant_and_the_default_call_uses_it(f16):
    import torch
    sh = ConvShape("t_tune", 2, 24, 20, 18, 40, 3, 3, 2, 1, 1, 10, 9, dist="uniform")
    _say("case tune", sh.name, "f16" if f16 else "fp32")
    rng = np.random.default_rng(23)
    go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
    w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
    ref = _oracle(sh, go, w)
    dev = torch.device("cuda", 0)
    tgo, tw = torch.from_numpy(go).to(dev), torch.from_numpy(w).to(dev)
    gi = torch.full(sh.gi_shape, float("nan"), device=dev)
    p = c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w, sh.out_channels,
                        sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h, sh.padding_w)
    v = c2b.tune(gi, tgo, tw, p, f16=f16)
    torch.cuda.synchronize()
    assert 0 <= v < c2b.num_variants() and c2b.variant_is_f16(v) == int(f16)
    assert rel_err(gi.cpu().numpy(), ref) <= TOL[f16]          # tune leaves the result
    assert c2b.planned_variant(p, f16) == v
    got = run_gpu(sh, go, w, f16=f16)                          # default call, tuned plan
    assert not np.any(np.isnan(got))
    assert rel_err(got, ref) <= TOL[f16]


# ---- 1x1, stride 1, unpadded: the GEMM over all images' pixels --------------
# Channel tiles of 128 with a ragged last one, pixel tiles of 128 that cross
# image boundaries, a contraction that is not a multiple of the 32-channel
# stage, Co = 1, images smaller than a quad row.
PW_SHAPES = [
    ConvShape("pw_ci4_2x2", 3, 4, 2, 2, 5, 1, 1, 1, 0, 0, 2, 2, dist="uniform"),
    ConvShape("pw_ci36_7x4", 5, 36, 7, 4, 33, 1, 1, 1, 0, 0, 7, 4, dist="uniform"),
    ConvShape("pw_ci132_10x20", 2, 132, 10, 20, 70, 1, 1, 1, 0, 0, 10, 20, dist="uniform"),
    ConvShape("pw_ci256_co1", 3, 256, 14, 14, 1, 1, 1, 1, 0, 0, 14, 14, dist="uniform"),
    ConvShape("pw_ci128_co40_12x12", 9, 128, 12, 12, 40, 1, 1, 1, 0, 0, 12, 12,
              dist="uniform"),
    # 294 tiles, more than the CUs: the two-buffer form, two workgroups per
    # CU (input gradient of the first, forward of the second)
    ConvShape("pw_ci700_co64_28x28", 8, 700, 28, 28, 64, 1, 1, 1, 0, 0, 28, 28,
              dist="uniform"),
    ConvShape("pw_ci64_co700_28x28", 8, 64, 28, 28, 700, 1, 1, 1, 0, 0, 28, 28,
              dist="uniform"),
]


@pytest.mark.parametrize("sh", PW_SHAPES, ids=[s.name for s in PW_SHAPES])
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_pointwise_gemm_shapes(sh, f16):
    _say("case pointwise", sh.name, "f16" if f16 else "fp32")
    p = c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w, sh.out_channels,
                        sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h, sh.padding_w)
    assert c2b.planned_variant(p, f16) == -1          # the GEMM path, not a variant
    rng = np.random.default_rng(zlib.crc32(sh.name.encode()))
    go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
    w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
    ref = _oracle(sh, go, w)
    got = run_gpu(sh, go, w, f16=f16)
    assert not np.any(np.isnan(got)), "unwritten grad_input elements"
    err = rel_err(got, ref)
    _say("  rel err", err)
    assert err <= TOL[f16], err
    if f16:
        assert rel_err(got, _oracle(sh, round_f16(go), round_f16(w))) <= 1e-5
    gi_, wi_ = draw_integers(sh, 9)
    got_i = run_gpu(sh, gi_, wi_, f16=f16)
    assert np.array_equal(got_i.astype(np.float64), _oracle(sh, gi_, wi_))


@pytest.mark.parametrize("sh", PW_RANDOM, ids=[s.name for s in PW_RANDOM])
def test_pointwise_gemm_random_shapes(sh):
    """Random shapes on the 1x1 GEMM (the ones the host replay walks), on
    both paths, against the oracle."""
    _say("case pointwise random", sh)
    p = params_of(sh)
    rng = np.random.default_rng(zlib.crc32(sh.name.encode()))
    go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
    w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
    ref = _oracle(sh, go, w)
    for f16 in (False, True):
        assert c2b.planned_variant(p, f16) == -1
        got = run_gpu(sh, go, w, f16=f16)
        assert not np.any(np.isnan(got)), ("unwritten grad_input elements", f16)
        assert rel_err(got, ref) <= TOL[f16], (f16, rel_err(got, ref))


def test_pointwise_gemm_misaligned_tensor_takes_the_variant_kernels():
    """A grad_out that is not 16-byte aligned cannot use the 16-byte loads:
    the call must still be right (it runs on the variant kernels)."""
    import torch
    sh = PW_SHAPES[1]
    rng = np.random.default_rng(3)
    go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
    w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
    dev = torch.device("cuda", 0)
    n = go.size
    store = torch.zeros(n + 1, dtype=torch.float32, device=dev)
    store[1:] = torch.from_numpy(go.ravel()).to(dev)
    tgo = store[1:].view(sh.go_shape)                   # 4 bytes past a 256-byte boundary
    assert tgo.data_ptr() % 16 == 4
    tw = torch.from_numpy(w).to(dev)
    gi = torch.full(sh.gi_shape, float("nan"), device=dev)
    p = c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w, sh.out_channels, 1, 1,
                        1, 0, 0)
    c2b.grad_input_into(gi, tgo, tw, p)
    torch.cuda.synchronize()
    assert rel_err(gi.cpu().numpy(), _oracle(sh, go, w)) <= TOL[False]
