"""Whole-tensor parity at the workloads' full sizes, on the launch plans that
are timed: the planner's model plan (what a first call runs) and the plan
conv2d_tune chooses (what bench.py times after tuning).

Every element of the output is compared with the CPU oracle on the same
seeded inputs.  Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32 path),
<= 2e-2 (f16-staged path, which must also be within 1e-5 of the oracle on
f16-rounded inputs); every output element written (NaN pre-fill), nothing
outside it (guard canaries).  After tuning, the default entry point must
return bit for bit what the chosen variant returns when forced.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import CONFIGS, draw, draw_forward
from tests.gpu_helpers import (TOL, params_of, rel_err, round_f16, run_gpu,
                               run_gpu_forward)

pytestmark = pytest.mark.gpu

IDS = [c.name for c in CONFIGS]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


# ---- oracle results, once per workload and rounding -------------------------
@functools.lru_cache(maxsize=None)
def _gi_ref(idx, rounded):
    sh = CONFIGS[idx]
    go, w = draw(sh, idx)
    if rounded:
        go, w = round_f16(go), round_f16(w)
    _say("  oracle grad_input", sh.name, "f16-rounded" if rounded else "")
    return oracle.grad_input_gather(go, w, sh.in_h, sh.in_w, sh.stride, sh.padding_h,
                                    sh.padding_w)


@functools.lru_cache(maxsize=None)
def _fwd_ref(idx, rounded):
    sh = CONFIGS[idx]
    x, w = draw_forward(sh, idx)
    if rounded:
        x, w = round_f16(x), round_f16(w)
    _say("  oracle forward", sh.name, "f16-rounded" if rounded else "")
    return oracle.conv2d_forward(x, w, sh.out_h, sh.out_w, sh.stride, sh.padding_h,
                                 sh.padding_w)


def _check(got, idx, f16, ref_fn, what):
    assert not np.any(np.isnan(got)), "unwritten %s elements" % what
    err = rel_err(got, ref_fn(idx, False))
    _say("  %s rel err %.3e" % (what, err))
    assert err <= TOL[f16], (what, err)
    if f16:
        err16 = rel_err(got, ref_fn(idx, True))
        _say("  %s rel err vs f16-rounded oracle %.3e" % (what, err16))
        assert err16 <= 1e-5, (what, err16)


def _tensors(sh, a, w, out_shape):
    import torch
    dev = torch.device("cuda", 0)
    return (torch.from_numpy(a).to(dev), torch.from_numpy(w).to(dev),
            torch.empty(out_shape, dtype=torch.float32, device=dev))


# ---- input gradient ----------------------------------------------------------
@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=IDS)
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_grad_input_whole_tensor_model_and_tuned_plans(idx, f16):
    sh = CONFIGS[idx]
    p = params_of(sh)
    go, w = draw(sh, idx)
    c2b.select_variant(p, f16, -1)                 # the planner's model plan
    model = c2b.planned_variant(p, f16)
    _say("case grad_input full", sh.name, "f16" if f16 else "fp32", "model variant", model)
    _check(run_gpu(sh, go, w, f16=f16), idx, f16, _gi_ref, "model plan")

    tgo, tw, gi = _tensors(sh, go, w, sh.gi_shape)
    tuned = c2b.tune(gi, tgo, tw, p, f16=f16)     # as bench.py does
    _say("  tuned variant", tuned)
    assert c2b.planned_variant(p, f16) == tuned
    got = run_gpu(sh, go, w, f16=f16)
    _check(got, idx, f16, _gi_ref, "tuned plan")
    if tuned < 0:   # a shape on the 1x1 GEMM: no variant to choose
        assert model == -1
        return
    assert np.array_equal(got, run_gpu(sh, go, w, variant=tuned)), \
        "default call after tuning differs from the chosen variant"
    if tuned != model:
        # a selection made in another process restores the same plan
        c2b.select_variant(p, f16, model)
        assert np.array_equal(run_gpu(sh, go, w, f16=f16),
                              run_gpu(sh, go, w, variant=model))
        c2b.select_variant(p, f16, tuned)


# ---- forward convolution -----------------------------------------------------
@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=IDS)
@pytest.mark.parametrize("f16", [False, True], ids=["fp32", "f16"])
def test_forward_whole_tensor_model_and_tuned_plans(idx, f16):
    sh = CONFIGS[idx]
    p = params_of(sh)
    x, w = draw_forward(sh, idx)
    model = c2b.planned_forward_variant(p, f16)
    if model >= 0:
        c2b.select_forward_variant(p, f16, -1)
        model = c2b.planned_forward_variant(p, f16)
    _say("case forward full", sh.name, "f16" if f16 else "fp32", "model variant", model)
    _check(run_gpu_forward(sh, x, w, f16=f16), idx, f16, _fwd_ref, "model plan")

    tx, tw, y = _tensors(sh, x, w, sh.go_shape)
    tuned = c2b.tune_forward(y, tx, tw, p, f16=f16)
    _say("  tuned variant", tuned)
    assert c2b.planned_forward_variant(p, f16) == tuned
    got = run_gpu_forward(sh, x, w, f16=f16)
    _check(got, idx, f16, _fwd_ref, "tuned plan")
    if tuned >= 0:
        assert np.array_equal(got, run_gpu_forward(sh, x, w, variant=tuned))


# ---- weight gradient ---------------------------------------------------------
@pytest.mark.parametrize("idx", range(len(CONFIGS)), ids=IDS)
def test_grad_weight_whole_tensor(idx):
    from tests.test_gpu_grad_weight import run_gw
    sh = CONFIGS[idx]
    go, _ = draw(sh, idx)
    x, _ = draw_forward(sh, idx + 1)
    _say("case grad_weight full", sh.name)
    ref = oracle.grad_weight(go, x, sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h,
                             sh.padding_w)
    got = run_gw(sh, go, x)
    assert not np.any(np.isnan(got)), "unwritten grad_weight elements"
    err = rel_err(got, ref)
    _say("  rel err %.3e" % err)
    assert err <= TOL[False], err
