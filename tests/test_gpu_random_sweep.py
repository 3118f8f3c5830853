"""Randomized parity over all three convolution entry points.

300 seeded random shapes (strides 1-4, kernels up to 7x7, asymmetric padding
up to the kernel, up to 70 channels and 48x48 images, ragged everywhere):
the input gradient on both paths, the forward convolution on both paths and
the weight gradient, each against the oracle at the usual bar
(max|gpu - oracle| / max|oracle| <= 1e-4 fp32, 2e-2 f16-staged), with every
output element written (NaN pre-fill) and nothing written outside it (guard
canaries).  Each shape's launches are replayed on the host before the GPU
runs them.
"""
import sys

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import random_shape
from tests.gpu_helpers import TOL, params_of, rel_err, run_gpu, run_gpu_forward
from tests.test_gpu_grad_weight import run_gw

pytestmark = pytest.mark.gpu

CHUNK = 50
SMALL, LARGE = 200, 100   # shapes of each size class


def _shape(i):
    rng = np.random.default_rng(20000 + i)
    if i < SMALL:
        sh = random_shape(rng, max_n=3, max_c=40, max_hw=30, max_k=7, max_s=4, name="s%d" % i)
    else:
        sh = random_shape(rng, max_n=4, max_c=70, max_hw=48, max_k=7, max_s=4, name="b%d" % i)
    return sh, rng


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.mark.parametrize("chunk", range((SMALL + LARGE) // CHUNK))
def test_random_shapes_all_entry_points(chunk):
    failures = []
    for i in range(chunk * CHUNK, (chunk + 1) * CHUNK):
        sh, rng = _shape(i)
        print("case", sh, flush=True)
        sys.stdout.flush()
        p = params_of(sh)
        for f16 in (False, True):
            assert c2b.check_indexing(p, f16)[0] == 0, (sh, f16)
            assert c2b.check_indexing_forward(p, f16)[0] == 0, (sh, f16)
        assert c2b.check_indexing_grad_weight(p)[0] == 0, sh
        go = rng.uniform(-1, 1, size=sh.go_shape).astype(np.float32)
        w = rng.uniform(-1, 1, size=sh.w_shape).astype(np.float32)
        x = rng.uniform(-1, 1, size=sh.gi_shape).astype(np.float32)
        gi_ref = oracle.grad_input_gather(go, w, sh.in_h, sh.in_w, sh.stride, sh.padding_h,
                                          sh.padding_w)
        y_ref = oracle.conv2d_forward(x, w, sh.out_h, sh.out_w, sh.stride, sh.padding_h,
                                      sh.padding_w)
        gw_ref = oracle.grad_weight(go, x, sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h,
                                    sh.padding_w)
        for f16 in (False, True):
            for what, got, ref in (("grad_input", run_gpu(sh, go, w, f16=f16), gi_ref),
                                   ("forward", run_gpu_forward(sh, x, w, f16=f16), y_ref)):
                err = rel_err(got, ref)
                if np.isnan(got).any() or err > TOL[f16]:
                    failures.append((sh.name, what, f16, err))
        got = run_gw(sh, go, x)
        err = rel_err(got, gw_ref)
        if np.isnan(got).any() or err > TOL[False]:
            failures.append((sh.name, "grad_weight", False, err))
    assert not failures, failures


# ---- the RMSNorm-fused product and attention dV on random shapes -------------

def _rms_shape(i):
    """Half the shapes have k and n multiples of 4 (the direct-to-LDS kernel),
    half any sizes (the register-path kernel)."""
    from conv2d_backward_implicit_amd.workloads import RmsShape
    rng = np.random.default_rng(30000 + i)
    m = int(rng.integers(1, 300))
    k, n = int(rng.integers(1, 600)), int(rng.integers(1, 400))
    if i % 2 == 0:
        k, n = 4 * max(1, k // 4), 4 * max(1, n // 4)
    eps = float(rng.choice([1e-6, 1e-3, 0.1]))
    return RmsShape("rms%d" % i, m, k, n, eps=eps)


def test_rms_norm_matmul_random_shapes():
    from conv2d_backward_implicit_amd.workloads import draw_rms
    from tests.test_gpu_rms_matmul import TOL as RMS_TOL, rel_err as rms_err, run_rms
    failures = []
    for i in range(60):
        sh = _rms_shape(i)
        print("case", sh, flush=True)
        rc, msg = c2b.check_indexing_rms_norm_matmul(c2b.make_rms_params(sh.m, sh.n, sh.k,
                                                                          sh.eps))
        assert rc == 0, (sh, rc, msg)
        x, g, w = draw_rms(sh, 40 + i)
        err = rms_err(run_rms(x, g, w, sh.eps), oracle.rms_norm_matmul(x, g, w, sh.eps))
        if err > RMS_TOL:
            failures.append((sh.name, err))
    assert not failures, failures


def _mha_shape(i):
    """Grouped kv heads (heads a multiple of kv_heads), with or without a
    window; causal shapes have q_seq = kv_seq, as the entry point requires."""
    from conv2d_backward_implicit_amd.workloads import MhaShape
    rng = np.random.default_rng(40000 + i)
    kv_heads = int(rng.integers(1, 4))
    heads = kv_heads * int(rng.integers(1, 4))
    causal = bool(i % 2 == 0)
    kv_seq = int(rng.integers(1, 200))
    q_seq = kv_seq if causal else int(rng.integers(1, 200))
    window = int(rng.integers(1, 100)) if i % 3 == 0 else 0
    return MhaShape("mha%d" % i, q_seq, kv_seq, heads, kv_heads, window=window, causal=causal)


def test_mha_grad_v_random_shapes():
    from conv2d_backward_implicit_amd.workloads import draw_mha
    from tests.test_gpu_mha_grad_v import TOL as MHA_TOL, run_dv
    failures = []
    for i in range(40):
        sh = _mha_shape(i)
        print("case", sh, flush=True)
        rc, msg = c2b.check_indexing_mha_grad_v(c2b.make_mha_params(
            sh.q_seq, sh.kv_seq, sh.heads, sh.kv_heads, sh.head_dim, sh.window, sh.causal))
        assert rc == 0, (sh, rc, msg)
        q, k, g = draw_mha(sh, 50 + i)
        lse = oracle.attention_lse(q, k, sh.kv_heads, sh.window, sh.causal).astype(np.float32)
        ref = oracle.mha_grad_v(g, q, k, lse, sh.window, sh.causal)
        got = run_dv(sh, q, k, g, lse)
        scale = max(float(np.max(np.abs(ref))), 1e-30)
        err = float(np.max(np.abs(got.astype(np.float64) - ref))) / scale
        if err > MHA_TOL:
            failures.append((sh.name, err))
    assert not failures, failures
