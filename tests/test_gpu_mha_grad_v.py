"""Parity of the attention dV kernel (mha_grad_v) with the CPU oracle's,
through the C ABI.

The forward's row statistics (lse) come from the oracle's attention_lse on
the same seeded q and k.  Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32
operands, fp32 accumulation, hardware exp); every dV element written (NaN
pre-fill) and nothing around it touched (guard bands).
"""
import sys

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import MHA_CONFIGS, MhaShape, draw_mha
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


def run_dv(sh, q, k, g, lse):
    import torch
    dev = torch.device("cuda", 0)
    tq, tk, tg, tl = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
                      for a in (q, k, g, lse))
    n = int(np.prod(k.shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch.float32, device=dev)
    buf[:GUARD] = CANARY
    buf[GUARD + n:] = CANARY
    dv = buf[GUARD:GUARD + n].view(k.shape)
    c2b.mha_grad_v_into(dv, tg, tq, tk, tl, sh.window, sh.causal)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == np.float32(CANARY)), "write before dv"
    assert np.all(host[GUARD + n:] == np.float32(CANARY)), "write after dv"
    got = host[GUARD:GUARD + n].reshape(k.shape)
    assert not np.any(np.isnan(got)), "unwritten dv elements"
    return got


def _check(sh: MhaShape, seed: int):
    q, k, g = draw_mha(sh, seed)
    lse = oracle.attention_lse(q, k, sh.kv_heads, sh.window, sh.causal).astype(np.float32)
    ref = oracle.mha_grad_v(g, q, k, lse, sh.window, sh.causal)
    got = run_dv(sh, q, k, g, lse)
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) / scale
    _say("  %s rel err %.3e" % (sh.name, err))
    assert err <= TOL, (sh.name, err)


@pytest.mark.parametrize("idx", range(len(MHA_CONFIGS)), ids=[c.name for c in MHA_CONFIGS])
def test_mha_grad_v_configs(idx):
    _say("case mha", MHA_CONFIGS[idx].name)
    _check(MHA_CONFIGS[idx], 70 + idx)


EDGE = [
    MhaShape("one_key", 1, 1, 1, 1),
    MhaShape("ragged_causal", 65, 65, 3, 3, window=5),
    MhaShape("noncausal_q_gt_kv", 100, 70, 4, 2, causal=False),
    MhaShape("noncausal_window", 100, 70, 4, 2, window=9, causal=False),
    MhaShape("window_block", 130, 130, 8, 2, window=64),
    MhaShape("q_lt_kv", 7, 200, 2, 1, window=3, causal=False),
    MhaShape("mqa", 200, 200, 6, 1),
    # causal units split over two workgroups by heads (group 2), and an odd
    # group that stays whole
    MhaShape("split_heads_causal", 130, 130, 4, 2),
    MhaShape("odd_group_causal", 100, 100, 3, 1),
]


@pytest.mark.parametrize("sh", EDGE, ids=[s.name for s in EDGE])
def test_mha_grad_v_edges(sh):
    _say("case mha", sh.name)
    _check(sh, 5)


def test_mha_grad_v_causal_split_is_deterministic():
    """The causal config's units are split over two workgroups whose partial
    dV meet on a zeroed dv by exactly two atomic adds: repeated calls must
    agree bit for bit."""
    sh = next(c for c in MHA_CONFIGS if c.causal and c.window == 0)
    _say("case mha determinism", sh.name)
    q, k, g = draw_mha(sh, 71)
    lse = oracle.attention_lse(q, k, sh.kv_heads, sh.window, sh.causal).astype(np.float32)
    first = run_dv(sh, q, k, g, lse)
    for _ in range(2):
        assert np.array_equal(run_dv(sh, q, k, g, lse), first)


def test_mha_grad_v_errors_and_empty():
    import torch
    dev = torch.device("cuda", 0)
    q = torch.zeros(8, 2, 64, device=dev)
    k = torch.zeros(8, 1, 64, device=dev)
    lse = torch.zeros(8, 2, 2, device=dev)
    p = c2b.make_mha_params(8, 8, 2, 1)
    assert c2b.mha_grad_v_raw(q.data_ptr(), q.data_ptr(), k.data_ptr(), lse.data_ptr(),
                              k.data_ptr(), p) == -3                   # dv is k
    assert c2b.mha_grad_v_raw(q.data_ptr(), q.data_ptr(), k.data_ptr(), lse.data_ptr(),
                              k.data_ptr(), c2b.make_mha_params(8, 8, 2, 1, 32)) == -2
    # heads == 0: zeros
    dv = torch.full((8, 1, 64), float("nan"), device=dev)
    p0 = c2b.make_mha_params(8, 8, 0, 1)
    assert c2b.mha_grad_v_raw(q.data_ptr(), q.data_ptr(), k.data_ptr(), lse.data_ptr(),
                              dv.data_ptr(), p0) == 0
    torch.cuda.synchronize()
    assert bool((dv == 0).all())
