"""The allocation-free weight gradient (conv2d_grad_weight_noalloc) against
the workspace entry point (conv2d_grad_weight) on the same inputs.

Both run the same plan, so their results must agree bit for bit (the bar is
the fp32 tolerance; equality is stricter).  Two calls in a row share the
library's scratch array: a full-size layer, then a smaller ragged one, so the
second call runs over what the first left in the scratch.  Every
grad_weight element must be written (NaN pre-fill), nothing outside it
(guard canaries), and the call must not allocate through torch.
"""
import sys

import numpy as np
import pytest

import oracle
import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import CONFIGS, ConvShape, draw, draw_forward
from tests.gpu_helpers import CANARY, GUARD, params_of, rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _pair(sh, seed):
    """(noalloc result, workspace-entry result, grad_out, x) as numpy."""
    import torch
    dev = torch.device("cuda", 0)
    go, _ = draw(sh, seed)
    x, _ = draw_forward(sh, seed + 1)
    tgo, tx = torch.from_numpy(go).to(dev), torch.from_numpy(x).to(dev)
    p = params_of(sh)
    ref = torch.empty(sh.w_shape, dtype=torch.float32, device=dev)
    c2b.grad_weight_into(ref, tgo, tx, p)          # own workspace
    n = int(np.prod(sh.w_shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch.float32, device=dev)
    buf[:GUARD] = CANARY
    buf[GUARD + n:] = CANARY
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(dev)
    c2b.grad_weight_noalloc_into(buf[GUARD:GUARD + n].view(sh.w_shape), tgo, tx, p)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(dev) == before, "the call allocated device memory"
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == np.float32(CANARY)), "write before grad_weight"
    assert np.all(host[GUARD + n:] == np.float32(CANARY)), "write after grad_weight"
    return host[GUARD:GUARD + n].reshape(sh.w_shape), ref.cpu().numpy(), go, x


def test_noalloc_matches_workspace_entry_on_two_calls_in_a_row():
    big = CONFIGS[1]   # ResNet stage-1 layer: 16.5 MB of partial sums
    small = ConvShape("noalloc_small_s2", 3, 37, 15, 14, 70, 3, 3, 2, 1, 0, 8, 6,
                      dist="uniform")
    assert c2b.grad_weight_workspace_size(params_of(big)) > \
        4 * c2b.grad_weight_workspace_size(params_of(small))
    for sh, seed in ((big, 1), (small, 41)):
        _say("case noalloc", sh.name, "workspace bytes",
             c2b.grad_weight_workspace_size(params_of(sh)))
        got, ref, go, x = _pair(sh, seed)
        assert not np.any(np.isnan(got)), "unwritten grad_weight elements"
        assert np.array_equal(got, ref), float(np.max(np.abs(got - ref)))
        if sh is small:
            want = oracle.grad_weight(go, x, sh.kernel_h, sh.kernel_w, sh.stride,
                                      sh.padding_h, sh.padding_w)
            assert rel_err(got, want) <= 1e-4, rel_err(got, want)


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    import torch
    dev = torch.device("cuda", 0)
    p = c2b.make_params(1, 1024, 8, 8, 1024, 3, 3, 1, 1, 1)
    go = torch.zeros((1, 1024, 8, 8), device=dev)
    x = torch.zeros((1, 1024, 8, 8), device=dev)
    dw = torch.full((1024, 1024, 3, 3), 7.0, device=dev)
    with pytest.raises(c2b.Conv2dError) as e:
        c2b.grad_weight_noalloc_into(dw, go, x, p)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert bool(torch.all(dw == 7.0)), "nothing may be written on an error"
