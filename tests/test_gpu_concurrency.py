"""Calls from several host threads at once, each on a stream of its own: the
entry points are reentrant (the plan memo is guarded by a mutex, nothing else
is shared between calls), so every call must give the single-threaded
result bit for bit.  ctypes releases the interpreter lock for the duration of
each foreign call, so the threads do overlap inside the library, planning
included: the shapes are new to the process when the threads start."""
import random
import threading

import numpy as np
import pytest

import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import ConvShape, draw
from tests.gpu_helpers import params_of

pytestmark = pytest.mark.gpu

THREADS, ROUNDS = 4, 6
SHAPES = [
    ConvShape("t_s1", 2, 24, 19, 17, 20, 3, 3, 1, 1, 1, 19, 17, dist="uniform"),
    ConvShape("t_s2", 2, 33, 22, 21, 18, 3, 3, 2, 1, 1, 11, 11, dist="uniform"),
    ConvShape("t_stem", 1, 3, 40, 38, 16, 7, 7, 2, 3, 3, 20, 19, dist="uniform"),
    ConvShape("t_pw", 3, 64, 10, 10, 48, 1, 1, 1, 0, 0, 10, 10, dist="uniform"),
    ConvShape("t_k5", 1, 10, 15, 13, 9, 5, 5, 1, 2, 2, 15, 13, dist="uniform"),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def test_concurrent_calls_from_host_threads():
    import torch
    dev = torch.device("cuda", 0)
    for sh in SHAPES:
        for f16 in (0, 1):
            assert c2b.check_indexing(params_of(sh), f16)[0] == 0, sh
    inputs = []
    for i, sh in enumerate(SHAPES):
        go, w = draw(sh, 90 + i)
        inputs.append((torch.from_numpy(go).to(dev), torch.from_numpy(w).to(dev)))
    torch.cuda.synchronize()
    results = {}
    errors = []

    def worker(t):
        try:
            stream = torch.cuda.Stream()
            order = [(i, f16) for i in range(len(SHAPES)) for f16 in (False, True)]
            rnd = random.Random(t)
            outs = {}
            for _ in range(ROUNDS):
                rnd.shuffle(order)
                for i, f16 in order:
                    sh = SHAPES[i]
                    tgo, tw = inputs[i]
                    with torch.cuda.stream(stream):
                        out = torch.empty(sh.gi_shape, device=dev)
                    c2b.grad_input_into(out, tgo, tw, params_of(sh), f16=f16, stream=stream)
                    stream.synchronize()
                    outs.setdefault((i, f16), []).append(out.cpu().numpy())
            results[t] = outs
        except Exception as e:   # reported by the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    # the single-threaded result of each call, after the threads
    for i, sh in enumerate(SHAPES):
        tgo, tw = inputs[i]
        for f16 in (False, True):
            ref = torch.empty(sh.gi_shape, device=dev)
            c2b.grad_input_into(ref, tgo, tw, params_of(sh), f16=f16)
            torch.cuda.synchronize()
            ref = ref.cpu().numpy()
            for t in range(THREADS):
                for got in results[t][(i, f16)]:
                    assert np.array_equal(got, ref), (sh.name, f16, t)
