"""Helpers for the GPU tests: run the HIP path through the C ABI on seeded
host arrays, with a NaN-filled output (every element must be written) framed
by guard bands (no element outside grad_input may change)."""
from __future__ import annotations

import numpy as np

import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import ConvShape

GUARD = 1024          # float32 elements of canary before and after grad_input
CANARY = -12345.678   # any value the kernels never produce from these inputs

TOL = {False: 1e-4, True: 2e-2}   # max|gpu - ref| / max|ref|, fp32 / f16-staged


def params_of(sh: ConvShape):
    return c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w,
                           sh.out_channels, sh.kernel_h, sh.kernel_w, sh.stride,
                           sh.padding_h, sh.padding_w, sh.out_h, sh.out_w)


def run_gpu(sh: ConvShape, go: np.ndarray, w: np.ndarray, f16: bool = False,
            stream=None, check_guards: bool = True, variant=None) -> np.ndarray:
    """grad_input of the HIP path, as a float32 numpy array (``variant``
    forces a kernel variant through conv2d_grad_input_variant)."""
    import torch
    dev = torch.device("cuda", 0)
    tgo = torch.from_numpy(np.ascontiguousarray(go, dtype=np.float32)).to(dev)
    tw = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev)
    n = int(np.prod(sh.gi_shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch.float32, device=dev)
    buf[:GUARD] = CANARY
    buf[GUARD + n:] = CANARY
    gi = buf[GUARD:GUARD + n].view(sh.gi_shape)
    c2b.grad_input_into(gi, tgo, tw, params_of(sh), f16=f16, stream=stream, variant=variant)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    if check_guards:
        assert np.all(host[:GUARD] == np.float32(CANARY)), "write before grad_input"
        assert np.all(host[GUARD + n:] == np.float32(CANARY)), "write after grad_input"
    return host[GUARD:GUARD + n].reshape(sh.gi_shape)


def run_gpu_forward(sh: ConvShape, x: np.ndarray, w: np.ndarray, f16: bool = False,
                    stream=None, variant=None) -> np.ndarray:
    """Forward convolution y of the HIP path (NaN-filled, guarded output), as
    a float32 numpy array."""
    import torch
    dev = torch.device("cuda", 0)
    tx = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    tw = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev)
    n = int(np.prod(sh.go_shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), dtype=torch.float32, device=dev)
    buf[:GUARD] = CANARY
    buf[GUARD + n:] = CANARY
    y = buf[GUARD:GUARD + n].view(sh.go_shape)
    c2b.forward_into(y, tx, tw, params_of(sh), f16=f16, stream=stream, variant=variant)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:GUARD] == np.float32(CANARY)), "write before y"
    assert np.all(host[GUARD + n:] == np.float32(CANARY)), "write after y"
    return host[GUARD:GUARD + n].reshape(sh.go_shape)


# Shapes every kernel variant is run on (GPU) and replayed on (CPU): ragged
# channel and pixel tiles, deep stages of a 1x1 kernel with a ragged last
# channel chunk, stride-2 classes with 1, 2 and 4 taps, a Ci = 3 stem, a
# 5x5 kernel with asymmetric padding.
VARIANT_SHAPES = [
    ConvShape("v_3x3_ragged", 2, 70, 13, 17, 40, 3, 3, 1, 1, 1, 13, 17, dist="uniform"),
    ConvShape("v_1x1_deep", 2, 33, 9, 10, 300, 1, 1, 1, 0, 0, 9, 10, dist="uniform"),
    ConvShape("v_3x3_s2", 1, 20, 15, 14, 37, 3, 3, 2, 1, 1, 8, 7, dist="uniform"),
    ConvShape("v_7x7_s2_ci3", 1, 3, 22, 19, 19, 7, 7, 2, 3, 3, 11, 10, dist="uniform"),
    ConvShape("v_5x5_asym", 1, 17, 11, 12, 21, 5, 5, 1, 2, 1, 11, 10, dist="uniform"),
]


def _shape(name, n, ci, h, w, co, kh, kw, s, ph, pw):
    return ConvShape(name, n, ci, h, w, co, kh, kw, s, ph, pw,
                     (h + 2 * ph - kh) // s + 1, (w + 2 * pw - kw) // s + 1, dist="uniform")


# Few-input-channel shapes for the variants that put column taps in the
# matrix rows: Ci from 1 to 5, column-tap counts from 1 to 9 (several input
# channels per 16 rows, or one), strides 1 to 4 (with classes no tap reaches),
# asymmetric padding, ragged rows, and rows split into several bands.
SMALL_CI_SHAPES = [
    _shape("c_ci1_7x7_s1", 2, 1, 20, 23, 9, 7, 7, 1, 3, 2),
    _shape("c_ci2_5x3_s2", 1, 2, 17, 30, 12, 5, 3, 2, 2, 1),
    _shape("c_ci3_7x7_s2", 2, 3, 31, 29, 20, 7, 7, 2, 3, 3),
    _shape("c_ci4_3x3_s3", 1, 4, 25, 26, 17, 3, 3, 3, 1, 0),
    _shape("c_ci3_1x9_s1", 1, 3, 9, 40, 7, 1, 9, 1, 0, 4),
    _shape("c_ci5_2x2_s2", 2, 5, 12, 13, 33, 2, 2, 2, 0, 0),
    _shape("c_ci2_3x3_s4", 1, 2, 15, 15, 6, 3, 3, 4, 1, 1),
    _shape("c_ci3_stem_rows", 1, 3, 120, 100, 64, 7, 7, 2, 3, 3),
]


# Stride-2 shapes for the multi-class variants: odd extents (the four
# classes differ in rows and columns), 2x2, 3x2 and 3x3 kernels, asymmetric,
# zero and double padding, channels off the 64-channel tile and the stage
# depth, and rows wide enough for several bands.
MC_SHAPES = [
    _shape("mc_3x3_odd", 2, 70, 13, 17, 40, 3, 3, 2, 1, 1),
    _shape("mc_2x2", 1, 20, 12, 14, 37, 2, 2, 2, 0, 0),
    _shape("mc_3x2_asym", 2, 33, 15, 10, 21, 3, 2, 2, 1, 0),
    _shape("mc_3x3_pad0", 1, 64, 16, 16, 64, 3, 3, 2, 0, 0),
    _shape("mc_3x3_pad2", 1, 17, 9, 11, 19, 3, 3, 2, 2, 2),
    _shape("mc_3x3_wide", 1, 16, 6, 130, 24, 3, 3, 2, 1, 1),
    _shape("mc_3x3_tiny", 3, 5, 3, 2, 6, 3, 3, 2, 1, 1),
]


def pw_random_shapes(rng: np.random.Generator, count: int, name: str) -> list:
    """Random shapes the 1x1 GEMM takes (1x1 kernel, stride 1, no padding,
    Ci and H*W multiples of 4): Ci up to 316 and Co up to 299 leave ragged
    128-row tiles and 32-deep stages; H*W from 4 to 380 pixels, so pixel
    tiles cross image boundaries."""
    out = []
    for i in range(count):
        n = int(rng.integers(1, 5))
        h, w = int(rng.integers(1, 20)), 4 * int(rng.integers(1, 6))   # H W % 4 == 0
        if i % 2:
            h, w = w, h
        ci = 4 * int(rng.integers(1, 80))
        co = int(rng.integers(1, 300))
        out.append(ConvShape("%s%d" % (name, i), n, ci, h, w, co, 1, 1, 1, 0, 0, h, w,
                             dist="uniform"))
    return out


# Replayed on the host (every access of both directions) and run on the GPU.
PW_RANDOM = pw_random_shapes(np.random.default_rng(97), 40, "pw")


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(got.astype(np.float64) - ref)))
    if scale == 0.0:
        return diff
    return diff / scale


def round_f16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest float16 (ties to even, numpy's cast) -> float64."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float64)
