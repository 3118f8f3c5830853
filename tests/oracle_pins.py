"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` (the committed build or a
deliberately mutated copy) and raises ``AssertionError`` when the oracle
disagrees with the fact it checks.  tests/test_oracle.py runs them on the
committed oracle; tests/test_oracle_mutants.py runs them on mutants and
requires that every mutant trips at least one pin.

What the pins rest on:
* torch's CPU routines ``torch.nn.grad.conv2d_input``,
  ``torch.nn.grad.conv2d_weight`` and ``torch.nn.functional.conv2d`` in
  float64 (third-party library; run, not copied);
* the adjoint identities <grad_input(g), x> = <g, conv2d(x)> and
  <grad_weight(g, x), V> = <g, conv2d(x, V)>, which define the gradients of
  a bilinear map;
* closed forms: all-ones inputs (tap counts from interval lengths), delta
  weights and delta grad_out (placement by strided array slicing), the 1x1
  stride-1 case as a plain matrix product (numpy matmul), exact zeros at
  pixels no tap reaches (stride > kernel);
* integer inputs, for which float64 sums are exact;
* hand-worked tap-count tables under tests/golden/ (no program made them);
* for the RMSNorm-fused product: torch's CPU ``rms_norm`` and matrix product
  in float64, constant rows (normalised to their sign), the one-column case
  written out, scale invariance at eps = 0, linearity in W and in g, and
  zero rows.
"""
from __future__ import annotations

import os

import numpy as np

from conv2d_backward_implicit_amd.workloads import ConvShape, random_shape

# Small random shapes used by the comparison pins (fixed seed, varied
# strides, asymmetric padding up to the kernel size, non-square images).
_RNG_SEED = 20261202
_N_RANDOM = 40


def _random_shapes(count=_N_RANDOM, seed=_RNG_SEED):
    rng = np.random.default_rng(seed)
    shapes = [random_shape(rng, name="rand%d" % i) for i in range(count)]
    # always include asymmetric padding, stride > kernel and Ci != Co cases
    shapes += [
        ConvShape("asym", 2, 3, 7, 9, 4, 3, 5, 1, 0, 2, 5, 9, dist="uniform"),
        ConvShape("s3k2", 1, 2, 8, 7, 3, 2, 2, 3, 1, 0, 3, 2, dist="uniform"),
        ConvShape("s2k3p0", 1, 3, 9, 8, 2, 3, 3, 2, 0, 0, 4, 3, dist="uniform"),
        ConvShape("k5p1", 1, 2, 9, 9, 3, 5, 5, 1, 1, 1, 7, 7, dist="uniform"),
    ]
    return shapes


def _inputs(shape: ConvShape, seed: int):
    rng = np.random.default_rng(seed)
    go = rng.uniform(-1, 1, size=shape.go_shape)
    w = rng.uniform(-1, 1, size=shape.w_shape)
    return go, w


def _gather(orc, shape, go, w):
    return orc.grad_input_gather(go, w, shape.in_h, shape.in_w, shape.stride,
                                 shape.padding_h, shape.padding_w)


def _rel_err(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale) if a.size else 0.0


def pin_torch_grad_input(orc):
    """Gather and scatter agree with torch.nn.grad.conv2d_input (float64)."""
    import torch
    for i, sh in enumerate(_random_shapes()):
        go, w = _inputs(sh, i)
        ref = torch.nn.grad.conv2d_input(
            sh.gi_shape, torch.from_numpy(w), torch.from_numpy(go),
            stride=sh.stride, padding=(sh.padding_h, sh.padding_w)).numpy()
        got = _gather(orc, sh, go, w)
        assert _rel_err(got, ref) < 1e-12, ("gather", sh, _rel_err(got, ref))
        sc = orc.grad_input_scatter(go, w, sh.in_h, sh.in_w, sh.stride,
                                    sh.padding_h, sh.padding_w)
        assert _rel_err(sc, ref) < 1e-12, ("scatter", sh, _rel_err(sc, ref))


def pin_torch_forward(orc):
    """The forward conv agrees with torch.nn.functional.conv2d (float64)."""
    import torch
    for i, sh in enumerate(_random_shapes()):
        rng = np.random.default_rng(1000 + i)
        x = rng.uniform(-1, 1, size=sh.gi_shape)
        w = rng.uniform(-1, 1, size=sh.w_shape)
        ref = torch.nn.functional.conv2d(
            torch.from_numpy(x), torch.from_numpy(w), stride=sh.stride,
            padding=(sh.padding_h, sh.padding_w)).numpy()
        assert ref.shape == sh.go_shape, (ref.shape, sh)
        got = orc.conv2d_forward(x, w, sh.out_h, sh.out_w, sh.stride,
                                 sh.padding_h, sh.padding_w)
        assert _rel_err(got, ref) < 1e-12, (sh, _rel_err(got, ref))


def pin_adjoint(orc):
    """<gather(g), x> equals <g, forward(x)> to float64 rounding."""
    for i, sh in enumerate(_random_shapes()):
        rng = np.random.default_rng(2000 + i)
        g = rng.uniform(-1, 1, size=sh.go_shape)
        w = rng.uniform(-1, 1, size=sh.w_shape)
        x = rng.uniform(-1, 1, size=sh.gi_shape)
        lhs = float(np.sum(_gather(orc, sh, g, w) * x))
        y = orc.conv2d_forward(x, w, sh.out_h, sh.out_w, sh.stride, sh.padding_h,
                               sh.padding_w)
        rhs = float(np.sum(g * y))
        scale = float(np.sum(np.abs(g)) * np.sum(np.abs(w)) + 1.0)
        assert abs(lhs - rhs) <= 1e-12 * scale, (sh, lhs, rhs)


def pin_gather_vs_scatter(orc):
    """The two independent formulations agree on every random shape."""
    for i, sh in enumerate(_random_shapes()):
        go, w = _inputs(sh, 3000 + i)
        a = _gather(orc, sh, go, w)
        b = orc.grad_input_scatter(go, w, sh.in_h, sh.in_w, sh.stride,
                                   sh.padding_h, sh.padding_w)
        assert _rel_err(a, b) < 1e-12, (sh, _rel_err(a, b))


def _tap_count(i, p, k, s, o):
    """How many kernel offsets t in [0, k) reach input index i: those with
    i + p - t = s*m for an integer m in [0, o).  Counted as the number of m in
    an interval: t = i + p - s*m must lie in [0, k)."""
    m_lo = max(0, -((-(i + p - (k - 1))) // s))   # ceil((i + p - k + 1) / s)
    m_hi = min(o - 1, (i + p) // s)                 # floor((i + p) / s)
    return max(0, m_hi - m_lo + 1)


def pin_all_ones(orc):
    """All-ones inputs: grad_input = Co * Th(ih) * Tw(iw), exactly.

    On the 8x8, 3x3, pad 1, stride 1 shape with 16 output channels this is
    16*9 = 144 inside, 16*6 = 96 on edges and 16*4 = 64 at corners."""
    tiny = ConvShape("tiny", 1, 8, 8, 8, 16, 3, 3, 1, 1, 1, 8, 8)
    go = np.ones(tiny.go_shape)
    w = np.ones(tiny.w_shape)
    gi = _gather(orc, tiny, go, w)
    assert gi[0, 0, 3, 4] == 144.0 and gi[0, 5, 0, 4] == 96.0, gi[0, 0]
    assert gi[0, 7, 7, 7] == 64.0 and gi[0, 2, 0, 0] == 64.0, gi[0, 0]
    for sh in _random_shapes() + [tiny]:
        go = np.ones(sh.go_shape)
        w = np.ones(sh.w_shape)
        gi = _gather(orc, sh, go, w)
        th = np.array([_tap_count(i, sh.padding_h, sh.kernel_h, sh.stride, sh.out_h)
                       for i in range(sh.in_h)], dtype=np.float64)
        tw = np.array([_tap_count(i, sh.padding_w, sh.kernel_w, sh.stride, sh.out_w)
                       for i in range(sh.in_w)], dtype=np.float64)
        exp = sh.out_channels * np.outer(th, tw)
        assert np.array_equal(gi, np.broadcast_to(exp, gi.shape)), sh


def _placement_slices(sh, kh, kw):
    """For tap (kh, kw): which grad_out rows/cols land on which input
    rows/cols, as (oh_slice, ih_slice, ow_slice, iw_slice) with in-range
    bounds.  Input row of output row oh is oh*s - ph + kh."""
    def axis(o, s, p, k, n):
        pairs = [(m, m * s - p + k) for m in range(o) if 0 <= m * s - p + k < n]
        return pairs
    rows = axis(sh.out_h, sh.stride, sh.padding_h, kh, sh.in_h)
    cols = axis(sh.out_w, sh.stride, sh.padding_w, kw, sh.in_w)
    return rows, cols


def pin_delta_weight(orc):
    """weight = delta(co0, ci0, kh0, kw0): channel ci0 of grad_input is grad_out
    channel co0 placed at (oh*s - ph + kh0, ow*s - pw + kw0); every other
    channel is zero.  Pins the orientation of the kernel (no flip) and of the
    padding of each axis."""
    for i, sh in enumerate(_random_shapes()[:25]):
        rng = np.random.default_rng(4000 + i)
        go = rng.uniform(-1, 1, size=sh.go_shape)
        co0 = int(rng.integers(sh.out_channels))
        ci0 = int(rng.integers(sh.in_channels))
        kh0 = int(rng.integers(sh.kernel_h))
        kw0 = int(rng.integers(sh.kernel_w))
        w = np.zeros(sh.w_shape)
        w[co0, ci0, kh0, kw0] = 1.0
        exp = np.zeros(sh.gi_shape)
        rows, cols = _placement_slices(sh, kh0, kw0)
        if rows and cols:
            oh = np.array([r[0] for r in rows]); ih = np.array([r[1] for r in rows])
            ow = np.array([c[0] for c in cols]); iw = np.array([c[1] for c in cols])
            exp[:, ci0][:, ih[:, None], iw[None, :]] = go[:, co0][:, oh[:, None], ow[None, :]]
        got = _gather(orc, sh, go, w)
        assert np.array_equal(got, exp), (sh, co0, ci0, kh0, kw0)


def pin_delta_grad_out(orc):
    """grad_out = delta(n0, co0, oh0, ow0): grad_input[n0, :, oh0*s-ph+kh,
    ow0*s-pw+kw] = weight[co0, :, kh, kw] at in-range positions, zero
    elsewhere.  Pins where each kernel tap lands."""
    for i, sh in enumerate(_random_shapes()[:25]):
        rng = np.random.default_rng(5000 + i)
        w = rng.uniform(-1, 1, size=sh.w_shape)
        n0 = int(rng.integers(sh.batch))
        co0 = int(rng.integers(sh.out_channels))
        oh0 = int(rng.integers(sh.out_h))
        ow0 = int(rng.integers(sh.out_w))
        go = np.zeros(sh.go_shape)
        go[n0, co0, oh0, ow0] = 1.0
        exp = np.zeros(sh.gi_shape)
        for kh in range(sh.kernel_h):
            ih = oh0 * sh.stride - sh.padding_h + kh
            if not 0 <= ih < sh.in_h:
                continue
            for kw in range(sh.kernel_w):
                iw = ow0 * sh.stride - sh.padding_w + kw
                if 0 <= iw < sh.in_w:
                    exp[n0, :, ih, iw] = w[co0, :, kh, kw]
        got = _gather(orc, sh, go, w)
        assert np.array_equal(got, exp), (sh, n0, co0, oh0, ow0)


def pin_pointwise_gemm(orc):
    """1x1 kernel, stride 1, no padding: grad_input[n] = W^T @ grad_out[n]
    (numpy matmul over channels, float64)."""
    rng = np.random.default_rng(6000)
    for (n, ci, co, h, w_) in [(2, 5, 7, 3, 4), (1, 16, 9, 5, 5), (3, 1, 4, 2, 6)]:
        sh = ConvShape("pw", n, ci, h, w_, co, 1, 1, 1, 0, 0, h, w_)
        go = rng.uniform(-1, 1, size=sh.go_shape)
        w = rng.uniform(-1, 1, size=sh.w_shape)
        wt = w[:, :, 0, 0].T                       # [Ci, Co]
        exp = np.matmul(wt[None], go.reshape(n, co, h * w_)).reshape(sh.gi_shape)
        got = _gather(orc, sh, go, w)
        assert _rel_err(got, exp) < 1e-13, sh


def pin_zero_structure(orc):
    """1x1 kernel with stride 2 and no padding: only even (ih, iw) are reached
    by a tap; odd rows/cols are exactly zero and even ones are W^T @ grad_out."""
    rng = np.random.default_rng(7000)
    sh = ConvShape("s2k1", 2, 3, 7, 6, 4, 1, 1, 2, 0, 0, 4, 3)
    go = rng.uniform(-1, 1, size=sh.go_shape)
    w = rng.uniform(-1, 1, size=sh.w_shape)
    got = _gather(orc, sh, go, w)
    assert np.all(got[:, :, 1::2, :] == 0.0) and np.all(got[:, :, :, 1::2] == 0.0)
    exp = np.einsum("oc,nohw->nchw", w[:, :, 0, 0], go)
    assert _rel_err(got[:, :, ::2, ::2], exp) < 1e-13


def pin_gather_at(orc):
    """Sampled evaluation returns exactly the full gather at those indices."""
    for i, sh in enumerate(_random_shapes()[:15]):
        go, w = _inputs(sh, 8000 + i)
        full = _gather(orc, sh, go, w).ravel()
        rng = np.random.default_rng(8000 + i)
        idx = rng.integers(0, full.size, size=min(64, full.size))
        got = orc.grad_input_gather_at(go, w, sh.in_h, sh.in_w, sh.stride,
                                       sh.padding_h, sh.padding_w, idx)
        assert np.array_equal(got, full[idx]), sh


def pin_integer_exact(orc):
    """Integer inputs give the same exact integers as torch's float64 routine
    (all partial sums are small integers, so every order is exact)."""
    import torch
    for i, sh in enumerate(_random_shapes()[:20]):
        rng = np.random.default_rng(9000 + i)
        go = rng.integers(-4, 5, size=sh.go_shape).astype(np.float64)
        w = rng.integers(-4, 5, size=sh.w_shape).astype(np.float64)
        ref = torch.nn.grad.conv2d_input(
            sh.gi_shape, torch.from_numpy(w), torch.from_numpy(go),
            stride=sh.stride, padding=(sh.padding_h, sh.padding_w)).numpy()
        got = _gather(orc, sh, go, w)
        assert np.array_equal(got, ref), sh
        assert np.array_equal(got, np.round(got)), sh


GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_tap_count_tables(path=os.path.join(GOLDEN_DIR, "all_ones_tap_counts.txt")):
    """(ConvShape, row counts, column counts) for every case in the table."""
    cases, cur = [], {}
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        cur[line[0]] = [int(v) for v in line[1:]]
        if line[0] == "cols":
            sh = ConvShape("golden%d" % len(cases), *cur["shape"])
            assert len(cur["rows"]) == sh.in_h and len(cur["cols"]) == sh.in_w
            cases.append((sh, cur["rows"], cur["cols"]))
            cur = {}
    return cases


def pin_golden_tap_counts(orc):
    """All-ones inputs against the hand-worked tables: Co * rows[ih] * cols[iw]."""
    cases = load_tap_count_tables()
    assert len(cases) == 4
    for sh, rows, cols in cases:
        gi = _gather(orc, sh, np.ones(sh.go_shape), np.ones(sh.w_shape))
        exp = sh.out_channels * np.outer(np.array(rows, float), np.array(cols, float))
        assert np.array_equal(gi, np.broadcast_to(exp, gi.shape)), (sh, gi[0, 0], exp)


def pin_degenerate(orc):
    """No output channels: the sum is empty and grad_input is all zeros."""
    sh = ConvShape("co0", 1, 3, 5, 5, 0, 3, 3, 1, 1, 1, 5, 5)
    go = np.zeros(sh.go_shape)
    w = np.zeros(sh.w_shape)
    got = _gather(orc, sh, go, w)
    assert got.shape == sh.gi_shape and np.all(got == 0.0)


def _gw_inputs(sh, seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(-1, 1, size=sh.go_shape), rng.uniform(-1, 1, size=sh.gi_shape)


def pin_torch_grad_weight(orc):
    """The weight gradient agrees with torch.nn.grad.conv2d_weight (float64)."""
    import torch
    for i, sh in enumerate(_random_shapes()):
        go, x = _gw_inputs(sh, 4000 + i)
        ref = torch.nn.grad.conv2d_weight(
            torch.from_numpy(x), sh.w_shape, torch.from_numpy(go), stride=sh.stride,
            padding=(sh.padding_h, sh.padding_w)).numpy()
        got = orc.grad_weight(go, x, sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h,
                              sh.padding_w)
        assert got.shape == sh.w_shape, (got.shape, sh)
        assert _rel_err(got, ref) < 1e-12, (sh, _rel_err(got, ref))


def pin_grad_weight_adjoint(orc):
    """<grad_weight(g, x), V> equals <g, forward(x, V)> to float64 rounding:
    the weight gradient of the linear map V -> forward(x, V)."""
    for i, sh in enumerate(_random_shapes()):
        rng = np.random.default_rng(5000 + i)
        g = rng.uniform(-1, 1, size=sh.go_shape)
        x = rng.uniform(-1, 1, size=sh.gi_shape)
        v = rng.uniform(-1, 1, size=sh.w_shape)
        gw = orc.grad_weight(g, x, sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h,
                             sh.padding_w)
        lhs = float(np.sum(gw * v))
        y = orc.conv2d_forward(x, v, sh.out_h, sh.out_w, sh.stride, sh.padding_h,
                               sh.padding_w)
        rhs = float(np.sum(g * y))
        scale = float(np.sum(np.abs(g)) * np.sum(np.abs(x)) + 1.0)
        assert abs(lhs - rhs) <= 1e-12 * scale, (sh, lhs, rhs)


def pin_grad_weight_pointwise(orc):
    """1x1 kernel, stride 1, no padding: grad_weight[co, ci] is the plain
    product sum_n grad_out[n] x[n]^T over pixels (numpy matmul)."""
    sh = ConvShape("gw1x1", 3, 5, 6, 7, 4, 1, 1, 1, 0, 0, 6, 7, dist="uniform")
    go, x = _gw_inputs(sh, 6000)
    N = sh.batch
    ref = sum(go[n].reshape(4, -1) @ x[n].reshape(5, -1).T for n in range(N))
    got = orc.grad_weight(go, x, 1, 1, 1, 0, 0)[:, :, 0, 0]
    assert _rel_err(got, ref) < 1e-12, _rel_err(got, ref)


def _pixel_count(k, p, s, o, n):
    """Output positions m in [0, o) whose source index m*s - p + k lies in
    [0, n): an interval count."""
    lo = max(0, -((-(p - k)) // s))          # ceil((p - k) / s)
    hi = min(o - 1, (n - 1 + p - k) // s)    # floor((n - 1 + p - k) / s)
    return max(0, hi - lo + 1)


def pin_grad_weight_all_ones(orc):
    """All-ones inputs: grad_weight[co, ci, kh, kw] = N * Ph(kh) * Pw(kw),
    with Ph(kh) the output rows whose tap kh lands inside the image."""
    for sh in _random_shapes()[:12] + [ConvShape("gwo", 2, 3, 8, 8, 5, 3, 3, 1, 1, 1, 8, 8)]:
        go = np.ones(sh.go_shape)
        x = np.ones(sh.gi_shape)
        got = orc.grad_weight(go, x, sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h,
                              sh.padding_w)
        for kh in range(sh.kernel_h):
            for kw in range(sh.kernel_w):
                want = sh.batch * _pixel_count(kh, sh.padding_h, sh.stride, sh.out_h,
                                               sh.in_h) * \
                    _pixel_count(kw, sh.padding_w, sh.stride, sh.out_w, sh.in_w)
                assert np.all(got[:, :, kh, kw] == want), (sh, kh, kw, want)


# ---- RMSNorm-fused matrix product (second page, matmul_rms_norm.wgsl) --------

_RMS_SHAPES = [(1, 1, 1), (3, 1, 4), (5, 7, 3), (9, 33, 17), (16, 64, 20), (2, 130, 5)]


def _rms_inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K)), 1.0 + 0.3 * rng.standard_normal(K),
            rng.standard_normal((K, N)))


def pin_torch_rms_norm_matmul(orc):
    """torch's CPU rms_norm (float64, with the norm weight and eps) followed by
    torch's matrix product: an implementation that is not this oracle."""
    import torch
    for i, (M, K, N) in enumerate(_RMS_SHAPES):
        x, g, w = _rms_inputs(M, K, N, 300 + i)
        for eps in (1e-6, 0.25):
            ref = (torch.nn.functional.rms_norm(torch.from_numpy(x), (K,),
                                                weight=torch.from_numpy(g), eps=eps)
                   @ torch.from_numpy(w)).numpy()
            err = _rel_err(orc.rms_norm_matmul(x, g, w, eps), ref)
            assert err <= 1e-12, ((M, K, N), eps, err)


def pin_rms_constant_rows(orc):
    """Row i constant c_i != 0 and eps = 0: the mean square is c_i^2, so the
    normalised row is sign(c_i) everywhere and C[i] = sign(c_i) * (g @ W)."""
    rng = np.random.default_rng(41)
    for M, K, N in [(4, 6, 5), (3, 50, 9), (2, 1, 3)]:
        c = rng.uniform(0.5, 3.0, M) * rng.choice([-1.0, 1.0], M)
        x = np.repeat(c[:, None], K, axis=1)
        g = rng.standard_normal(K)
        w = rng.standard_normal((K, N))
        want = np.sign(c)[:, None] * (g @ w)[None, :]
        err = _rel_err(orc.rms_norm_matmul(x, g, w, 0.0), want)
        assert err <= 1e-13, ((M, K, N), err)


def pin_rms_one_column(orc):
    """K = 1: C[i, j] = x_i / sqrt(x_i^2 + eps) * g * w[0, j], written out for
    chosen numbers (eps large enough to matter)."""
    x = np.array([[2.0], [-0.5], [0.0]])
    g = np.array([3.0])
    w = np.array([[1.0, -2.0]])
    eps = 0.25
    got = orc.rms_norm_matmul(x, g, w, eps)
    # 2/sqrt(4.25)*3 = 2.910427..., -0.5/sqrt(0.5)*3 = -2.121320...
    want = np.array([[6.0 / np.sqrt(4.25), -12.0 / np.sqrt(4.25)],
                     [-1.5 / np.sqrt(0.5), 3.0 / np.sqrt(0.5)],
                     [0.0, 0.0]])
    assert np.max(np.abs(got - want)) <= 1e-14, got


def pin_rms_scale_and_linearity(orc):
    """With eps = 0 a positive scale of a row leaves C unchanged; C is linear
    in W and in g; the all-zero row gives a zero row for eps > 0."""
    x, g, w = _rms_inputs(6, 40, 7, 77)
    alpha = np.array([0.5, 1.0, 2.0, 7.5, 1e-3, 123.0])
    assert _rel_err(orc.rms_norm_matmul(alpha[:, None] * x, g, w, 0.0),
                    orc.rms_norm_matmul(x, g, w, 0.0)) <= 1e-13
    _, g2, w2 = _rms_inputs(6, 40, 7, 78)
    for eps in (0.0, 0.3):
        a = orc.rms_norm_matmul(x, g, w + w2, eps)
        b = orc.rms_norm_matmul(x, g, w, eps) + orc.rms_norm_matmul(x, g, w2, eps)
        assert _rel_err(a, b) <= 1e-13
        a = orc.rms_norm_matmul(x, g + g2, w, eps)
        b = orc.rms_norm_matmul(x, g, w, eps) + orc.rms_norm_matmul(x, g2, w, eps)
        assert _rel_err(a, b) <= 1e-13
    xz = x.copy()
    xz[2] = 0.0
    c = orc.rms_norm_matmul(xz, g, w, 1e-6)
    assert np.all(c[2] == 0.0) and np.all(np.isfinite(c))


def pin_rms_rows(orc):
    """Chosen rows alone equal the same rows of the full product."""
    x, g, w = _rms_inputs(11, 20, 9, 5)
    full = orc.rms_norm_matmul(x, g, w, 1e-5)
    rows = [10, 0, 3, 3]
    assert np.array_equal(orc.rms_norm_matmul(x, g, w, 1e-5, rows=rows), full[rows])


# ---- attention dV (third page, mha_grad_v.wgsl) ----------------------------------

# (q_seq, kv_seq, H, HKV, D, window, causal)
_MHA_CASES = [(9, 9, 4, 2, 8, 0, True), (11, 11, 6, 3, 4, 3, True), (7, 12, 2, 2, 8, 0, False),
              (10, 6, 4, 1, 8, 2, False), (16, 16, 8, 8, 4, 5, True), (5, 5, 3, 1, 6, 1, True)]


def _visible(q_seq, kv_seq, window, causal):
    """[q_seq, kv_seq] mask: query pos sees key t (the page's position loop
    read from the key side: pos in [causal ? t : 0, t + window))."""
    pos = np.arange(q_seq)[:, None]
    t = np.arange(kv_seq)[None, :]
    m = np.ones((q_seq, kv_seq), dtype=bool)
    if causal:
        m &= t <= pos
    if window > 0:
        m &= pos < t + window
    return m


def pin_torch_mha_grad_v(orc):
    """torch autograd of masked softmax attention in float64 (O = softmax(QK^T
    / sqrt(D)) V per head, kv head h // (H / HKV)): dV of <O, dO>; and the
    row statistics against torch.logsumexp."""
    import torch
    for i, (qs, ks, H, HKV, D, win, causal) in enumerate(_MHA_CASES):
        rng = np.random.default_rng(500 + i)
        q, k, v, g = (rng.standard_normal(s_) for s_ in
                      ((qs, H, D), (ks, HKV, D), (ks, HKV, D), (qs, H, D)))
        mask = torch.from_numpy(_visible(qs, ks, win, causal))
        tq, tk, tg = (torch.from_numpy(a) for a in (q, k, g))
        tv = torch.from_numpy(v).requires_grad_(True)
        grp = H // HKV
        out = torch.zeros(qs, H, D, dtype=torch.float64)
        lse_ref = torch.zeros(qs, H, dtype=torch.float64)
        seen_t = mask.any(dim=1)   # rows with no visible key attend to nothing
        for h in range(H):
            sc = (tq[:, h, :] @ tk[:, h // grp, :].T) / np.sqrt(D)
            sc = sc.masked_fill(~mask, float("-inf"))
            lse_ref[:, h] = torch.logsumexp(sc, dim=1)
            sc = torch.where(seen_t[:, None], sc, torch.zeros_like(sc))
            pr = torch.softmax(sc, dim=1) * seen_t[:, None]
            out[:, h, :] = pr @ tv[:, h // grp, :]
        (out * tg).sum().backward()
        lse = orc.attention_lse(q, k, HKV, win, causal)
        seen = _visible(qs, ks, win, causal).any(axis=1)   # rows that see a key
        assert np.max(np.abs((lse[..., 0] + lse[..., 1] - lse_ref.numpy())[seen])) <= 1e-12, i
        assert np.all(lse[~seen] == 0.0), i
        dv = orc.mha_grad_v(g, q, k, lse, win, causal)
        err = _rel_err(dv, tv.grad.numpy())
        assert err <= 1e-12, (i, err)


def pin_torch_attention_row_max(orc):
    """The statistics' first entry on its own: for a row that sees a key, the
    maximum of the scaled scores q . k / sqrt(D) over the keys the mask lets
    through, by torch's masked max in float64 (a row that sees none: 0).
    Their sum with the second entry is invariant to the choice of maximum,
    so this is pinned separately."""
    import torch
    for i, (qs, ks, H, HKV, D, win, causal) in enumerate(_MHA_CASES):
        rng = np.random.default_rng(700 + i)
        q, k = rng.standard_normal((qs, H, D)), rng.standard_normal((ks, HKV, D))
        vis = _visible(qs, ks, win, causal)
        mask = torch.from_numpy(vis)
        grp = H // HKV
        want = np.zeros((qs, H))
        for h in range(H):
            sc = (torch.from_numpy(q[:, h, :]) @ torch.from_numpy(k[:, h // grp, :]).T)
            sc = (sc / np.sqrt(D)).masked_fill(~mask, float("-inf"))
            mx = sc.max(dim=1).values.numpy()
            want[:, h] = np.where(vis.any(axis=1), mx, 0.0)
        lse = orc.attention_lse(q, k, HKV, win, causal)
        assert np.max(np.abs(lse[..., 0] - want)) <= 1e-12, i


def pin_mha_uniform_scores(orc):
    """K = 0: every score is 0, so P = 1 / (number of keys query pos sees)
    and dV[t] = sum over the queries that see t and the group's heads of
    dO / count, with the counts taken from the mask."""
    for i, (qs, ks, H, HKV, D, win, causal) in enumerate(_MHA_CASES):
        rng = np.random.default_rng(600 + i)
        q, g = rng.standard_normal((qs, H, D)), rng.standard_normal((qs, H, D))
        k = np.zeros((ks, HKV, D))
        vis = _visible(qs, ks, win, causal)
        cnt = vis.sum(axis=1)
        want = np.zeros((ks, HKV, D))
        grp = H // HKV
        for t in range(ks):
            for pos in range(qs):
                if vis[pos, t]:
                    for h in range(H):
                        want[t, h // grp] += g[pos, h] / cnt[pos]
        lse = orc.attention_lse(q, k, HKV, win, causal)
        assert _rel_err(orc.mha_grad_v(g, q, k, lse, win, causal), want) <= 1e-13, i


def pin_mha_single_dout(orc):
    """dO nonzero at one (query, head) only: dV is nonzero only for that
    head's kv head and the keys the query sees."""
    qs, ks, H, HKV, D, win, causal = 12, 12, 6, 2, 4, 4, True
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal((qs, H, D)), rng.standard_normal((ks, HKV, D))
    g = np.zeros((qs, H, D))
    pos0, h0 = 7, 4
    g[pos0, h0] = rng.standard_normal(D)
    dv = orc.mha_grad_v(g, q, k, orc.attention_lse(q, k, HKV, win, causal), win, causal)
    vis = _visible(qs, ks, win, causal)[pos0]
    kvh0 = h0 // (H // HKV)
    for t in range(ks):
        for kvh in range(HKV):
            nz = np.any(dv[t, kvh] != 0.0)
            assert nz == (kvh == kvh0 and vis[t]), (t, kvh)


def pin_mha_exponent_clamp(orc):
    """The exponent is clamped at 0: with a row max far below the scores,
    P = exp(-log_sum) for every visible key."""
    qs, ks, H, HKV, D = 6, 6, 2, 1, 4
    rng = np.random.default_rng(8)
    q, k, g = (rng.standard_normal(s_) for s_ in ((qs, H, D), (ks, HKV, D), (qs, H, D)))
    lse = np.zeros((qs, H, 2))
    lse[..., 0] = -1e6
    lse[..., 1] = 0.5
    dv = orc.mha_grad_v(g, q, k, lse, 0, True)
    want = np.zeros((ks, HKV, D))
    for t in range(ks):
        for pos in range(t, qs):
            want[t, 0] += np.exp(-0.5) * g[pos].sum(axis=0)
    assert _rel_err(dv, want) <= 1e-13


ALL_PINS = [
    pin_torch_grad_input,
    pin_torch_forward,
    pin_adjoint,
    pin_gather_vs_scatter,
    pin_all_ones,
    pin_golden_tap_counts,
    pin_delta_weight,
    pin_delta_grad_out,
    pin_pointwise_gemm,
    pin_zero_structure,
    pin_gather_at,
    pin_integer_exact,
    pin_degenerate,
    pin_torch_grad_weight,
    pin_grad_weight_adjoint,
    pin_grad_weight_pointwise,
    pin_grad_weight_all_ones,
    pin_torch_rms_norm_matmul,
    pin_rms_constant_rows,
    pin_rms_one_column,
    pin_rms_scale_and_linearity,
    pin_rms_rows,
    pin_torch_mha_grad_v,
    pin_torch_attention_row_max,
    pin_mha_uniform_scores,
    pin_mha_single_dout,
    pin_mha_exponent_clamp,
]
