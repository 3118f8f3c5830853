"""CPU oracle for conv2d grad-input (and the forward convolution and weight
gradient beside it): TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding in ``conv2d_backward_implicit_amd``) never imports it, and
this package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain loop nests in double precision,
OpenMP over independent output elements).  This module only builds that file
with the host C compiler and marshals numpy arrays to it.

Source cited as [p3]: the docs.rs source page of meganeura 0.2.0,
``src/shaders/conv2d_grad_input_gemm_coop.wgsl``.

Functions (all take float64-convertible arrays and return float64 arrays):

* ``grad_input_gather``    -- the definition ([p3] header comment, weight_T
  staging, the stride > 1 im2col rule applied to every stride).
* ``grad_input_gather_at`` -- the same sum at chosen flat output indices.
* ``grad_input_scatter``   -- independent scatter form (transpose of forward).
* ``conv2d_forward``       -- forward cross-correlation, for the adjoint check.
* ``grad_weight``          -- the weight gradient of the same forward
  cross-correlation (not on the pages; its index map is the forward one).
* ``attention_lse``        -- the forward statistics (row max, log sum) of
  attention under the third page's causal and window bounds.
* ``mha_grad_v``           -- dV of multi-head attention with grouped kv
  heads, ``src/shaders/mha_grad_v.wgsl`` (the third page).
* ``rms_norm_matmul``      -- C = RmsNorm(X, g) x W of the second page,
  ``src/shaders/matmul_rms_norm.wgsl`` (header comment, per-row rsqrt
  prologue, normalise-on-load), in that order, optionally for chosen rows.

Every function is pinned by tests/test_oracle.py to facts outside the oracle
itself (closed forms, delta inputs, a library GEMM, torch's CPU convolution
routines, the adjoint identity), and tests/test_oracle_mutants.py shows that
those pins fail for planted mistakes.  No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_I64 = ctypes.c_int64
_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int64)


def compile_source(src: str, out: str) -> str:
    """Compile one C file into a shared library with gcc -O2 -fopenmp."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(SOURCE)):
        return _LIB_PATH
    return compile_source(SOURCE, _LIB_PATH)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_DP)


def _dims(go_shape, w_shape, H, W, stride, padding_h, padding_w):
    N, Co, OH, OW = (int(v) for v in go_shape)
    Co2, Ci, KH, KW = (int(v) for v in w_shape)
    if Co2 != Co:
        raise ValueError("grad_out channels %d != weight out-channels %d" % (Co, Co2))
    if stride < 1:
        raise ValueError("stride must be >= 1")
    return [N, Ci, int(H), int(W), Co, KH, KW, int(stride), int(padding_h),
            int(padding_w), OH, OW]


class Oracle:
    """ctypes wrapper around one build of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        sig = [_DP, _DP, _DP] + [_I64] * 12
        for name in ("oracle_grad_input_gather", "oracle_grad_input_scatter",
                     "oracle_conv2d_forward", "oracle_grad_weight"):
            fn = getattr(lib, name)
            fn.argtypes = sig
            fn.restype = None
        lib.oracle_grad_input_gather_at.argtypes = [_DP, _DP, _IP, _I64, _DP] + [_I64] * 12
        lib.oracle_grad_input_gather_at.restype = None
        lib.oracle_rms_norm_matmul.argtypes = [_DP, _DP, _DP, _DP, _I64, _I64, _I64,
                                               ctypes.c_double, _IP, _I64]
        lib.oracle_rms_norm_matmul.restype = None
        lib.oracle_attention_lse.argtypes = [_DP, _DP, _DP] + [_I64] * 7
        lib.oracle_attention_lse.restype = None
        lib.oracle_mha_grad_v.argtypes = [_DP] * 5 + [_I64] * 7
        lib.oracle_mha_grad_v.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self._lib = lib
        self.path = path

    def grad_input_gather(self, grad_out, weight, H, W, stride, padding_h, padding_w):
        """grad_input [N, Ci, H, W] by the direct gather definition (float64)."""
        go, w = _f64(grad_out), _f64(weight)
        d = _dims(go.shape, w.shape, H, W, stride, padding_h, padding_w)
        gi = np.empty((d[0], d[1], d[2], d[3]), dtype=np.float64)
        self._lib.oracle_grad_input_gather(_ptr(go), _ptr(w), _ptr(gi), *d)
        return gi

    def grad_input_gather_at(self, grad_out, weight, H, W, stride, padding_h,
                             padding_w, flat_idx):
        """The gather definition evaluated at flat grad_input indices (float64)."""
        go, w = _f64(grad_out), _f64(weight)
        d = _dims(go.shape, w.shape, H, W, stride, padding_h, padding_w)
        idx = np.ascontiguousarray(flat_idx, dtype=np.int64)
        total = d[0] * d[1] * d[2] * d[3]
        if idx.size and (idx.min() < 0 or idx.max() >= total):
            raise IndexError("flat index out of range")
        out = np.empty(idx.shape, dtype=np.float64)
        self._lib.oracle_grad_input_gather_at(
            _ptr(go), _ptr(w), idx.ctypes.data_as(_IP), int(idx.size), _ptr(out), *d)
        return out

    def grad_input_scatter(self, grad_out, weight, H, W, stride, padding_h, padding_w):
        """grad_input [N, Ci, H, W] by the scatter formulation (float64)."""
        go, w = _f64(grad_out), _f64(weight)
        d = _dims(go.shape, w.shape, H, W, stride, padding_h, padding_w)
        gi = np.empty((d[0], d[1], d[2], d[3]), dtype=np.float64)
        self._lib.oracle_grad_input_scatter(_ptr(go), _ptr(w), _ptr(gi), *d)
        return gi

    def conv2d_forward(self, x, weight, OH, OW, stride, padding_h, padding_w):
        """Forward cross-correlation y [N, Co, OH, OW] (float64)."""
        xx, w = _f64(x), _f64(weight)
        N, Ci, H, W = (int(v) for v in xx.shape)
        Co, Ci2, KH, KW = (int(v) for v in w.shape)
        if Ci2 != Ci:
            raise ValueError("x channels %d != weight in-channels %d" % (Ci, Ci2))
        y = np.empty((N, Co, int(OH), int(OW)), dtype=np.float64)
        self._lib.oracle_conv2d_forward(_ptr(xx), _ptr(w), _ptr(y), N, Ci, H, W,
                                        Co, KH, KW, int(stride), int(padding_h),
                                        int(padding_w), int(OH), int(OW))
        return y

    def grad_weight(self, grad_out, x, KH, KW, stride, padding_h, padding_w):
        """Weight gradient [Co, Ci, KH, KW] of the forward cross-correlation
        (float64); grad_out [N, Co, OH, OW], x [N, Ci, H, W]."""
        go, xx = _f64(grad_out), _f64(x)
        N, Co, OH, OW = (int(v) for v in go.shape)
        N2, Ci, H, W = (int(v) for v in xx.shape)
        if N2 != N:
            raise ValueError("grad_out batch %d != x batch %d" % (N, N2))
        gw = np.empty((Co, Ci, int(KH), int(KW)), dtype=np.float64)
        self._lib.oracle_grad_weight(_ptr(go), _ptr(xx), _ptr(gw), N, Ci, H, W, Co,
                                     int(KH), int(KW), int(stride), int(padding_h),
                                     int(padding_w), OH, OW)
        return gw

    def rms_norm_matmul(self, x, g, w, eps, rows=None):
        """C [M, N] = RmsNorm(x [M, K], g [K], eps) x w [K, N] (float64).  With
        ``rows`` (indices), only those rows are computed and returned, as a
        [len(rows), N] array."""
        xx, gg, ww = _f64(x), _f64(g), _f64(w)
        M, K = (int(v) for v in xx.shape)
        K2, N = (int(v) for v in ww.shape)
        if K2 != K or gg.shape != (K,):
            raise ValueError("shapes x %s, g %s, w %s do not chain" % (xx.shape, gg.shape,
                                                                     ww.shape))
        if K < 1:
            raise ValueError("the mean over K needs K >= 1")
        sel = np.arange(M, dtype=np.int64) if rows is None else \
            np.ascontiguousarray(rows, dtype=np.int64)
        if sel.size and (sel.min() < 0 or sel.max() >= M):
            raise IndexError("row index out of range")
        # each row once: the C routine computes its rows in parallel, in place
        todo = np.ascontiguousarray(np.unique(sel), dtype=np.int64)
        c = np.zeros((M, N), dtype=np.float64)
        self._lib.oracle_rms_norm_matmul(_ptr(xx), _ptr(gg), _ptr(ww), _ptr(c), M, K, N,
                                         float(eps), todo.ctypes.data_as(_IP), int(todo.size))
        return c if rows is None else c[sel]

    def attention_lse(self, q, k, num_kv_heads, window=0, causal=True):
        """(max, log sum exp) per query row and head [q_seq, H, 2] (float64);
        q [q_seq, H, D], k [kv_seq, HKV, D]."""
        qq, kk = _f64(q), _f64(k)
        q_seq, H, D = (int(v) for v in qq.shape)
        kv_seq, HKV, D2 = (int(v) for v in kk.shape)
        if D2 != D or HKV != int(num_kv_heads) or H % HKV:
            raise ValueError("shapes q %s, k %s do not match" % (qq.shape, kk.shape))
        lse = np.empty((q_seq, H, 2), dtype=np.float64)
        self._lib.oracle_attention_lse(_ptr(qq), _ptr(kk), _ptr(lse), q_seq, kv_seq, H, HKV, D,
                                       int(window), int(bool(causal)))
        return lse

    def mha_grad_v(self, dout, q, k, lse, window=0, causal=True):
        """dV [kv_seq, HKV, D] (float64); dout, q [q_seq, H, D], k
        [kv_seq, HKV, D], lse [q_seq, H, 2]."""
        g, qq, kk, ll = _f64(dout), _f64(q), _f64(k), _f64(lse)
        q_seq, H, D = (int(v) for v in qq.shape)
        kv_seq, HKV, D2 = (int(v) for v in kk.shape)
        if g.shape != qq.shape or D2 != D or H % HKV or ll.shape != (q_seq, H, 2):
            raise ValueError("shapes do not match")
        dv = np.empty((kv_seq, HKV, D), dtype=np.float64)
        self._lib.oracle_mha_grad_v(_ptr(g), _ptr(qq), _ptr(kk), _ptr(ll), _ptr(dv), q_seq,
                                    kv_seq, H, HKV, D, int(window), int(bool(causal)))
        return dv

    def num_threads(self) -> int:
        """OpenMP threads the oracle routines use in this process."""
        return int(self._lib.oracle_num_threads())


_default = None
_lock = threading.Lock()


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing/stale)."""
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build(force=False))
    return _default


def grad_input_gather(*a, **k):
    return default().grad_input_gather(*a, **k)


def grad_input_gather_at(*a, **k):
    return default().grad_input_gather_at(*a, **k)


def grad_input_scatter(*a, **k):
    return default().grad_input_scatter(*a, **k)


def conv2d_forward(*a, **k):
    return default().conv2d_forward(*a, **k)


def grad_weight(*a, **k):
    return default().grad_weight(*a, **k)


def attention_lse(*a, **k):
    return default().attention_lse(*a, **k)


def mha_grad_v(*a, **k):
    return default().mha_grad_v(*a, **k)


def rms_norm_matmul(*a, **k):
    return default().rms_norm_matmul(*a, **k)


def num_threads() -> int:
    return default().num_threads()
