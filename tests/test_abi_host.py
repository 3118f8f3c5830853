"""Host-side checks of the C ABI: no GPU needed, no kernel is launched.

The library must load on a machine without a GPU, export every function the
header declares, and turn every invalid argument into its status code before
any HIP call is made.
"""
import ctypes
import glob
import os
import re

import pytest

import conv2d_backward_implicit_amd as c2b
from conv2d_backward_implicit_amd.workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv2d_bwd.h")

OK, NULL, BAD, ALIAS, OVF, UNSUP = 0, -1, -2, -3, -4, -5


HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _header_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text,
                                flags=re.M))
    return sorted(names)


def _p(**kw):
    base = dict(batch=1, in_channels=3, in_h=8, in_w=8, out_channels=4,
                kernel_h=3, kernel_w=3, stride=1, padding_h=1, padding_w=1)
    base.update(kw)
    return c2b.make_params(**base)


def test_library_loads_and_exports_every_declared_symbol():
    lib = c2b.load_library()
    declared = _header_functions()
    assert declared == sorted(c2b.EXPORTED_SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_params_struct_layout_matches_header():
    assert ctypes.sizeof(c2b.Conv2dParams) == 48
    text = open(HEADER).read()
    body = re.search(r"typedef struct conv2d_params \{(.*?)\} conv2d_params;", text,
                     re.S).group(1)
    fields = re.findall(r"uint32_t (\w+);", body)
    assert fields == [f for f, _ in c2b.Conv2dParams._fields_]
    assert ctypes.sizeof(c2b.PlanInfo) == 48


def test_status_strings():
    for code in (OK, NULL, BAD, ALIAS, OVF, UNSUP, -6):
        s = c2b.status_string(code)
        assert s and s != "unknown status", code
    assert c2b.status_string(12345) == "unknown status"


def test_valid_shapes_ok():
    for cfg in CONFIGS:
        p = c2b.make_params(cfg.batch, cfg.in_channels, cfg.in_h, cfg.in_w,
                            cfg.out_channels, cfg.kernel_h, cfg.kernel_w, cfg.stride,
                            cfg.padding_h, cfg.padding_w, cfg.out_h, cfg.out_w)
        assert c2b.check_params(p) == OK, cfg.name


def test_null_params():
    lib = c2b.load_library()
    assert lib.conv2d_check_params(None) == NULL
    info = c2b.PlanInfo()
    assert lib.conv2d_describe_plan(None, 0, ctypes.byref(info)) == NULL
    assert lib.conv2d_describe_plan(ctypes.byref(_p()), 0, None) == NULL


@pytest.mark.parametrize("kw", [
    dict(stride=0, out_h=1, out_w=1),
    dict(kernel_h=0, out_h=10),
    dict(kernel_w=0, out_w=10),
    dict(out_h=7),                       # forward extent is 8
    dict(out_w=9),
    dict(in_h=1, padding_h=0, out_h=1),  # padded input smaller than kernel
    dict(in_w=2, padding_w=0, kernel_w=3, out_w=1),
])
def test_bad_shape(kw):
    assert c2b.check_params(_p(**kw)) == BAD


def test_padding_axes_are_separate():
    # out_h follows padding_h and out_w follows padding_w
    p = _p(in_h=9, in_w=9, padding_h=0, padding_w=2, out_h=7, out_w=11)
    assert c2b.check_params(p) == OK
    p = _p(in_h=9, in_w=9, padding_h=0, padding_w=2, out_h=11, out_w=7)
    assert c2b.check_params(p) == BAD


def test_overflow():
    # per-image grad_input plane of 2^31 elements
    p = _p(in_channels=2 ** 11, in_h=2 ** 10, in_w=2 ** 10)
    assert c2b.check_params(p) == OVF
    # weight of 2^31 elements
    p = _p(in_channels=2 ** 16, out_channels=2 ** 15, kernel_h=1, kernel_w=1,
           padding_h=0, padding_w=0)
    assert c2b.check_params(p) == OVF
    # a large batch alone is fine (64-bit batch offsets)
    p = _p(batch=2 ** 20)
    assert c2b.check_params(p) == OK


def test_unsupported_kernel_window():
    # a 40x40 stride-1 kernel window cannot be staged on chip
    p = _p(in_h=64, in_w=64, kernel_h=40, kernel_w=40, padding_h=0, padding_w=0)
    assert c2b.check_params(p) == UNSUP
    # the same kernel with stride 4 splits into 16 classes of 10x10 taps
    p = _p(in_h=64, in_w=64, kernel_h=40, kernel_w=40, padding_h=0, padding_w=0,
           stride=4)
    assert c2b.check_params(p) == OK


def test_degenerate_sizes_ok():
    for kw in (dict(batch=0), dict(in_channels=0), dict(out_channels=0),
               dict(in_h=0, padding_h=1, kernel_h=1, out_h=2)):
        assert c2b.check_params(_p(**kw)) == OK, kw
    info = c2b.describe_plan(_p(batch=0))
    assert info["tiles"] == 0 and info["launches"] == 0


def _call(fn, go, w, gi, p):
    return fn(go, w, gi, p, 0)


@pytest.mark.parametrize("fn", [c2b.conv2d_grad_input, c2b.conv2d_grad_input_f16])
def test_entry_points_reject_before_any_device_call(fn):
    p = _p()
    # shape errors come first
    assert _call(fn, 0x1000, 0x2000, 0x3000, _p(stride=0, out_h=1, out_w=1)) == BAD
    # null pointers of non-empty tensors
    assert _call(fn, 0, 0x2000, 0x100000, p) == NULL
    assert _call(fn, 0x1000, 0, 0x100000, p) == NULL
    assert _call(fn, 0x1000, 0x2000, 0, p) == NULL
    # grad_input overlapping grad_out or weight
    gi_bytes = 1 * 3 * 8 * 8 * 4
    assert _call(fn, 0x100000, 0x900000, 0x100000, p) == ALIAS
    assert _call(fn, 0x100000 + gi_bytes - 4, 0x900000, 0x100000, p) == ALIAS
    assert _call(fn, 0x100000, 0x900000 + 4, 0x900000, p) == ALIAS
    lib = c2b.load_library()
    assert getattr(lib, fn.__name__)(ctypes.c_void_p(1), ctypes.c_void_p(2),
                                     ctypes.c_void_p(3), None, None) == NULL


def test_plan_phases_and_work():
    by = {c.name.split("_")[0]: c for c in CONFIGS}
    def plan(c, f16=False):
        p = c2b.make_params(c.batch, c.in_channels, c.in_h, c.in_w, c.out_channels,
                            c.kernel_h, c.kernel_w, c.stride, c.padding_h,
                            c.padding_w, c.out_h, c.out_w)
        return c2b.describe_plan(p, f16)
    # stride 1: one class; stride 2: four classes, none empty for 3x3 / 7x7
    assert plan(by["resnet"])["phases"] == 1
    assert plan(by["strided"])["phases"] == 4
    assert plan(by["stem"])["phases"] == 4
    for c in CONFIGS:
        info = plan(c, c.f16_staged)
        assert info["zero_phases"] == 0
        assert info["useful_macs"] * 2 == c.useful_flops
        # the residue split never issues the 4x structural-zero work of a
        # dense im2col GEMM: issued MACs stay within tile padding of useful
        assert info["macs"] >= info["useful_macs"]
    # ResNet stage-1, fp32: at most one tile per workgroup slot (256 CUs, at
    # most two workgroups each), in one launch, >= 90% of issued lanes useful
    r = plan(by["resnet"])
    assert r["tiles"] <= 2 * 256 and r["launches"] == 1
    assert r["useful_macs"] >= 0.9 * r["macs"]
    # strided: issued work within 1.25x of useful (no 4x zero work)
    s = plan(by["strided"])
    assert s["macs"] <= 1.25 * s["useful_macs"]


def test_plan_zero_classes_when_stride_exceeds_kernel():
    # 1x1 kernel, stride 2: only the class (0, 0) is reached by a tap
    p = _p(in_h=7, in_w=6, kernel_h=1, kernel_w=1, padding_h=0, padding_w=0,
           stride=2, out_h=4, out_w=3)
    info = c2b.describe_plan(p)
    assert info["phases"] == 4 and info["zero_phases"] == 3
    # stride 3 with a 2x2 kernel: 9 classes, 5 of them without taps
    p = _p(in_h=8, in_w=7, kernel_h=2, kernel_w=2, padding_h=1, padding_w=0,
           stride=3, out_h=3, out_w=2)
    info = c2b.describe_plan(p)
    assert info["phases"] == 9 and info["zero_phases"] == 5


def test_library_shares_torchs_hip_runtime():
    """Loaded first thing in a fresh process, the library must still bind to
    the HIP runtime torch carries: with two runtimes in one process, every
    launch on a torch stream fails."""
    import subprocess
    import sys
    code = (
        "import conv2d_backward_implicit_amd as c2b\n"
        "c2b.load_library()\n"
        "paths = set()\n"
        "for line in open('/proc/self/maps'):\n"
        "    if 'libamdhip64' in line:\n"
        "        paths.add(line.split()[-1])\n"
        "print(len(paths))\n"
        "print('\\n'.join(sorted(paths)))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = out.stdout.split()
    assert lines[0] == "1", out.stdout
    import torch
    assert os.path.dirname(torch.__file__) in lines[1], out.stdout


def test_tune_rejects_before_any_device_call():
    lib = c2b.load_library()
    chosen = ctypes.c_int(7)

    def tune(go, w, gi, p, f16=0):
        return lib.conv2d_tune(ctypes.c_void_p(go), ctypes.c_void_p(w), ctypes.c_void_p(gi),
                               ctypes.byref(p), f16, None, ctypes.byref(chosen))
    p = _p()
    assert tune(0x1000, 0x2000, 0x3000, _p(stride=0, out_h=1, out_w=1)) == BAD
    assert tune(0, 0x2000, 0x100000, p) == NULL
    assert tune(0x100000, 0x900000, 0x100000, p, 1) == ALIAS
    assert chosen.value == 7   # untouched on a validation error


def test_planned_variant_is_a_variant_of_the_path():
    for f16 in (False, True):
        v = c2b.planned_variant(_p(in_channels=40, out_channels=24), f16)
        assert 0 <= v < c2b.num_variants() and c2b.variant_is_f16(v) == int(f16)
    assert c2b.planned_variant(_p(batch=0)) == -1
    with pytest.raises(c2b.Conv2dError):
        c2b.planned_variant(_p(stride=0, out_h=1, out_w=1))
    lib = c2b.load_library()
    assert lib.conv2d_planned_variant(ctypes.byref(_p()), 0, None) == NULL


def test_select_variant_sets_the_default_plan_and_survives_other_shapes():
    """A chosen variant is the default plan's until changed, however many
    other shapes are planned afterwards (the plan memo is bounded, the table
    of chosen variants is not evicted)."""
    p = _p(batch=3, in_channels=56, in_h=9, in_w=11, out_channels=30)
    for f16 in (False, True):
        model = c2b.planned_variant(p, f16)
        others = [v for v in range(c2b.num_variants())
                  if c2b.variant_is_f16(v) == int(f16) and v != model
                  and _tiles(p, v)]
        assert others
        chosen = others[-1]
        c2b.select_variant(p, f16, chosen)
        assert c2b.planned_variant(p, f16) == chosen
        assert c2b.planned_variant(p, not f16) != chosen      # per path
        # plan 150 other shapes (more than the memo holds), each with every
        # variant of the path forced through describe and the default plan
        for i in range(150):
            q = _p(batch=1 + i % 3, in_channels=8 + i, in_h=7, in_w=9, out_channels=12)
            c2b.planned_variant(q, f16)
        assert c2b.planned_variant(p, f16) == chosen
        c2b.select_variant(p, f16, -1)                          # back to the model
        assert c2b.planned_variant(p, f16) == model


def _tiles(p, v):
    try:
        c2b.describe_plan_variant(p, v)
        return True
    except c2b.Conv2dError:
        return False


def test_select_variant_rejects():
    lib = c2b.load_library()
    p = _p(in_channels=40, out_channels=24)
    n = c2b.num_variants()
    fp32 = next(v for v in range(n) if c2b.variant_is_f16(v) == 0)
    assert lib.conv2d_select_variant(ctypes.byref(p), 0, n) == UNSUP
    assert lib.conv2d_select_variant(ctypes.byref(p), 0, -2) == UNSUP
    assert lib.conv2d_select_variant(ctypes.byref(p), 1, fp32) == UNSUP   # other path
    assert lib.conv2d_select_variant(None, 0, fp32) == NULL
    assert lib.conv2d_select_variant(ctypes.byref(_p(stride=0, out_h=1, out_w=1)), 0,
                                     fp32) == BAD
    assert lib.conv2d_select_variant(ctypes.byref(p), 0, -1) == OK        # nothing chosen


def test_describe_plan_variant_matches_forced_plans():
    p = _p(in_channels=40, out_channels=24)
    for v in range(c2b.num_variants()):
        try:
            info = c2b.describe_plan_variant(p, v)
        except c2b.Conv2dError as e:
            assert e.status == -5, (v, e.status)
            continue
        assert info["useful_macs"] == 1 * 24 * 8 * 8 * 40 * 9
        assert info["macs"] >= info["useful_macs"] and info["tiles"] >= 1
    with pytest.raises(c2b.Conv2dError):
        c2b.describe_plan_variant(p, c2b.num_variants())


# ---- forward convolution entry points ---------------------------------------

@pytest.mark.parametrize("fn", [c2b.conv2d_forward, c2b.conv2d_forward_f16])
def test_forward_entry_points_reject_before_any_device_call(fn):
    p = _p()
    assert _call(fn, 0x1000, 0x2000, 0x3000, _p(stride=0, out_h=1, out_w=1)) == BAD
    # null pointers of non-empty tensors (x, weight, y)
    assert _call(fn, 0, 0x2000, 0x100000, p) == NULL
    assert _call(fn, 0x1000, 0, 0x100000, p) == NULL
    assert _call(fn, 0x1000, 0x2000, 0, p) == NULL
    # y (1 x 4 x 8 x 8 fp32) overlapping x or weight
    y_bytes = 1 * 4 * 8 * 8 * 4
    assert _call(fn, 0x100000, 0x900000, 0x100000, p) == ALIAS
    assert _call(fn, 0x100000 + y_bytes - 4, 0x900000, 0x100000, p) == ALIAS
    assert _call(fn, 0x100000, 0x900000 + 4, 0x900000, p) == ALIAS
    # x may end where y begins
    x_bytes = 1 * 3 * 8 * 8 * 4
    lib = c2b.load_library()
    assert getattr(lib, fn.__name__)(ctypes.c_void_p(1), ctypes.c_void_p(2),
                                     ctypes.c_void_p(3), None, None) == NULL
    assert x_bytes < y_bytes


def test_forward_variant_and_tune_reject_before_any_device_call():
    lib = c2b.load_library()
    p = _p()
    n = c2b.num_variants()
    assert c2b.conv2d_forward_variant(0x1000, 0x2000, 0x100000, p, n) == UNSUP
    cm = [v for v in range(n) if c2b.variant_uses_column_taps(v) == 1]
    assert c2b.conv2d_forward_variant(0x1000, 0x2000, 0x100000, p, cm[0]) == UNSUP
    chosen = ctypes.c_int(7)

    def tune(x, w, y, q, f16=0):
        return lib.conv2d_tune_forward(ctypes.c_void_p(x), ctypes.c_void_p(w),
                                       ctypes.c_void_p(y), ctypes.byref(q), f16, None,
                                       ctypes.byref(chosen))
    assert tune(0x1000, 0x2000, 0x3000, _p(stride=0, out_h=1, out_w=1)) == BAD
    assert tune(0, 0x2000, 0x100000, p) == NULL
    assert tune(0x100000, 0x900000, 0x100000, p, 1) == ALIAS
    assert chosen.value == 7


def test_forward_plans():
    p = _p(in_channels=40, out_channels=24)
    for f16 in (False, True):
        v = c2b.planned_forward_variant(p, f16)
        assert 0 <= v < c2b.num_variants() and c2b.variant_is_f16(v) == int(f16)
        assert c2b.variant_uses_column_taps(v) == 0
        info = c2b.describe_forward_plan(p, f16)
        assert info["useful_macs"] == 1 * 24 * 8 * 8 * 40 * 9
        assert info["launches"] == 1 and info["phases"] == 1 and info["tiles"] >= 1
    for v in range(c2b.num_variants()):
        if c2b.variant_uses_column_taps(v) == 1 or c2b.variant_is_multi_class(v) == 1:
            with pytest.raises(c2b.Conv2dError):   # no forward instance
                c2b.describe_forward_plan_variant(p, v)
            continue
        info = c2b.describe_forward_plan_variant(p, v)
        assert info["macs"] >= info["useful_macs"] > 0
    # no image or no output channel: nothing to write; no input channel: y
    # still gets its zeros
    assert c2b.describe_forward_plan(_p(batch=0))["tiles"] == 0
    assert c2b.describe_forward_plan(_p(out_channels=0))["tiles"] == 0
    zero = c2b.describe_forward_plan(_p(in_channels=0))
    assert zero["tiles"] >= 1 and zero["macs"] == 0
    assert c2b.planned_forward_variant(_p(batch=0)) == -1
    with pytest.raises(c2b.Conv2dError):
        c2b.describe_forward_plan(_p(stride=0, out_h=1, out_w=1))


def test_forward_few_channel_route():
    """fp32 forward with 1-15 input channels runs the im2col GEMM, which has
    no variant; a batch too large for that kernel's 32-bit whole-tensor
    offsets takes the variant kernels (which offset per image) instead of
    failing."""
    lib = c2b.load_library()
    stem = c2b.make_params(16, 3, 224, 224, 64, 7, 7, 2, 3, 3)
    assert c2b.planned_forward_variant(stem, False) == -1
    assert lib.conv2d_select_forward_variant(ctypes.byref(stem), 0, 0) == UNSUP
    assert lib.conv2d_select_forward_variant(ctypes.byref(stem), 0, -1) == OK
    v16 = c2b.planned_forward_variant(stem, True)            # f16: variant family
    assert v16 >= 0 and c2b.variant_is_f16(v16) == 1
    # x of 4000 x 3 x 224 x 224 fp32 is 2.4 GB, past 2^31 bytes
    big = c2b.make_params(4000, 3, 224, 224, 64, 7, 7, 2, 3, 3)
    assert c2b.check_params(big) == OK
    v = c2b.planned_forward_variant(big, False)
    assert v >= 0 and c2b.variant_is_f16(v) == 0 and c2b.variant_uses_column_taps(v) == 0
    c2b.select_forward_variant(big, False, v)
    assert c2b.planned_forward_variant(big, False) == v
    c2b.select_forward_variant(big, False, -1)


def test_multi_class_planning():
    """Multi-class variants tile only fp32 stride-2 input gradients whose four
    residue classes all have pixels and taps (kernel of at most 9 taps); on
    such a layer every class is in the one launch, and the model picks a
    multi-class variant for the strided workload.  They issue fewer MACs
    than a per-class plan would pad, never fewer than the useful ones."""
    mc = [v for v in range(c2b.num_variants()) if c2b.variant_is_multi_class(v) == 1]
    assert len(mc) == 3 and all(c2b.variant_is_f16(v) == 0 for v in mc)
    strided = c2b.make_params(32, 128, 56, 56, 256, 3, 3, 2, 1, 1)
    assert c2b.planned_variant(strided, False) in mc
    for v in mc:
        info = c2b.describe_plan_variant(strided, v)
        assert info["launches"] == 1 and info["phases"] == 4 and info["zero_phases"] == 0
        assert info["useful_macs"] <= info["macs"] <= 1.07 * info["useful_macs"]
    for bad in (c2b.make_params(4, 16, 20, 20, 8, 3, 3, 1, 1, 1),    # stride 1
                c2b.make_params(4, 16, 20, 20, 8, 5, 5, 2, 2, 2),    # 25 taps
                c2b.make_params(4, 16, 20, 20, 8, 1, 1, 2, 0, 0),    # three classes without taps
                c2b.make_params(4, 16, 20, 20, 8, 3, 3, 3, 1, 1)):   # stride 3
        for v in mc:
            with pytest.raises(c2b.Conv2dError):
                c2b.describe_plan_variant(bad, v)
    # the f16-staged path has no multi-class variant
    assert c2b.planned_variant(strided, True) not in mc


def test_forward_pointwise_route():
    """1x1, stride-1, unpadded forward shapes run on the 1x1 GEMM (no
    variant), except those with fewer than 16 input channels on the fp32
    path, which the im2col GEMM takes; the plan description reports one
    launch of ceil(Co/128) x ceil(N H W/128) tiles."""
    lib = c2b.load_library()
    p = c2b.make_params(64, 256, 14, 14, 1024, 1, 1, 1, 0, 0)
    for f16 in (False, True):
        assert c2b.planned_forward_variant(p, f16) == -1
        assert lib.conv2d_select_forward_variant(ctypes.byref(p), int(f16), 0) == UNSUP
        assert lib.conv2d_select_forward_variant(ctypes.byref(p), int(f16), -1) == OK
        info = c2b.describe_forward_plan(p, f16)
        assert info["launches"] == 1 and info["phases"] == 1
        assert info["tiles"] == 8 * ((64 * 14 * 14 + 127) // 128)
        assert info["useful_macs"] == 64 * 14 * 14 * 256 * 1024
    # the input gradient of the same shape: ceil(Ci/128) row tiles
    assert c2b.describe_plan(p, False)["tiles"] == 2 * ((64 * 14 * 14 + 127) // 128)
    # a 1x1 stride-2 shape is not on the GEMM: a variant runs it
    p2 = c2b.make_params(4, 64, 14, 14, 32, 1, 1, 2, 0, 0)
    assert c2b.planned_forward_variant(p2, False) >= 0


# ---- weight gradient entry points ---------------------------------------------

def test_grad_weight_rejects_before_any_device_call():
    lib = c2b.load_library()
    p = _p()                       # go 1x4x8x8, x 1x3x8x8, dw 4x3x3x3
    need = c2b.grad_weight_workspace_size(p)
    assert need > 0

    def call(go, x, dw, q, ws=0x7000000, wsb=None):
        return c2b.conv2d_grad_weight(go, x, dw, q, ws, need if wsb is None else wsb)
    assert call(0x1000, 0x2000, 0x3000, _p(stride=0, out_h=1, out_w=1)) == BAD
    assert call(0, 0x200000, 0x400000, p) == NULL
    assert call(0x100000, 0, 0x400000, p) == NULL
    assert call(0x100000, 0x200000, 0, p) == NULL
    # workspace missing or too small
    assert call(0x100000, 0x200000, 0x400000, p, ws=0) == -7
    assert call(0x100000, 0x200000, 0x400000, p, wsb=need - 4) == -7
    assert call(0x100000, 0x200000, 0x400000, p, ws=0x7000004) == -7   # not 16-byte aligned
    # grad_weight or workspace overlapping an input or each other
    assert call(0x100000, 0x200000, 0x100000, p) == ALIAS
    assert call(0x100000, 0x200000, 0x400000, p, ws=0x200000) == ALIAS
    assert call(0x100000, 0x200000, 0x400000, p, ws=0x400000) == ALIAS
    assert lib.conv2d_grad_weight(None, None, None, None, None, 0, None) == NULL
    assert c2b.status_string(-7).startswith("workspace")


def test_grad_weight_workspace_size():
    lib = c2b.load_library()
    assert lib.conv2d_grad_weight_workspace_size(ctypes.byref(_p()), None) == NULL
    with pytest.raises(c2b.Conv2dError):
        c2b.grad_weight_workspace_size(_p(stride=0, out_h=1, out_w=1))
    # no pixel or no output: nothing to split
    assert c2b.grad_weight_workspace_size(_p(batch=0)) == 0
    assert c2b.grad_weight_workspace_size(_p(out_channels=0)) == 0
    assert c2b.grad_weight_workspace_size(_p(in_channels=0)) == 0
    # one 64 x 64 partial tile per (chunk, co tile, column tile), enough
    # column slots for every weight column
    for sh in CONFIGS:
        p = c2b.make_params(sh.batch, sh.in_channels, sh.in_h, sh.in_w, sh.out_channels,
                            sh.kernel_h, sh.kernel_w, sh.stride, sh.padding_h, sh.padding_w)
        for v in [-1] + list(range(c2b.GRAD_WEIGHT_VARIANTS)):
            n = c2b.grad_weight_workspace_size(p, v)
            d = c2b.describe_grad_weight_plan(p, v)
            assert n == d["chunks"] * d["co_tiles"] * d["column_tiles"] * 64 * 64 * 4, (sh.name, v)
            assert d["co_tiles"] * 64 >= sh.out_channels
            assert d["column_tiles"] * 64 >= sh.in_channels * sh.kernel_h * sh.kernel_w
            assert d["chunks"] * d["chunk_pixels"] >= sh.batch * sh.out_h * sh.out_w
            if v >= 0:
                assert d["variant"] == v


def test_grad_weight_variants_host():
    lib = c2b.load_library()
    p = _p()
    need = c2b.grad_weight_workspace_size(p, 0)
    for v in (-2, c2b.GRAD_WEIGHT_VARIANTS):
        assert c2b.conv2d_grad_weight_variant(0x100000, 0x200000, 0x400000, p, 0x7000000,
                                              need, 0, v) == -5
        with pytest.raises(c2b.Conv2dError):
            c2b.describe_grad_weight_plan(p, v)
        assert c2b.check_indexing_grad_weight_variant(p, v)[0] == -5
    assert lib.conv2d_describe_grad_weight_plan(None, -1, None, 0) == NULL
    # tap tiles: 64 (channel, tap) slots, 1, 2 or 4 taps
    for v, taps in ((1, 1), (2, 2), (3, 4)):
        d = c2b.describe_grad_weight_plan(p, v)
        assert (d["tile_taps"], d["tile_channels"]) == (taps, 64 // taps)
    # the planner: tap tiles for many channels, flat tiles for a few-channel
    # big kernel (the 7x7 stem), the fewest slots among the tap layouts
    assert c2b.describe_grad_weight_plan(_p(in_channels=64, out_channels=64))["variant"] == 1
    stem = c2b.make_params(16, 3, 224, 224, 64, 7, 7, 2, 3, 3)
    assert c2b.describe_grad_weight_plan(stem)["variant"] == 0
    assert c2b.describe_grad_weight_plan(_p(in_channels=32))["variant"] == 2
    assert c2b.describe_grad_weight_plan(_p(in_channels=16))["variant"] == 3


# ---- RMSNorm-fused matrix product entry point ------------------------------------

def test_rms_norm_matmul_rejects_before_any_device_call():
    lib = c2b.load_library()
    p = c2b.make_rms_params(4, 3, 5)
    call = c2b.conv2d_rms_norm_matmul_raw
    assert lib.rms_norm_matmul(None, None, None, None, None, None) == NULL
    assert call(0, 0x2000, 0x3000, 0x4000, p) == NULL
    assert call(0x1000, 0, 0x3000, 0x4000, p) == NULL
    assert call(0x1000, 0x2000, 0, 0x4000, p) == NULL
    assert call(0x1000, 0x2000, 0x3000, 0, p) == NULL
    assert call(0x1000, 0x2000, 0x3000, 0x4000, c2b.make_rms_params(4, 3, 0)) == BAD
    assert call(0x1000, 0x2000, 0x3000, 0x4000, c2b.make_rms_params(4, 3, 5, -1e-3)) == BAD
    # out overlapping x, the norm weight or the projection
    assert call(0x1000, 0x2000, 0x3000, 0x1000 + 8, p) == ALIAS
    assert call(0x1000, 0x2000, 0x3000, 0x2000 - 8, p) == ALIAS
    assert call(0x1000, 0x2000, 0x3000, 0x3000 + 40, p) == ALIAS
    assert call(0x1000, 0x2000, 0x3000, 0x4000, c2b.make_rms_params(1 << 16, 8, 1 << 13)) == OVF
    # empty outputs launch nothing and succeed
    assert call(0x1000, 0x2000, 0x3000, 0x4000, c2b.make_rms_params(0, 3, 5)) == OK
    assert call(0x1000, 0x2000, 0x3000, 0x4000, c2b.make_rms_params(4, 0, 5)) == OK


def test_rms_params_struct_layout():
    assert ctypes.sizeof(c2b.RmsMatmulParams) == 16


# ---- attention dV entry point --------------------------------------------------------

def test_mha_grad_v_rejects_before_any_device_call():
    lib = c2b.load_library()
    p = c2b.make_mha_params(8, 8, 2, 1)        # q, dout 8 x 2 x 64; k, dv 8 x 1 x 64
    call = c2b.mha_grad_v_raw
    assert lib.mha_grad_v(None, None, None, None, None, None, None) == NULL
    assert call(0, 0x100000, 0x200000, 0x300000, 0x400000, p) == NULL
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0, p) == NULL
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x400000,
                c2b.make_mha_params(8, 8, 2, 1, 128)) == BAD          # head_dim
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x400000,
                c2b.make_mha_params(8, 8, 3, 2)) == BAD               # groups
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x400000,
                c2b.make_mha_params(8, 9, 2, 1)) == BAD               # causal q != kv
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x400004, p) == BAD   # unaligned dv
    # dv overlapping an input
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x200000, p) == ALIAS
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x100000 + 64, p) == ALIAS
    # no key: nothing to do
    assert call(0x10000, 0x100000, 0x200000, 0x300000, 0x400000,
                c2b.make_mha_params(8, 0, 2, 1, causal=False)) == OK


def test_mha_params_struct_layout():
    assert ctypes.sizeof(c2b.MhaGradVParams) == 28


def test_grad_weight_noalloc_rejects_before_any_device_call():
    """Argument errors of the allocation-free weight gradient come back
    before any HIP call (this machine may have no GPU), including a shape
    whose partial sums exceed the library's scratch array."""
    lib = c2b.load_library()

    def call(go, x, dw, q):
        return lib.conv2d_grad_weight_noalloc(ctypes.c_void_p(go), ctypes.c_void_p(x),
                                              ctypes.c_void_p(dw), q, None)
    p = _p()
    assert call(1, 2, 3, None) == NULL
    assert call(0x1000, 0x2000, 0x3000, ctypes.byref(_p(stride=0, out_h=1, out_w=1))) == BAD
    assert call(0, 0x200000, 0x100000, ctypes.byref(p)) == NULL
    assert call(0x300000, 0, 0x100000, ctypes.byref(p)) == NULL
    assert call(0x300000, 0x200000, 0, ctypes.byref(p)) == NULL
    assert call(0x100000, 0x200000, 0x100000, ctypes.byref(p)) == ALIAS   # dw on grad_out
    # 1024 x 1024 channels, 3 x 3: 2304 tiles of 64 x 64 -> 37.7 MB of partial
    # sums, more than the 32 MiB scratch
    big = _p(batch=1, in_channels=1024, in_h=8, in_w=8, out_channels=1024)
    assert call(0x1000000, 0x2000000, 0x3000000, ctypes.byref(big)) == -8
    assert c2b.status_string(-8) != "unknown status"
    need = c2b.grad_weight_workspace_size(big)
    assert need > 32 << 20, need
