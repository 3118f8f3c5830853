"""Planted mistakes in the oracle must trip at least one pin.

Each mutant is a copy of oracle/oracle.c with one plausible slip (a flipped
kernel, a wrong sign, swapped paddings, a transposed weight, a dropped tap or
divisibility test, a shifted bound, a wrong initial value), compiled on the
CPU into a temporary library.  The committed oracle passes every pin (see
test_oracle.py); each mutant must fail at least one.
"""
import os

import pytest

import oracle
from tests import oracle_pins

# (name, function the slip goes into, text to replace, replacement)
MUTANTS = [
    ("gather_flipped_kernel", "oracle_grad_input_gather",
     "w[((co * Ci + ci) * KH + kh) * KW + kw]",
     "w[((co * Ci + ci) * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)]"),
    ("gather_sign_h", "oracle_grad_input_gather",
     "i64 th = ih + ph - kh;", "i64 th = ih - ph + kh;"),
    ("gather_padding_swapped", "oracle_grad_input_gather",
     "i64 tw = iw + pw - kw;", "i64 tw = iw + ph - kw;"),
    ("gather_weight_transposed", "oracle_grad_input_gather",
     "w[((co * Ci + ci)", "w[((ci * Co + co)"),
    ("gather_no_divisibility", "oracle_grad_input_gather",
     "if (th % s != 0 || tw % s != 0) continue;", ""),
    ("gather_last_row_dropped", "oracle_grad_input_gather",
     "if (oh >= OH || ow >= OW) continue;", "if (oh >= OH - 1 || ow >= OW) continue;"),
    ("gather_last_tap_dropped", "oracle_grad_input_gather",
     "kw < KW; ++kw", "kw < KW - 1; ++kw"),
    ("gather_no_stride_divide", "oracle_grad_input_gather",
     "i64 oh = th / s;", "i64 oh = th;"),
    ("gather_bad_init", "oracle_grad_input_gather",
     "double acc = 0.0;", "double acc = 1e-3;"),
    ("gather_at_sign_w", "oracle_grad_input_gather_at",
     "i64 tw = iw + pw - kw;", "i64 tw = iw - pw + kw;"),
    ("scatter_sign_h", "oracle_grad_input_scatter",
     "i64 ih = oh * s - ph + kh;", "i64 ih = oh * s + ph - kh;"),
    ("scatter_flipped_kernel", "oracle_grad_input_scatter",
     "w[((co * Ci + ci) * KH + kh) * KW + kw]",
     "w[((co * Ci + ci) * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)]"),
    ("forward_padding_swapped", "oracle_conv2d_forward",
     "i64 iw = ow * s - pw + kw;", "i64 iw = ow * s - ph + kw;"),
    ("forward_flipped_kernel", "oracle_conv2d_forward",
     "w[((co * Ci + ci) * KH + kh) * KW + kw]",
     "w[((co * Ci + ci) * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)]"),
    ("grad_weight_sign_h", "oracle_grad_weight",
     "i64 ih = oh * s - ph + kh;", "i64 ih = oh * s + ph - kh;"),
    ("grad_weight_padding_swapped", "oracle_grad_weight",
     "i64 iw = ow * s - pw + kw;", "i64 iw = ow * s - ph + kw;"),
    ("grad_weight_flipped_kernel", "oracle_grad_weight",
     "i64 ih = oh * s - ph + kh;", "i64 ih = oh * s - ph + (KH - 1 - kh);"),
    ("grad_weight_last_row_dropped", "oracle_grad_weight",
     "oh < OH; ++oh", "oh < OH - 1; ++oh"),
    ("grad_weight_bad_init", "oracle_grad_weight",
     "double acc = 0.0;", "double acc = 1e-3;"),
    ("rms_sum_not_mean", "oracle_rms_norm_matmul",
     "ss / (double)K + eps", "ss + eps"),
    ("rms_eps_dropped", "oracle_rms_norm_matmul",
     "ss / (double)K + eps", "ss / (double)K"),
    ("rms_sqrt_not_rsqrt", "oracle_rms_norm_matmul",
     "1.0 / sqrt(ss / (double)K + eps)", "sqrt(ss / (double)K + eps)"),
    ("rms_scale_dropped", "oracle_rms_norm_matmul",
     "xi[k] * r * g[k]", "xi[k] * r"),
    ("rms_scale_on_columns", "oracle_rms_norm_matmul",
     "ci[j] += a * wk[j];", "ci[j] += a / g[k] * g[j % K] * wk[j];"),
    ("rms_w_transposed", "oracle_rms_norm_matmul",
     "const double* wk = w + k * N;", "const double* wk = w + k;"),
    ("rms_last_k_dropped", "oracle_rms_norm_matmul",
     "for (i64 k = 0; k < K; ++k) {", "for (i64 k = 0; k < K - 1; ++k) {"),
    ("rms_bad_init", "oracle_rms_norm_matmul",
     "ci[j] = 0.0;", "ci[j] = 1e-3;"),
    ("mha_causal_off_by_one", "oracle_mha_grad_v",
     "const i64 start = causal ? t : 0;", "const i64 start = causal ? t + 1 : 0;"),
    ("mha_window_off_by_one", "oracle_mha_grad_v",
     "(q_seq < t + window ? q_seq : t + window)", "(q_seq < t + window - 1 ? q_seq : t + window - 1)"),
    ("mha_heads_interleaved", "oracle_mha_grad_v",
     "const i64 h = kvh * group + r;", "const i64 h = kvh + r * HKV;"),
    ("mha_scale_dropped", "oracle_mha_grad_v",
     "    s *= scale;\n          const double* l", "    const double* l"),
    ("mha_clamp_dropped", "oracle_mha_grad_v",
     "if (e > 0.0) e = 0.0;", ""),
    ("mha_log_sum_ignored", "oracle_mha_grad_v",
     "exp(e - l[1])", "exp(e)"),
    ("lse_log_dropped", "oracle_attention_lse",
     "log(sum)", "sum"),
    ("lse_sum_unscaled", "oracle_attention_lse",
     "sum += exp(s * scale - mx);", "sum += exp(s - mx);"),
    # the row maximum alone (its sum with the log-sum is unchanged by these)
    ("lse_window_off_by_one", "oracle_attention_lse",
     "(window > 0 && pos >= t + window)", "(window > 0 && pos >= t + window - 1)"),
    ("lse_max_unscaled", "oracle_attention_lse",
     "        s *= scale;\n        if (s > mx) mx = s;", "        if (s > mx) mx = s;"),
]


def _mutate(src, func, old, new):
    start = src.index("void %s(" % func)
    nxt = src.find("\nvoid ", start + 1)
    end = len(src) if nxt < 0 else nxt
    body = src[start:end]
    assert old in body, (func, old)
    return src[:start] + body.replace(old, new, 1) + src[end:]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[0])
def test_mutant_is_caught(mutant, tmp_path):
    name, func, old, new = mutant
    with open(oracle.SOURCE) as f:
        src = f.read()
    path = os.path.join(str(tmp_path), name + ".c")
    with open(path, "w") as f:
        f.write(_mutate(src, func, old, new))
    lib = oracle.compile_source(path, os.path.join(str(tmp_path), name + ".so"))
    orc = oracle.Oracle(lib)
    tripped = None
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            tripped = pin.__name__   # one pin is enough
            break
    assert tripped, "mutant %s passed every pin" % name
