"""The oracle's pins must catch plausible mistakes: each mutant below plants
one mistake in a copy of the oracle's C source (built into a temporary
library on the CPU), and at least one pin in test_oracle_pins.py has to fail
against it."""
import ctypes
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_attention_pins as apins
from tests import test_oracle_gated_pins as gpins
from tests import test_oracle_producer_pins as ppins
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ss_oracle.c")

MUTANTS = {
    "decay_sign": ("exp(d * A_row[n])", "exp(-d * A_row[n])"),
    "b_not_discretised": ("d * Bt[n * bc_stride] * xv", "Bt[n * bc_stride] * xv"),
    "B_C_swapped": ("s6_token(N, h, d, x[i], A + c * N, Bm + b * N * L + t, Cm + b * N * L + t, L, rs)",
                    "s6_token(N, h, d, x[i], A + c * N, Cm + b * N * L + t, Bm + b * N * L + t, L, rs)"),
    "y_reads_old_state": ("h[n] = a * h[n] + d * Bt[n * bc_stride] * xv;\n        y += Ct[n * bc_stride] * h[n];",
                          "y += Ct[n * bc_stride] * h[n];\n        h[n] = a * h[n] + d * Bt[n * bc_stride] * xv;"),
    "skip_term_dropped": ("yt += (D ? D[c] : 0.0) * x[i];", "yt += 0.0;"),
    "gate_before_skip": ("yt += (D ? D[c] : 0.0) * x[i];\n            if (z) yt *= silu(z[i]);",
                         "if (z) yt *= silu(z[i]);\n            yt += (D ? D[c] : 0.0) * x[i];"),
    "softplus_wrong": ("return fmax(v, 0.0) + log1p(exp(-fabs(v)));", "return fmax(v, 0.0) + exp(-fabs(v));"),
    "bias_ignored": ("double v = dt_raw + (dt_bias ? dt_bias[c] : 0.0);", "double v = dt_raw;"),
    "reset_zeroes_write_too": ("h[n] = a * h[n] + d * Bt[n * bc_stride] * xv;",
                               "h[n] = reset ? 0.0 : a * h[n] + d * Bt[n * bc_stride] * xv;"),
    "reset_ignored": ("double a = reset ? 0.0 : exp(d * A_row[n]);", "double a = exp(d * A_row[n]);"),
    "A_wrong_index": ("exp(d * A_row[n])", "exp(d * A_row[0])"),
    "A_of_channel_0": ("s6_token(N, h, d, x[i], A + c * N,", "s6_token(N, h, d, x[i], A,"),
    "decode_A_of_channel_0": ("s6_token(N, state + r * N, d, x[r], A + c * N,", "s6_token(N, state + r * N, d, x[r], A,"),
    "h0_ignored": ("h[n] = h0 ? h0[r * N + n] : 0.0;", "h[n] = 0.0;"),
    "silu_is_sigmoid": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "decode_no_skip": ("yt += (D ? D[c] : 0.0) * x[r];", "yt += 0.0;"),
    # scalar-gated state scan
    "gated_gate_after_write": ("S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];",
                               "S[i * dv + j] = g * (S[i * dv + j] + kt[i] * vt[j]);"),
    "gated_y_reads_old_state": ("""            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];
                y[(b * L + t) * dv + j] = acc;
            }""", """            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];
                y[(b * L + t) * dv + j] = acc;
            }
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];"""),
    "gated_query_is_key": ("acc += qt[i] * S[i * dv + j];", "acc += kt[i] * S[i * dv + j];"),
    "gated_initial_state_ignored": ("S[e] = s0 ? s0[b * dk * dv + e] : 0.0;", "S[e] = 0.0;"),
    "gated_gate_of_next_token": ("const double g = gamma[b * L + t];",
                                 "const double g = gamma[b * L + (t + 1 < L ? t + 1 : t)];"),
    # effective attention
    "attn_product_includes_j": ("if (i > j)\n                    for (int64_t n = 0; n < N; ++n) prod[n] *=",
                                "if (i >= j)\n                    for (int64_t n = 0; n < N; ++n) prod[n] *="),
    "attn_decay_of_column_token": ("prod[n] *= exp(A[c * N + n] * d[i]);", "prod[n] *= exp(A[c * N + n] * d[j]);"),
    "attn_B_C_swapped": ("Cb[n * L + i] * prod[n] * Bb[n * L + j]", "Bb[n * L + i] * prod[n] * Cb[n * L + j]"),
    "attn_not_causal": ("i >= j ? Cb[n * L + i]", "1 ? Cb[n * L + i]"),
    "attn_row_scaled": ("Bb[n * L + j] * colscale", "Bb[n * L + j] * (include_dt ? d[i] : 1.0)"),
    # input-side producers
    "conv_taps_reversed": ("acc += conv_w[c * W + k] * x_pre[r * L + s];",
                           "acc += conv_w[c * W + (W - 1 - k)] * x_pre[r * L + s];"),
    "conv_off_by_one": ("const int64_t s = t - (W - 1) + k;", "const int64_t s = t - W + k;"),
    "conv_reset_ignored": ("if (reset && reset[b * L + t]) doc_start = t;", "if (0) doc_start = t;"),
    "conv_bias_dropped": ("double acc = conv_b ? conv_b[c] : 0.0;", "double acc = 0.0;"),
    "conv_no_silu": ("x[r * L + t] = silu(acc);", "x[r * L + t] = acc;"),
    "dtproj_delta_index": ("acc += w_dt[c * R + k] * delta[(b * L + t) * R + k];",
                           "acc += w_dt[c * R + k] * delta[(b * L + (L - 1 - t)) * R + k];"),
    "dtproj_bias_outside_softplus": ("oracle_softplus(acc + (dt_bias ? dt_bias[c] : 0.0))",
                                     "oracle_softplus(acc) + (dt_bias ? dt_bias[c] : 0.0)"),
}


def _pin_callables():
    calls = []
    for name in dir(pins):
        if not name.startswith("test_pin"):
            continue
        fn = getattr(pins, name)
        if name == "test_pin6_hand_worked_cases":
            for case in pins._hand_cases():
                calls.append((f"{name}[{case['name']}]", lambda fn=fn, case=case: fn(case)))
        else:
            calls.append((name, fn))
    for name in dir(gpins):
        if not name.startswith("test_gpin"):
            continue
        fn = getattr(gpins, name)
        if name == "test_gpin5_hand_worked_cases":
            for case in gpins._hand_cases():
                calls.append((f"{name}[{case['name']}]", lambda fn=fn, case=case: fn(case)))
        elif name in ("test_gpin1_unrolled_sum",):
            calls.append((name, lambda fn=fn: fn(2, True)))
        else:
            calls.append((name, fn))
    for name in dir(apins):
        if not name.startswith("test_apin"):
            continue
        fn = getattr(apins, name)
        if name == "test_apin1_reconstructs_the_scan":
            calls.append((name, lambda fn=fn: fn(True)))
        else:
            calls.append((name, fn))
    for name in dir(ppins):
        if not name.startswith("test_ppin"):
            continue
        fn = getattr(ppins, name)
        if name == "test_ppin1_matches_numpy_convolve":
            calls.append((name, lambda fn=fn: fn(4)))
        elif name == "test_ppin5_dt_proj_matches_numpy_matmul":
            calls.append((name, lambda fn=fn: fn(True)))
        else:
            calls.append((name, fn))
    return calls


def _build_mutant(old, new, tmp):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    path_c = os.path.join(tmp, "mut.c")
    path_so = os.path.join(tmp, "mut.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", path_so, path_c, "-lm"])
    return path_so


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    old, new = MUTANTS[mutant]
    real = oracle._load()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(old, new, tmp)
        lib = ctypes.CDLL(so)
        for fn in ("oracle_scan", "oracle_update", "oracle_softplus", "oracle_gated_scan",
                   "oracle_effective_attention", "oracle_conv1d_silu", "oracle_dt_proj"):
            getattr(lib, fn).restype = getattr(real, fn).restype
            getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        monkeypatch.setattr(oracle, "_lib", lib)
        failed = []
        for name, call in _pin_callables():
            try:
                call()
            except AssertionError:
                failed.append(name)
        assert failed, f"no pin catches mutant {mutant}"
