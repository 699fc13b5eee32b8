"""The pins must catch plausible mistakes: each test builds a copy of the C oracle with one
planted mistake (on the CPU, in a temporary directory), points the oracle wrapper at it and
checks that at least one pin fails.  The real oracle is never modified."""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mamba_oracle.c")

# (name, exact source text, replacement)
MUTANTS = [
    ("abar_without_delta", "double abar = exp(dt * Arow[n]);", "double abar = exp(Arow[n]);"),
    ("abar_wrong_sign", "double abar = exp(dt * Arow[n]);", "double abar = exp(-dt * Arow[n]);"),
    ("bbar_without_delta", "double bx = dt * Bp[n * bstride] * x;",
     "double bx = Bp[n * bstride] * x;"),
    ("b_and_c_swapped", "y += Cp[n * bstride] * h[n];", "y += Bp[n * bstride] * h[n];"),
    ("readout_before_update",
     "    h[n] = abar * h[n] + bx;\n    y += Cp[n * bstride] * h[n];",
     "    y += Cp[n * bstride] * h[n];\n    h[n] = abar * h[n] + bx;"),
    ("bias_dropped", "double dt = draw + bias;", "double dt = draw;"),
    ("softplus_before_bias",
     "double dt = draw + bias;\n  if (softplus_flag) dt = sp(dt);",
     "double dt = draw;\n  if (softplus_flag) dt = sp(dt);\n  dt += bias;"),
    ("softplus_ignored", "if (softplus_flag) dt = sp(dt);", "(void)softplus_flag;"),
    ("skip_dropped", "if (has_D) y += Dd * x;", "(void)Dd;"),
    ("gate_is_sigmoid", "if (has_z) y *= silu(zz);", "if (has_z) y *= 1.0 / (1.0 + exp(-zz));"),
    ("gate_before_skip", "  if (has_D) y += Dd * x;\n  if (has_z) y *= silu(zz);",
     "  if (has_z) y *= silu(zz);\n  if (has_D) y += Dd * x;"),
    ("B_indexed_by_channel", "B + b * dstate * seqlen + t, C + b * dstate * seqlen + t",
     "B + (d % batch) * dstate * seqlen + t, C + b * dstate * seqlen + t"),
    ("state_not_zeroed", "double* h = (double*)calloc((size_t)dstate, sizeof(double));",
     "double* h = (double*)malloc((size_t)dstate * sizeof(double)); "
     "for (int64_t q = 0; q < dstate; ++q) h[q] = 0.25;"),
    ("affine_scan_add_first", "s = a[t] * s + b[t];", "s = a[t] * (s + b[t]);"),
    ("time_reversed_B", "B + b * dstate * seqlen + t,",
     "B + b * dstate * seqlen + (seqlen - 1 - t),"),
    ("softplus_naive_sign", "return fmax(x, 0.0) + log1p(exp(-fabs(x)));",
     "return fmax(x, 0.0) + log1p(exp(fabs(x)));"),
]

PIN_TESTS = [
    pins.test_p1_fixed_gate_printed_values,
    pins.test_p2_selective_gate_printed_values,
    pins.test_p3_composition_printed_example,
    pins.test_p4_scalar_zero_order_hold,
    pins.test_p5_time_invariant_equals_convolution,
    lambda: pins.test_p6_tree_scans_match_sequential(pins._tree_blelloch),
    pins.test_p7_constant_coefficients_closed_form,
    pins.test_p8_zero_step_keeps_state,
    pins.test_p9_large_step_forgets_history,
    pins.test_p10_scan_equals_steps,
    pins.test_p11_structural_invariants,
    pins.test_p12_unrolled_products_brute_force,
    pins.test_p13_softplus_silu_library,
    pins.test_bias_then_softplus_reading,
    pins.test_gate_and_skip_readings,
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(so),
                    str(path), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    for fn in ("ref_scan_fwd_f64", "ref_state_update_f64", "ref_affine_scan_f64",
               "ref_softplus_f64", "ref_silu_f64", "ref_set_threads", "ref_max_threads"):
        f = getattr(mut, fn)
        f.argtypes = getattr(real, fn).argtypes
        f.restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mut)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name}"


# planted mistakes in the hand-written adjoint (ref_scan_bwd_f64)
BWD_MUTANTS = [
    ("bwd_carry_without_abar", "lam[n] = l * a_t;", "lam[n] = l;"),
    ("bwd_dA_without_delta", "gA[n] += l * a_t * dt * hp;", "gA[n] += l * a_t * hp;"),
    ("bwd_ddelta_drops_input_term", "gdt += l * (a_t * Arow[n] * hp + Bb[n * L + t] * x);",
     "gdt += l * (a_t * Arow[n] * hp);"),
    ("bwd_dC_uses_previous_state", "myC[(b * N + n) * L + t] += dy * H[t * N + n];",
     "myC[(b * N + n) * L + t] += dy * hp;"),
    ("bwd_dlast_ignored", "lam[n] = dlast ? dlast[(b * dim + d) * N + n] : 0.0;",
     "lam[n] = 0.0;"),
    ("bwd_no_softplus_derivative", "const double graw = gdt * sig[t];",
     "const double graw = gdt;"),
    ("bwd_gate_derivative_is_sigmoid",
     "dz[row + t] = dout[row + t] * ypre[t] * s * (1.0 + zz * (1.0 - s));",
     "dz[row + t] = dout[row + t] * ypre[t] * s;"),
    ("bwd_du_skip_dropped", "double gu = dy * Dd, gdt = 0.0;", "double gu = 0.0, gdt = 0.0;"),
]


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_planted_adjoint_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    from tests import test_oracle_backward as bw
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    for fn in ("ref_scan_bwd_f64", "ref_scan_fwd_f64", "ref_set_threads", "ref_max_threads"):
        f = getattr(mut, fn)
        f.argtypes = getattr(real, fn).argtypes
        f.restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mut)
    failures = 0
    for flags in bw.FLAGS + [dict(softplus=True, D=True, z=False, bias=True)]:
        try:
            bw.test_c_adjoint_matches_autograd(flags, (2, 3, 17))
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name}"


# planted mistakes in the causal conv1d + SiLU oracle
CONV_MUTANTS = [
    ("conv_taps_reversed", "if (s >= 0) acc += w[d * W + k] * xr[s];",
     "if (s >= 0) acc += w[d * W + (W - 1 - k)] * xr[s];"),
    ("conv_bias_dropped", "double acc = bias ? bias[d] : 0.0;", "double acc = 0.0;"),
    ("conv_looks_ahead", "const int64_t s = t - (W - 1) + k;", "const int64_t s = t + k;"),
    ("conv_no_silu", "u[ch * L + t] = silu(acc);", "u[ch * L + t] = acc;"),
    ("conv_off_by_one", "const int64_t s = t - (W - 1) + k;", "const int64_t s = t - W + k;"),
]


@pytest.mark.parametrize("name,old,new", CONV_MUTANTS, ids=[m[0] for m in CONV_MUTANTS])
def test_planted_conv_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    from tests import test_oracle_conv as cv
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    mut = ctypes.CDLL(so)
    for fn in ("ref_causal_conv1d_silu_f64", "ref_scan_fwd_f64", "ref_set_threads",
               "ref_max_threads"):
        f = getattr(mut, fn)
        f.argtypes = getattr(real, fn).argtypes
        f.restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mut)
    pins = [lambda: cv.test_conv_matches_torch_conv1d(4, (2, 3, 17)),
            lambda: cv.test_conv_matches_torch_conv1d(1, (1, 5, 2)),
            cv.test_conv_impulse_response, cv.test_conv_is_causal,
            cv.test_conv_width_one_is_pointwise]
    failures = 0
    for t in pins:
        try:
            t()
        except (AssertionError, IndexError):
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name}"
