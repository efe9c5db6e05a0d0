"""Planted mistakes in the oracle must fail at least one of its pins.

The pins only mean something if a plausible slip in the oracle breaks one of
them.  Each case here copies an oracle source with one textual change (a
dropped term, a wrong index, a flipped sign, a wrong power of the
denominator, a non-exact sign decision, a truncated error scale, a rounding
that breaks ties the wrong way ...) and runs the pins against the copy:

* the C oracle (``oracle/grkan_oracle.c``): the mutant is compiled with the
  oracle's own gcc flags into a temporary directory and the activation and
  PAU pin files run in a child pytest whose ``GRKAN_ORACLE_LIB`` points at it;
  the child must fail.
* the Python oracles (``oracle/layer.py``, ``oracle/chebykan.py``): the
  mutant module is executed in a fresh namespace, its functions and constants
  are patched over the real module's, and the pin functions of that oracle
  are called in-process; at least one must raise.

Nothing here touches a GPU or the HIP path.
"""
import os
import subprocess
import sys
import types

import pytest

from oracle import chebykan, layer
import test_oracle_pins_chebykan as pins_cheby
import test_oracle_pins_layer as pins_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "grkan_oracle.c")

# (name, original text, mutated text): each original occurs exactly once.
C_MUTANTS = [
    ("numerator_drops_a0", "for (int i = 0; i <= m; ++i) {\n        P += a[i] * xp[i];",
     "for (int i = 1; i <= m; ++i) {\n        P += a[i] * xp[i];"),
    ("numerator_shifted_power", "P += a[i] * xp[i];", "P += a[i] * xp[i + 1];"),
    ("denominator_derivative_index", "Qd += (double)j * b[j - 1] * xp[j - 1];",
     "Qd += (double)j * b[j - 1] * xp[j];"),
    ("denominator_derivative_no_factor", "Qd += (double)j * b[j - 1] * xp[j - 1];",
     "Qd += b[j - 1] * xp[j - 1];"),
    ("dx_quotient_rule_sign", "double dFdx = Pd / D - (double)s * P * Qd / D2;",
     "double dFdx = Pd / D + (double)s * P * Qd / D2;"),
    ("dx_quotient_rule_power", "double dFdx = Pd / D - (double)s * P * Qd / D2;",
     "double dFdx = Pd / D - (double)s * P * Qd / D;"),
    ("sign_not_exact", "return sign_q_exact(x, n, b);", "return sign_of(q);"),
    ("dA_term_power", "out[ORC_T + i] = dy * xp[i] / D;", "out[ORC_T + i] = dy * xp[i] / D2;"),
    ("dB_term_power", "out[ORC_T + m + j] = -dy * (double)s * P * xp[j] / D2;",
     "out[ORC_T + m + j] = -dy * (double)s * P * xp[j] / D;"),
    ("dB_term_sign", "out[ORC_T + m + j] = -dy * (double)s * P * xp[j] / D2;",
     "out[ORC_T + m + j] = dy * (double)s * P * xp[j] / D2;"),
    ("dB_term_index", "out[ORC_T + m + j] = -dy * (double)s * P * xp[j] / D2;",
     "out[ORC_T + m + j] = -dy * (double)s * P * xp[j - 1] / D2;"),
    ("denominator_without_abs", "double D = 1.0 + fabs(Q);", "double D = 1.0 + Q;"),
    ("error_scale_truncated", "out[ORC_FMAG] = (Pabs + aP * Qabs / D) / D;", "out[ORC_FMAG] = Pabs / D;"),
    ("rows_group_coefficients_off_by_one", "A + (long)(m + 1) * g, B + (long)n * g, out);",
     "A + (long)(m + 1) * ((g + 1) % n_g), B + (long)n * g, out);"),
    ("rows_group_span_short", "for (long c = g * dg; c < (g + 1) * dg; ++c) {",
     "for (long c = g * dg; c < (g + 1) * dg - 1; ++c) {"),
    ("rows_sum_of_squares_unsquared", "acc2[k] += t * t;", "acc2[k] += t;"),
    ("points_group_from_row", "long c = idx[k] % d;", "long c = idx[k] / d;"),
    ("dx_error_scale_truncated", "+ (Pabs * aQd + aP * Qdabs + 2.0 * aP * aQd * Qabs / D) / D2);",
     "+ (Pabs * aQd) / D2);"),
    ("dA_term_scale_truncated", "out[ORC_T + nk + i] = ady * axp[i] * (1.0 + Qabs / D) / D;",
     "out[ORC_T + nk + i] = ady * axp[i] / D;"),
    ("dB_term_scale_truncated", "out[ORC_T + nk + m + j] = ady * axp[j] * (Pabs + 2.0 * aP * Qabs / D) / D2;",
     "out[ORC_T + nk + m + j] = ady * axp[j] * aP / D2;"),
]


def _mutate(text, old, new):
    assert text.count(old) == 1, f"mutation target occurs {text.count(old)} times: {old!r}"
    return text.replace(old, new)


@pytest.fixture(scope="module")
def c_source():
    with open(C_SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_oracle_mutant_fails_a_pin(tmp_path, c_source, name, old, new):
    src = tmp_path / f"{name}.c"
    src.write_text(_mutate(c_source, old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(so), str(src), "-lm"], check=True)
    env = dict(os.environ, GRKAN_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_oracle_pins.py", "tests/test_oracle_pins_pau.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, (f"mutant {name} passed every pin (exit {r.returncode}):\n"
                               + r.stdout[-2000:] + r.stderr[-2000:])


def test_unmutated_c_oracle_passes_through_the_same_route(tmp_path, c_source):
    """Control: the unchanged source, loaded the same way, passes (so the failures above come
    from the mutations, not from the route)."""
    src = tmp_path / "same.c"
    src.write_text(c_source)
    so = tmp_path / "libsame.so"
    subprocess.run(["gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(so), str(src), "-lm"], check=True)
    env = dict(os.environ, GRKAN_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


PY_MUTANTS = [
    (layer, pins_layer, "bf16_ties_away_from_zero",
     "q = np.rint(np.ldexp(v, -shift))", "q = np.trunc(np.ldexp(v, -shift) + np.copysign(0.5, v))"),
    (layer, pins_layer, "bf16_seven_bits", "shift = np.maximum(exp - 8, -133)", "shift = np.maximum(exp - 7, -133)"),
    (layer, pins_layer, "bf16_no_subnormals", "shift = np.maximum(exp - 8, -133)", "shift = exp - 8"),
    (layer, pins_layer, "activation_ambiguity_dropped",
     "width = np.where(lo != hi, hi - lo, 0.0)\n    return fb, width",
     "width = np.zeros_like(fb)\n    return fb, width"),
    (layer, pins_layer, "activation_not_rounded", "fb = bf16_round(f)\n", "fb = f\n"),
    (layer, pins_layer, "upstream_not_rounded", "return bf16_round(dy), np.where", "return dy, np.where"),
    (layer, pins_layer, "upstream_ambiguity_dropped",
     "err = k * 2.0 ** -24 * (np.abs(dz) @ np.abs(W))", "err = 0.0 * (np.abs(dz) @ np.abs(W))"),
    (layer, pins_layer, "weight_gradient_transposed", '"dW": dz.T @ fb', '"dW": (fb.T @ dz).T[::-1]'),
    (layer, pins_layer, "weight_gradient_unrounded_activation",
     "fb, wf = activation_operand(x_bits, A, B, n_groups)\n    out = {\"dW\": dz.T @ fb",
     "fb, wf = activation_operand(x_bits, A, B, n_groups)\n    out = {\"dW\": dz.T @ "
     "oracle.run(x_bits, A, B, n_groups, io=\"bf16\")[\"y\"]"),
    (layer, pins_layer, "forward_weight_not_transposed", '{"z": fb @ W.T', '{"z": fb @ W[:, ::-1].T'),
    (chebykan, pins_cheby, "recurrence_sign",
     "out[..., k + 1] = 2.0 * t * out[..., k] - out[..., k - 1]",
     "out[..., k + 1] = 2.0 * t * out[..., k] + out[..., k - 1]"),
    (chebykan, pins_cheby, "recurrence_factor",
     "out[..., k + 1] = 2.0 * t * out[..., k] - out[..., k - 1]",
     "out[..., k + 1] = t * out[..., k] - out[..., k - 1]"),
    (chebykan, pins_cheby, "derivative_without_k", "out[..., k] = k * u[..., k - 1]", "out[..., k] = u[..., k - 1]"),
    (chebykan, pins_cheby, "derivative_index", "out[..., k] = k * u[..., k - 1]",
     "out[..., k] = k * u[..., min(k, degree - 1)]"),
    (chebykan, pins_cheby, "dx_without_tanh_derivative", "s = 1.0 - t * t\n", "s = 1.0 + 0.0 * t\n"),
    (chebykan, pins_cheby, "dx_tanh_derivative_sign", "s = 1.0 - t * t\n", "s = 1.0 + t * t\n"),
    (chebykan, pins_cheby, "basis_without_tanh", "t = np.tanh(x)\n    T = chebyshev_t", "t = x\n    T = chebyshev_t"),
    (chebykan, pins_cheby, "basis_error_too_small", "return (k * k + 1) * 2.0 ** -20", "return (k * k + 1) * 2.0 ** -26"),
    (chebykan, pins_cheby, "dC_not_reshaped_per_input",
     '"dC": (dy.T @ bb).reshape(d_out, d_in, nb)',
     '"dC": (dy.T @ bb).reshape(d_out, nb, d_in).transpose(0, 2, 1)'),
]


def _pin_functions(pin_module):
    return [getattr(pin_module, n) for n in sorted(dir(pin_module))
            if n.startswith("test_") and callable(getattr(pin_module, n))]


def _load_mutant(module, old, new):
    with open(module.__file__) as f:
        text = _mutate(f.read(), old, new)
    mutant = types.ModuleType(module.__name__ + "_mutant")
    mutant.__package__ = module.__package__
    mutant.__file__ = module.__file__
    exec(compile(text, module.__file__ + " (mutant)", "exec"), mutant.__dict__)
    return mutant


def _patch_module(monkeypatch, module, mutant):
    for name, value in mutant.__dict__.items():
        if name.startswith("__"):
            continue
        orig = getattr(module, name, None)
        if isinstance(value, types.FunctionType) and getattr(value, "__module__", None) == mutant.__name__:
            monkeypatch.setattr(module, name, value)
        elif isinstance(value, float) and isinstance(orig, float):
            monkeypatch.setattr(module, name, value)


@pytest.mark.parametrize("module,pins,name,old,new", PY_MUTANTS, ids=[m[2] for m in PY_MUTANTS])
def test_python_oracle_mutant_fails_a_pin(monkeypatch, module, pins, name, old, new):
    mutant = _load_mutant(module, old, new)
    _patch_module(monkeypatch, module, mutant)
    failed = []
    for fn in _pin_functions(pins):
        try:
            fn()
        except Exception as e:   # an assertion or any error the mutant causes counts as a failed pin
            failed.append(f"{fn.__name__}: {type(e).__name__}")
            break
    assert failed, f"mutant {name} passed every pin of {pins.__name__}"


def test_unmutated_python_oracles_pass_through_the_same_route(monkeypatch):
    """Control: reloading each module unchanged through the same route keeps every pin green."""
    for module, pins in ((layer, pins_layer), (chebykan, pins_cheby)):
        mutant = _load_mutant(module, "from __future__ import annotations", "from __future__ import annotations")
        _patch_module(monkeypatch, module, mutant)
        for fn in _pin_functions(pins):
            fn()
