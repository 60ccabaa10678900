"""Plant plausible mistakes in a copy of the oracle (CPU only) and check the pins catch each.

Each mutant is the oracle's C source with one textual change, compiled to a
temporary library and swapped in for the real one while a set of pin tests
runs.  A mutant that every pin accepts would mean the pins cannot tell that
mistake from the definition.
"""
import ctypes
import os
import subprocess

import pytest
import torch

import oracle
from tests import test_oracle_pins as pins


@pytest.fixture(autouse=True, scope="module")
def _float64_default():
    """The pins run with float64 as torch's default dtype (restored after this module)."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)

SRC = os.path.join(os.path.dirname(oracle.__file__), "titans_oracle.c")

READ = "            mlp_forward(L, n, theta, q + t * tok_stride, y + t * y_stride, fwork);\n"
UPDATE = ("                s[i] = bt * s[i] + (1.0 - bt) * g[i];\n"
          "                theta[i] = (1.0 - a) * theta[i] - e * s[i];\n"
          "            }\n")

MUTANTS = {
    "read_after_write": [(READ, ""), (UPDATE, UPDATE + READ)],
    "grad_at_current_weights": [("mlp_grad(L, n, theta_c, k", "mlp_grad(L, n, theta, k")],
    "momentum_weights_swapped": [("s[i] = bt * s[i] + (1.0 - bt) * g[i];",
                                  "s[i] = (1.0 - bt) * s[i] + bt * g[i];")],
    "write_uses_previous_momentum": [(UPDATE,
                                      "                theta[i] = (1.0 - a) * theta[i] - e * s[i];\n"
                                      "                s[i] = bt * s[i] + (1.0 - bt) * g[i];\n"
                                      "            }\n")],
    "loss_without_factor_two": [("    return 2.0 * r;\n}", "    return r;\n}")],
    "huber_slope_not_capped": [("a <= prm ? 2.0 * r : (r > 0 ? 2.0 * prm : -2.0 * prm)", "2.0 * r")],
    "huber_loss_not_continuous": [("2.0 * prm * a - prm * prm", "2.0 * prm * a")],
    "lp_gradient_exponent": [("double m = prm * pow(a, prm - 1.0);", "double m = prm * pow(a, prm);")],
    "lp_gradient_sign_dropped": [("return r > 0 ? m : -m;", "return m;")],
    "surprise_without_root": [("surprise[t * surprise_stride] = sqrt(gg);",
                               "surprise[t * surprise_stride] = gg;")],
    "wrong_silu_derivative": [("return s * (1.0 + z * (1.0 - s));", "return s * (1.0 + z * s);")],
    "gradient_step_sign": [("theta[i] = (1.0 - a) * theta[i] - e * s[i];",
                            "theta[i] = (1.0 - a) * theta[i] + e * s[i];")],
    "decay_on_wrong_side": [("theta[i] = (1.0 - a) * theta[i] - e * s[i];",
                             "theta[i] = (1.0 - a) * (theta[i] - e * s[i]);")],
    "backward_drops_activation_derivative": [("dprev[j] = acc * silu_prime(zp[j]);",
                                              "dprev[j] = acc;")],
    "read_with_transposed_weights": [
        ("for (int j = 0; j < n[l - 1]; ++j) z += W[(int64_t)i * n[l - 1] + j] * cur[j];",
         "for (int j = 0; j < n[l - 1]; ++j) z += W[(int64_t)j * n[l] + i] * cur[j];")],
    "gradient_forward_transposed": [
        ("acc += Wl[l][(int64_t)i * n[l - 1] + j] * hin[j];",
         "acc += Wl[l][(int64_t)j * n[l] + i] * hin[j];")],
    "chunk_freezes_one_token_late": [
        ("memcpy(theta_c, theta, sizeof(double) * P);   /* frozen for this chunk's gradients */",
         "")],
}

PIN_CASES = [
    (pins.test_grad_matches_central_differences, dict(widths=(4, 8, 4))),
    (pins.test_grad_matches_central_differences, dict(widths=(5, 7, 3))),
    (pins.test_forward_and_grad_match_torch_library, dict(widths=(5, 7, 3))),
    (pins.test_linear_memory_no_momentum_no_decay_is_delta_rule, dict(C=1)),
    (pins.test_linear_memory_no_momentum_no_decay_is_delta_rule, dict(C=4)),
    (pins.test_orthonormal_keys_exact_recall_and_read_before_write, {}),
    (pins.test_eta_zero_is_pure_decay, dict(C=5)),
    (pins.test_alpha_one_beta_zero_keeps_one_token, {}),
    (pins.test_scalar_memory_momentum_and_decay_closed_form, dict(s0_val=0.7)),
    (pins.test_bias_loss_values_by_hand, {}),
    (pins.test_bias_grad_matches_central_differences, dict(widths=(4, 8, 4), bias=("huber", 0.3))),
    (pins.test_bias_grad_matches_central_differences, dict(widths=(4, 8, 4), bias=("lp", 3.0))),
    (pins.test_linear_memory_biased_delta_rule, dict(bias=("huber", 0.2), C=4)),
    (pins.test_linear_memory_biased_delta_rule, dict(bias=("lp", 3.0), C=1)),
    (pins.test_surprise_of_a_linear_memory_closed_form, {}),
]


def _build_mutant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"mutation {name}: pattern not found in the oracle source"
        src = src.replace(old, new, 1)
    if name == "chunk_freezes_one_token_late":
        # theta_c never refreshed at chunk starts: refresh it after the first token instead
        src = src.replace("            double a = alpha[t * gate_stride]",
                          "            if (t == c0 + 1) memcpy(theta_c, theta, sizeof(double) * P);\n"
                          "            double a = alpha[t * gate_stride]", 1)
        src = src.replace("    memcpy(s, s0, sizeof(double) * P);\n",
                          "    memcpy(s, s0, sizeof(double) * P);\n"
                          "    memcpy(theta_c, theta, sizeof(double) * P);\n", 1)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path),
                           "-o", str(so), "-lm"])
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path, monkeypatch):
    so = _build_mutant(tmp_path, name, MUTANTS[name])
    real = oracle._load()
    mutant = ctypes.CDLL(so)
    for fn in ("oracle_param_count", "oracle_mlp_forward", "oracle_mlp_loss", "oracle_mlp_grad",
               "oracle_scan", "oracle_retrieve", "oracle_mlp_loss_bias", "oracle_mlp_grad_bias",
               "oracle_scan_bias", "oracle_scan_full"):
        getattr(mutant, fn).restype = getattr(real, fn).restype
        getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", mutant)
    caught = []
    for fn, kw in PIN_CASES:
        try:
            fn(**kw)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"no pin rejects the planted mistake {name!r}"
