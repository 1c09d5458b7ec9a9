"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutation edits the oracle's source text (a dropped term, a wrong sign,
a wrong operand, an off-by-one, a missing rounding) and loads the edited copy
as a separate module; the real oracle is untouched.
"""
import importlib.util
import os
import types

import pytest

from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "muon_oracle.py")

MUTATIONS = {
    "drop_c_term": ("B = b * A + c * (A @ A)", "B = b * A"),
    "drop_b_term": ("B = b * A + c * (A @ A)", "B = c * (A @ A)"),
    "sign_of_BX": ("return a * x + B @ x", "return a * x - B @ x"),
    "drop_aX": ("return a * x + B @ x", "return B @ x"),
    "gram_wrong_side": ("A = x @ x.T", "A = (x.T @ x)[: x.shape[0], : x.shape[0]]"),
    "norm_without_sqrt": ("u / (np.sqrt(np.sum(u * u)) + eps)", "u / (np.sum(u * u) + eps)"),
    "eps_inside_sqrt": ("u / (np.sqrt(np.sum(u * u)) + eps)", "u / np.sqrt(np.sum(u * u) + eps)"),
    "max_norm_instead_of_fro": ("u / (np.sqrt(np.sum(u * u)) + eps)", "u / (np.max(np.abs(u)) + eps)"),
    "no_transpose_back": ("return x.T.copy() if tall else x.copy()", "return x.copy()"),
    "one_step_short": ("for _ in range(int(steps)):", "for _ in range(max(int(steps) - 1, 0)):"),
    "coeffs_swapped": ("x = ns_polynomial_step(x, a, b, c)", "x = ns_polynomial_step(x, a, c, b)"),
    "nesterov_old_buffer": ("u = g + mu * new_buf if nesterov", "u = g + mu * buf if nesterov"),
    "nesterov_ignored": ("u = g + mu * new_buf if nesterov else new_buf.copy()", "u = new_buf.copy()"),
    "buffer_not_rounded": ("new_buf = round_exact_sum(hi, lo, buf_dtype)", "new_buf = hi + lo"),
    "buffer_rounded_via_fp32": ("new_buf = round_exact_sum(hi, lo, buf_dtype)",
                                "new_buf = _ROUND[buf_dtype](fp32_round(hi))"),
    "buffer_rounded_from_f64_sum": ("new_buf = round_exact_sum(hi, lo, buf_dtype)",
                                    "new_buf = _ROUND[buf_dtype](hi)"),
    "tie_direction_flipped": ("np.where(lo > 0, up, down)", "np.where(lo < 0, up, down)"),
    "two_sum_error_dropped": ("e = (a - (s - bb)) + (b - bb)", "e = 0.0 * s"),
    "ema_momentum": ("hi, lo = two_sum(mu * buf, g)", "hi, lo = two_sum(mu * buf, (1 - mu) * g)"),
    "bf16_7_bits": ("np.rint(np.ldexp(f[normal], 8)), e[normal] - 8)",
                    "np.rint(np.ldexp(f[normal], 7)), e[normal] - 7)"),
    "bf16_truncate": ("np.rint(np.ldexp(f[normal], 8))", "np.trunc(np.ldexp(f[normal], 8))"),
    "bf16_half_up": ("np.rint(np.ldexp(f[normal], 8))", "np.floor(np.ldexp(f[normal], 8) + 0.5)"),
    "apply_sign": ("res = w * (1.0 - lr_eff * wd_eff) - lr_eff * x",
                   "res = w * (1.0 - lr_eff * wd_eff) + lr_eff * x"),
    "apply_no_wd_mul": ("wd_eff = float(wd) * float(wd_mul)", "wd_eff = float(wd)"),
    "apply_no_lr_mul": ("lr_eff = float(lr) * float(lr_mul)", "lr_eff = float(lr)"),
    "apply_decay_no_lr": ("res = w * (1.0 - lr_eff * wd_eff) - lr_eff * x",
                          "res = w * (1.0 - wd_eff) - lr_eff * x"),
    "adam_no_m_correction": ("m_hat = m_new / (1.0 - beta1 ** t)", "m_hat = m_new"),
    "adam_no_v_correction": ("v_hat = v_new / (1.0 - beta2 ** t)", "v_hat = v_new"),
    "adam_betas_swapped": ("m_new = fp32_round(beta1 * m + (1.0 - beta1) * g)",
                           "m_new = fp32_round(beta2 * m + (1.0 - beta2) * g)"),
    "adam_eps_inside_sqrt": ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    "adam_v_not_squared": ("(1.0 - beta2) * g * g)", "(1.0 - beta2) * np.abs(g))"),
    "adam_decay_without_lr": ("p * (1.0 - rate * decay) - rate * m_hat",
                              "p * (1.0 - decay) - rate * m_hat"),
    "adam_no_lr_mul": ("rate = float(lr) * float(lr_mul)", "rate = float(lr)"),
    "adam_no_wd_mul": ("decay = float(wd) * float(wd_mul)", "decay = float(wd)"),
    "adam_moments_not_rounded": ("m_new = fp32_round(beta1 * m + (1.0 - beta1) * g)",
                                 "m_new = beta1 * m + (1.0 - beta1) * g"),
    "adam_step_off_by_one": ("t = int(step)", "t = int(step) + 1"),
    "apply_multipliers_swapped": ("lr_eff = float(lr) * float(lr_mul)\n    wd_eff = float(wd) * float(wd_mul)",
                                  "lr_eff = float(lr) * float(wd_mul)\n    wd_eff = float(wd) * float(lr_mul)"),
    "apply_not_rounded": ("        return bf16_round(res)\n    if dtype == \"fp32\"",
                          "        return res\n    if dtype == \"fp32\""),
}


def load_mutant(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    spec = importlib.util.spec_from_loader(mod.__name__, loader=None)
    mod.__spec__ = spec
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mutant = load_mutant(name, *MUTATIONS[name])
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception:            # AssertionError, or a shape error
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutation {name}"
