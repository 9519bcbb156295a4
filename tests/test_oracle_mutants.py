"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the
pins catch every one of them: a dropped term, a wrong sign, a transposed operand,
a wrong index."""
import importlib.util
import os
import types

import pytest

import _pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "ce_tvd.py")).read()

MUTANTS = {
    "tvd_without_half": ('out["tvd"][valid] = 0.5 * np.sum(', 'out["tvd"][valid] = 1.0 * np.sum('),
    "forward_sign_flipped": ("    d = p - q\n", "    d = q - p\n"),
    "backward_sign_flipped": ("s = np.sign(p - q)", "s = np.sign(q - p)"),
    "onehot_dropped": ("gv = g_ce * (p - onehot)", "gv = g_ce * p"),
    "sigma_term_dropped": ("0.5 * p * (s - sigma)", "0.5 * p * s"),
    "sigma_weights_q": ("sigma = np.sum(p * s, axis=-1, keepdims=True)", "sigma = np.sum(q * s, axis=-1, keepdims=True)"),
    "ce_from_teacher": ('out["ce"][valid] = lse_s - zv[', 'out["ce"][valid] = lse_s - decode(u_raw)[valid]['),
    "lse_missing_max": ("(m + np.log(", "(0 * m + np.log("),
    "p_uses_teacher_lse": ("p = probs_rows(zv, lse_s)", "p = probs_rows(zv, lse_t)"),
    "target_off_by_one": ("onehot[rows, t] = 1.0", "onehot[rows, (t + 1) % V] = 1.0"),
    "tvd_grad_half_dropped": ("g_tvd * 0.5 * p * (s - sigma)", "g_tvd * p * (s - sigma)"),
    "row_weights_swapped": ("g_ce = np.broadcast_to(np.asarray(g_ce,", "g_ce = np.broadcast_to(np.asarray(g_tvd,"),
    "row_weights_unmasked": ("(R,))[valid][:, None]\n    g_tvd", "(R,))[:, None][:1]\n    g_tvd"),
    "binary16_read_as_bf16": ("    if raw.dtype == np.uint16:", "    if raw.dtype in (np.uint16, np.float16):\n        raw = raw.view(np.uint16)"),
    "linear_grad_x_sign": ('out["grad_x_s"] = g @ ws', 'out["grad_x_s"] = -g @ ws'),
    "linear_grad_w_from_teacher_hidden": ('out["grad_w_s"] = g.T @ xs', 'out["grad_w_s"] = g.T @ (xs if x_t_raw is None else decode(x_t_raw)[:, :xs.shape[1]])'),
    "linear_teacher_logits_transposed": ("decode(x_t_raw) @ decode(w_t_raw).T", "(decode(w_t_raw) @ decode(x_t_raw).T).T[:, ::-1]"),
    "branch_signs_ignored_in_forward": ("s = np.sign(d) if signs is None else", "s = np.sign(d) if True else"),
    "branch_signs_ignored_in_backward": ("s = np.sign(p - q) if signs is None else", "s = np.sign(p - q) if True else"),
    "ignored_rows_not_zeroed": ('valid = _valid_mask(target, V, ignore_index)\n    grad', 'valid = _valid_mask(target, V, ignore_index) | True\n    grad'),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation anchor for {name} not found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant(name)
    caught = []
    for pin in _pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"mutant {name} passed every pin"
