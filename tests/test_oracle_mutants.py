"""Planted mistakes in copies of the oracle must each make some pin fail.

Each mutant is the oracle's source with one plausible slip (a dropped term, a
wrong sign or index, a swapped operand, a different reading); it is executed as a
throwaway module on the CPU and the pins are run against it.
"""
import inspect
import types

import pytest

from oracle import fwmem_oracle
from tests import oracle_pins

MUTANTS = {
    "residual_sign": ('r = vt - np.einsum("nij,ni->nj", S, x)',
                      'r = vt + np.einsum("nij,ni->nj", S, x)'),
    "same_index_pairing": ("x = np.where(has[:, None], unit(xprev), 0.0)",
                           "x = np.where(has[:, None], kt, 0.0)"),
    "no_ridge_decay": ("decay = 1.0 - (", "decay = 1.0 + 0.0 * ("),
    "no_key_energy": ("den = np.sum(x * x, axis=1) + lam_hat + eps",
                      "den = 1.0 + lam_hat + eps"),
    "no_lambda_in_eta": ("den = np.sum(x * x, axis=1) + lam_hat + eps",
                         "den = np.sum(x * x, axis=1) + eps"),
    "first_step_writes": ("eta = np.where(has, Bt[:, t] / np.where(has, den, 1.0), 0.0)",
                          "eta = Bt[:, t] / den"),
    "mean_channel_reading": ("lam_hat = lam_t.max(axis=1)", "lam_hat = lam_t.mean(axis=1)"),
    "transposed_read": ('O[:, t] = np.einsum("nij,ni->nj", S, qt)',
                        'O[:, t] = np.einsum("nji,ni->nj", S, qt)'),
    "additive_no_decay": ("S = gam * S + b", "S = S + b"),
    "additive_no_beta": ("S = gam * S + b[:, None, None] *", "S = gam * S + 1.0 *"),
    "elu_no_shift": ("np.where(x > 0, x + 1.0,", "np.where(x > 0, x,"),
    "residual_uses_query": ('r = vt - np.einsum("nij,ni->nj", S, x)',
                            'r = vt - np.einsum("nij,ni->nj", S, qt)'),
    "write_uses_value_not_residual": ("eta[:, None, None] * x[:, :, None] * r[:, None, :]",
                                      "eta[:, None, None] * x[:, :, None] * vt[:, None, :]"),
    "inner_writes_residual": ("eta[:, None, None] * x[:, :, None] * vt[:, None, :]",
                              "eta[:, None, None] * x[:, :, None] * (vt - np.einsum(\"nij,ni->nj\", S, x))[:, None, :]"),
    "inner_same_index_pairing": ("* x[:, :, None] * vt[:, None, :]", "* kt[:, :, None] * vt[:, None, :]"),
    "inner_no_decay": ("S = decay[:, :, None] * S + eta[:, None, None] * x[:, :, None] * vt",
                       "S = S + eta[:, None, None] * x[:, :, None] * vt"),
    "inner_unnormalised_step": ("eta[:, None, None] * x[:, :, None] * vt[:, None, :]",
                                "Bt[:, t][:, None, None] * x[:, :, None] * vt[:, None, :]"),
    "qk_norm_skips_carried_key": ("x = np.where(has[:, None], unit(xprev), 0.0)",
                                  "x = np.where(has[:, None], xprev, 0.0)"),
    "qk_norm_skips_query": ("qt = unit(phi(Q[:, t], phi_kind))", "qt = phi(Q[:, t], phi_kind)"),
    "qk_norm_rms_length_one": ('length = 1.0 if qk_norm == "l2" else float(np.sqrt(dk))', "length = 1.0"),
    "retention_uses_softplus": ("Lm = sigmoid(Lm) if rule == RULE_ADDITIVE else softplus(Lm)",
                                "Lm = softplus(Lm)"),
    "beta_range_one": ('Bt = {"sigmoid": 1.0, "sigmoid2": 2.0}[beta_act] * sigmoid(Bt)', "Bt = sigmoid(Bt)"),
    "bwd_no_residual_state_term": ("G_prev = (a[:, None] if per_channel else a) * G - np.outer(x, dr)",
                                   "G_prev = (a[:, None] if per_channel else a) * G"),
    "bwd_den_sign": ("dden = -eta * deta / den", "dden = eta * deta / den"),
    "bwd_no_phi_grad_on_shifted_key": ("g[\"k\"][n, t - 1] += dx * phi_grad(K[n, t - 1], phi_kind)",
                                       "g[\"k\"][n, t - 1] += dx"),
    "bwd_same_index_key": ("g[\"k\"][n, t - 1] += dx * phi_grad(K[n, t - 1], phi_kind)",
                           "g[\"k\"][n, t] += dx * phi_grad(K[n, t], phi_kind)"),
    "bwd_lambda_hat_not_routed": ("                            dlt[imax] += dden\n", ""),
    "bwd_read_after_undo": ("                G = G + np.outer(qf, dOh[n, t])\n", ""),
    "pv_shared_step": ("Bt[:, t, :] / np.where(has, den_pv, 1.0)[:, None]",
                       "Bt[:, t, :1] / np.where(has, den_pv, 1.0)[:, None] + 0.0 * Bt[:, t, :]"),
    "pv_decay_on_rows": ("(1.0 - eta_pv * lam_pv[:, None])[:, None, :] * S",
                         "(1.0 - eta_pv * lam_pv[:, None])[:, :, None] * S"),
    "pv_residual_sign": ('r_pv = vt - np.einsum("ni,nij->nj", x, S)', 'r_pv = vt + np.einsum("ni,nij->nj", x, S)'),
    "pv_no_ridge_in_step": ("den_pv = np.sum(x * x, axis=1) + lam_pv + eps",
                            "den_pv = np.sum(x * x, axis=1) + eps"),
    "pv_same_index_pairing": ("x = unit(xprev) * has[:, None]", "x = kt * has[:, None]"),
    "ridge_not_scaled": ("lam_t = lam_t * (energy[:, None] if per_channel else energy)", "lam_t = lam_t"),
    "ridge_hat_not_scaled": ("lam_hat = lam_hat * energy", "lam_hat = lam_hat"),
    "ridge_scaled_by_norm": ("energy = np.sum(x * x, axis=1)", "energy = np.sqrt(np.sum(x * x, axis=1))"),
    "znorm_no_decay": ("z = gam[:, :, 0] * z + b[:, None] * kt", "z = z + b[:, None] * kt"),
    "znorm_no_beta": ("z = gam[:, :, 0] * z + b[:, None] * kt", "z = gam[:, :, 0] * z + kt"),
    "bwd_softplus_derivative_dropped": ("Lm, dLm = softplus(Lm), sl", "Lm, dLm = softplus(Lm), 1.0"),
    "bwd_sigmoid2_derivative_halved": ("Bt, dBt = scale * sb, scale * sb * (1.0 - sb)",
                                       "Bt, dBt = scale * sb, sb * (1.0 - sb)"),
    "bwd_norm_projection_dropped": ("return f * (g - u * np.sum(u * g, axis=-1, keepdims=True))",
                                    "return f * g"),
    "bwd_scaled_ridge_key_term_dropped": ("dx = dx + 2.0 * x * (np.sum(dlt * lt) if per_channel else dlt * lt)",
                                          "dx = dx"),
    "bwd_pv_decay_on_rows": ("G_prev = G * a[None, :] - np.outer(x, dr)", "G_prev = G * a[:, None] - np.outer(x, dr)"),
    "bwd_znorm_z_not_decayed": ("                Gz = gam * Gz\n", ""),
    "decay_after_write": ("S = decay[:, :, None] * S + eta[:, None, None] * x[:, :, None] * r[:, None, :]",
                          "S = decay[:, :, None] * (S + eta[:, None, None] * x[:, :, None] * r[:, None, :])"),
}


def _mutant(old, new):
    src = inspect.getsource(fwmem_oracle)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash caused by the slip
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutant {name}"
