"""Planted mistakes in the oracle (on the CPU): every plausible slip must fail a pin.

Each mutant below is the oracle's token step with exactly one mistake (a dropped term, a
wrong sign, a stale operand, a transposed operand, a wrong feature-map argument).  The
mutant is patched into the oracle module and a fixed set of pins from ``test_oracle.py``
is run against it; at least one pin must fail.  This is what makes the pins a pin of the
oracle and not of itself.
"""

import numpy as np
import pytest

import oracle.vla_oracle as vo
from tests import test_oracle as pins


def _mutant_step(mutation):
    def step(S, A, n, q_t, k_t, v_t, u_t, eps=1e-6, gain="unit"):
        S, A, n = (np.asarray(x, dtype=np.float64) for x in (S, A, n))
        q_t, k_t, v_t, u_t = (np.asarray(x, dtype=np.float64) for x in (q_t, k_t, v_t, u_t))
        khat = vo._unit(k_t)
        z = np.matmul(A, (k_t if mutation == "z_from_k" else u_t)[..., None])[..., 0]
        delta = (0.0 if mutation == "drop_one" else 1.0) + np.sum(u_t * z, axis=-1)
        sign = 1.0 if mutation == "sm_plus" else -1.0
        A_new = A + sign * (z[..., :, None] * z[..., None, :]) / delta[..., None, None]
        A_gate = A if mutation == "gate_old_A" else A_new
        y = np.matmul(A_gate, khat[..., None])[..., 0]
        if mutation == "gate_is_khat":
            y = khat
        ahat = vo._unit(y) if gain == "unit" else y
        Sk = np.swapaxes(S, -1, -2) if mutation == "transpose_S" else S
        kr = k_t if mutation == "resid_raw_k" else khat
        resid = v_t - np.matmul(Sk, kr[..., None])[..., 0]
        S_new = S + resid[..., :, None] * ahat[..., None, :]
        fq = vo.phi(q_t)
        n_new = n + (vo.phi(khat) if mutation == "phi_khat" else vo.phi(k_t))
        S_read = S if mutation == "read_old_S" else S_new
        num = np.matmul(S_read, fq[..., None])[..., 0]
        den = np.sum((n if mutation == "old_n" else n_new) * fq, axis=-1) + eps
        o = num if mutation == "no_ratio" else num / den[..., None]
        return {"S": S_new, "A": A_new, "n": n_new, "o": o, "khat": khat, "z": z,
                "delta": delta, "y": y, "ahat": ahat, "resid": resid, "den": den}
    return step


PIN_CALLS = [
    lambda: pins.test_A_equals_direct_inverse_of_penalty(3, 0.5),
    pins.test_A_symmetric_positive_definite,
    pins.test_unit_key_and_gate,
    pins.test_residual_identity,
    lambda: pins.test_bruteforce_per_step_argmin(6, 3, 1),
    pins.test_rls_special_case_equals_ridge_regression,
    pins.test_u_zero_is_delta_rule,
    pins.test_d1_closed_form,
    pins.test_T1_closed_form,
    pins.test_hand_worked_example,
    pins.test_key_scale_invariance,
    pins.test_penalty_scale_invariance,
]

MUTATIONS = ["z_from_k", "drop_one", "sm_plus", "gate_old_A", "gate_is_khat", "transpose_S",
             "resid_raw_k", "phi_khat", "read_old_S", "old_n", "no_ratio"]


def test_unmutated_step_passes_all_selected_pins(monkeypatch):
    monkeypatch.setattr(vo, "vla_step", _mutant_step(None))
    monkeypatch.setattr(pins, "vla_step", _mutant_step(None))
    for call in PIN_CALLS:
        call()


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_planted_mistake_is_caught(monkeypatch, mutation):
    step = _mutant_step(mutation)
    monkeypatch.setattr(vo, "vla_step", step)
    monkeypatch.setattr(pins, "vla_step", step)
    failed = []
    for i, call in enumerate(PIN_CALLS):
        try:
            with np.errstate(all="ignore"):
                call()
        except (AssertionError, np.linalg.LinAlgError, FloatingPointError, ValueError):
            failed.append(i)
    assert failed, f"no pin caught the planted mistake {mutation!r}"
