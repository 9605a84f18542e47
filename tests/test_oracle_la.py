"""Pins of the linear-attention oracle (CPU): the quadratic (attention) form written out as a
double loop, the T = 1 closed form, a hand-worked example, the state as one matrix product,
causality and continuation; and planted mistakes that each of them must catch.

The recurrence (oracle/la_oracle.py) and the quadratic form compute the same numbers by
different routes: the recurrence carries a d x d state, the quadratic form sums the causal
token pairs (s <= t) with explicit feature-map values, with no state at all.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle.la_oracle as lo
from oracle import la_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _phi_scalar(x):
    return x + 1.0 if x > 0.0 else math.exp(x)


def _quadratic_form(q, k, v, eps):
    """o_t = sum_{s<=t} v_s w_ts / (sum_{s<=t} w_ts + eps), w_ts = phi(k_s) . phi(q_t)."""
    T, d = q.shape
    out = np.zeros((T, d))
    for t in range(T):
        fq = [_phi_scalar(x) for x in q[t]]
        num = [0.0] * d
        den = 0.0
        for s in range(t + 1):
            w = sum(_phi_scalar(k[s][j]) * fq[j] for j in range(d))
            den += w
            for i in range(d):
                num[i] += v[s][i] * w
        out[t] = [x / (den + eps) for x in num]
    return out


def _inputs(T, d, seed, streams=1):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((streams, T, d)) for _ in range(3))


# pins, each taking the forward under test (so planted mistakes can be run through them)

def pin_quadratic_form(fwd):
    for T, d, seed in ((1, 3, 0), (7, 4, 1), (13, 5, 2)):
        q, k, v = _inputs(T, d, seed)
        out, _, _ = fwd(q, k, v, eps=1e-6)
        np.testing.assert_allclose(out[0], _quadratic_form(q[0], k[0], v[0], 1e-6), rtol=1e-12,
                                   atol=1e-12)


def pin_T1_closed_form(fwd):
    q, k, v = _inputs(1, 6, 3)
    c = sum(_phi_scalar(a) * _phi_scalar(b) for a, b in zip(k[0, 0], q[0, 0]))
    out, S, n = fwd(q, k, v, eps=0.25)
    np.testing.assert_allclose(out[0, 0], v[0, 0] * c / (c + 0.25), rtol=1e-13)


def pin_hand_example(fwd):
    with open(os.path.join(GOLDEN, "la_hand_t2_d2.json")) as f:
        g = json.load(f)
    out, S, n = fwd(np.array([g["q"]]), np.array([g["k"]]), np.array([g["v"]]), eps=g["eps"])
    np.testing.assert_allclose(out[0], g["out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0], g["S_T"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(n[0], g["n_T"], rtol=0, atol=1e-15)


def pin_state_is_one_product(fwd):
    q, k, v = _inputs(9, 5, 4, streams=2)
    _, S, n = fwd(q, k, v)
    fk = np.vectorize(_phi_scalar)(k)
    for s in range(2):
        np.testing.assert_allclose(S[s], v[s].T @ fk[s], rtol=1e-12)
        np.testing.assert_allclose(n[s], fk[s].sum(axis=0), rtol=1e-12)


PINS = [pin_quadratic_form, pin_T1_closed_form, pin_hand_example, pin_state_is_one_product]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_meets_pin(pin):
    pin(la_forward)


def test_causality_and_streams():
    q, k, v = _inputs(10, 4, 5, streams=3)
    out, _, _ = la_forward(q, k, v)
    q2, k2, v2 = (x.copy() for x in (q, k, v))
    for x in (q2, k2, v2):
        x[:, 6:] += 3.0
    out2, _, _ = la_forward(q2, k2, v2)
    np.testing.assert_array_equal(out[:, :6], out2[:, :6])
    one, _, _ = la_forward(q[1], k[1], v[1])
    np.testing.assert_allclose(out[1], one, rtol=1e-15)


def test_continuation_equals_one_call():
    q, k, v = _inputs(20, 4, 6)
    out, S, n = la_forward(q, k, v)
    a = la_forward(q[:, :8], k[:, :8], v[:, :8])
    b = la_forward(q[:, 8:], k[:, 8:], v[:, 8:], state=(a[1], a[2]))
    np.testing.assert_allclose(np.concatenate([a[0], b[0]], axis=1), out, rtol=1e-13)
    np.testing.assert_allclose(b[1], S, rtol=1e-13)


def _mutant(mutation):
    def fwd(q, k, v, eps=1e-6, state=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        batch, T, d = q.shape[:-2], q.shape[-2], q.shape[-1]
        S = np.zeros(batch + (d, d))
        n = np.zeros(batch + (d,))
        out = np.empty(q.shape)
        for t in range(T):
            fk = lo.phi(k[..., t, :]) if mutation != "raw_key" else k[..., t, :]
            fq = lo.phi(q[..., t, :]) if mutation != "raw_query" else q[..., t, :]
            S_old = S
            outer = v[..., t, :, None] * fk[..., None, :]
            S = S + (np.swapaxes(outer, -1, -2) if mutation == "transposed_outer" else outer)
            n = n + (lo.phi(k[..., t, :]) if mutation != "n_raw_key" else k[..., t, :])
            S_read = S_old if mutation == "read_old_S" else S
            num = np.matmul(S_read, fq[..., None])[..., 0]
            den = np.sum(n * fq, axis=-1) + (0.0 if mutation == "drop_eps" else eps)
            out[..., t, :] = num / den[..., None] if mutation != "no_ratio" else num
        return out, S, n
    return fwd


MUTATIONS = ["raw_key", "raw_query", "transposed_outer", "n_raw_key", "read_old_S", "drop_eps",
             "no_ratio"]


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_planted_mistake_fails_a_pin(mutation):
    fwd = _mutant(mutation)
    failed = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutation {mutation} passed every pin"
