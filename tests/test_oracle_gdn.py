"""Pins for the float64 Gated DeltaNet oracle (CPU only).

Checks the product form against the expanded delta-rule form, special gate
values with closed-form results, the Proposition 2 identity by direct
recurrence, Proposition 1's split and its constructive counter-example, and
the footprint counts.
"""
import math

import numpy as np
import pytest

from oracle import gdn


def _coeffs(rng, steps, dk, dv, alpha_lo=0.5):
    ks = [g / np.linalg.norm(g) for g in rng.standard_normal((steps, dk))]
    vs = list(rng.standard_normal((steps, dv)))
    alphas = list(rng.uniform(alpha_lo, 1.0, steps))
    betas = list(rng.uniform(0.0, 1.0, steps))
    return alphas, betas, ks, vs


def test_product_form_equals_delta_rule_form():
    """S A + B equals alpha S + beta (v - alpha S k) k^T (the two forms of the
    update the pages give)."""
    rng = np.random.default_rng(0)
    dk, dv = 5, 7
    S = rng.standard_normal((dv, dk))
    (a,), (b,), (k,), (v,) = _coeffs(rng, 1, dk, dv)
    delta = a * S + b * np.outer(v - a * (S @ k), k)
    assert np.allclose(gdn.gdn_step(S, a, b, k, v), delta, rtol=1e-13, atol=1e-13)


def test_beta_one_writes_value_exactly():
    """With beta = 1 and a unit key, the new state maps k to v:
    S_i k = alpha (1 - beta) S_{i-1} k + beta v = v."""
    rng = np.random.default_rng(1)
    S = rng.standard_normal((6, 4))
    k = rng.standard_normal(4)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(6)
    S1 = gdn.gdn_step(S, 0.93, 1.0, k, v)
    assert np.allclose(S1 @ k, v, rtol=1e-13, atol=1e-13)


def test_alpha_one_beta_zero_keeps_state():
    rng = np.random.default_rng(2)
    S = rng.standard_normal((3, 3))
    k = np.array([0.6, 0.8, 0.0])
    assert np.array_equal(gdn.gdn_step(S, 1.0, 0.0, k, rng.standard_normal(3)), S)


def test_zero_state_single_write():
    """From S_0 = 0 one step gives beta v k^T (the write alone)."""
    k = np.array([0.0, 1.0, 0.0])
    v = np.array([2.0, -1.0])
    S1 = gdn.gdn_step(np.zeros((2, 3)), 0.9, 0.5, k, v)
    assert np.array_equal(S1, [[0.0, 1.0, 0.0], [0.0, -0.5, 0.0]])


@pytest.mark.parametrize("dk,dv", [(4, 4), (5, 8), (8, 6)])
def test_proposition2_unrolled_identity(dk, dv):
    """S_{t+j} = S_t P_j + W_j for j = 0..7 along one continuation, and
    o_{t+j} = S_t (P_j q) + W_j q."""
    rng = np.random.default_rng(dk * 10 + dv)
    t, J = 5, 7
    al, be, ks, vs = _coeffs(rng, t + J, dk, dv)
    states = gdn.gdn_run(np.zeros((dv, dk)), al, be, ks, vs)
    St = states[t]
    Ps, Ws = gdn.unrolled_products(al[t:], be[t:], ks[t:], vs[t:], dv)
    assert np.array_equal(Ps[0], np.eye(dk)) and np.all(Ws[0] == 0)
    for j in range(J + 1):
        ref = states[t + j]
        err = np.max(np.abs(St @ Ps[j] + Ws[j] - ref)) / np.max(np.abs(ref))
        assert err <= 1e-12, (j, err)
        q = rng.standard_normal(dk)
        o = gdn.readout(ref, q)
        o_split = St @ (Ps[j] @ q) + Ws[j] @ q
        assert np.allclose(o, o_split, rtol=1e-12, atol=1e-12)


def test_proposition1_split_and_counterexample():
    rng = np.random.default_rng(7)
    dv, dk, m = 5, 6, 3
    S = rng.standard_normal((dv, dk))
    Q = rng.standard_normal((dk, m))
    q_star = rng.standard_normal(dk)
    first, second = gdn.query_span_split(S, Q, q_star)
    assert np.allclose(first + second, S @ q_star, rtol=1e-10, atol=1e-10)
    # q* inside the span: the second term vanishes and (SQ) alone determines S q*
    q_in = Q @ rng.standard_normal(m)
    f_in, s_in = gdn.query_span_split(S, Q, q_in)
    assert np.max(np.abs(s_in)) <= 1e-10
    assert np.allclose(f_in, S @ q_in, rtol=1e-10, atol=1e-10)
    # outside the span: S' = S + u w^T agrees on every exposed readout, differs on q*
    Pi = Q @ np.linalg.pinv(Q)
    w = (np.eye(dk) - Pi) @ q_star
    assert np.linalg.norm(w) > 1e-6
    u = rng.standard_normal(dv)
    S2 = S + np.outer(u, w)
    assert np.allclose(S2 @ Q, S @ Q, rtol=1e-10, atol=1e-10)
    assert np.allclose(S2 @ q_star - S @ q_star, u * np.dot(w, w), rtol=1e-10, atol=1e-10)
    # the split sees the change only in the second term
    f2, s2 = gdn.query_span_split(S2, Q, q_star)
    assert np.allclose(f2, first, rtol=1e-10, atol=1e-10)
    assert np.allclose(s2 - second, u * np.dot(w, w), rtol=1e-10, atol=1e-10)


def test_proposition1_full_row_rank_projector_is_identity():
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((4, 9))              # rank 4 = d_k
    Pi = Q @ gdn.pinv(Q)
    assert np.allclose(Pi, np.eye(4), atol=1e-12)
    S = rng.standard_normal((3, 4))
    q_star = rng.standard_normal(4)
    _, second = gdn.query_span_split(S, Q, q_star)
    assert np.max(np.abs(second)) <= 1e-10


def test_pinv_brute_force_properties():
    """The four Moore-Penrose conditions on a rank-deficient matrix."""
    rng = np.random.default_rng(9)
    Q = rng.standard_normal((6, 2)) @ rng.standard_normal((2, 4))   # rank 2
    X = gdn.pinv(Q)
    assert np.allclose(Q @ X @ Q, Q, atol=1e-10)
    assert np.allclose(X @ Q @ X, X, atol=1e-10)
    assert np.allclose((Q @ X).T, Q @ X, atol=1e-10)
    assert np.allclose((X @ Q).T, X @ Q, atol=1e-10)


def test_footprint_counts():
    # Wide-heads shape: 2 layers x 48 heads, 128 x 128 states, t = 16384
    s, kv = gdn.footprint(96, 16384, 128, 128)
    assert s == 1_572_864 and kv == 402_653_184 and kv // s == 256
    # the crossover t = d_v d_k / (d_k + d_v) = 64 gives equal counts
    s, kv = gdn.footprint(2, 64, 128, 128)
    assert s == kv
    # paper shape: 32 pairs at t = 4096 -> 1 : 64
    s, kv = gdn.footprint(32, 4096, 128, 128)
    assert kv == 64 * s
    assert math.isclose(gdn.footprint(1, 1, 3, 5)[1], 8)
