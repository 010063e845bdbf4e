"""Pins for the Log-Linear Gated DeltaNet oracle (``oracle/gdn.py``), each
against something other than its own formula: the recurrent form over
Fenwick level states, Gated DeltaNet's own single-state recurrence
(lambda = 1), the Mamba-2 form's oracle (orthogonal keys), a hand-worked
two-token example, and one-hot level weights."""

import numpy as np
import pytest

import oracle
from oracle import gdn


def _inputs(rng, B, H, T, dk, dv, L, unit_keys=True):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    a = -np.abs(rng.standard_normal((B, H, T))) * 0.2
    beta = rng.random((B, H, T))
    lam = rng.random((B, H, T, L))
    return q, k, v, a, beta, lam


def _L(T):
    return 1 if T <= 1 else 1 + (T - 1).bit_length()


@pytest.mark.parametrize("T", [1, 2, 3, 8, 13, 37])
def test_pairwise_equals_recurrent_levels(T):
    rng = np.random.default_rng(500 + T)
    q, k, v, a, beta, lam = _inputs(rng, 1, 2, T, 4, 3, _L(T))
    np.testing.assert_allclose(gdn.gdn_fwd(q, k, v, a, beta, lam), gdn.gdn_recurrent(q, k, v, a, beta, lam),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("T", [1, 9, 40])
def test_unit_lambda_is_gated_deltanet(T):
    rng = np.random.default_rng(520 + T)
    q, k, v, a, beta, _ = _inputs(rng, 2, 1, T, 5, 3, _L(T))
    lam = np.ones((2, 1, T, _L(T)))
    np.testing.assert_allclose(gdn.gdn_fwd(q, k, v, a, beta, lam), gdn.gdn_serial(q, k, v, a, beta),
                               rtol=1e-11, atol=1e-12)


def test_orthogonal_keys_reduce_to_the_mamba2_form():
    """Keys pairwise orthogonal: each M_r leaves every other key's direction
    alone up to alpha_r, so A[t,s] = beta_s exp(sum a) (k_s . q_t), the
    Mamba-2 form with v_s scaled by beta_s (checked against that form's own
    C oracle)."""
    rng = np.random.default_rng(540)
    T, dk, dv = 16, 16, 3
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[rng.permutation(dk)[:T]][None, None]          # [1,1,T,dk] orthonormal rows
    q = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    a = -np.abs(rng.standard_normal((1, 1, T))) * 0.3
    beta = rng.random((1, 1, T))
    lam = rng.random((1, 1, T, _L(T)))
    got = gdn.gdn_fwd(q, k, v, a, beta, lam)
    want = oracle.fwd(q, k, v * beta[..., None], a, lam)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_hand_example_two_tokens():
    """dk = dv = 1.  o_0 = lam_0[0] b_0 k_0 q_0 v_0 = 1 * 0.5 * 1 * 2 * 3 = 3.
    o_1 = lam_1[0] b_1 k_1 q_1 v_1 + lam_1[1] b_0 k_0 alpha_1 (1 - b_1 k_1^2) q_1 v_0
        = 0.5 * 0.25 * 4 + 2 * 0.5 * 0.5 * 0.75 * 3 = 0.5 + 1.125 = 1.625."""
    q = np.array([2.0, 1.0]).reshape(1, 1, 2, 1)
    k = np.array([1.0, 1.0]).reshape(1, 1, 2, 1)
    v = np.array([3.0, 4.0]).reshape(1, 1, 2, 1)
    a = np.array([0.0, np.log(0.5)]).reshape(1, 1, 2)
    beta = np.array([0.5, 0.25]).reshape(1, 1, 2)
    lam = np.array([[1.0, 7.0], [0.5, 2.0]]).reshape(1, 1, 2, 2)
    got = gdn.gdn_fwd(q, k, v, a, beta, lam)[0, 0, :, 0]
    np.testing.assert_allclose(got, [3.0, 1.625], rtol=1e-14)
    np.testing.assert_allclose(gdn.gdn_recurrent(q, k, v, a, beta, lam)[0, 0, :, 0], [3.0, 1.625], rtol=1e-14)


def test_one_hot_level_reads_only_its_bucket():
    """lambda one-hot at level l: only keys s with level(t, s) = l reach o_t,
    each with its full A[t, s] (the M factors of the keys in between stay)."""
    rng = np.random.default_rng(560)
    T, dk, dv = 23, 4, 2
    q, k, v, a, beta, _ = _inputs(rng, 1, 1, T, dk, dv, _L(T))
    for l in range(_L(T)):
        lam = np.zeros((1, 1, T, _L(T)))
        lam[..., l] = 1.0
        got = gdn.gdn_fwd(q, k, v, a, beta, lam)
        lam1 = np.ones((1, 1, T, _L(T)))
        for t in range(T):
            keep = np.array([oracle.level(t, s) == l for s in range(T)], dtype=float)
            vt = v * keep[None, None, :, None]
            full = gdn.gdn_fwd(q, k, vt, a, beta, lam1)
            np.testing.assert_allclose(got[0, 0, t], full[0, 0, t], rtol=1e-11, atol=1e-12)


def test_rows_match_full():
    rng = np.random.default_rng(580)
    T = 29
    q, k, v, a, beta, lam = _inputs(rng, 2, 2, T, 4, 3, _L(T))
    full = gdn.gdn_fwd(q, k, v, a, beta, lam)
    rows = np.array([[0, 0], [1, 28], [2, 13], [3, 7]])
    got = gdn.gdn_fwd_rows(q, k, v, a, beta, lam, rows)
    for i, (bh, t) in enumerate(rows):
        np.testing.assert_allclose(got[i], full.reshape(4, T, 3)[bh, t], rtol=1e-13, atol=1e-14)
