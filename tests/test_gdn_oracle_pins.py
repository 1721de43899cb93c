"""Pins of the oracle's gated delta rule ([Kazeia] "Le kernel actuel": per token, decay
the state by the gate, form delta = (v - S^T k) beta, add k delta^T, read S^T q) against
what the mathematics fixes: closed forms, the delta rule's write-then-read identity,
state passing, and the chunkwise algorithm of the same page (an independent derivation,
tests/gdn_chunkwise.py).  CPU only."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gdn_chunkwise import gdn_chunkwise


def _inputs(B=2, H=3, P=150, dk=16, dv=8, seed=0, state=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, P, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, P, dk))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)  # unit keys
    v = rng.standard_normal((B, H, P, dv)).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((B, H, P))))).astype(np.float32)
    alpha = (-np.log1p(np.exp(rng.standard_normal((B, H, P)) - 2))).astype(np.float32)
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32) * 0.1 if state else None
    return q, k, v, beta, alpha, s0


def test_chunkwise_algorithm_equals_token_recurrence():
    q, k, v, beta, alpha, s0 = _inputs()
    o_ref, s_ref = O.gdn(q, k, v, beta, alpha, s0)
    for C in (64, 16, 7):  # chunks spanning the sequence, with a ragged last one
        o, s = gdn_chunkwise(q, k, v, beta, alpha, s0, C=C)
        assert np.abs(o - o_ref).max() <= 1e-9 * np.abs(o_ref).max()
        assert np.abs(s - s_ref).max() <= 1e-9 * np.abs(s_ref).max()


def test_no_update_is_pure_decay():
    """beta = 0: the state only decays, S_t = prod(g_1..g_t) S0, out_t = S_t^T q_t."""
    q, k, v, beta, alpha, s0 = _inputs(B=1, H=2, P=20)
    beta[:] = 0
    o, s = O.gdn(q, k, v, beta, alpha, s0)
    G = np.exp(np.cumsum(alpha.astype(np.float64), axis=-1))  # [B,H,P]
    ref = G[..., None] * np.einsum("bhpi,bhij->bhpj", q.astype(np.float64), s0.astype(np.float64))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, G[..., -1, None, None] * s0, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_store_values_exactly():
    """No decay, beta = 1, key t = e_t, empty state: token t writes v_t into row t, so
    out_t = sum_{s<=t} q_t[s] v_s (a causal linear attention)."""
    P, dk, dv = 12, 16, 5
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, P, dk)).astype(np.float32)
    v = rng.standard_normal((1, 1, P, dv)).astype(np.float32)
    k = np.zeros((1, 1, P, dk), np.float32)
    k[0, 0, np.arange(P), np.arange(P)] = 1
    o, s = O.gdn(q, k, v, np.ones((1, 1, P), np.float32), np.zeros((1, 1, P), np.float32))
    qq, vv = q[0, 0].astype(np.float64), v[0, 0].astype(np.float64)
    ref = np.array([(qq[t, :t + 1, None] * vv[:t + 1]).sum(0) for t in range(P)])
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s[0, 0, :P], vv, rtol=0, atol=0)


def test_delta_rule_reads_back_the_value_just_written():
    """No decay, beta = 1, unit key: after token t the state maps k_t to v_t exactly
    (the error-correcting write)."""
    q, k, v, beta, alpha, s0 = _inputs(B=1, H=1, P=9, dk=8, dv=4)
    beta[:] = 1
    alpha[:] = 0
    # keys of four entries +-1/2: |k|^2 = 1 exactly in fp32
    rng = np.random.default_rng(5)
    k[:] = 0
    for t in range(9):
        idx = rng.choice(8, 4, replace=False)
        k[0, 0, t, idx] = rng.choice([-0.5, 0.5], 4)
    for t in range(9):
        _, s = O.gdn(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1], beta[:, :, :t + 1],
                     alpha[:, :, :t + 1], s0)
        np.testing.assert_allclose(s[0, 0].T @ k[0, 0, t].astype(np.float64),
                                   v[0, 0, t].astype(np.float64), rtol=1e-9, atol=1e-9)


def test_state_carries_across_calls():
    """Two calls with the state handed over equal one call over the whole sequence."""
    q, k, v, beta, alpha, s0 = _inputs(P=70)
    o, s = O.gdn(q, k, v, beta, alpha, s0)
    P1 = 31
    o1, s1 = O.gdn(q[:, :, :P1], k[:, :, :P1], v[:, :, :P1], beta[:, :, :P1], alpha[:, :, :P1],
                   s0)
    # the oracle takes an fp32 state: hand over the fp64 one through float32 and compare
    # the second half against a reference that starts from the same rounded state
    s1f = s1.astype(np.float32)
    o2, s2 = O.gdn(q[:, :, P1:], k[:, :, P1:], v[:, :, P1:], beta[:, :, P1:], alpha[:, :, P1:],
                   s1f)
    o2r, s2r = gdn_chunkwise(q[:, :, P1:], k[:, :, P1:], v[:, :, P1:], beta[:, :, P1:],
                             alpha[:, :, P1:], s1f)
    np.testing.assert_allclose(o[:, :, :P1], o1, rtol=0, atol=0)
    np.testing.assert_allclose(o2, o2r, rtol=1e-9, atol=1e-12)
    assert np.abs(o[:, :, P1:] - o2).max() <= 1e-5 * np.abs(o).max()
    assert np.abs(s - s2).max() <= 1e-5 * np.abs(s).max()


def test_zero_length_and_zero_state():
    q, k, v, beta, alpha, _ = _inputs(P=0)
    o, s = O.gdn(q, k, v, beta, alpha, None)
    assert o.shape == (2, 3, 0, 8) and not s.any()
