"""CPU pins of the contraction bound that lets the prefill scan a long sequence in segments.

One token's state map is S -> (I - beta k k^T) Diag(alpha) S (plus a term that does not
depend on S).  Its spectral norm is at most max_c alpha_c * max(1, |1 - beta |k|^2|): the
projection is symmetric with eigenvalues 1 (k's complement) and 1 - beta |k|^2, and
Diag(alpha) has norm max_c alpha_c.  Over a tail of tokens the map is the product, so two
runs of the token recurrence that differ only in the state entering the tail differ at its
end by at most the product of the bounds times the norm of that difference.  The segmented
scan takes the state at a segment boundary as the tail run from a zero state once that
product is at most 2^-160.  These tests check the bound against brute-force transition
matrices and the claim against the fp64 oracle, with masked tokens (the identity), keys
that are not unit-norm (beta |k|^2 > 2 makes the factor exceed 1) and slow gates.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _token_bound_log2(la_row, beta, k_row, valid=True):
    if not valid:
        return 0.0
    f = abs(1.0 - beta * float(k_row @ k_row))
    return float(np.max(la_row)) / np.log(2.0) + np.log2(max(1.0, f))


def _transition(la_row, beta, k_row):
    K = k_row.shape[0]
    return (np.eye(K) - beta * np.outer(k_row, k_row)) @ np.diag(np.exp(la_row))


@pytest.mark.parametrize("case", ["unit_keys", "long_keys", "slow_gates"])
def test_token_and_tail_bound_brute_force(case):
    r = np.random.default_rng({"unit_keys": 1, "long_keys": 2, "slow_gates": 3}[case])
    K, T = 8, 40
    k = r.standard_normal((T, K))
    if case == "long_keys":
        k *= 1.7 / np.sqrt(K)                      # |k|^2 around 2.9: beta |k|^2 often above 2
    else:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal(T)))
    shift = 6.0 if case == "slow_gates" else 0.0
    la = -np.log1p(np.exp(r.standard_normal((T, K)) - shift))
    valid = r.random(T) > 0.2
    M = np.eye(K)
    total = 0.0
    for t in range(T):
        b = _token_bound_log2(la[t], beta[t], k[t], valid[t])
        Tt = _transition(la[t], beta[t], k[t]) if valid[t] else np.eye(K)
        assert np.log2(np.linalg.norm(Tt, 2)) <= b + 1e-12
        M = Tt @ M
        total += b
        assert np.log2(max(np.linalg.norm(M, 2), 1e-300)) <= total + 1e-9
    if case == "long_keys":
        assert any(beta[t] * (k[t] @ k[t]) > 2 for t in range(T) if valid[t]), "the case must exercise the factor"


def test_tail_from_zero_matches_within_bound(oracle):
    """The fp64 oracle run over a tail from a state S0 and from zero differ by at most
    2^(sum of the tail's bounds) * |S0| (Frobenius), for growing tails; with this workload's
    gates the bound falls below 2^-160 within a few hundred tokens, where the two runs agree
    to fp64 rounding."""
    r = np.random.default_rng(7)
    B, T, H, dk, dv = 1, 1600, 1, 32, 8
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    la = -np.log1p(np.exp(r.standard_normal((B, T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    mask = (r.random((B, T)) > 0.1).astype(np.uint8)
    s0 = 1e3 * r.standard_normal((B, H, dk, dv))           # a large entry state
    bounds = np.array([_token_bound_log2(la[0, t, 0], beta[0, t, 0], k[0, t, 0], bool(mask[0, t]))
                       for t in range(T)])
    reached = False
    for L in (16, 64, 256, 800, 1600):
        sl = slice(0, L)
        args = dict(q=q[:, sl], k=k[:, sl], v=v[:, sl], log_alpha=la[:, sl], beta=beta[:, sl], mask=mask[:, sl])
        _, s_from = oracle.c_prefill(**args, init_state=s0)
        _, s_zero = oracle.c_prefill(**args)
        diff = np.linalg.norm(s_from - s_zero)
        bound = 2.0 ** bounds[:L].sum() * np.linalg.norm(s0)
        assert diff <= bound * (1 + 1e-9) + 1e-12 * np.linalg.norm(s_zero), (L, diff, bound)
        if bounds[:L].sum() <= -160:
            reached = True
            assert diff <= 1e-12 * max(1.0, np.linalg.norm(s_zero))
    assert reached, "the workload's gates should forget within 1600 tokens"
