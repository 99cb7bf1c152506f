"""Pins of the oracle's gradient (np_prefill_backward) on the CPU: central finite
differences of the C oracle's forward (an independent implementation of the recurrence,
itself pinned in test_oracle_pins.py), a closed form for the identity case, and the
linearity of the gradient in the output cotangent.  The loss is
L = sum_t <do_t, o_t> + <dfinal, S_T>."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D


def _loss(O, inp, do, dfinal, mask, s0, l2=False):
    o, s = O.c_prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], mask=mask,
                       init_state=s0, l2norm_qk=l2, nthreads=1)
    return float(np.sum(o * do) + np.sum(s * dfinal))


def _case(seed, B=2, T=9, H=2, dk=3, dv=4, masked=True):
    rng = np.random.default_rng(seed)
    inp = {n: x.astype(np.float64) for n, x in D.np_kda_inputs(B, T, H, dk, dv, "fp32", seed=seed, unit_qk=False).items()}
    inp["beta"] = rng.uniform(0.1, 0.9, (B, T, H))
    s0 = rng.normal(0, 0.5, (B, H, dk, dv))
    do = rng.normal(0, 1, (B, T, H, dv))
    dfinal = rng.normal(0, 1, (B, H, dk, dv))
    mask = None
    if masked:
        mask = np.ones((B, T), np.uint8)
        mask[0, 2] = 0
        mask[1, :3] = 0
        mask[1, 7] = 0
    return inp, s0, do, dfinal, mask


@pytest.mark.parametrize("masked,l2", [(False, False), (True, False), (True, True)])
def test_gradient_matches_central_differences(oracle, masked, l2):
    """With l2, the C forward normalises q and k itself (its own code, pinned against the NumPy
    twin), so the differences also pin the chain rule through the normalisation."""
    inp, s0, do, dfinal, mask = _case(3, masked=masked)
    g = oracle.np_prefill_backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, dfinal,
                                   mask=mask, init_state=s0, l2norm_qk=l2)
    eps = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "beta": "dbeta"}
    for n, gn in list(names.items()) + [("s0", "dinit_state")]:
        base = s0 if n == "s0" else inp[n]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            keep = base[idx]
            base[idx] = keep + eps
            lp = _loss(oracle, inp, do, dfinal, mask, s0, l2)
            base[idx] = keep - eps
            lm = _loss(oracle, inp, do, dfinal, mask, s0, l2)
            base[idx] = keep
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - g[gn]))
        scale = max(1.0, np.max(np.abs(fd)))
        assert err <= 1e-6 * scale, f"{gn}: max |analytic - central difference| = {err:.3e}"
    if masked:                                  # masked positions have zero gradients
        for gn in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
            assert np.all(g[gn][mask == 0] == 0)


def test_gradient_identity_case_closed_form(oracle):
    """beta = 0 and log_alpha = 0 leave S = S0, so o_t = S0^T q_t: dS0 = sum_t q_t do_t^T +
    dfinal and dq_t = S0 do_t exactly."""
    inp, s0, do, dfinal, _ = _case(5, masked=False)
    inp["beta"][:] = 0.0
    inp["log_alpha"][:] = 0.0
    g = oracle.np_prefill_backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, dfinal,
                                   init_state=s0)
    want_s0 = np.einsum("bthi,bthj->bhij", inp["q"], do) + dfinal
    want_q = np.einsum("bhij,bthj->bthi", s0, do)
    assert np.allclose(g["dinit_state"], want_s0, rtol=1e-13, atol=1e-13)
    assert np.allclose(g["dq"], want_q, rtol=1e-13, atol=1e-13)
    assert np.all(g["dv"] == 0)                 # dv = beta du = 0


def test_gradient_is_linear_in_the_cotangents(oracle):
    inp, s0, do, dfinal, mask = _case(7)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    g1 = oracle.np_prefill_backward(*args, do, dfinal, mask=mask, init_state=s0)
    g2 = oracle.np_prefill_backward(*args, 2.0 * do, 2.0 * dfinal, mask=mask, init_state=s0)
    g0 = oracle.np_prefill_backward(*args, 0.0 * do, None, mask=mask, init_state=s0)
    for n in g1:
        assert np.allclose(g2[n], 2.0 * g1[n], rtol=1e-12, atol=1e-12), n
        assert np.all(g0[n] == 0), n


def test_gradient_l2_radial_direction_is_null(oracle):
    """Scaling a row of q or k leaves its normalised row unchanged (up to the eps), so with
    the norm inside the call the raw gradient has no radial part: x . dx ~ 0 for every row,
    while without the norm it does not vanish."""
    inp, s0, do, dfinal, mask = _case(11, masked=False)
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, dfinal)
    g = oracle.np_prefill_backward(*args, init_state=s0, l2norm_qk=True)
    g0 = oracle.np_prefill_backward(*args, init_state=s0)
    for n, x in (("dq", inp["q"]), ("dk", inp["k"])):
        radial = np.abs(np.sum(x * g[n], axis=-1))
        scale = np.linalg.norm(x, axis=-1) * np.linalg.norm(g[n], axis=-1)
        # the eps leaves a radial part of relative size eps / |x|^2
        assert np.all(radial <= 1e-5 * scale + 1e-12), n
        assert np.max(np.abs(np.sum(x * g0[n], axis=-1))) > 1e-3, n
