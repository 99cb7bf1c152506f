"""KDA oracle (Python side) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  It shares no code with the HIP path.

Contents
--------
* ``c_prefill`` / ``c_decode_step`` / ``c_short_conv``: ctypes calls into the
  plain-C fp64 oracle (``kda_oracle.c``), OpenMP over (b, h).
* ``np_prefill`` / ``np_decode_step`` / ``np_short_conv``: an independent NumPy
  twin of the same token-by-token definitions (vectorised over (b, h) only).
* ``np_chunked_prefill``: the chunk (WY) form in fp64, derived from the
  token recurrence; the Kimi Linear summary page names it (256-token chunks,
  WY representation, batched rank-1 updates turned into triangular solves)
  without printing formulas.  It exists to pin the sequential form
  ("chunked equals sequential") and to host the injected faults used as
  positive controls for the prefix-invariance audit (dev.to audit page,
  "Two auditing norms": a clean verdict needs a positive control).
* ``l2norm``: x / sqrt(sum x^2 + 1e-6), the reading taken for the configs'
  "L2-normalised per head".
* ``np_prefill_backward``: the fp64 gradients of the token recurrence for the loss
  sum_t <do_t, o_t> + <dfinal, S_T> (reverse-mode differentiation of the token loop; with
  l2norm_qk, through the q/k normalisation as well), pinned by central finite differences
  of the C forward in tests/test_oracle_grad.py.

The recurrence (Kimi Linear summary page, recurrent-layers paragraph; the
remio.ai page's section on KDA's recurrent memory): per (b, h), with rows of
the dk x dv state S indexed by key channel,
S' = Diag(alpha_t) S;  u = beta_t (v_t - S'^T k_t);  S = S' + k_t u^T;
o_t = S^T q_t.  Masked positions leave S alone and give o_t = 0
(Transformers issue report on Kimi Linear cached continuation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None
L2_EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        up = ctypes.POINTER(ctypes.c_uint8)
        i = ctypes.c_int
        lib.kda_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, up, dp, dp, dp, i, i, i, i, i, i, i]
        lib.kda_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, up, dp, dp, i, i, i, i, i, i]
        lib.kda_oracle_short_conv.argtypes = [dp, dp, dp, up, dp, dp, dp, i, i, i, i, i]
        for f in (lib.kda_oracle_prefill, lib.kda_oracle_decode_step, lib.kda_oracle_short_conv):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> exact upcast on the host
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _u8(m):
    if m is None:
        return None
    if hasattr(m, "detach"):
        m = m.detach().cpu().numpy()
    return np.ascontiguousarray(m, dtype=np.uint8)


def _dp(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _up(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def host_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# ------------------------------------------------------------------ C oracle

def c_prefill(q, k, v, log_alpha, beta, mask=None, init_state=None, l2norm_qk=False,
              nthreads=None):
    """Token-by-token fp64 prefill.  Returns (o [B,T,H,dv], final_state [B,H,dk,dv])."""
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    mask, s0 = _u8(mask), _f64(init_state)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    fs = np.zeros((B, H, dk, dv))
    rc = _load().kda_oracle_prefill(_dp(q), _dp(k), _dp(v), _dp(la), _dp(beta), _up(mask),
                                    _dp(s0), _dp(o), _dp(fs), B, T, H, dk, dv, int(l2norm_qk),
                                    int(nthreads or host_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_prefill failed")
    return o, fs


def c_decode_step(q, k, v, log_alpha, beta, state, mask=None, l2norm_qk=False, nthreads=None):
    """One fp64 decode step.  ``state`` [B,H,dk,dv] is copied, not modified.
    Returns (o [B,H,dv], new_state)."""
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    mask = _u8(mask)
    st = np.array(_f64(state), copy=True)
    B, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, H, dv))
    rc = _load().kda_oracle_decode_step(_dp(q), _dp(k), _dp(v), _dp(la), _dp(beta), _up(mask),
                                        _dp(st), _dp(o), B, H, dk, dv, int(l2norm_qk),
                                        int(nthreads or host_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode_step failed")
    return o, st


def c_short_conv(x, w, bias=None, mask=None, cache=None, silu=False):
    """Masked depthwise causal conv over the compacted sequence.
    Returns (y [B,T,D], new_cache [B,W-1,D])."""
    x, w, bias, cache = _f64(x), _f64(w), _f64(bias), _f64(cache)
    mask = _u8(mask)
    B, T, D = x.shape
    W = w.shape[1]
    y = np.zeros((B, T, D))
    nc = np.zeros((B, W - 1, D))
    rc = _load().kda_oracle_short_conv(_dp(x), _dp(w), _dp(bias), _up(mask), _dp(cache),
                                       _dp(y), _dp(nc), B, T, D, W, int(silu))
    if rc != 0:
        raise RuntimeError("kda_oracle_short_conv failed")
    return y, nc


# ------------------------------------------------------------------ NumPy twin

def l2norm(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def np_prefill(q, k, v, log_alpha, beta, mask=None, init_state=None, l2norm_qk=False):
    """Independent NumPy version of the token loop, vectorised over (b, h)."""
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if l2norm_qk:
        q, k = l2norm(q), l2norm(k)
    S = np.zeros((B, H, dk, dv)) if init_state is None else np.array(_f64(init_state), copy=True)
    m = np.ones((B, T), bool) if mask is None else (_u8(mask) != 0)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        sel = m[:, t]
        if not sel.any():
            continue
        St = S[sel]                                             # [b,H,dk,dv]
        Sd = np.exp(la[sel, t])[..., None] * St                 # decay key channels
        kt, qt = k[sel, t], q[sel, t]
        pred = np.einsum("bhij,bhi->bhj", Sd, kt)               # S'^T k
        u = beta[sel, t][..., None] * (v[sel, t] - pred)
        Sn = Sd + kt[..., :, None] * u[..., None, :]
        o[sel, t] = np.einsum("bhij,bhi->bhj", Sn, qt)
        S[sel] = Sn
    return o, S


def np_prefill_backward(q, k, v, log_alpha, beta, do, dfinal=None, mask=None, init_state=None,
                        l2norm_qk=False):
    """Gradients of the token recurrence (the blockwise training the remio.ai page names in
    its KDA section needs them): for the loss L = sum_t <do_t, o_t> + <dfinal, S_T>, the
    derivatives of L with respect to q, k, v, log_alpha, beta and the initial state, in fp64.

    Reverse-mode differentiation of the token loop of np_prefill, written out step by step
    (all per-token states are kept, so for small inputs only).  With S' = Diag(a) S_{t-1},
    a = exp(log_alpha_t), r = v_t - S'^T k_t, u = beta_t r, S_t = S' + k_t u^T and
    o_t = S_t^T q_t, and lam = dL/dS_t:
        lam += q_t do_t^T;  dq_t = S_t do_t
        du = lam^T k_t;  dk_t = lam u;  dbeta_t = du . r;  dv_t = beta_t du
        dS' = lam - k_t (beta_t du)^T;  dk_t -= S' (beta_t du)
        dlog_alpha_t = rowsum(dS' * S');  lam <- Diag(a) dS'
    A masked position leaves lam alone and has zero gradients.  With l2norm_qk the loop runs
    on q and k normalised as in np_prefill, x_hat = s x with s = (|x|^2 + eps)^(-1/2), and dq,
    dk are taken back to the raw rows by the chain rule through that map:
        dx = s dx_hat - s^3 x (x . dx_hat).
    Returns a dict with dq, dk, dv, dlog_alpha, dbeta, dinit_state (the last is returned even
    without an initial state: it is the gradient with respect to the zero state)."""
    q, k, v, la, beta, do = map(_f64, (q, k, v, log_alpha, beta, do))
    raw = None
    if l2norm_qk:
        raw = {"dq": q, "dk": k}
        q, k = l2norm(q), l2norm(k)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if init_state is None else np.array(_f64(init_state), copy=True)
    m = np.ones((B, T), bool) if mask is None else (_u8(mask) != 0)
    # forward, keeping every state
    states = [S0]
    S = S0.copy()
    for t in range(T):
        Sn = S.copy()
        for b in range(B):
            if not m[b, t]:
                continue
            for h in range(H):
                Sp = np.exp(la[b, t, h])[:, None] * S[b, h]
                u = beta[b, t, h] * (v[b, t, h] - Sp.T @ k[b, t, h])
                Sn[b, h] = Sp + np.outer(k[b, t, h], u)
        S = Sn
        states.append(S)
    lam = np.zeros((B, H, dk, dv)) if dfinal is None else np.array(_f64(dfinal), copy=True)
    g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("dbeta", beta))}
    for t in range(T - 1, -1, -1):
        for b in range(B):
            if not m[b, t]:
                continue
            for h in range(H):
                Sprev, St = states[t][b, h], states[t + 1][b, h]
                a = np.exp(la[b, t, h])
                Sp = a[:, None] * Sprev
                kt, qt, vt, bt = k[b, t, h], q[b, t, h], v[b, t, h], beta[b, t, h]
                r = vt - Sp.T @ kt
                u = bt * r
                L = lam[b, h] + np.outer(qt, do[b, t, h])
                g["dq"][b, t, h] = St @ do[b, t, h]
                du = L.T @ kt
                g["dbeta"][b, t, h] = du @ r
                dr = bt * du
                g["dv"][b, t, h] = dr
                g["dk"][b, t, h] = L @ u - Sp @ dr
                dSp = L - np.outer(kt, dr)
                g["dlog_alpha"][b, t, h] = np.sum(dSp * Sp, axis=1)
                lam[b, h] = a[:, None] * dSp
    g["dinit_state"] = lam
    if raw is not None:
        for n, x in raw.items():
            sc = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)
            gx = g[n]
            g[n] = sc * gx - sc ** 3 * x * np.sum(x * gx, axis=-1, keepdims=True)
    return g


def np_decode_step(q, k, v, log_alpha, beta, state, mask=None, l2norm_qk=False):
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    o, s = np_prefill(q[:, None], k[:, None], v[:, None], la[:, None], beta[:, None],
                      None if mask is None else _u8(mask)[:, None], state, l2norm_qk)
    return o[:, 0], s


def np_short_conv(x, w, bias=None, mask=None, cache=None, silu=False):
    """Compacted-sequence short conv via NumPy correlation over [cache, valid x]."""
    x, w = _f64(x), _f64(w)
    B, T, D = x.shape
    W = w.shape[1]
    cache = np.zeros((B, W - 1, D)) if cache is None else _f64(cache)
    m = np.ones((B, T), bool) if mask is None else (_u8(mask) != 0)
    y = np.zeros((B, T, D))
    nc = np.zeros((B, W - 1, D))
    for b in range(B):
        idx = np.nonzero(m[b])[0]
        seq = np.concatenate([cache[b], x[b, idx]], axis=0)      # [W-1+n, D]
        n = len(idx)
        acc = np.zeros((n, D))
        for j in range(W):
            acc += w[:, j][None, :] * seq[j:j + n]
        if bias is not None:
            acc += _f64(bias)[None, :]
        if silu:
            acc = acc / (1.0 + np.exp(-acc))
        y[b, idx] = acc
        nc[b] = seq[len(seq) - (W - 1):] if W > 1 else nc[b]
    return y, nc


# ------------------------------------------------------------------ fp64 chunk (WY) form

def np_chunked_prefill(q, k, v, log_alpha, beta, chunk, mask=None, init_state=None,
                       fault=None):
    """Chunkwise-parallel form of the same recurrence, in fp64.

    Within a chunk that starts from state S0, let G be the inclusive cumulative
    sum of log_alpha from the chunk start (per key channel) and Gamma = exp(G).
    With Kt = K*Gamma, the per-token corrections u satisfy the unit
    lower-triangular system (I + A) U = Diag(beta) (V - Kt S0), where
    A[t,j] = beta_t sum_c k[t,c] k[j,c] exp(G[t,c] - G[j,c]) for j < t.
    Then O = (Q*Gamma) S0 + P U with P[t,j] = sum_c q[t,c] k[j,c]
    exp(G[t,c] - G[j,c]) for j <= t, and the state leaving the chunk is
    Diag(Gamma_last) S0 + (K * Gamma_last / Gamma)^T U.

    Masked positions get log_alpha = 0, beta = 0 and zero q/k/v, which makes
    them exact no-ops; their output is set to 0.

    ``fault`` plants a defect for positive controls:
      * "future_chunk":  each chunk reads the state *after* itself (an
        inter-chunk reduction over the wrong axis), leaking the future with
        onset at a chunk boundary;
      * "diag_leak":  P includes j = t + 1 (a non-strict triangle).
    """
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    m = np.ones((B, T), bool) if mask is None else (_u8(mask) != 0)
    mm = m[:, :, None, None]
    q, k, v, la = q * mm, k * mm, v * mm, la * mm
    beta = beta * m[:, :, None]
    S = np.zeros((B, H, dk, dv)) if init_state is None else np.array(_f64(init_state), copy=True)
    nch = (T + chunk - 1) // chunk
    states = [S]
    pieces = []
    for n in range(nch):
        t0, t1 = n * chunk, min(T, (n + 1) * chunk)
        Cn = t1 - t0
        Q, K, V, L = (np.moveaxis(x[:, t0:t1], 1, 2) for x in (q, k, v, la))   # [B,H,C,*]
        bt = np.moveaxis(beta[:, t0:t1], 1, 2)                                  # [B,H,C]
        G = np.cumsum(L, axis=2)
        Gam = np.exp(G)
        strict = np.tril(np.ones((Cn, Cn), bool), -1)
        incl = np.tril(np.ones((Cn, Cn), bool), 1 if fault == "diag_leak" else 0)
        Ediff = G[:, :, :, None, :] - G[:, :, None, :, :]                       # G[t]-G[j]
        Dinc = np.exp(np.where(incl[None, None, :, :, None], Ediff, -np.inf))
        Dstr = np.exp(np.where(strict[None, None, :, :, None], Ediff, -np.inf))
        A = bt[..., None] * np.einsum("bhtc,bhjc,bhtjc->bhtj", K, K, Dstr)
        P = np.einsum("bhtc,bhjc,bhtjc->bhtj", Q, K, Dinc)
        S0 = states[-1]
        rhs = bt[..., None] * (V - np.einsum("bhtc,bhcv->bhtv", K * Gam, S0))
        U = np.linalg.solve(np.eye(Cn)[None, None] + A, rhs)   # unit lower-triangular system
        Sn = Gam[:, :, -1, :, None] * S0 + np.einsum(
            "bhtc,bhtv->bhcv", K * np.exp(G[:, :, -1:, :] - G), U)
        states.append(Sn)
        pieces.append((t0, t1, Q * Gam, P, U))
    o = np.zeros((B, T, H, dv))
    for n, (t0, t1, Qt, P, U) in enumerate(pieces):
        Sread = states[n + 1] if fault == "future_chunk" else states[n]
        On = np.einsum("bhtc,bhcv->bhtv", Qt, Sread) + np.einsum("bhtj,bhjv->bhtv", P, U)
        o[:, t0:t1] = np.moveaxis(On, 2, 1)
    return o * mm, states[-1]


# ------------------------------------------------------------------ pipeline helpers

def pipeline(xq, xk, xv, wq, wk, wv, log_alpha, beta, H, dk, dv, mask=None,
             caches=None, init_state=None, silu=False, impl="c"):
    """raw x -> short conv (q,k,v) -> L2-norm(q,k) -> recurrence.

    Returns a dict of every stage's output (for per-stage prefix audits):
    yq, yk, yv (conv outputs [B,T,H*d]), qn, kn (normalised), o, state, caches.
    """
    conv = c_short_conv if impl == "c" else np_short_conv
    pre = c_prefill if impl == "c" else np_prefill
    caches = caches or (None, None, None)
    yq, cq = conv(xq, wq, None, mask, caches[0], silu)
    yk, ck = conv(xk, wk, None, mask, caches[1], silu)
    yv, cv = conv(xv, wv, None, mask, caches[2], silu)
    B, T, _ = yq.shape
    qn = l2norm(yq.reshape(B, T, H, dk))
    kn = l2norm(yk.reshape(B, T, H, dk))
    o, s = pre(qn, kn, yv.reshape(B, T, H, dv), log_alpha, beta, mask, init_state, False)
    return dict(yq=yq, yk=yk, yv=yv, qn=qn, kn=kn, o=o, state=s, caches=(cq, ck, cv))


def prefix_delta(stages_a: dict, stages_b: dict, p: int, keys=("yq", "yk", "yv", "qn", "kn", "o")):
    """Per-stage max |a - b| over positions [0, p) (dev.to audit page, audit steps)."""
    return {key: float(np.max(np.abs(np.asarray(stages_a[key])[:, :p] - np.asarray(stages_b[key])[:, :p]),
                              initial=0.0)) for key in keys}
