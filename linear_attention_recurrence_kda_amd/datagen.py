"""Seeded synthetic inputs for the KDA path.

This module is shared by the oracle tests, the GPU tests and the benchmark.
It holds only the input recipe (which distributions, which shapes, how values
are rounded to the storage dtype); none of the recurrence's arithmetic lives
here.

Recipe (shapes and distributions of the workloads the Kimi Linear pages
describe: long-context prefill and batched decode):

* q, k ~ N(0, 1) drawn in fp32, then scaled to unit L2 norm over the key
  dimension per (b, t, h), then rounded to the storage dtype (bf16: round to
  nearest even).
* v ~ N(0, 1), rounded to the storage dtype.
* log_alpha = -softplus(z), z ~ N(0, 1), fp32, one value per key channel
  (the per-channel forget gate).  The "slow" variant uses -softplus(z - 5),
  i.e. alpha close to 0.993, so that state survives for hundreds of tokens.
* beta = sigmoid(z), z ~ N(0, 1), fp32, one scalar per (b, t, h).

Two generators implement the same recipe:

* ``np_*``: NumPy PCG64 with one ``SeedSequence([seed, tensor_id, b, h])``
  stream per (tensor, b, h), so any head can be regenerated on its own.
* ``torch_*``: torch's device generator, for inputs too large to draw on the
  host (the 128k/512k-token prefill and the decode workload).  The GPU
  parity tests copy the heads they check back to the host.
"""
from __future__ import annotations

import numpy as np

# tensor ids for the per-(tensor, b, h) streams
TID_Q, TID_K, TID_V, TID_LA, TID_BETA, TID_S0 = 1, 2, 3, 4, 5, 6
TID_XQ, TID_XK, TID_XV, TID_CONVW, TID_CACHE, TID_LEN = 7, 8, 9, 10, 11, 12
TID_MASK, TID_PROBE = 13, 14


def _rng(seed: int, tid: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b, h])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return fp32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # NaN stays NaN (not produced by this recipe, kept for completeness)
    return np.where(np.isnan(x), x, out)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z.astype(np.float64))


def np_kda_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                  seed: int = 0, unit_qk: bool = True, decay: str = "default") -> dict:
    """q,k,v,log_alpha,beta as fp32 NumPy arrays, layout [B,T,H,*].

    q/k/v values are exactly representable in ``dtype``.
    """
    q = np.empty((B, T, H, dk), np.float32)
    k = np.empty((B, T, H, dk), np.float32)
    v = np.empty((B, T, H, dv), np.float32)
    la = np.empty((B, T, H, dk), np.float32)
    beta = np.empty((B, T, H), np.float32)
    shift = {"default": 0.0, "slow": 5.0}[decay]
    for b in range(B):
        for h in range(H):
            qq = _rng(seed, TID_Q, b, h).standard_normal((T, dk), dtype=np.float32)
            kk = _rng(seed, TID_K, b, h).standard_normal((T, dk), dtype=np.float32)
            if unit_qk:
                qq, kk = _unit_rows(qq), _unit_rows(kk)
            q[b, :, h] = to_storage(qq, dtype)
            k[b, :, h] = to_storage(kk, dtype)
            v[b, :, h] = to_storage(_rng(seed, TID_V, b, h).standard_normal((T, dv), dtype=np.float32), dtype)
            z = _rng(seed, TID_LA, b, h).standard_normal((T, dk), dtype=np.float32)
            la[b, :, h] = (-_softplus(z - shift)).astype(np.float32)
            zb = _rng(seed, TID_BETA, b, h).standard_normal((T,), dtype=np.float32)
            beta[b, :, h] = (1.0 / (1.0 + np.exp(-zb.astype(np.float64)))).astype(np.float32)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta)


def np_state(B: int, H: int, dk: int, dv: int, std: float, seed: int = 0) -> np.ndarray:
    s = np.empty((B, H, dk, dv), np.float32)
    for b in range(B):
        for h in range(H):
            s[b, h] = std * _rng(seed, TID_S0, b, h).standard_normal((dk, dv), dtype=np.float32)
    return s


def np_raw_x(B: int, T: int, D: int, dtype: str, seed: int, tid: int) -> np.ndarray:
    """Raw pre-convolution activations [B,T,D], N(0,1)."""
    x = np.empty((B, T, D), np.float32)
    for b in range(B):
        x[b] = to_storage(_rng(seed, tid, b).standard_normal((T, D), dtype=np.float32), dtype)
    return x


def np_conv_weight(D: int, W: int = 4, seed: int = 0, tid: int = TID_CONVW) -> np.ndarray:
    """Depthwise taps [D,W] ~ U(-1/2, 1/2) (default fan-in-4 init bound 1/sqrt(4))."""
    return _rng(seed, tid).uniform(-0.5, 0.5, (D, W)).astype(np.float32)


def np_conv_cache(B: int, W: int, D: int, dtype: str, seed: int = 0, tid: int = TID_CACHE) -> np.ndarray:
    c = np.empty((B, W - 1, D), np.float32)
    for b in range(B):
        c[b] = to_storage(_rng(seed, tid, b).standard_normal((W - 1, D), dtype=np.float32), dtype)
    return c


def padded_layout(lengths, Tpad: int, sides) -> np.ndarray:
    """0/1 mask [B,Tpad] with ``lengths[b]`` valid positions packed left ('right' padding)
    or right ('left' padding)."""
    m = np.zeros((len(lengths), Tpad), np.uint8)
    for b, (n, s) in enumerate(zip(lengths, sides)):
        if s == "left":
            m[b, Tpad - n:] = 1
        else:
            m[b, :n] = 1
    return m


def continuation_lengths(n_seq: int, seed: int = 0, prefix_max: int = 8192,
                         cont_min: int = 3, cont_max: int = 512):
    """Cached-prefix lengths U{1..prefix_max} and continuation lengths U{cont_min..cont_max};
    even sequences are left-padded, odd ones right-padded."""
    r = _rng(seed, TID_LEN)
    prefix = r.integers(1, prefix_max + 1, n_seq)
    cont = r.integers(cont_min, cont_max + 1, n_seq)
    sides = ["left" if b % 2 == 0 else "right" for b in range(n_seq)]
    return [int(x) for x in prefix], [int(x) for x in cont], sides


# ---------------------------------------------------------------- torch (device) generator

def torch_kda_inputs(B: int, T: int, H: int, dk: int, dv: int, device, dtype: str = "bf16",
                     seed: int = 0, decay: str = "default"):
    """Same recipe as ``np_kda_inputs`` drawn with torch's generator on ``device``
    (values differ from the NumPy streams; used where host generation is too slow)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    shift = {"default": 0.0, "slow": 5.0}[decay]

    def unit(x):
        return x / x.double().pow(2).sum(-1, keepdim=True).sqrt().clamp_min(1e-30).float()

    q = unit(torch.randn(B, T, H, dk, device=device, generator=g)).to(tdt)
    k = unit(torch.randn(B, T, H, dk, device=device, generator=g)).to(tdt)
    v = torch.randn(B, T, H, dv, device=device, generator=g).to(tdt)
    la = -torch.nn.functional.softplus(torch.randn(B, T, H, dk, device=device, generator=g) - shift)
    beta = torch.sigmoid(torch.randn(B, T, H, device=device, generator=g))
    return dict(q=q, k=k, v=v, log_alpha=la.contiguous(), beta=beta.contiguous())
