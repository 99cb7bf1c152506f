"""Gated DeltaNet's gate (KDA_FLAG_SCALAR_GATE): one log forget gate per (token, head).
It is KDA with that gate on every key channel.  With fp32 rows (and in the decode kernels)
the scalar-gate path runs the per-channel arithmetic on the one value, so it gives bit for
bit what the per-channel path gives for the broadcast gate.  With bf16 rows the prefill
takes its own prep (A and P as Gram products of the raw rows times the scalar decay mask),
which differs from the broadcast path by rounding only; it is held to the fp64 oracle fed
the broadcast gate."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _run(kda, inp, dtype, dev, chunk, la, scalar, mask=None, s0=None, l2=False):
    d = {n: to_dev(inp[n], dtype if n in "qkv" else None, dev) for n in ("q", "k", "v", "beta")}
    return kda.chunk_prefill(d["q"], d["k"], d["v"], to_dev(la, dev=dev), d["beta"],
                             mask=None if mask is None else to_dev(mask, dev=dev),
                             initial_state=None if s0 is None else to_dev(s0, dev=dev),
                             chunk_size=chunk, scalar_gate=scalar, l2norm_qk=l2)


@pytest.mark.parametrize("dtype,chunk,decay,dk,l2", [("bf16", 64, "default", 128, False),
                                                     ("fp32", 32, "default", 128, False),
                                                     ("fp32", 64, "strong", 64, True),
                                                     ("bf16", 64, "strong", 128, False),
                                                     ("bf16", 32, "default", 16, True),
                                                     ("bf16", 16, "strong", 64, True)])
def test_prefill_scalar_gate_vs_broadcast(oracle, dtype, chunk, decay, dk, l2):
    """Masks, an initial state, head sizes down to 16, the q/k norm, and chunks whose decay
    passes 2^-120 (where the per-channel path takes its exact pairwise branch): fp32 bit for
    bit equal to the broadcast gate; both paths within the bar of the oracle."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dv = 2, 203, 3, 64
    say(f"[case] prefill scalar gate {dtype} chunk={chunk} decay={decay} dk={dk} l2={l2}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=21, unit_qk=not l2)
    g = np.ascontiguousarray(inp["log_alpha"][..., 0])                       # [B,T,H]
    if decay == "strong":
        g[:, 70:74] = -40.0
    gb = np.ascontiguousarray(np.repeat(g[..., None], dk, axis=-1))          # [B,T,H,dk]
    s0 = D.np_state(B, H, dk, dv, 0.1, seed=21)
    mask = np.ones((B, T), np.uint8)
    mask[1, 150:] = 0
    mask[0, :5] = 0
    o1, s1 = _run(kda, inp, dtype, dev, chunk, g, True, mask, s0, l2)
    o2, s2 = _run(kda, inp, dtype, dev, chunk, gb, False, mask, s0, l2)
    torch.cuda.synchronize()
    if dtype == "fp32":
        assert torch.equal(o1, o2)
        assert torch.equal(s1, s2)
    else:                                   # the per-head prep ran (other roundings)
        assert not torch.equal(s1, s2)
    ref = dict(inp)
    ref["log_alpha"] = gb
    ro, rs = oracle.c_prefill(**ref, mask=mask, init_state=s0, l2norm_qk=l2)
    check(f"gate per head o ({dtype})", host(o1), ro, dtype)
    check(f"gate per head state ({dtype})", host(s1), rs, dtype)
    check(f"broadcast gate o ({dtype})", host(o2), ro, dtype)
    check(f"broadcast gate state ({dtype})", host(s2), rs, dtype)


def test_prefill_scalar_gate_matches_oracle(oracle):
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 1, 300, 2, 64, 128
    say("[case] prefill scalar gate vs oracle")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=22)
    g = np.ascontiguousarray(inp["log_alpha"][..., 0])
    o, s = _run(kda, inp, "bf16", dev, 64, g, True)
    ref = dict(inp)
    ref["log_alpha"] = np.repeat(g[..., None], dk, axis=-1)
    ro, rs = oracle.c_prefill(**ref)
    check("gdn o", host(o), ro, "bf16")
    check("gdn state", host(s), rs, "bf16")


def test_decode_scalar_gate_equals_broadcast():
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv = 3, 4, 128, 128
    say("[case] decode and fused decode, scalar gate")
    g = D.np_kda_inputs(B, 1, H, dk, dv, "bf16", seed=23)
    inp = {n: np.ascontiguousarray(x[:, 0]) for n, x in g.items()}
    gs = np.ascontiguousarray(inp["log_alpha"][..., 0])                      # [B,H]
    gb = np.ascontiguousarray(np.repeat(gs[..., None], dk, axis=-1))
    s0 = to_dev(D.np_state(B, H, dk, dv, 0.2, seed=23), dev=dev)
    qkv = [to_dev(inp[n], "bf16", dev) for n in ("q", "k", "v")]
    beta = to_dev(inp["beta"], dev=dev)
    st1, st2 = s0.clone(), s0.clone()
    o1 = kda.decode_step(*qkv, to_dev(gs, dev=dev), beta, st1, l2norm_qk=True, scalar_gate=True)
    o2 = kda.decode_step(*qkv, to_dev(gb, dev=dev), beta, st2, l2norm_qk=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)
    # the fused step: raw inputs through the convolutions, same gate check
    W = 4
    x = {n: to_dev(D.np_raw_x(B, 1, H * d, "bf16", 23, t)[:, 0], "bf16", dev)
         for n, d, t in (("q", dk, D.TID_XQ), ("k", dk, D.TID_XK), ("v", dv, D.TID_XV))}
    w = {n: to_dev(D.np_conv_weight(H * d, W, seed=i), dev=dev) for i, (n, d) in enumerate((("q", dk), ("k", dk), ("v", dv)))}
    c1 = {n: to_dev(D.np_conv_cache(B, W, H * d, "bf16", seed=i), "bf16", dev)
          for i, (n, d) in enumerate((("q", dk), ("k", dk), ("v", dv)))}
    c2 = {n: c1[n].clone() for n in c1}
    st1, st2 = s0.clone(), s0.clone()
    f1 = kda.decode_step_fused(x["q"], x["k"], x["v"], w["q"], w["k"], w["v"], c1["q"], c1["k"], c1["v"],
                               to_dev(gs, dev=dev), beta, st1, H, l2norm_qk=True, scalar_gate=True)
    f2 = kda.decode_step_fused(x["q"], x["k"], x["v"], w["q"], w["k"], w["v"], c2["q"], c2["k"], c2["v"],
                               to_dev(gb, dev=dev), beta, st2, H, l2norm_qk=True)
    torch.cuda.synchronize()
    assert torch.equal(f1, f2) and torch.equal(st1, st2)
