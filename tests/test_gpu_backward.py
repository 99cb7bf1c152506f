"""GPU parity of kda_chunk_prefill_backward (through the C ABI) against the oracle's fp64
gradient np_prefill_backward, itself pinned by finite differences on the CPU.

Bar, per gradient: the forward's bars applied relative to the gradient's scale
(max(1, max|ref|)), since gradients are not O(1): bf16 inputs rel-L2 <= 5e-3 and
max-abs <= 2e-2 * scale; fp32 inputs rel-L2 <= 1e-4 and max-abs <= 1e-4 * scale."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import device, host, metrics, say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinit_state")
TOL_G = {"bf16": (5e-3, 2e-2), "fp32": (1e-4, 1e-4)}     # (rel-L2, max-abs per unit scale)


def _check(tag, got, ref, dtype):
    REL, ABS = TOL_G[dtype]
    for n in NAMES:
        g, r = host(got[n]), np.asarray(ref[n], np.float64)
        assert g.shape == r.shape, f"{tag} {n}: shape {g.shape} vs {r.shape}"
        max_abs, rel = metrics(g, r)
        scale = max(1.0, float(np.max(np.abs(r), initial=0.0)))
        say(f"[parity] {tag} {n}: max_abs={max_abs:.3e} (scale {scale:.2e}) rel_l2={rel:.3e}")
        assert np.all(np.isfinite(g)), f"{tag} {n}: non-finite values"
        assert max_abs <= ABS * scale, f"{tag} {n}: max_abs {max_abs:.3e} > {ABS * scale:.3e}"
        assert rel <= REL, f"{tag} {n}: rel_l2 {rel:.3e} > {REL}"


def _cotangents(B, T, H, dk, dv, dtype, seed, with_final=True):
    rng = np.random.default_rng(1000 + seed)
    do = D.to_storage(rng.normal(0, 1, (B, T, H, dv)).astype(np.float32), dtype)
    dfinal = rng.normal(0, 1, (B, H, dk, dv)).astype(np.float32) if with_final else None
    return do, dfinal


def _run(inp, do, dfinal, dtype, dev, mask=None, s0=None):
    from linear_attention_recurrence_kda_amd import kda
    return kda.chunk_prefill_backward(
        to_dev(inp["q"], dtype, dev), to_dev(inp["k"], dtype, dev), to_dev(inp["v"], dtype, dev),
        to_dev(inp["log_alpha"], dev=dev), to_dev(inp["beta"], dev=dev), to_dev(do, dtype, dev),
        d_final_state=None if dfinal is None else to_dev(dfinal, dev=dev),
        mask=None if mask is None else to_dev(mask, dev=dev),
        initial_state=None if s0 is None else to_dev(s0, dev=dev))


def _ref(oracle, inp, do, dfinal, mask=None, s0=None, l2=False):
    return oracle.np_prefill_backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do,
                                      dfinal, mask=mask, init_state=s0, l2norm_qk=l2)


def test_backward_tiny_fp32(oracle):
    """B=1, H=2, T=64, dk=dv=16, fp32, zero initial state, no final-state cotangent."""
    dev = device()
    say("[case] backward tiny fp32")
    inp = D.np_kda_inputs(1, 64, 2, 16, 16, "fp32", seed=0)
    do, _ = _cotangents(1, 64, 2, 16, 16, "fp32", 0, with_final=False)
    _check("tiny", _run(inp, do, None, "fp32", dev), _ref(oracle, inp, do, None), "fp32")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_masked_with_state(oracle, dtype):
    """T=300 (18 full 16-token segments and a 12-token tail), masks at the start, middle and end."""
    dev = device()
    B, T, H, dk, dv = 2, 300, 3, 128, 128
    say(f"[case] backward {dtype} T={T} masked+state+dfinal")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=1)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=1)
    mask = np.ones((B, T), np.uint8)
    mask[0, :37] = 0
    mask[1, 250:] = 0
    mask[1, 100:103] = 0
    do, dfinal = _cotangents(B, T, H, dk, dv, dtype, 1)
    got = _run(inp, do, dfinal, dtype, dev, mask, s0)
    _check(f"masked {dtype}", got, _ref(oracle, inp, do, dfinal, mask, s0), dtype)
    for n in ("dq", "dk", "dv", "dlog_alpha"):
        assert np.all(host(got[n])[mask == 0] == 0.0), f"{n} nonzero at a masked position"
    assert np.all(host(got["dbeta"])[mask == 0] == 0.0)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (64, 64), (128, 32), (16, 64), (128, 16)])
def test_backward_head_sizes(oracle, dk, dv):
    dev = device()
    B, T, H = 2, 137, 2
    say(f"[case] backward bf16 dk={dk} dv={dv}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=2)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=2)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 2)
    _check(f"dk{dk} dv{dv}", _run(inp, do, dfinal, "bf16", dev, s0=s0), _ref(oracle, inp, do, dfinal, s0=s0), "bf16")


@pytest.mark.parametrize("T", [0, 1, 17, 63, 64, 65, 130])
def test_backward_short_sequences(oracle, T):
    """No token (dinit = dfinal), one token, and lengths around one and two 64-token chunks."""
    dev = device()
    B, H, dk, dv = 1, 2, 64, 64
    say(f"[case] backward T={T}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "fp32", seed=3)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=3)
    do, dfinal = _cotangents(B, T, H, dk, dv, "fp32", 3)
    got = _run(inp, do, dfinal, "fp32", dev, s0=s0)
    _check(f"T{T}", got, _ref(oracle, inp, do, dfinal, s0=s0), "fp32")
    if T == 0:
        assert np.array_equal(host(got["dinit_state"]), dfinal.astype(np.float64))


def test_backward_all_masked_passes_dfinal_through(oracle):
    dev = device()
    B, T, H, dk, dv = 2, 40, 2, 32, 32
    say("[case] backward all masked")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=4)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 4)
    mask = np.zeros((B, T), np.uint8)
    got = _run(inp, do, dfinal, "bf16", dev, mask)
    for n in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        assert np.all(host(got[n]) == 0.0), n
    assert np.array_equal(host(got["dinit_state"]), dfinal.astype(np.float64))


def test_backward_is_deterministic():
    dev = device()
    say("[case] backward determinism")
    inp = D.np_kda_inputs(1, 100, 4, 128, 128, "bf16", seed=5)
    do, dfinal = _cotangents(1, 100, 4, 128, 128, "bf16", 5)
    a = _run(inp, do, dfinal, "bf16", dev)
    b = _run(inp, do, dfinal, "bf16", dev)
    for n in NAMES:
        assert np.array_equal(host(a[n]), host(b[n])), n


def test_backward_training_size_sampled_heads(oracle):
    """B=4, H=32, T=4096, dk=dv=128, bf16 (the chunked-prefill shape): the whole batch on
    the GPU, three (b, h) heads checked against the oracle run on those heads alone (the
    recurrence of one head does not see the others)."""
    dev = device()
    B, T, H, dk, dv = 4, 4096, 32, 128, 128
    say(f"[case] backward bf16 B={B} T={T} H={H} sampled heads")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=6)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 6)
    got = _run(inp, do, dfinal, "bf16", dev)
    for b, h in ((0, 0), (2, 17), (3, 31)):
        one = {n: x[b:b + 1, :, h:h + 1] for n, x in inp.items()}
        ref = _ref(oracle, one, do[b:b + 1, :, h:h + 1], dfinal[b:b + 1, h:h + 1])
        sub = {n: (got[n][b:b + 1, h:h + 1] if n == "dinit_state" else got[n][b:b + 1, :, h:h + 1])
               for n in NAMES}
        _check(f"full b{b} h{h}", sub, ref, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_extreme_decay_chunks(oracle, dtype):
    """Chunks in which some channels decay below 2^-120 (log_alpha = -3 over 64 tokens) take
    the entry-by-entry path; the chunks around them stay on the factorised one."""
    dev = device()
    B, T, H, dk, dv = 1, 200, 2, 64, 64
    say(f"[case] backward {dtype} extreme decay")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=7)
    inp["log_alpha"][:, 64:128, 0, :5] = -3.0
    inp["log_alpha"][:, 140:, 1, 40:] = -6.0
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=7)
    do, dfinal = _cotangents(B, T, H, dk, dv, dtype, 7)
    _check(f"extreme {dtype}", _run(inp, do, dfinal, dtype, dev, s0=s0), _ref(oracle, inp, do, dfinal, s0=s0), dtype)


def test_backward_slow_gates(oracle):
    """Slow gates (log_alpha = -softplus(z - 5), per-token decay about 0.993): the state keeps
    hundreds of tokens, the regime where rounding in the reverse scan accumulates most."""
    dev = device()
    B, T, H, dk, dv = 1, 1024, 2, 128, 128
    say("[case] backward bf16 slow gates")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=8, decay="slow")
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 8)
    _check("slow gates", _run(inp, do, dfinal, "bf16", dev), _ref(oracle, inp, do, dfinal), "bf16")


def test_backward_wide_scan_tiles_equal_narrow():
    """With 64 or more (b, h) pairs and bf16 the reverse scan takes 32 dv columns per
    workgroup; every column sees the same operations in the same order as with 16, so
    one call over 64 pairs equals two calls over 32 pairs each, bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 2, 200, 32, 128, 128
    say("[case] backward wide vs narrow scan tiles")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=9)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 9)
    mask = np.ones((B, T), np.uint8)
    mask[1, 150:] = 0
    full = _run(inp, do, dfinal, "bf16", dev, mask)
    for b in range(B):
        one = {n: x[b:b + 1] for n, x in inp.items()}
        part = _run(one, do[b:b + 1], dfinal[b:b + 1], "bf16", dev, mask[b:b + 1])
        for n in NAMES:
            got = full[n][b:b + 1]
            assert torch.equal(got, part[n]), f"{n} differs for batch row {b}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_scalar_gate_equals_broadcast(dtype):
    """KDA_FLAG_SCALAR_GATE (one gate per token and head), fed the chunk-end states of the
    per-head training forward: dq, dk, dv, dbeta and dinit equal those of the per-channel call
    fed the broadcast gate and the same states bit for bit, and the gate's gradient is that
    call's per-channel dlog_alpha summed over the channels.  Without the states the call runs
    the per-head forward itself and gives the same gradients bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 2, 200, 3, 64, 128
    say(f"[case] backward scalar gate = broadcast gate, {dtype}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=11)
    la1 = np.ascontiguousarray(inp["log_alpha"][..., 0])
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=11)
    mask = np.ones((B, T), np.uint8)
    mask[1, :30] = 0
    do, dfinal = _cotangents(B, T, H, dk, dv, dtype, 11)
    q, k, v = (to_dev(inp[n], dtype, dev) for n in ("q", "k", "v"))
    beta, dm, ds0 = to_dev(inp["beta"], dev=dev), to_dev(mask, dev=dev), to_dev(s0, dev=dev)
    ddo, dfin = to_dev(do, dtype, dev), to_dev(dfinal, dev=dev)
    la_s = to_dev(la1, dev=dev)
    la_b = la_s.unsqueeze(-1).expand(B, T, H, dk).contiguous()
    _, _, ck = kda.chunk_prefill_states(q, k, v, la_s, beta, mask=dm, initial_state=ds0, chunk_size=64,
                                        state_interval=64, scalar_gate=True)
    got = kda.chunk_prefill_backward(q, k, v, la_s, beta, ddo, d_final_state=dfin, mask=dm, initial_state=ds0,
                                     chunk_states=ck, scalar_gate=True)
    rec = kda.chunk_prefill_backward(q, k, v, la_s, beta, ddo, d_final_state=dfin, mask=dm, initial_state=ds0,
                                     scalar_gate=True)
    ref = kda.chunk_prefill_backward(q, k, v, la_b, beta, ddo, d_final_state=dfin, mask=dm, initial_state=ds0,
                                     chunk_states=ck)
    torch.cuda.synchronize()
    for n in got:
        assert torch.equal(got[n], rec[n]), f"given states vs recompute: {n}"
    for n in ("dq", "dk", "dv", "dbeta", "dinit_state"):
        assert torch.equal(got[n], ref[n]), n
    assert got["dlog_alpha"].shape == (B, T, H)
    summed = ref["dlog_alpha"].double().sum(-1)
    err = (got["dlog_alpha"].double() - summed).abs().max().item()
    assert err <= 1e-5 * max(1.0, summed.abs().max().item()), err
    assert torch.all(got["dlog_alpha"][1, :30] == 0)


def test_backward_scalar_gate_vs_oracle(oracle):
    """The per-head gate's gradients against the oracle's gradient with the gate broadcast to
    every channel (its dlog_alpha summed over the channels: the chain rule through the
    broadcast), with the states of a scalar-gate training forward handed in."""
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 1, 300, 2, 128, 128
    say("[case] backward scalar gate vs oracle")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=12)
    la1 = np.ascontiguousarray(inp["log_alpha"][..., 0])
    one = dict(inp, log_alpha=np.ascontiguousarray(np.broadcast_to(la1[..., None], inp["log_alpha"].shape)))
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=12)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 12)
    q, k, v = (to_dev(inp[n], "bf16", dev) for n in ("q", "k", "v"))
    la_s, beta, ds0 = to_dev(la1, dev=dev), to_dev(inp["beta"], dev=dev), to_dev(s0, dev=dev)
    _, _, ck = kda.chunk_prefill_states(q, k, v, la_s, beta, initial_state=ds0, state_interval=64, scalar_gate=True)
    got = kda.chunk_prefill_backward(q, k, v, la_s, beta, to_dev(do, "bf16", dev), d_final_state=to_dev(dfinal, dev=dev),
                                     initial_state=ds0, chunk_states=ck, scalar_gate=True)
    ref = _ref(oracle, one, do, dfinal, s0=s0)
    ref = dict(ref, dlog_alpha=np.asarray(ref["dlog_alpha"]).sum(-1))
    _check("scalar gate", got, ref, "bf16")


def test_backward_128k_sampled_head(oracle):
    """One 131072-token sequence (2048 chunk steps of the reverse scan), bf16, 2 heads on the
    GPU; head 1 against the oracle's fp64 gradient over the whole sequence."""
    dev = device()
    B, T, H, dk, dv = 1, 131072, 2, 128, 128
    say(f"[case] backward bf16 T={T} sampled head")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=13)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 13)
    got = _run(inp, do, dfinal, "bf16", dev)
    h = 1
    one = {n: x[:, :, h:h + 1] for n, x in inp.items()}
    ref = _ref(oracle, one, do[:, :, h:h + 1], dfinal[:, h:h + 1])
    sub = {n: (got[n][:, h:h + 1] if n == "dinit_state" else got[n][:, :, h:h + 1]) for n in NAMES}
    _check(f"128k h{h}", sub, ref, "bf16")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("fp32", 64, 32), ("bf16", 16, 64)])
def test_backward_l2norm_vs_oracle(oracle, dtype, dk, dv):
    """With the q/k L2-norm flag the call differentiates the prefill that normalises q and k
    itself: raw N(0,1) rows (norms near sqrt(dk)), masks, an initial state and a final-state
    cotangent, against the oracle's gradient with the norm.  NaN in q and k at masked
    positions gives the same gradients as zeros there, bit for bit, and zero gradients."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H = 2, 300, 2
    say(f"[case] backward l2 norm {dtype} dk={dk} dv={dv}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=61, unit_qk=False)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=61)
    mask = np.ones((B, T), np.uint8)
    mask[0, :21] = 0
    mask[1, 150:170] = 0
    do, dfinal = _cotangents(B, T, H, dk, dv, dtype, 61)
    zeroed = {n: x.copy() for n, x in inp.items()}
    for n in ("q", "k"):
        zeroed[n][mask == 0] = 0.0
    ref = _ref(oracle, zeroed, do, dfinal, mask, s0, l2=True)

    def run(src):
        return kda.chunk_prefill_backward(
            *(to_dev(src[n], dtype if n in "qkv" else None, dev) for n in ("q", "k", "v", "log_alpha", "beta")),
            to_dev(do, dtype, dev), d_final_state=to_dev(dfinal, dev=dev), mask=to_dev(mask, dev=dev),
            initial_state=to_dev(s0, dev=dev), l2norm_qk=True)
    got = run(zeroed)
    _check(f"l2 {dtype}", got, ref, dtype)
    poisoned = {n: x.copy() for n, x in zeroed.items()}
    for n in ("q", "k"):
        poisoned[n][mask == 0] = np.nan
    bad = run(poisoned)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(bad[n], got[n]), f"NaN at masked positions changed {n}"
    for n in ("dq", "dk"):
        assert np.all(host(got[n])[mask == 0] == 0.0), n


def test_backward_l2norm_given_states_equals_recompute():
    """States saved by kda_chunk_prefill_states with the L2-norm flag, handed to the backward
    with the flag, give the gradients of the call that runs that forward again, bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 2, 260, 3, 128, 128
    say("[case] backward l2 norm, given states vs recompute")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=62, unit_qk=False)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 62)
    args = tuple(to_dev(inp[n], "bf16" if n in "qkv" else None, dev) for n in ("q", "k", "v", "log_alpha", "beta"))
    ddo, dfin = to_dev(do, "bf16", dev), to_dev(dfinal, dev=dev)
    _, _, ck = kda.chunk_prefill_states(*args, chunk_size=64, state_interval=64, l2norm_qk=True)
    got = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin, chunk_states=ck, l2norm_qk=True)
    ref = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin, l2norm_qk=True)
    plain = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(got[n], ref[n]), n
    # the flag matters for rows that are not unit-norm
    assert not torch.equal(got["dq"], plain["dq"])
