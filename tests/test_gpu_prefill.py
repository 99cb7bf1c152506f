"""GPU parity and invariance tests of kda_chunk_prefill (through the C ABI)."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _dev_inputs(inp, dtype, dev):
    return dict(q=to_dev(inp["q"], dtype, dev), k=to_dev(inp["k"], dtype, dev),
                v=to_dev(inp["v"], dtype, dev), log_alpha=to_dev(inp["log_alpha"], dev=dev),
                beta=to_dev(inp["beta"], dev=dev))


def _run(inp, dtype, dev, chunk, mask=None, s0=None, l2norm=False):
    from linear_attention_recurrence_kda_amd import kda
    d = _dev_inputs(inp, dtype, dev)
    o, s = kda.chunk_prefill(**d, mask=None if mask is None else to_dev(mask, dev=dev),
                             initial_state=None if s0 is None else to_dev(s0, dev=dev),
                             chunk_size=chunk, l2norm_qk=l2norm)
    return o, s


def test_tiny_fp32_config(oracle):
    """B=1, H=2, T=64, dk=dv=16, fp32, chunk 16, zero initial state, seed 0."""
    dev = device()
    say("[case] prefill tiny fp32")
    inp = D.np_kda_inputs(1, 64, 2, 16, 16, "fp32", seed=0)
    o, s = _run(inp, "fp32", dev, 16)
    ro, rs = oracle.c_prefill(**inp)
    check("tiny o", host(o), ro, "fp32")
    check("tiny state", host(s), rs, "fp32")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_masked_with_state(oracle, chunk, dtype):
    dev = device()
    B, T, H, dk, dv = 2, 300, 3, 128, 128
    say(f"[case] prefill {dtype} chunk={chunk} T={T} masked+state")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=1)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=1)
    mask = np.ones((B, T), np.uint8)
    mask[0, :37] = 0
    mask[1, 250:] = 0
    mask[1, 100:103] = 0
    o, s = _run(inp, dtype, dev, chunk, mask, s0)
    ro, rs = oracle.c_prefill(**inp, mask=mask, init_state=s0)
    check("masked o", host(o), ro, dtype)
    check("masked state", host(s), rs, dtype)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (64, 64), (128, 32), (16, 64)])
def test_prefill_head_sizes(oracle, dk, dv):
    dev = device()
    B, T, H = 2, 130, 2
    say(f"[case] prefill bf16 dk={dk} dv={dv}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=2)
    s0 = D.np_state(B, H, dk, dv, 0.1, seed=2)
    o, s = _run(inp, "bf16", dev, 64, None, s0)
    ro, rs = oracle.c_prefill(**inp, init_state=s0)
    check(f"dk{dk}dv{dv} o", host(o), ro, "bf16")
    check(f"dk{dk}dv{dv} state", host(s), rs, "bf16")


@pytest.mark.parametrize("T", [1, 64, 65, 128])
def test_prefill_one_or_two_chunks(oracle, T):
    """One or two 64-token chunks: the scan's prologue and its odd/even tails, where the
    next chunk's operands (and the decay/valid slots two chunks ahead) are clamped."""
    dev = device()
    B, H, dk, dv = 2, 3, 128, 128
    say(f"[case] prefill bf16 chunk=64 T={T}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=9)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=9)
    o, s = _run(inp, "bf16", dev, 64, None, s0)
    ro, rs = oracle.c_prefill(**inp, init_state=s0)
    check(f"T{T} o", host(o), ro, "bf16")
    check(f"T{T} state", host(s), rs, "bf16")


@pytest.mark.parametrize("decay", ["slow", "strong"])
def test_prefill_decay_regimes(oracle, decay):
    """Slow gates (state lives for hundreds of tokens) and strong gates (some channels decay
    below 2^-100 within one chunk, which takes the exact pairwise-decay path)."""
    dev = device()
    B, T, H, dk, dv = 1, 256, 2, 128, 128
    say(f"[case] prefill decay={decay}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=3, decay="slow" if decay == "slow" else "default")
    if decay == "strong":
        inp["log_alpha"][0, 70:75, 0, :5] = -40.0
        inp["log_alpha"][0, 140, 1, 7] = -90.0
    o, s = _run(inp, "bf16", dev, 64)
    ro, rs = oracle.c_prefill(**inp)
    check(f"{decay} o", host(o), ro, "bf16")
    check(f"{decay} state", host(s), rs, "bf16")


def test_prefill_l2norm_flag(oracle):
    dev = device()
    B, T, H, dk, dv = 2, 100, 2, 128, 64
    say("[case] prefill l2norm flag")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=4, unit_qk=False)
    o, s = _run(inp, "bf16", dev, 64, l2norm=True)
    ro, rs = oracle.c_prefill(**inp, l2norm_qk=True)
    check("l2norm o", host(o), ro, "bf16")
    check("l2norm state", host(s), rs, "bf16")


def test_prefill_zero_length_copies_state(oracle):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    say("[case] prefill T=0")
    s0 = to_dev(D.np_state(2, 3, 64, 64, 1.0, seed=5), dev=dev)
    e = torch.empty(2, 0, 3, 64, dtype=torch.bfloat16, device=dev)
    o, s = kda.chunk_prefill(e, e, e, torch.empty(2, 0, 3, 64, device=dev), torch.empty(2, 0, 3, device=dev),
                             initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(s, s0)


@pytest.mark.parametrize("p", [63, 64, 65, 191])
def test_prefix_invariance_is_exact(p):
    """dev.to audit page: outputs before the perturbed position must not move at all; the
    sequence (192) is three chunks of 64 so the inter-chunk step is exercised."""
    import torch
    dev = device()
    B, T, H, dk, dv = 1, 192, 2, 128, 128
    say(f"[case] prefix invariance p={p}")
    a = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=6)
    b = {n: x.copy() for n, x in a.items()}
    b["v"][:, p] = D.round_bf16(b["v"][:, p] + 1.0)
    b["k"][:, p] = -b["k"][:, p]
    b["log_alpha"][:, p] *= 0.5
    b["beta"][:, p] = 0.9
    oa, _ = _run(a, "bf16", dev, 64)
    ob, _ = _run(b, "bf16", dev, 64)
    torch.cuda.synchronize()
    assert torch.equal(oa[:, :p], ob[:, :p])
    assert not torch.equal(oa[:, p], ob[:, p])


def test_prefill_is_deterministic():
    import torch
    dev = device()
    say("[case] determinism")
    inp = D.np_kda_inputs(2, 200, 4, 128, 128, "bf16", seed=7)
    o1, s1 = _run(inp, "bf16", dev, 64)
    o2, s2 = _run(inp, "bf16", dev, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_split_and_chunk_invariance(oracle):
    """prefill(T) == prefill(T1) -> prefill(T-T1) == prefill(T1) -> decode steps, and chunk
    sizes 16/32/64 agree (remio.ai page, serving checks: state at chunk boundaries)."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv, T1 = 2, 160, 2, 128, 128, 97
    say("[case] split and chunk invariance")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=8)
    o_full, s_full = _run(inp, "bf16", dev, 64)
    first = {n: x[:, :T1] for n, x in inp.items()}
    rest = {n: x[:, T1:] for n, x in inp.items()}
    o1, s1 = _run(first, "bf16", dev, 64)
    o2, s2 = _run(rest, "bf16", dev, 64, s0=host(s1).astype(np.float32))
    check("split o", np.concatenate([host(o1), host(o2)], 1), host(o_full), "bf16")
    check("split state", host(s2), host(s_full), "bf16")
    st = s1.clone()
    outs = []
    for t in range(T - T1):
        step = _dev_inputs({n: x[:, t] for n, x in rest.items()}, "bf16", dev)
        outs.append(host(kda.decode_step(**step, state=st)))
    check("prefill->decode o", np.stack(outs, 1), host(o2), "bf16")
    check("prefill->decode state", host(st), host(s2), "bf16")
    for c in (16, 32):
        oc, sc = _run(inp, "bf16", dev, c)
        check(f"chunk{c} vs chunk64 o", host(oc), host(o_full), "bf16")
    torch.cuda.synchronize()


def test_needle_across_chunks(oracle):
    """k_0 = e_0, later keys orthogonal to e_0, channel 0 never decays: the last token reads
    beta_0 v_0 exactly, across 16 chunks (remio.ai page, serving section: needle retrieval
    after long prefill; a transposed state layout fails this)."""
    dev = device()
    T, dk, dv = 1024, 128, 128
    say("[case] needle")
    inp = D.np_kda_inputs(1, T, 1, dk, dv, "bf16", seed=9)
    inp["k"][0, :, 0, 0] = 0.0
    inp["k"][0, 0, 0] = 0.0
    inp["k"][0, 0, 0, 0] = 1.0
    inp["log_alpha"][0, :, 0, 0] = 0.0
    inp["q"][0, -1, 0] = 0.0
    inp["q"][0, -1, 0, 0] = 1.0
    o, _ = _run(inp, "bf16", dev, 64)
    want = np.float64(inp["beta"][0, 0, 0]) * inp["v"][0, 0, 0]
    check("needle", host(o)[0, -1, 0], want, "bf16")


def test_chunked_prefill_full_size_sampled(oracle):
    """B=4, H=32, T=4096, dk=dv=128, bf16, chunk 64, zero state: the full workload in the
    benchmark's launch configuration, with sampled heads checked against the oracle."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 4, 4096, 32, 128, 128
    say("[case] prefill full size 4x4096x32, sampled heads")
    x = D.torch_kda_inputs(B, T, H, dk, dv, dev, "bf16", seed=0)
    o, s = kda.chunk_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], chunk_size=64)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (1, 17), (3, 31), (2, 8)]:
        one = {n: host(t[b:b + 1, :, h:h + 1]) for n, t in x.items()}
        ro, rs = oracle.c_prefill(**one)
        check(f"full o b{b}h{h}", host(o[b:b + 1, :, h:h + 1]), ro, "bf16")
        check(f"full state b{b}h{h}", host(s[b:b + 1, h:h + 1]), rs, "bf16")


def test_long_prefill_sampled_heads(oracle):
    """B=1, H=32, T=524288, dk=dv=128, bf16, zero state: the long-prefill workload in one
    call; three heads checked against the oracle over every position and the final state."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 1, 524288, 32, 128, 128
    say("[case] prefill long 1x524288x32, sampled heads")
    x = D.torch_kda_inputs(B, T, H, dk, dv, dev, "bf16", seed=3)
    o, s = kda.chunk_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], chunk_size=64)
    torch.cuda.synchronize()
    heads = [0, 15, 31]
    one = {n: host(t[:, :, heads]) for n, t in x.items()}
    ro, rs = oracle.c_prefill(**one)
    for i, h in enumerate(heads):
        check(f"long o h{h}", host(o[:, :, h]), ro[:, :, i], "bf16")
        check(f"long state h{h}", host(s[:, h]), rs[:, i], "bf16")


@pytest.mark.parametrize("chunk", [64, 32])
def test_wide_scan_tiles_equal_narrow(chunk):
    """With 64 or more (b, h) pairs and dv = 128 in bf16 the scan takes 32 dv columns per
    workgroup instead of 16; every column sees the same operations in the same order, so a
    batch that takes that path equals each of its rows run alone (16-column path) bit for
    bit, padding mask, initial state and L2 norm included."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 4, 300, 16, 128, 128
    say(f"[case] 32-column scan tiles vs 16 chunk={chunk}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=40)
    s0 = D.np_state(B, H, dk, dv, 0.1, seed=40)
    mask = np.ones((B, T), np.uint8)
    mask[1, 250:] = 0
    mask[3, :37] = 0
    o, s = _run(inp, "bf16", dev, chunk, mask=mask, s0=s0, l2norm=True)
    for b in range(B):
        ob, sb = _run({n: x[b:b + 1] for n, x in inp.items()}, "bf16", dev, chunk, mask=mask[b:b + 1],
                      s0=s0[b:b + 1], l2norm=True)
        torch.cuda.synchronize()
        assert torch.equal(o[b:b + 1], ob), f"o of row {b}"
        assert torch.equal(s[b:b + 1], sb), f"state of row {b}"
