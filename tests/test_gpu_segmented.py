"""GPU tests of the segmented scan of kda_chunk_prefill (through the C ABI).

With bf16 inputs, dv = 128, fewer than 64 (b, h) pairs and at least 128 chunks, the call
cuts each head's sequence into G segments scanned side by side; the state entering segment g
is the run from a zero state over a tail of chunks whose per-token contraction bounds
multiply to at most 2^-160, and a head with a boundary lacking such a tail is scanned as one
chain.  The tests check the results against the fp64 oracle (every position, final state),
the fallback bit for bit against KDA_FLAG_SERIAL_SCAN, and which heads were segmented by
reading the plan the call leaves at the end of its workspace.
"""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu

DK = DV = 128


def _segments(nbh, NC):
    """The segment count the library chooses (mirrors its rule: double while there are
    fewer than 64 chains and every segment keeps at least 64 chunks)."""
    G = 1
    while nbh * G < 64 and NC // (2 * G) >= 64:
        G *= 2
    return G


def _run(inp, dev, mask=None, s0=None, l2norm=False, serial=False, scalar_gate=False, inplace=False):
    """Returns (o, final_state, plan or None): the plan is read from the workspace tail."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    B, T, H, _ = inp["q"].shape
    d = dict(q=to_dev(inp["q"], "bf16", dev), k=to_dev(inp["k"], "bf16", dev), v=to_dev(inp["v"], "bf16", dev),
             log_alpha=to_dev(inp["log_alpha"], dev=dev), beta=to_dev(inp["beta"], dev=dev))
    need = kda.prefill_workspace_size(B, T, H, DK, DV, 64, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    init = None if s0 is None else to_dev(s0, dev=dev)
    fin = init if inplace else None
    o, s = kda.chunk_prefill(**d, mask=None if mask is None else to_dev(mask, dev=dev), initial_state=init,
                             chunk_size=64, l2norm_qk=l2norm, workspace=ws, scalar_gate=scalar_gate,
                             serial_scan=serial, final_state=fin)
    torch.cuda.synchronize()
    G = _segments(B * H, (T + 63) // 64)
    plan = None
    if G > 1 and not serial:
        plan = ws[need - B * H * G * 4:need].view(torch.int32).cpu().numpy().reshape(B * H, G)
    return o, s, plan


def _check_all(name, o, s, ro, rs):
    check(f"{name} o", host(o), ro, "bf16")
    check(f"{name} state", host(s), rs, "bf16")


@pytest.mark.parametrize("T", [8192, 16384 + 37])
def test_segmented_fast_gates_vs_oracle(oracle, T):
    """Default gates forget within a few chunks: every head is segmented (G = 2 at 8192
    tokens, 4 at 16421 with two heads); o at every position and the final state against the
    oracle, and against the single-chain call within the same bar."""
    dev = device()
    B, H = 1, 2
    say(f"[case] segmented fast gates T={T}")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=51)
    s0 = D.np_state(B, H, DK, DV, 0.1, seed=51)
    o, s, plan = _run(inp, dev, s0=s0)
    assert plan is not None and plan.shape[1] == _segments(B * H, (T + 63) // 64)
    say(f"[plan] {plan.tolist()}")
    assert np.all(plan[:, 0] == 1), "every head should be segmented"
    G = plan.shape[1]
    seg_nc = -(-((T + 63) // 64) // G)
    for g in range(1, G):
        assert np.all((plan[:, g] >= (g - 1) * seg_nc) & (plan[:, g] < g * seg_nc)), "tail inside the segment before"
    ro, rs = oracle.c_prefill(**inp, init_state=s0)
    _check_all("segmented", o, s, ro, rs)
    os_, ss, _ = _run(inp, dev, s0=s0, serial=True)
    _check_all("serial", os_, ss, ro, rs)


def test_segmented_slow_gates_fall_back_bitwise():
    """Slow gates (the state lives for thousands of tokens): no boundary has a forgetting
    tail, so every head runs as one chain, bit for bit the KDA_FLAG_SERIAL_SCAN call."""
    import torch
    dev = device()
    B, T, H = 1, 8192 + 5, 3
    say("[case] segmented slow gates fall back")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=52, decay="slow")
    s0 = D.np_state(B, H, DK, DV, 0.1, seed=52)
    o, s, plan = _run(inp, dev, s0=s0)
    assert plan is not None and np.all(plan[:, 0] == 0), f"no head should be segmented: {plan[:, 0]}"
    os_, ss, _ = _run(inp, dev, s0=s0, serial=True)
    assert torch.equal(o, os_) and torch.equal(s, ss)


def test_segmented_mixed_heads(oracle):
    """Heads 0 and 2 forget fast, head 1 has one slow channel: heads 0 and 2 are segmented,
    head 1 runs as one chain and equals its single-chain run bit for bit; all three against
    the oracle, with a padding mask (left padding and a hole) and an initial state."""
    import torch
    dev = device()
    B, T, H = 1, 8192 + 100, 3
    say("[case] segmented mixed heads")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=53)
    inp["log_alpha"][0, :, 1, 5] = -1e-4                  # one channel that almost never decays
    mask = np.ones((B, T), np.uint8)
    mask[0, :300] = 0
    mask[0, 5000:5400] = 0
    s0 = D.np_state(B, H, DK, DV, 0.1, seed=53)
    o, s, plan = _run(inp, dev, mask=mask, s0=s0)
    assert plan[:, 0].tolist() == [1, 0, 1], plan[:, 0]
    os_, ss, _ = _run(inp, dev, mask=mask, s0=s0, serial=True)
    assert torch.equal(o[:, :, 1], os_[:, :, 1]) and torch.equal(s[:, 1], ss[:, 1])
    assert torch.all(o[0, :300] == 0) and torch.all(o[0, 5000:5400] == 0), "masked positions give o = 0"
    ro, rs = oracle.c_prefill(**inp, mask=mask, init_state=s0)
    _check_all("mixed", o, s, ro, rs)


def _poison(a, m):
    """Copy of a with NaN / +Inf / -Inf cycling over the masked positions (mask m [B,T])."""
    out = a.copy()
    bad = np.array([np.nan, np.inf, -np.inf], np.float32)
    for i, (b, t) in enumerate(np.argwhere(m == 0)):
        out[b, t] = bad[i % 3]
    return out


def test_segmented_masked_garbage_and_padding(oracle):
    """Masked positions never enter the contraction bound or the scan: with NaN, +Inf and
    -Inf at every masked position of q, k, v, log_alpha and beta (left padding, a hole across
    the segment boundary and its tail, right padding) the segmented call equals, bit for bit,
    the call with zeros there, which is checked against the oracle.  A masked run counts as
    the identity in the bound, so padding longer than the first segment leaves the boundary
    without a forgetting tail (the state entering it is the initial state, not forgotten):
    that head must fall back to one chain, bit for bit the serial call."""
    import torch
    dev = device()
    B, T, H = 1, 8192 + 77, 2
    NC = (T + 63) // 64
    seg_nc = -(-NC // _segments(B * H, NC))
    say("[case] segmented masked garbage")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=56)
    s0 = D.np_state(B, H, DK, DV, 0.1, seed=56)
    mask = np.ones((B, T), np.uint8)
    mask[0, :200] = 0
    mask[0, 64 * seg_nc - 700:64 * seg_nc + 300] = 0       # over the boundary and its tail
    mask[0, T - 150:] = 0
    zero = {n: a.copy() for n, a in inp.items()}
    for a in zero.values():
        a[mask == 0] = 0.0
    bad = {n: _poison(a, mask) for n, a in inp.items()}
    oz, sz, pz = _run(zero, dev, mask=mask, s0=s0)
    ob, sb, pb = _run(bad, dev, mask=mask, s0=s0)
    assert np.all(pz[:, 0] == 1) and np.array_equal(pz, pb), (pz.tolist(), pb.tolist())
    assert torch.equal(oz, ob) and torch.equal(sz, sb), "masked NaN/Inf changed the segmented result"
    ro, rs = oracle.c_prefill(**zero, mask=mask, init_state=s0)
    _check_all("masked garbage", oz, sz, ro, rs)

    say("[case] segmented padding past the first segment falls back")
    mask2 = np.ones((B, T), np.uint8)
    mask2[0, :64 * seg_nc + 10] = 0
    bad2 = {n: _poison(a, mask2) for n, a in inp.items()}
    o2, s2, p2 = _run(bad2, dev, mask=mask2, s0=s0)
    assert np.all(p2[:, 0] == 0), p2.tolist()
    os2, ss2, _ = _run(bad2, dev, mask=mask2, s0=s0, serial=True)
    assert torch.equal(o2, os2) and torch.equal(s2, ss2)
    assert torch.all(o2[0, :64 * seg_nc + 10] == 0)


def test_segmented_flags_and_inplace(oracle):
    """The q/k L2-norm flag on raw rows and the per-head gate, each with the final state
    written over the initial state (the plan kernel copies it before pass 2 overwrites it),
    and a ragged tail; against the oracle."""
    dev = device()
    B, T, H = 1, 8192 + 63, 2
    s0 = D.np_state(B, H, DK, DV, 0.1, seed=54)
    say("[case] segmented l2norm in place")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=54, unit_qk=False)
    o, s, plan = _run(inp, dev, s0=s0, l2norm=True, inplace=True)
    assert np.all(plan[:, 0] == 1)
    ro, rs = oracle.c_prefill(**inp, init_state=s0, l2norm_qk=True)
    _check_all("l2norm", o, s, ro, rs)
    say("[case] segmented per-head gate in place")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=55)
    gate = np.ascontiguousarray(inp["log_alpha"][..., 0])                    # [B,T,H]
    run = dict(inp, log_alpha=gate)
    o, s, plan = _run(run, dev, s0=s0, scalar_gate=True, inplace=True)
    assert np.all(plan[:, 0] == 1)
    ro, rs = oracle.c_prefill(**dict(inp, log_alpha=np.repeat(gate[..., None], DK, axis=-1)), init_state=s0)
    _check_all("per-head gate", o, s, ro, rs)


def test_segmented_deterministic():
    """Two calls on the same inputs give the same bits (the plan is made on the device from
    the inputs alone)."""
    import torch
    dev = device()
    B, T, H = 2, 8192, 4
    say("[case] segmented determinism")
    inp = D.np_kda_inputs(B, T, H, DK, DV, "bf16", seed=56)
    o1, s1, p1 = _run(inp, dev)
    o2, s2, p2 = _run(inp, dev)
    assert np.all(p1[:, 0] == 1)
    assert torch.equal(o1, o2) and torch.equal(s1, s2) and np.array_equal(p1, p2)


@pytest.mark.parametrize("dk,chunk", [(64, 64), (128, 32), (32, 16)])
def test_segmented_other_shapes(oracle, dk, chunk):
    """Segmentation depends only on bf16, dv = 128, B*H < 64 and the chunk count: key sizes 64
    and 32 and 32- and 16-token chunks (run inside the 32-row chunk kernels) segment too;
    two batch rows with their own initial states, against the oracle."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H = 2, 2
    T = 128 * chunk + 21                                  # at least 128 chunks: segmented
    say(f"[case] segmented dk={dk} chunk={chunk} T={T}")
    inp = D.np_kda_inputs(B, T, H, dk, DV, "bf16", seed=57)
    s0 = D.np_state(B, H, dk, DV, 0.1, seed=57)
    d = dict(q=to_dev(inp["q"], "bf16", dev), k=to_dev(inp["k"], "bf16", dev), v=to_dev(inp["v"], "bf16", dev),
             log_alpha=to_dev(inp["log_alpha"], dev=dev), beta=to_dev(inp["beta"], dev=dev))
    need = kda.prefill_workspace_size(B, T, H, dk, DV, chunk, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    o, s = kda.chunk_prefill(**d, initial_state=to_dev(s0, dev=dev), chunk_size=chunk, workspace=ws)
    torch.cuda.synchronize()
    G = _segments(B * H, (T + chunk - 1) // chunk)
    assert G >= 2
    plan = ws[need - B * H * G * 4:need].view(torch.int32).cpu().numpy().reshape(B * H, G)
    assert np.all(plan[:, 0] == 1), plan
    ro, rs = oracle.c_prefill(**inp, init_state=s0)
    _check_all(f"dk{dk} chunk{chunk}", o, s, ro, rs)


def test_segmented_noalloc_equals_workspace_call():
    """kda_chunk_prefill_noalloc takes the same segmented path from its static scratch: bit
    for bit the workspace call, twice in a row (the second call smaller but still segmented)."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    for T, H in ((16384 + 3, 2), (8192, 1)):
        say(f"[case] segmented noalloc T={T} H={H}")
        inp = D.np_kda_inputs(1, T, H, DK, DV, "bf16", seed=58)
        d = dict(q=to_dev(inp["q"], "bf16", dev), k=to_dev(inp["k"], "bf16", dev), v=to_dev(inp["v"], "bf16", dev),
                 log_alpha=to_dev(inp["log_alpha"], dev=dev), beta=to_dev(inp["beta"], dev=dev))
        o1, s1 = kda.chunk_prefill(**d, chunk_size=64)
        o2, s2 = kda.chunk_prefill_noalloc(**d, chunk_size=64)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)


def _sweep_cases(n=10, seed=4242):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        chunk = int(r.choice([16, 32, 64]))
        out.append(dict(dk=int(r.choice([32, 64, 128])), chunk=chunk, B=int(r.integers(1, 3)),
                        H=int(r.choice([1, 2, 3])), T=int(r.integers(128 * chunk, 160 * chunk + 64)),
                        mask=str(r.choice(["none", "left", "right", "holes"])), s0=bool(r.integers(0, 2)),
                        l2=bool(r.integers(0, 2)), scalar=bool(r.integers(0, 2)),
                        slow_head=bool(r.random() < 0.3), seed=300 + i))
    return out


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[f"s{i}" for i in range(len(SWEEP))])
def test_segmented_sweep(oracle, case):
    """Seeded sweep over shapes that take the segmented path (bf16, dv = 128, B*H < 64, at
    least 128 chunks): key size, chunk, batch, heads, length, mask pattern, initial state, the
    two flags, and sometimes one head with a slow channel (which then runs as one chain); o and
    the final state against the oracle, and the plan's per-head decision checked against which
    head was made slow."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    c = case
    B, T, H, dk, chunk = c["B"], c["T"], c["H"], c["dk"], c["chunk"]
    say(f"[case] segmented sweep {c}")
    inp = D.np_kda_inputs(B, T, H, dk, DV, "bf16", seed=c["seed"], unit_qk=not c["l2"])
    if c["slow_head"]:
        inp["log_alpha"][0, :, 0, :] *= 1e-3                   # (b 0, h 0) forgets too slowly
    ref_la = inp["log_alpha"]
    if c["scalar"]:
        inp["log_alpha"] = np.ascontiguousarray(inp["log_alpha"][..., 0])
        ref_la = np.repeat(inp["log_alpha"][..., None], dk, axis=-1)
    mask = None
    if c["mask"] != "none":
        r = np.random.default_rng(c["seed"])
        mask = np.ones((B, T), np.uint8)
        for b in range(B):
            cut = int(r.integers(0, T // 4))
            if c["mask"] == "left":
                mask[b, :cut] = 0
            elif c["mask"] == "right":
                mask[b, T - cut:] = 0
            else:
                mask[b, r.random(T) < 0.15] = 0
    s0 = D.np_state(B, H, dk, DV, 0.1, seed=c["seed"]) if c["s0"] else None
    d = dict(q=to_dev(inp["q"], "bf16", dev), k=to_dev(inp["k"], "bf16", dev), v=to_dev(inp["v"], "bf16", dev),
             log_alpha=to_dev(inp["log_alpha"], dev=dev), beta=to_dev(inp["beta"], dev=dev))
    need = kda.prefill_workspace_size(B, T, H, dk, DV, chunk, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    o, s = kda.chunk_prefill(**d, mask=None if mask is None else to_dev(mask, dev=dev),
                             initial_state=None if s0 is None else to_dev(s0, dev=dev), chunk_size=chunk,
                             l2norm_qk=c["l2"], scalar_gate=c["scalar"], workspace=ws)
    torch.cuda.synchronize()
    G = _segments(B * H, (T + chunk - 1) // chunk)
    assert G >= 2
    plan = ws[need - B * H * G * 4:need].view(torch.int32).cpu().numpy().reshape(B * H, G)
    want = np.ones(B * H, np.int32)
    if c["slow_head"]:
        want[0] = 0
    assert np.array_equal(plan[:, 0], want), plan[:, 0]
    ro, rs = oracle.c_prefill(q=inp["q"], k=inp["k"], v=inp["v"], log_alpha=ref_la, beta=inp["beta"], mask=mask,
                              init_state=s0, l2norm_qk=c["l2"])
    _check_all("sweep", o, s, ro, rs)


@pytest.mark.parametrize("B,H,dk", [(1, 40, 128), (7, 9, 128), (2, 3, 16)])
def test_segmented_chain_counts(oracle, B, H, dk):
    """Between 33 and 63 (b, h) pairs the call still segments (G = 2: 80 and 126 chains, not
    multiples of the eight chains an XCD group takes), and a 16-channel key runs inside the
    32-channel kernels; sampled (b, h) pairs against the oracle over every position."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    T = 8192 + 77
    say(f"[case] segmented chain counts B={B} H={H} dk={dk} T={T}")
    x = D.torch_kda_inputs(B, T, H, dk, DV, dev, "bf16", seed=59)
    need = kda.prefill_workspace_size(B, T, H, dk, DV, 64, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    o, s = kda.chunk_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], chunk_size=64, workspace=ws)
    torch.cuda.synchronize()
    G = _segments(B * H, (T + 63) // 64)
    assert G == 2 if B * H < 64 else G == 1
    plan = ws[need - B * H * G * 4:need].view(torch.int32).cpu().numpy().reshape(B * H, G)
    assert np.all(plan[:, 0] == 1), plan[:, 0]
    picks = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})
    for b, h in picks:
        one = {n: host(t[b:b + 1, :, h:h + 1]) for n, t in x.items()}
        ro, rs = oracle.c_prefill(**one)
        _check_all(f"b{b}h{h}", o[b:b + 1, :, h:h + 1], s[b:b + 1, h:h + 1], ro, rs)


def test_segmented_headline_128k(oracle):
    """The benchmarked call itself: B=1, H=32, T=131072, dk=dv=128, bf16, chunk 64, zero
    state, in the launch configuration bench.py times (two segments per head, 64 chains of
    32-column tiles); three heads against the oracle over every position and the final
    state, and every head segmented."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H = 1, 131072, 32
    say("[case] segmented headline 1x131072x32, sampled heads")
    x = D.torch_kda_inputs(B, T, H, DK, DV, dev, "bf16", seed=0)
    need = kda.prefill_workspace_size(B, T, H, DK, DV, 64, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o, s = kda.chunk_prefill(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], chunk_size=64, workspace=ws)
    torch.cuda.synchronize()
    G = _segments(B * H, T // 64)
    assert G == 2
    plan = ws[need - H * G * 4:need].view(torch.int32).cpu().numpy().reshape(H, G)
    assert np.all(plan[:, 0] == 1), plan[:, 0]
    say(f"[plan] tails start at chunks {sorted(set(plan[:, 1].tolist()))} (boundary 1024)")
    heads = [0, 13, 31]
    one = {n: host(t[:, :, heads]) for n, t in x.items()}
    ro, rs = oracle.c_prefill(**one)
    for i, h in enumerate(heads):
        _check_all(f"128k h{h}", o[:, :, h], s[:, h], ro[:, :, i], rs[:, i])


# ---------------------------------------------------------------- packed sequences
def _packed(lengths, H, dk, seed, decay="default"):
    T = int(sum(lengths))
    inp = {n: np.ascontiguousarray(x[0]) for n, x in D.np_kda_inputs(1, T, H, dk, DV, "bf16", seed=seed,
                                                                        decay=decay).items()}
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return inp, cu


def _dev_packed(inp, dev):
    return {n: to_dev(x, "bf16" if n in "qkv" else None, dev) for n, x in inp.items()}


@pytest.mark.parametrize("H", [2, 40])
def test_varlen_segments_like_lone_runs(oracle, H):
    """With fewer than 64 (sequence, head) pairs (H = 2) packed sequences are segmented one
    by one, each as its lone kda_chunk_prefill run is (the same rule on its chunk count and
    the head count): long ones (9000 and 8256 tokens) among short and empty ones, with
    initial states, equal their lone runs bit for bit.  With more pairs (H = 40: 240) the
    chip is full of single chains and every sequence equals its lone run with
    KDA_FLAG_SERIAL_SCAN.  The long ones against the oracle too."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [9000, 300, 0, 8256, 17, 1]
    N = len(lengths)
    say(f"[case] varlen segmented H={H} lengths={lengths}")
    inp, cu = _packed(lengths, H, DK, seed=61)
    d = _dev_packed(inp, dev)
    s0 = to_dev(D.np_state(N, H, DK, DV, 0.1, seed=61), dev=dev)
    o, sN = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                     initial_state=s0, chunk_size=64)
    torch.cuda.synchronize()
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        oi, si = kda.chunk_prefill(*(d[n][a:b].unsqueeze(0).contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                   initial_state=s0[i:i + 1].contiguous(), chunk_size=64,
                                   serial_scan=N * H >= 64)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], oi[0]), f"o of sequence {i} (length {b - a}) differs from its lone run"
        assert torch.equal(sN[i], si[0]), f"state of sequence {i} differs from its lone run"
    heads = [0, H - 1]
    for i in (0, 3):
        a, b = int(cu[i]), int(cu[i + 1])
        one = {n: x[a:b][None][:, :, heads] for n, x in inp.items()}
        ro, rs = oracle.c_prefill(**one, init_state=host(s0[i:i + 1, heads]))
        _check_all(f"seq{i}", o[a:b][None][:, :, heads], sN[i:i + 1, heads], ro, rs)


def test_varlen_segmented_slots_checkpoints_serial():
    """With state slots (the pool updated in place) the segmented packed call equals the
    lone runs bit for bit; with checkpoints, or with KDA_FLAG_SERIAL_SCAN, it scans each
    sequence as one chain and equals the single-chain lone runs bit for bit; a sequence with
    slow gates falls back to one chain."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H = 2
    lengths = [8192 + 40, 500, 8192 + 64]
    N = len(lengths)
    say(f"[case] varlen segmented slots/checkpoints/serial lengths={lengths}")
    inp, cu = _packed(lengths, H, DK, seed=62)
    inp["log_alpha"][int(cu[2]):int(cu[3])] *= 1e-3          # sequence 2: slow gates
    d = _dev_packed(inp, dev)
    cu_d = to_dev(cu, dev=dev)
    s0 = to_dev(D.np_state(N, H, DK, DV, 0.1, seed=62), dev=dev)
    lone, lone_serial, flags = [], [], []
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        args = [d[n][a:b].unsqueeze(0).contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
        need = kda.prefill_workspace_size(1, b - a, H, DK, DV, 64, 0)
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        lone.append(kda.chunk_prefill(*args, initial_state=s0[i:i + 1].contiguous(), chunk_size=64, workspace=ws))
        lone_serial.append(kda.chunk_prefill(*args, initial_state=s0[i:i + 1].contiguous(), chunk_size=64,
                                             serial_scan=True))
        G = _segments(H, (b - a + 63) // 64)
        flags.append(ws[need - H * G * 4:need].view(torch.int32).cpu().numpy().reshape(H, G)[:, 0].tolist()
                     if G > 1 else None)
    torch.cuda.synchronize()
    assert flags == [[1, 1], None, [0, 0]], flags      # 0 segmented, 1 too short, 2 slow gates
    assert torch.equal(lone[2][0], lone_serial[2][0]) and torch.equal(lone[2][1], lone_serial[2][1])
    # slots: sequence i in slot 3 - i of a pool of 4, updated in place
    pool = torch.zeros(4, H, DK, DV, dtype=torch.float32, device=dev)
    for i in range(N):
        pool[3 - i] = s0[i]
    slot = torch.tensor([3 - i for i in range(N)], dtype=torch.int32, device=dev)
    o, _ = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], cu_d, initial_state=pool,
                                    final_state=pool, slot=slot, chunk_size=64)
    torch.cuda.synchronize()
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        assert torch.equal(o[a:b], lone[i][0][0]) and torch.equal(pool[3 - i], lone[i][1][0]), f"slots: sequence {i}"
    # a slot outside the pool: the segmented sequence 0 starts from zero (no entry state is
    # copied for it) and keeps no state; it equals its lone run without an initial state
    a0, b0 = int(cu[0]), int(cu[1])
    args0 = [d[n][a0:b0].unsqueeze(0).contiguous() for n in ("q", "k", "v", "log_alpha", "beta")]
    o_zero, s_zero = kda.chunk_prefill(*args0, chunk_size=64)
    pool2 = pool.clone()
    before = pool2.clone()
    slot2 = torch.tensor([-1, 1, 0], dtype=torch.int32, device=dev)
    o2, _ = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], cu_d, initial_state=pool2,
                                     final_state=pool2, slot=slot2, chunk_size=64)
    torch.cuda.synchronize()
    assert torch.equal(o2[a0:b0], o_zero[0]), "slot outside the pool: sequence 0 from zero"
    assert torch.equal(pool2[2], before[2]) and torch.equal(pool2[3], before[3]), "no state kept for slot -1"
    for i in (1, 2):
        a, b = int(cu[i]), int(cu[i + 1])
        assert torch.equal(o2[a:b], kda.chunk_prefill(*[d[n][a:b].unsqueeze(0).contiguous() for n in
                                                        ("q", "k", "v", "log_alpha", "beta")],
                                                      initial_state=before[2 - i:3 - i].contiguous(),
                                                      chunk_size=64)[0][0]), f"slot {2 - i}: sequence {i}"
    # checkpoints and the serial flag: single chains
    for kw in (dict(state_interval=64), dict(serial_scan=True)):
        res = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], cu_d, initial_state=s0,
                                       chunk_size=64, **kw)
        torch.cuda.synchronize()
        o, sN = res[0], res[1]
        for i in range(N):
            a, b = int(cu[i]), int(cu[i + 1])
            assert torch.equal(o[a:b], lone_serial[i][0][0]) and torch.equal(sN[i], lone_serial[i][1][0]), \
                f"{kw}: sequence {i}"
