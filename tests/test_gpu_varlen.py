"""GPU parity of kda_chunk_prefill_varlen: N sequences of different lengths packed end to end.

Each packed sequence must give, bit for bit, what kda_chunk_prefill gives for that sequence
alone (its chunks start at its own first token, so the arithmetic is the same) and what the
right-padded, masked batch gives; and it must match the fp64 oracle run on each sequence.
Prefix reuse: the state a packed call leaves after a prefix, fed back as the initial state of
a later packed call holding the continuation beside fresh prompts, continues the sequence."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _packed_inputs(lengths, H, dk, dv, dtype, seed, scalar=False):
    T = int(sum(lengths))
    inp = {n: x[0] for n, x in D.np_kda_inputs(1, max(T, 1), H, dk, dv, dtype, seed=seed).items()}
    inp = {n: np.ascontiguousarray(x[:T]) for n, x in inp.items()}
    if scalar:
        inp["log_alpha"] = np.ascontiguousarray(inp["log_alpha"][..., 0])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return inp, cu


def _dev(inp, dtype, dev):
    return {n: to_dev(x, dtype if n in "qkv" else None, dev) for n, x in inp.items()}


def _varlen(kda, d, cu, dev, chunk, s0=None, l2=False, scalar=False):
    return kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                    initial_state=s0, chunk_size=chunk, l2norm_qk=l2, scalar_gate=scalar)


@pytest.mark.parametrize("dtype,chunk,l2,scalar", [("bf16", 64, False, False), ("bf16", 32, True, False),
                                                   ("fp32", 16, False, False), ("bf16", 64, False, True),
                                                   ("fp32", 64, True, True)])
def test_varlen_equals_each_sequence_alone_and_padded_batch(dtype, chunk, l2, scalar):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [0, 1, 63, 64, 65, 200, 130, 0, 17]
    N, H, dk, dv = len(lengths), 3, 128, 64
    say(f"[case] varlen vs alone and padded {dtype} chunk={chunk} l2={l2} scalar={scalar}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, dtype, seed=31, scalar=scalar)
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=31), dev=dev)
    d = _dev(inp, dtype, dev)
    o, sN = _varlen(kda, d, cu, dev, chunk, s0=s0, l2=l2, scalar=scalar)
    # right-padded batch: sequence i in row i, positions past its length masked
    Tmax = max(lengths)
    pad = {n: torch.zeros((N, Tmax) + x.shape[1:], dtype=x.dtype, device=dev) for n, x in d.items()}
    for i in range(N):
        for n in pad:
            pad[n][i, :lengths[i]] = d[n][int(cu[i]):int(cu[i + 1])]
    mask = to_dev(D.padded_layout(lengths, Tmax, ["right"] * N), dev=dev)
    op, sp = kda.chunk_prefill(pad["q"], pad["k"], pad["v"], pad["log_alpha"], pad["beta"], mask=mask,
                               initial_state=s0, chunk_size=chunk, l2norm_qk=l2, scalar_gate=scalar)
    torch.cuda.synchronize()
    assert torch.equal(sN, sp), "final states differ from the padded batch"
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        oi, si = kda.chunk_prefill(*(d[n][a:b].unsqueeze(0).contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                   initial_state=s0[i:i + 1].contiguous(), chunk_size=chunk, l2norm_qk=l2,
                                   scalar_gate=scalar)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], oi[0]), f"o of sequence {i} (length {b - a}) differs from the lone run"
        assert torch.equal(sN[i], si[0]), f"state of sequence {i} differs from the lone run"
        assert torch.equal(o[a:b], op[i, :b - a]), f"o of sequence {i} differs from the padded batch"
        if b == a:
            assert torch.equal(sN[i], s0[i]), "an empty sequence must keep its initial state"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_varlen_matches_oracle(oracle, dtype):
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [100, 0, 257, 64, 3]
    N, H, dk, dv = len(lengths), 2, 64, 128
    say(f"[case] varlen vs oracle {dtype}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, dtype, seed=32)
    s0 = D.np_state(N, H, dk, dv, 0.1, seed=32)
    o, sN = _varlen(kda, _dev(inp, dtype, dev), cu, dev, 64, s0=to_dev(s0, dev=dev), l2=True)
    go, gs = host(o), host(sN)
    ro = np.zeros_like(go)
    rs = np.zeros_like(gs)
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        seq = {n: x[None, a:b] for n, x in inp.items()}
        oi, si = oracle.c_prefill(**seq, init_state=s0[i:i + 1], l2norm_qk=True)
        ro[a:b], rs[i] = oi[0], si[0]
    check("varlen o", go, ro, dtype)
    check("varlen state", gs, rs, dtype)


def test_varlen_prefix_reuse_in_a_mixed_batch(oracle):
    """Continuous batching with cached prefixes: call 1 packs the prefixes, call 2 packs the
    continuations (initial state = the cached one) beside a fresh prompt (zero state).  A
    prefix that ends on a chunk boundary continues bit for bit as the whole sequence run at
    once; every continuation matches the oracle run on prefix + continuation."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H, dk, dv = 4, 128, 128
    prefix, cont, _ = D.continuation_lengths(3, seed=33, prefix_max=700, cont_max=300)
    prefix[0] = 256                                            # chunk-aligned prefix
    say(f"[case] varlen prefix reuse prefixes={prefix} continuations={cont}")
    full = [p + c for p, c in zip(prefix, cont)]
    whole, _ = _packed_inputs(full, H, dk, dv, "bf16", seed=33)
    fresh_len = 190
    fresh, _ = _packed_inputs([fresh_len], H, dk, dv, "bf16", seed=34)
    starts = np.concatenate([[0], np.cumsum(full)])
    pre = {n: np.concatenate([x[s:s + p] for s, p in zip(starts, prefix)]) for n, x in whole.items()}
    con = {n: np.concatenate([x[s + p:s + p + c] for s, p, c in zip(starts, prefix, cont)] + [fresh[n]])
           for n, x in whole.items()}
    cu_pre = np.concatenate([[0], np.cumsum(prefix)]).astype(np.int32)
    cu_con = np.concatenate([[0], np.cumsum(cont + [fresh_len])]).astype(np.int32)
    _, cached = _varlen(kda, _dev(pre, "bf16", dev), cu_pre, dev, 64)
    s_in = torch.cat([cached, torch.zeros_like(cached[:1])]).contiguous()
    o2, s2 = _varlen(kda, _dev(con, "bf16", dev), cu_con, dev, 64, s0=s_in)
    o_all, s_all = _varlen(kda, _dev(whole, "bf16", dev), np.concatenate([[0], np.cumsum(full)]).astype(np.int32),
                           dev, 64)
    torch.cuda.synchronize()
    # the chunk-aligned prefix: the continuation equals the tail of the single run bit for bit
    a0 = int(cu_con[0])
    assert torch.equal(o2[a0:a0 + cont[0]], o_all[prefix[0]:full[0]])
    assert torch.equal(s2[0], s_all[0])
    go2, gs2 = host(o2), host(s2)
    for i in range(3):
        s, p, c = int(starts[i]), prefix[i], cont[i]
        seq = {n: x[None, s:s + p + c] for n, x in whole.items()}
        ro, rs = oracle.c_prefill(**seq)
        check(f"continuation {i} o", go2[cu_con[i]:cu_con[i + 1]], ro[0, p:], "bf16")
        check(f"continuation {i} state", gs2[i], rs[0], "bf16")
    ro, rs = oracle.c_prefill(**{n: x[None] for n, x in fresh.items()})
    check("fresh prompt o", go2[cu_con[3]:], ro[0], "bf16")
    check("fresh prompt state", gs2[3], rs[0], "bf16")


def test_varlen_state_in_place():
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [70, 0, 129]
    N, H, dk, dv = 3, 2, 128, 128
    say("[case] varlen final_state aliasing initial_state")
    inp, cu = _packed_inputs(lengths, H, dk, dv, "bf16", seed=35)
    d = _dev(inp, "bf16", dev)
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=35), dev=dev)
    o_ref, s_ref = _varlen(kda, d, cu, dev, 64, s0=s0.clone())
    st = s0.clone()
    o, s = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                    initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert s.data_ptr() == st.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(st, s_ref)


def test_varlen_serving_mix_equals_lone_runs():
    """A serving-sized pack: 16 prompts of 1 .. 4096 tokens (uniform), 32 heads of 128 x 128,
    bf16; every sequence equals its lone run bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    r = np.random.default_rng(36)
    lengths = [int(x) for x in r.integers(1, 4097, 16)]
    H, dk, dv = 32, 128, 128
    T = sum(lengths)
    say(f"[case] varlen serving mix T={T} lengths={lengths}")
    d = D.torch_kda_inputs(1, T, H, dk, dv, dev, "bf16", seed=36)
    d = {n: x[0].contiguous() for n, x in d.items()}
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    o, sN = _varlen(kda, d, cu, dev, 64)
    for i in range(len(lengths)):
        a, b = int(cu[i]), int(cu[i + 1])
        oi, si = kda.chunk_prefill(*(d[n][a:b].unsqueeze(0).contiguous() for n in ("q", "k", "v", "log_alpha", "beta")))
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], oi[0]), f"o of sequence {i} (length {b - a})"
        assert torch.equal(sN[i], si[0]), f"state of sequence {i}"


@pytest.mark.parametrize("dtype,chunk,interval", [("bf16", 64, 128), ("bf16", 32, 64), ("fp32", 64, 192)])
def test_varlen_state_checkpoints(dtype, chunk, interval):
    """Checkpoint j of sequence i is the state after its first j * interval tokens: bit for
    bit the final state of a packed run over those prefixes (one sequence per prefix)."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [300, 0, 2 * interval, 1000, interval - 1, interval]
    N, H, dk, dv = len(lengths), 2, 128, 128
    say(f"[case] varlen checkpoints {dtype} chunk={chunk} interval={interval}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, dtype, seed=37)
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=37), dev=dev)
    d = _dev(inp, dtype, dev)
    o, sN, ck = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                         initial_state=s0, chunk_size=chunk, state_interval=interval)
    counts = [L // interval for L in lengths]
    assert ck.shape[0] == sum(counts) == kda.num_checkpoints(cu, interval)
    # every prefix as its own packed sequence, each from its sequence's initial state
    pre_idx, pre_len, pre_seq = [], [], []
    for i, L in enumerate(lengths):
        for j in range(1, counts[i] + 1):
            pre_idx.append(np.arange(cu[i], cu[i] + j * interval))
            pre_len.append(j * interval)
            pre_seq.append(i)
    sel = torch.from_numpy(np.concatenate(pre_idx)).to(dev)
    dp = {n: x.index_select(0, sel).contiguous() for n, x in d.items()}
    cu_p = np.concatenate([[0], np.cumsum(pre_len)]).astype(np.int32)
    _, s_pre = kda.chunk_prefill_varlen(dp["q"], dp["k"], dp["v"], dp["log_alpha"], dp["beta"],
                                        to_dev(cu_p, dev=dev), initial_state=s0[pre_seq].contiguous(),
                                        chunk_size=chunk)
    torch.cuda.synchronize()
    assert torch.equal(ck, s_pre)
    # a sequence whose length is a multiple of the interval: its last checkpoint is its final state
    last = int(np.cumsum(counts)[2]) - 1
    assert torch.equal(ck[last], sN[2])
    # the outputs do not change when checkpoints are saved
    o2, s2 = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                      initial_state=s0, chunk_size=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(sN, s2)


def test_varlen_checkpoints_match_oracle_and_respect_capacity(oracle):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [200, 450]
    N, H, dk, dv, interval = 2, 2, 64, 64, 128
    say("[case] varlen checkpoints vs oracle, short checkpoint array")
    inp, cu = _packed_inputs(lengths, H, dk, dv, "bf16", seed=38)
    d = _dev(inp, "bf16", dev)
    M = kda.num_checkpoints(cu, interval)                       # 1 + 3
    _, _, ck = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                        l2norm_qk=True, state_interval=interval)
    got = host(ck)
    k = 0
    for i, L in enumerate(lengths):
        for j in range(1, L // interval + 1):
            a = int(cu[i])
            _, rs = oracle.c_prefill(**{n: x[None, a:a + j * interval] for n, x in inp.items()}, l2norm_qk=True)
            check(f"checkpoint {i}.{j}", got[k], rs[0], "bf16")
            k += 1
    assert k == M
    # an array that holds fewer entries than the checkpoints: those past it are not written
    big = torch.full((M, H, dk, dv), float("nan"), device=dev)
    kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                             l2norm_qk=True, state_interval=interval, chunk_states=big[:2])
    torch.cuda.synchronize()
    assert torch.equal(big[:2], ck[:2])
    assert torch.isnan(big[2:]).all()


@pytest.mark.parametrize("dk,dv,dtype,chunk", [(16, 16, "fp32", 16), (32, 128, "bf16", 32), (64, 32, "bf16", 64),
                                               (128, 16, "fp32", 64)])
def test_varlen_head_sizes_with_checkpoints(dk, dv, dtype, chunk):
    """Every supported head-size family through the packed path: each sequence equals its
    lone run, and every checkpoint equals the lone run over that prefix, bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    interval = 2 * chunk
    lengths = [3 * interval + 5, 0, interval, 77]
    N, H = len(lengths), 3
    say(f"[case] varlen dk={dk} dv={dv} {dtype} chunk={chunk}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, dtype, seed=39)
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=39), dev=dev)
    d = _dev(inp, dtype, dev)
    o, sN, ck = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                         initial_state=s0, chunk_size=chunk, l2norm_qk=True,
                                         state_interval=interval)
    k = 0
    for i, L in enumerate(lengths):
        a = int(cu[i])
        oi, si = kda.chunk_prefill(*(d[n][a:a + L].unsqueeze(0).contiguous()
                                     for n in ("q", "k", "v", "log_alpha", "beta")),
                                   initial_state=s0[i:i + 1].contiguous(), chunk_size=chunk, l2norm_qk=True)
        torch.cuda.synchronize()
        assert torch.equal(o[a:a + L], oi[0]) and torch.equal(sN[i], si[0]), f"sequence {i}"
        for j in range(1, L // interval + 1):
            _, sj = kda.chunk_prefill(*(d[n][a:a + j * interval].unsqueeze(0).contiguous()
                                        for n in ("q", "k", "v", "log_alpha", "beta")),
                                      initial_state=s0[i:i + 1].contiguous(), chunk_size=chunk, l2norm_qk=True)
            torch.cuda.synchronize()
            assert torch.equal(ck[k], sj[0]), f"checkpoint {j} of sequence {i}"
            k += 1
    assert k == ck.shape[0]


def test_prefill_calls_in_graph_replays():
    """The batch and the packed prefill captured once in a graph (workspace and outputs
    fixed) and replayed with new inputs copied in eagerly, with a synchronisation between
    replays: every replay equals the eager call bit for bit, checkpoints included."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H, dk, dv, chunk, interval = 2, 128, 128, 64, 128
    lengths = [130, 0, 256, 61]
    N, T = len(lengths), sum(lengths)
    say("[case] prefill and packed prefill in a graph")
    cu = to_dev(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), dev=dev)
    M = kda.num_checkpoints(cu, interval)

    def inputs(seed):
        inp, _ = _packed_inputs(lengths, H, dk, dv, "bf16", seed=seed)
        return _dev(inp, "bf16", dev)
    d0 = inputs(50)
    g = {n: x.clone() for n, x in d0.items()}                      # captured input buffers
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=50), dev=dev)
    out = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    ck = torch.empty(M, H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.prefill_varlen_workspace_size(N, T, H, dk, dv, chunk, kda.KDA_BF16), dtype=torch.uint8,
                     device=dev)
    gb = {n: x[None, :64].contiguous() for n, x in d0.items()}     # a batch call beside it
    ob = torch.empty(1, 64, H, dv, dtype=torch.bfloat16, device=dev)
    fb = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    wsb = torch.empty(kda.prefill_workspace_size(1, 64, H, dk, dv, chunk, kda.KDA_BF16), dtype=torch.uint8,
                      device=dev)

    def step():
        kda.chunk_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], cu, initial_state=s0,
                                 chunk_size=chunk, out=out, final_state=fs, workspace=ws,
                                 state_interval=interval, chunk_states=ck)
        kda.chunk_prefill(gb["q"], gb["k"], gb["v"], gb["log_alpha"], gb["beta"], chunk_size=chunk,
                          out=ob, final_state=fb, workspace=wsb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        d = inputs(60 + r)
        for n in g:
            g[n].copy_(d[n])
            gb[n].copy_(d[n][None, :64])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_e, s_e, c_e = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], cu,
                                                 initial_state=s0, chunk_size=chunk, state_interval=interval)
        ob_e, fb_e = kda.chunk_prefill(*(d[n][None, :64].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                       chunk_size=chunk)
        torch.cuda.synchronize()
        assert torch.equal(out, o_e) and torch.equal(fs, s_e) and torch.equal(ck, c_e), f"packed, replay {r}"
        assert torch.equal(ob, ob_e) and torch.equal(fb, fb_e), f"batch, replay {r}"


@pytest.mark.parametrize("scalar", [False, True])
def test_varlen_wide_tiles_equal_narrow_with_checkpoints(scalar):
    """16 packed sequences x 4 heads (64 pairs) run on 32-column scan tiles; the same
    sequences split into four packed calls of 4 (16 pairs, 16-column tiles) give the same
    outputs, final states and checkpoints bit for bit, with L2 norm, initial states and
    the per-head gate."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H, dk, dv, interval = 4, 128, 128, 128
    r = np.random.default_rng(41)
    lengths = [int(x) for x in r.integers(0, 700, 16)]
    lengths[3] = 0
    lengths[5] = 2 * interval
    N = len(lengths)
    say(f"[case] varlen wide vs narrow scalar={scalar} lengths={lengths}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, "bf16", seed=41, scalar=scalar)
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=41), dev=dev)
    d = _dev(inp, "bf16", dev)
    o, sN, ck = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                         initial_state=s0, l2norm_qk=True, scalar_gate=scalar,
                                         state_interval=interval)
    k = 0
    for g0 in range(0, N, 4):
        a, b = int(cu[g0]), int(cu[g0 + 4])
        cu_g = (cu[g0:g0 + 5] - cu[g0]).astype(np.int32)
        og, sg, cg = kda.chunk_prefill_varlen(*(d[n][a:b].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                              to_dev(cu_g, dev=dev), initial_state=s0[g0:g0 + 4].contiguous(),
                                              l2norm_qk=True, scalar_gate=scalar, state_interval=interval)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], og), f"o of sequences {g0}..{g0 + 3}"
        assert torch.equal(sN[g0:g0 + 4], sg), f"states of sequences {g0}..{g0 + 3}"
        assert torch.equal(ck[k:k + cg.shape[0]], cg), f"checkpoints of sequences {g0}..{g0 + 3}"
        k += cg.shape[0]
    assert k == ck.shape[0]


@pytest.mark.parametrize("heads", [2, 16])
def test_varlen_state_slots(heads):
    """States from a pool (in place): sequence i starts from pool[slot[i]] and leaves its
    final state there; other entries are untouched; a slot outside the pool starts from
    zero and keeps nothing.  Outputs equal the packed call on the gathered states bit for
    bit; with 16 heads the 80 (sequence, head) pairs take the 32-column scan tiles."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H, dk, dv, S = heads, 128, 128, 12
    lengths = [100, 0, 65, 200, 30]
    slot = np.array([7, 2, -1, 4, 12], np.int32)
    N = len(lengths)
    say(f"[case] varlen state slots H={H}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, "bf16", seed=42)
    d = _dev(inp, "bf16", dev)
    pool = to_dev(np.concatenate([D.np_state(1, H, dk, dv, 0.1, seed=200 + i) for i in range(S)]), dev=dev)
    before = pool.clone()
    valid = (slot >= 0) & (slot < S)
    gathered = torch.stack([before[int(s)] if ok else torch.zeros_like(before[0]) for s, ok in zip(slot, valid)])
    o_ref, s_ref = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                            initial_state=gathered.contiguous(), l2norm_qk=True)
    o, _ = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                    initial_state=pool, final_state=pool, slot=to_dev(slot, dev=dev), l2norm_qk=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for i in range(N):
        if valid[i]:
            assert torch.equal(pool[int(slot[i])], s_ref[i]), f"slot {slot[i]} of sequence {i}"
    for j in sorted(set(range(S)) - set(int(x) for x in slot[valid])):
        assert torch.equal(pool[j], before[j]), f"slot {j} changed"


def test_varlen_many_sequences_chunk_table():
    """2500 packed sequences: the chunk table is built in several passes of the setup
    workgroup (1024 sequences each), carrying chunk and checkpoint counts from pass to
    pass.  The result equals the same sequences packed in calls of at most 1000 (one pass
    each) bit for bit, outputs, final states and checkpoints."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H, dk, dv, chunk, interval = 2, 64, 64, 32, 32
    r = np.random.default_rng(43)
    lengths = [int(x) for x in r.integers(0, 100, 2500)]
    N = len(lengths)
    say(f"[case] varlen N={N} T={sum(lengths)}")
    inp, cu = _packed_inputs(lengths, H, dk, dv, "bf16", seed=43)
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=43), dev=dev)
    d = _dev(inp, "bf16", dev)
    o, sN, ck = kda.chunk_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], to_dev(cu, dev=dev),
                                         initial_state=s0, chunk_size=chunk, state_interval=interval)
    k = 0
    for g0 in range(0, N, 1000):
        g1 = min(N, g0 + 1000)
        a, b = int(cu[g0]), int(cu[g1])
        cu_g = (cu[g0:g1 + 1] - cu[g0]).astype(np.int32)
        og, sg, cg = kda.chunk_prefill_varlen(*(d[n][a:b].contiguous() for n in ("q", "k", "v", "log_alpha", "beta")),
                                              to_dev(cu_g, dev=dev), initial_state=s0[g0:g1].contiguous(),
                                              chunk_size=chunk, state_interval=interval)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], og), f"o of sequences {g0}..{g1 - 1}"
        assert torch.equal(sN[g0:g1], sg), f"states of sequences {g0}..{g1 - 1}"
        assert torch.equal(ck[k:k + cg.shape[0]], cg), f"checkpoints of sequences {g0}..{g1 - 1}"
        k += cg.shape[0]
    assert k == ck.shape[0] == sum(L // interval for L in lengths)


def test_varlen_all_empty_and_no_sequences():
    """Edge cases: every packed sequence empty (T = 0) copies each initial state to its
    final state (and to its slot); no sequences at all is a no-op."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    N, H, dk, dv = 3, 2, 64, 128
    say("[case] varlen all-empty, N = 0")
    e = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=dev)  # noqa: E731
    s0 = to_dev(D.np_state(N, H, dk, dv, 0.1, seed=44), dev=dev)
    cu = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    la = torch.empty(0, H, dk, dtype=torch.float32, device=dev)
    beta = torch.empty(0, H, dtype=torch.float32, device=dev)
    o, sN = kda.chunk_prefill_varlen(e(0, H, dk), e(0, H, dk), e(0, H, dv), la, beta, cu, initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (0, H, dv) and torch.equal(sN, s0)
    pool = to_dev(D.np_state(5, H, dk, dv, 0.1, seed=45), dev=dev)
    before = pool.clone()
    slot = torch.tensor([4, -1, 0], dtype=torch.int32, device=dev)
    kda.chunk_prefill_varlen(e(0, H, dk), e(0, H, dk), e(0, H, dv), la, beta, cu, initial_state=pool,
                             final_state=pool, slot=slot)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)                   # each used slot rewritten with itself
    o0, s00 = kda.chunk_prefill_varlen(e(0, H, dk), e(0, H, dk), e(0, H, dv), la, beta,
                                       torch.zeros(1, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert s00.shape == (0, H, dk, dv)
