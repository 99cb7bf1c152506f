"""GPU parity of kda_chunk_prefill_varlen_backward: the training backward over N sequences of
different lengths packed end to end.

Each sequence's chunks start at its own first token, so its gradients must equal, bit for bit,
those kda_chunk_prefill_backward gives for that sequence alone; a sequence of length 0 passes
d_final_state through to d_init_state.  The checkpoints kda_chunk_prefill_varlen writes at
state_interval = 64, handed in, give the gradients of the call that runs the forward again,
bit for bit; and each sequence's gradients are within the backward's bar of the fp64 oracle."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import device, host, say, to_dev
from tests.test_gpu_backward import _check, _ref

pytestmark = pytest.mark.gpu

INPUTS = ("q", "k", "v", "log_alpha", "beta")
TOKEN_GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta")


def _packed(lengths, H, dk, dv, dtype, seed, scalar=False, unit_qk=True):
    """Packed inputs, initial states and cotangents for the given lengths (numpy)."""
    T = int(sum(lengths))
    N = len(lengths)
    inp = {n: x[0] for n, x in D.np_kda_inputs(1, max(T, 1), H, dk, dv, dtype, seed=seed, unit_qk=unit_qk).items()}
    inp = {n: np.ascontiguousarray(x[:T]) for n, x in inp.items()}
    if scalar:
        inp["log_alpha"] = np.ascontiguousarray(inp["log_alpha"][..., 0])
    rng = np.random.default_rng(2000 + seed)
    do = D.to_storage(rng.normal(0, 1, (T, H, dv)).astype(np.float32), dtype)
    dfinal = rng.normal(0, 1, (N, H, dk, dv)).astype(np.float32)
    s0 = D.np_state(N, H, dk, dv, 0.05, seed=seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return inp, do, dfinal, s0, cu


def _lone(kda, d, ddo, dfin, ds0, cu, i, scalar, l2=False):
    """kda_chunk_prefill_backward on sequence i alone (B = 1)."""
    a, b = int(cu[i]), int(cu[i + 1])
    one = {n: x[a:b].unsqueeze(0).contiguous() for n, x in d.items()}
    return kda.chunk_prefill_backward(*(one[n] for n in INPUTS), ddo[a:b].unsqueeze(0).contiguous(),
                                      d_final_state=dfin[i:i + 1].contiguous(),
                                      initial_state=ds0[i:i + 1].contiguous(), scalar_gate=scalar, l2norm_qk=l2)


def _compare_with_lone_runs(kda, got, d, ddo, dfin, ds0, cu, lengths, scalar, tag, l2=False):
    import torch
    for i, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(got["dinit_state"][i], dfin[i]), f"{tag}: empty sequence {i}"
            continue
        ref = _lone(kda, d, ddo, dfin, ds0, cu, i, scalar, l2)
        torch.cuda.synchronize()
        a, b = int(cu[i]), int(cu[i + 1])
        for n in TOKEN_GRADS:
            assert torch.equal(got[n][a:b], ref[n][0]), f"{tag}: {n} of sequence {i} (length {L})"
        assert torch.equal(got["dinit_state"][i], ref["dinit_state"][0]), f"{tag}: dinit of sequence {i}"


@pytest.mark.parametrize("dtype,H,dk,dv,scalar,l2", [("bf16", 2, 128, 128, False, False),
                                                     ("fp32", 3, 64, 32, False, False),
                                                     ("bf16", 16, 128, 128, False, False),
                                                     ("bf16", 2, 64, 64, True, False),
                                                     ("bf16", 2, 128, 128, False, True)])
def test_varlen_backward_equals_lone_sequences(dtype, H, dk, dv, scalar, l2):
    """Lengths with empty sequences, single tokens, exact and ragged chunks: every gradient
    equals the lone sequence's backward bit for bit, with the states recomputed and with the
    packed forward's checkpoints handed in.  H = 16 puts N*H past 64 (the 32-column scan tiles);
    l2: the q/k norm inside the call, on raw rows that are not unit-norm."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [0, 1, 63, 64, 65, 200, 130, 0, 17]
    say(f"[case] varlen backward vs lone runs {dtype} H={H} dk={dk} dv={dv} scalar={scalar} l2={l2} "
        f"lengths={lengths}")
    inp, do, dfinal, s0, cu = _packed(lengths, H, dk, dv, dtype, seed=51, scalar=scalar, unit_qk=not l2)
    d = {n: to_dev(x, dtype if n in "qkv" else None, dev) for n, x in inp.items()}
    ddo, dfin, ds0, dcu = to_dev(do, dtype, dev), to_dev(dfinal, dev=dev), to_dev(s0, dev=dev), to_dev(cu, dev=dev)
    args = tuple(d[n] for n in INPUTS)
    got = kda.chunk_prefill_varlen_backward(*args, dcu, ddo, d_final_state=dfin, initial_state=ds0,
                                            scalar_gate=scalar, l2norm_qk=l2)
    _, _, ck = kda.chunk_prefill_varlen(*args, dcu, initial_state=ds0, chunk_size=64, state_interval=64,
                                        scalar_gate=scalar, l2norm_qk=l2)
    given = kda.chunk_prefill_varlen_backward(*args, dcu, ddo, d_final_state=dfin, initial_state=ds0,
                                              chunk_states=ck, scalar_gate=scalar, l2norm_qk=l2)
    torch.cuda.synchronize()
    for n in got:
        assert torch.equal(got[n], given[n]), f"states given vs recomputed: {n}"
    _compare_with_lone_runs(kda, got, d, ddo, dfin, ds0, cu, lengths, scalar, f"{dtype} H={H}", l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_varlen_backward_matches_oracle(oracle, dtype):
    """Each sequence of a packed call within the backward's bar of the oracle's fp64 gradient
    of that sequence alone."""
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lengths = [100, 0, 257, 64, 3]
    H, dk, dv = 2, 64, 64
    say(f"[case] varlen backward vs oracle {dtype} lengths={lengths}")
    inp, do, dfinal, s0, cu = _packed(lengths, H, dk, dv, dtype, seed=52)
    d = {n: to_dev(x, dtype if n in "qkv" else None, dev) for n, x in inp.items()}
    got = kda.chunk_prefill_varlen_backward(*(d[n] for n in INPUTS), to_dev(cu, dev=dev), to_dev(do, dtype, dev),
                                            d_final_state=to_dev(dfinal, dev=dev), initial_state=to_dev(s0, dev=dev))
    for i, L in enumerate(lengths):
        a, b = int(cu[i]), int(cu[i + 1])
        if L == 0:
            assert np.array_equal(host(got["dinit_state"][i]), dfinal[i])
            continue
        one = {n: x[None, a:b] for n, x in inp.items()}
        ref = _ref(oracle, one, do[None, a:b], dfinal[i:i + 1], s0=s0[i:i + 1])
        sub = {n: (x[i:i + 1] if n == "dinit_state" else x[a:b].unsqueeze(0)) for n, x in got.items()}
        _check(f"varlen {dtype} sequence {i} (length {L})", sub, ref, dtype)


def test_varlen_backward_training_mix():
    """The training shape as packed documents: 16384 tokens in 12 sequences of random lengths,
    32 heads, dk = dv = 128, bf16, with the packed forward's checkpoints; four sequences checked
    bit for bit against their lone backward, every gradient finite."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    r = np.random.default_rng(53)
    cuts = np.sort(r.choice(np.arange(1, 16384), 11, replace=False))
    lengths = [int(x) for x in np.diff(np.concatenate([[0], cuts, [16384]]))]
    H, dk, dv = 32, 128, 128
    say(f"[case] varlen backward training mix T={sum(lengths)} lengths={lengths}")
    inp, do, dfinal, s0, cu = _packed(lengths, H, dk, dv, "bf16", seed=53)
    d = {n: to_dev(x, "bf16" if n in "qkv" else None, dev) for n, x in inp.items()}
    ddo, dfin, ds0, dcu = to_dev(do, "bf16", dev), to_dev(dfinal, dev=dev), to_dev(s0, dev=dev), to_dev(cu, dev=dev)
    args = tuple(d[n] for n in INPUTS)
    _, _, ck = kda.chunk_prefill_varlen(*args, dcu, initial_state=ds0, chunk_size=64, state_interval=64)
    got = kda.chunk_prefill_varlen_backward(*args, dcu, ddo, d_final_state=dfin, initial_state=ds0, chunk_states=ck)
    torch.cuda.synchronize()
    for n, x in got.items():
        assert torch.isfinite(x).all(), n
    pick = [0, 3, 7, len(lengths) - 1]
    for i in pick:
        ref = _lone(kda, d, ddo, dfin, ds0, cu, i, False)
        torch.cuda.synchronize()
        a, b = int(cu[i]), int(cu[i + 1])
        for n in TOKEN_GRADS:
            assert torch.equal(got[n][a:b], ref[n][0]), f"{n} of sequence {i} (length {lengths[i]})"
        assert torch.equal(got["dinit_state"][i], ref["dinit_state"][0])
    say(f"[case] checked sequences {pick} of lengths {[lengths[i] for i in pick]}")


def test_varlen_backward_all_empty():
    """Every sequence empty (T = 0): d_init_state = d_final_state, nothing else is touched."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    H, dk, dv = 2, 64, 64
    say("[case] varlen backward, all sequences empty")
    e = torch.empty((0, H, dk), dtype=torch.bfloat16, device=dev)
    ev = torch.empty((0, H, dv), dtype=torch.bfloat16, device=dev)
    la = torch.empty((0, H, dk), dtype=torch.float32, device=dev)
    bt = torch.empty((0, H), dtype=torch.float32, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    dfin = torch.randn(3, H, dk, dv, device=dev)
    got = kda.chunk_prefill_varlen_backward(e, e, ev, la, bt, cu, ev, d_final_state=dfin)
    torch.cuda.synchronize()
    assert torch.equal(got["dinit_state"], dfin)
