"""GPU tests of kda_chunk_prefill_states (the batch prefill that saves the state every
state_interval tokens) and of kda_chunk_prefill_backward fed with those states instead of
running the forward again.  Checkpoints are compared with the oracle's state after the
same prefix (the forward bar); the outputs and the gradients are compared bit for bit with
the calls that save nothing / recompute the states."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu

INPUTS = ("q", "k", "v", "log_alpha", "beta")
GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinit_state")


def _dev(inp, dtype, dev):
    return {n: to_dev(x, dtype if n in ("q", "k", "v") else None, dev) for n, x in inp.items()}


@pytest.mark.parametrize("dtype,chunk,interval", [("bf16", 64, 64), ("bf16", 16, 128), ("fp32", 32, 96)])
def test_prefill_states_match_oracle(oracle, dtype, chunk, interval):
    """Row b's checkpoint j is its state after j * interval tokens (masked positions count
    as tokens that leave the state alone): the oracle's final state over that prefix.  The
    outputs equal those of kda_chunk_prefill bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 2, 300, 2, 64, 64
    say(f"[case] prefill states {dtype} chunk={chunk} interval={interval}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=41)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=41)
    mask = np.ones((B, T), np.uint8)
    mask[0, :20] = 0
    mask[1, 130:140] = 0
    d = _dev(inp, dtype, dev)
    dm, ds0 = to_dev(mask, dev=dev), to_dev(s0, dev=dev)
    o, fin, ck = kda.chunk_prefill_states(*(d[n] for n in INPUTS), mask=dm, initial_state=ds0,
                                          chunk_size=chunk, state_interval=interval)
    per = T // interval
    assert ck.shape == (B * per, H, dk, dv)
    o2, fin2 = kda.chunk_prefill(*(d[n] for n in INPUTS), mask=dm, initial_state=ds0, chunk_size=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    got = host(ck)
    for b in range(B):
        for j in range(1, per + 1):
            L = j * interval
            _, rs = oracle.c_prefill(**{n: x[b:b + 1, :L] for n, x in inp.items()}, mask=mask[b:b + 1, :L],
                                     init_state=s0[b:b + 1])
            check(f"row {b} checkpoint {j}", got[b * per + j - 1], rs[0], dtype)


def test_prefill_states_capacity_and_last_checkpoint():
    """Entries past num_states are not written; when T is a multiple of the interval the last
    checkpoint of a row is its final state."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 3, 256, 2, 128, 128
    say("[case] prefill states capacity")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=42)
    d = _dev(inp, "bf16", dev)
    _, fin, ck = kda.chunk_prefill_states(*(d[n] for n in INPUTS), state_interval=64)
    torch.cuda.synchronize()
    for b in range(B):
        assert torch.equal(ck[4 * b + 3], fin[b]), f"last checkpoint of row {b}"
    part = torch.full((B * 4, H, dk, dv), float("nan"), device=dev)
    kda.chunk_prefill_states(*(d[n] for n in INPUTS), state_interval=64, chunk_states=part[:5])
    torch.cuda.synchronize()
    assert torch.equal(part[:5], ck[:5])
    assert torch.isnan(part[5:]).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_with_given_states_equals_recompute(dtype):
    """States from kda_chunk_prefill_states (chunk 64, interval 64) handed to the backward give
    the gradients of the call that runs the forward again, bit for bit: masks, an initial
    state and a ragged tail included."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv = 2, 300, 3, 128, 128
    say(f"[case] backward with given states {dtype}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=43)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=43)
    mask = np.ones((B, T), np.uint8)
    mask[0, :37] = 0
    mask[1, 250:] = 0
    rng = np.random.default_rng(43)
    do = D.to_storage(rng.normal(0, 1, (B, T, H, dv)).astype(np.float32), dtype)
    dfin = to_dev(rng.normal(0, 1, (B, H, dk, dv)).astype(np.float32), dev=dev)
    d = _dev(inp, dtype, dev)
    dm, ds0, ddo = to_dev(mask, dev=dev), to_dev(s0, dev=dev), to_dev(do, dtype, dev)
    args = tuple(d[n] for n in INPUTS)
    _, _, ck = kda.chunk_prefill_states(*args, mask=dm, initial_state=ds0, chunk_size=64, state_interval=64)
    ref = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin, mask=dm, initial_state=ds0)
    got = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin, mask=dm, initial_state=ds0, chunk_states=ck)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(got[n], ref[n]), n


def test_backward_with_given_states_training_size(oracle):
    """B=4, H=32, T=4096, dk=dv=128, bf16 with the states of the forward call: bit for bit
    the recomputing call, and two heads within the gradient bar of the oracle."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    from tests.test_gpu_backward import _check, _cotangents, _ref
    dev = device()
    B, T, H, dk, dv = 4, 4096, 32, 128, 128
    say("[case] backward with given states, training size")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=44)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 44)
    d = _dev(inp, "bf16", dev)
    args = tuple(d[n] for n in INPUTS)
    ddo, dfin = to_dev(do, "bf16", dev), to_dev(dfinal, dev=dev)
    _, _, ck = kda.chunk_prefill_states(*args, chunk_size=64, state_interval=64)
    got = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin, chunk_states=ck)
    ref_gpu = kda.chunk_prefill_backward(*args, ddo, d_final_state=dfin)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(got[n], ref_gpu[n]), n
    for b, h in ((1, 5), (3, 30)):
        one = {n: x[b:b + 1, :, h:h + 1] for n, x in inp.items()}
        ref = _ref(oracle, one, do[b:b + 1, :, h:h + 1], dfinal[b:b + 1, h:h + 1])
        sub = {n: (got[n][b:b + 1, h:h + 1] if n == "dinit_state" else got[n][b:b + 1, :, h:h + 1])
               for n in GRADS}
        _check(f"given states b{b} h{h}", sub, ref, "bf16")


def test_backward_with_states_of_another_chunk_size(oracle):
    """States saved by a chunk-32 forward (interval 64) differ from the chunk-64 ones only by
    rounding: the gradients stay within the oracle's bar."""
    from linear_attention_recurrence_kda_amd import kda
    from tests.test_gpu_backward import _check, _cotangents, _ref
    dev = device()
    B, T, H, dk, dv = 1, 520, 2, 128, 128
    say("[case] backward with chunk-32 states")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=45)
    do, dfinal = _cotangents(B, T, H, dk, dv, "bf16", 45)
    d = _dev(inp, "bf16", dev)
    args = tuple(d[n] for n in INPUTS)
    _, _, ck = kda.chunk_prefill_states(*args, chunk_size=32, state_interval=64)
    got = kda.chunk_prefill_backward(*args, to_dev(do, "bf16", dev), d_final_state=to_dev(dfinal, dev=dev),
                                     chunk_states=ck)
    _check("chunk-32 states", got, _ref(oracle, inp, do, dfinal), "bf16")


@pytest.mark.parametrize("l2,scalar", [(True, False), (False, True)])
def test_prefill_states_equal_prefix_runs_with_flags(l2, scalar):
    """With the L2-norm flag or the per-head gate, checkpoint j of each row is bit for bit the
    final state of kda_chunk_prefill over that row's first j * interval tokens (the chunk
    boundaries of the prefix and of the whole row coincide)."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, H, dk, dv, interval = 2, 320, 2, 64, 64, 128
    say(f"[case] prefill states vs prefix runs, l2={l2} scalar_gate={scalar}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=46)
    if scalar:
        inp["log_alpha"] = np.ascontiguousarray(inp["log_alpha"][..., 0])
    d = _dev(inp, "bf16", dev)
    s0 = to_dev(D.np_state(B, H, dk, dv, 0.05, seed=46), dev=dev)
    _, fin, ck = kda.chunk_prefill_states(*(d[n] for n in INPUTS), initial_state=s0, chunk_size=32,
                                          state_interval=interval, l2norm_qk=l2, scalar_gate=scalar)
    per = T // interval
    for j in range(1, per + 1):
        L = j * interval
        pre = {n: x[:, :L].contiguous() for n, x in d.items()}
        _, sj = kda.chunk_prefill(*(pre[n] for n in INPUTS), initial_state=s0, chunk_size=32,
                                  l2norm_qk=l2, scalar_gate=scalar)
        torch.cuda.synchronize()
        for b in range(B):
            assert torch.equal(ck[b * per + j - 1], sj[b]), f"row {b} checkpoint {j}"


@pytest.mark.parametrize("T", [1, 40, 63])
def test_backward_with_no_state_boundary(T):
    """Sequences shorter than 64 tokens: the training forward saves no state (an empty tensor,
    which reaches the library as NULL); the backward handed it equals the recomputing call bit
    for bit, in the batch and the packed layouts."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv = 2, 2, 64, 64
    say(f"[case] backward with no 64-token boundary, T={T}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, "bf16", seed=47)
    rng = np.random.default_rng(47)
    do = to_dev(D.to_storage(rng.normal(0, 1, (B, T, H, dv)).astype(np.float32), "bf16"), "bf16", dev)
    dfin = to_dev(rng.normal(0, 1, (B, H, dk, dv)).astype(np.float32), dev=dev)
    d = _dev(inp, "bf16", dev)
    args = tuple(d[n] for n in INPUTS)
    _, _, ck = kda.chunk_prefill_states(*args, chunk_size=64, state_interval=64)
    assert ck.shape[0] == 0
    got = kda.chunk_prefill_backward(*args, do, d_final_state=dfin, chunk_states=ck)
    ref = kda.chunk_prefill_backward(*args, do, d_final_state=dfin)
    cu = to_dev(np.array([0, T, 2 * T], np.int32), dev=dev)
    flat = tuple(x.reshape(B * T, *x.shape[2:]).contiguous() for x in args)
    _, _, ckp = kda.chunk_prefill_varlen(*flat, cu, chunk_size=64, state_interval=64)
    gp = kda.chunk_prefill_varlen_backward(*flat, cu, do.reshape(B * T, H, dv).contiguous(), d_final_state=dfin,
                                           chunk_states=ckp)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(got[n], ref[n]), n
        want = ref[n] if n == "dinit_state" else ref[n].reshape(B * T, *ref[n].shape[2:])
        assert torch.equal(gp[n], want), f"packed {n}"
