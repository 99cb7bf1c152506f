"""Seeded sweep over the supported space of the prefill and its backward, each case against
the fp64 oracle: dtype, head sizes, chunk, batch, length (ragged tails, T below one chunk),
heads, mask pattern (none, left or right padding, scattered holes), initial state, and the two
flags (q/k L2 norm, per-head gate).  The forward is checked on o and the final state; the
backward, fed the chunk-end states of the training forward on the same inputs, on every
gradient.  The cases are drawn once from a fixed seed, so every run checks the same ones."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev
from tests.test_gpu_backward import _check

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(
            dtype=str(r.choice(["bf16", "fp32"])), dk=int(r.choice([16, 32, 64, 128])),
            dv=int(r.choice([16, 32, 64, 128])), chunk=int(r.choice([16, 32, 64])),
            B=int(r.integers(1, 4)), T=int(r.integers(1, 330)), H=int(r.choice([1, 2, 3, 5])),
            mask=str(r.choice(["none", "left", "right", "holes"])), s0=bool(r.integers(0, 2)),
            l2=bool(r.integers(0, 2)), scalar=bool(r.integers(0, 2)), seed=100 + i))
    return out


CASES = _cases()


def _mask(kind, B, T, seed):
    if kind == "none":
        return None
    r = np.random.default_rng(seed)
    m = np.ones((B, T), np.uint8)
    for b in range(B):
        cut = int(r.integers(0, T))
        if kind == "left":
            m[b, :cut] = 0
        elif kind == "right":
            m[b, T - cut:] = 0
        else:
            m[b, r.random(T) < 0.15] = 0
    return m


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_sweep_forward_and_backward(oracle, case):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    c = case
    B, T, H, dk, dv, dtype = c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"]
    say(f"[case] sweep {c}")
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=c["seed"], unit_qk=not c["l2"])
    if c["scalar"]:
        inp["log_alpha"] = np.ascontiguousarray(inp["log_alpha"][..., 0])
    mask = _mask(c["mask"], B, T, c["seed"])
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=c["seed"]) if c["s0"] else None
    rng = np.random.default_rng(c["seed"] + 7)
    do = D.to_storage(rng.normal(0, 1, (B, T, H, dv)).astype(np.float32), dtype)
    dfinal = rng.normal(0, 1, (B, H, dk, dv)).astype(np.float32)

    d = {n: to_dev(x, dtype if n in "qkv" else None, dev) for n, x in inp.items()}
    args = tuple(d[n] for n in ("q", "k", "v", "log_alpha", "beta"))
    dm = None if mask is None else to_dev(mask, dev=dev)
    ds0 = None if s0 is None else to_dev(s0, dev=dev)
    flags = dict(l2norm_qk=c["l2"], scalar_gate=c["scalar"])
    o, fin = kda.chunk_prefill(*args, mask=dm, initial_state=ds0, chunk_size=c["chunk"], **flags)
    _, _, ck = kda.chunk_prefill_states(*args, mask=dm, initial_state=ds0, chunk_size=64, state_interval=64,
                                       **flags)
    g = kda.chunk_prefill_backward(*args, to_dev(do, dtype, dev), d_final_state=to_dev(dfinal, dev=dev),
                                   mask=dm, initial_state=ds0, chunk_states=ck, **flags)
    torch.cuda.synchronize()

    la = inp["log_alpha"] if not c["scalar"] else np.repeat(inp["log_alpha"][..., None], dk, axis=-1)
    ro, rs = oracle.c_prefill(inp["q"], inp["k"], inp["v"], la, inp["beta"], mask=mask, init_state=s0,
                              l2norm_qk=c["l2"])
    check("sweep o", host(o), ro, dtype)
    check("sweep state", host(fin), rs, dtype)
    ref = oracle.np_prefill_backward(inp["q"], inp["k"], inp["v"], la, inp["beta"], do, dfinal, mask=mask,
                                     init_state=s0, l2norm_qk=c["l2"])
    if c["scalar"]:
        ref["dlog_alpha"] = ref["dlog_alpha"].sum(-1)
    _check("sweep", g, ref, dtype)


def _varlen_cases(n=8, seed=77):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(r.integers(1, 6))
        out.append(dict(
            dtype=str(r.choice(["bf16", "fp32"])), dk=int(r.choice([32, 64, 128])), dv=int(r.choice([16, 64, 128])),
            H=int(r.choice([1, 2, 3])), lengths=[int(x) for x in r.integers(0, 260, N)],
            s0=bool(r.integers(0, 2)), l2=bool(r.integers(0, 2)), scalar=bool(r.integers(0, 2)), seed=300 + i))
    return out


VCASES = _varlen_cases()


@pytest.mark.parametrize("case", VCASES, ids=[f"v{i}" for i in range(len(VCASES))])
def test_sweep_packed_forward_and_backward(oracle, case):
    """Packed sequences: every sequence's output, final state and gradients (the packed
    backward fed the packed forward's 64-token checkpoints) against the oracle run on that
    sequence alone."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    c = case
    H, dk, dv, dtype, lengths = c["H"], c["dk"], c["dv"], c["dtype"], c["lengths"]
    N, T = len(lengths), int(sum(lengths))
    say(f"[case] packed sweep {c}")
    inp = {n: x[0] for n, x in D.np_kda_inputs(1, max(T, 1), H, dk, dv, dtype, seed=c["seed"],
                                                 unit_qk=not c["l2"]).items()}
    inp = {n: np.ascontiguousarray(x[:T]) for n, x in inp.items()}
    if c["scalar"]:
        inp["log_alpha"] = np.ascontiguousarray(inp["log_alpha"][..., 0])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s0 = D.np_state(N, H, dk, dv, 0.05, seed=c["seed"]) if c["s0"] else None
    rng = np.random.default_rng(c["seed"] + 7)
    do = D.to_storage(rng.normal(0, 1, (T, H, dv)).astype(np.float32), dtype)
    dfinal = rng.normal(0, 1, (N, H, dk, dv)).astype(np.float32)

    d = {n: to_dev(x, dtype if n in "qkv" else None, dev) for n, x in inp.items()}
    args = tuple(d[n] for n in ("q", "k", "v", "log_alpha", "beta"))
    dcu = to_dev(cu, dev=dev)
    ds0 = None if s0 is None else to_dev(s0, dev=dev)
    flags = dict(l2norm_qk=c["l2"], scalar_gate=c["scalar"])
    o, fin, ck = kda.chunk_prefill_varlen(*args, dcu, initial_state=ds0, chunk_size=64, state_interval=64, **flags)
    g = kda.chunk_prefill_varlen_backward(*args, dcu, to_dev(do, dtype, dev), d_final_state=to_dev(dfinal, dev=dev),
                                          initial_state=ds0, chunk_states=ck, **flags)
    torch.cuda.synchronize()
    for i, L in enumerate(lengths):
        a, b = int(cu[i]), int(cu[i + 1])
        one = {n: x[None, a:b] for n, x in inp.items()}
        la = one["log_alpha"] if not c["scalar"] else np.repeat(one["log_alpha"][..., None], dk, axis=-1)
        si = None if s0 is None else s0[i:i + 1]
        if L == 0:
            want = np.zeros((H, dk, dv)) if si is None else si[0]
            assert np.array_equal(host(fin[i]), want), f"empty sequence {i}: final state"
            assert np.array_equal(host(g["dinit_state"][i]), dfinal[i]), f"empty sequence {i}: dinit"
            continue
        ro, rs = oracle.c_prefill(one["q"], one["k"], one["v"], la, one["beta"], init_state=si, l2norm_qk=c["l2"])
        check(f"packed sweep o[{i}]", host(o[a:b])[None], ro, dtype)
        check(f"packed sweep state[{i}]", host(fin[i:i + 1]), rs, dtype)
        ref = oracle.np_prefill_backward(one["q"], one["k"], one["v"], la, one["beta"], do[None, a:b],
                                         dfinal[i:i + 1], init_state=si, l2norm_qk=c["l2"])
        if c["scalar"]:
            ref["dlog_alpha"] = ref["dlog_alpha"].sum(-1)
        sub = {n: (x[i:i + 1] if n == "dinit_state" else x[a:b].unsqueeze(0)) for n, x in g.items()}
        _check(f"packed sweep grads[{i}]", sub, ref, dtype)
