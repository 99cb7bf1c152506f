"""GPU parity of kda_decode_step_fused: bit for bit against three kda_short_conv calls
followed by kda_decode_step on the same inputs, against the fp64 oracle composition
(convolution, rounding to the I/O dtype as the convolution stores it, then the decode step),
and its state slots."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, H, dk, dv, W, dtype, seed):
    dims = {"q": H * dk, "k": H * dk, "v": H * dv}
    tids = {"q": D.TID_XQ, "k": D.TID_XK, "v": D.TID_XV}
    x = {n: D.np_raw_x(B, 1, dims[n], dtype, seed, tids[n])[:, 0] for n in "qkv"}
    w = {n: D.np_conv_weight(dims[n], W, seed=3 * seed + i) for i, n in enumerate("qkv")}
    c = {n: D.np_conv_cache(B, W, dims[n], dtype, seed=3 * seed + i) for i, n in enumerate("qkv")}
    b = {n: np.linspace(-0.2, 0.2, dims[n]).astype(np.float32) * (i + 1) for i, n in enumerate("qkv")}
    g = D.np_kda_inputs(B, 1, H, dk, dv, dtype, seed=seed)
    return x, w, c, b, g["log_alpha"][:, 0], g["beta"][:, 0]


def _unfused(kda, xd, wd, cd, bd, la, beta, state, mask, H, silu):
    B = xd["q"].shape[0]
    ys = {}
    for n in "qkv":
        Dn = xd[n].shape[1]
        ys[n] = kda.short_conv(xd[n].view(B, 1, Dn), wd[n], None if bd is None else bd[n],
                               None if mask is None else mask.view(B, 1), cd[n], silu=silu)
    dk, dv = xd["q"].shape[1] // H, xd["v"].shape[1] // H
    return kda.decode_step(ys["q"].view(B, H, dk), ys["k"].view(B, H, dk), ys["v"].view(B, H, dv),
                           la, beta, state, mask=mask, l2norm_qk=True)


@pytest.mark.parametrize("dtype,W,silu,bias", [("bf16", 4, False, False), ("bf16", 3, True, True),
                                              ("fp32", 4, True, False), ("fp32", 2, False, True)])
def test_fused_equals_unfused_bitwise(dtype, W, silu, bias):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv, steps = 3, 4, 128, 64, 3
    say(f"[case] fused decode vs unfused {dtype} W={W} silu={silu} bias={bias}")
    s0 = to_dev(D.np_state(B, H, dk, dv, 0.2, seed=4), dev=dev)
    st_u, st_f = s0.clone(), s0.clone()
    cu = cf = None
    for s in range(steps):
        x, w, c, b, la, beta = _inputs(B, H, dk, dv, W, dtype, seed=40 + s)
        xd = {n: to_dev(x[n], dtype, dev) for n in "qkv"}
        wd = {n: to_dev(w[n], dev=dev) for n in "qkv"}
        bd = {n: to_dev(b[n], dev=dev) for n in "qkv"} if bias else None
        if cu is None:                                  # caches carried over the steps
            cu = {n: to_dev(c[n], dtype, dev) for n in "qkv"}
            cf = {n: cu[n].clone() for n in "qkv"}
        lad, betad = to_dev(la, dev=dev), to_dev(beta, dev=dev)
        mask = to_dev(np.array([1, 0 if s == 1 else 1, 1], np.uint8), dev=dev)
        o_u = _unfused(kda, xd, wd, cu, bd, lad, betad, st_u, mask, H, silu)
        o_f = kda.decode_step_fused(xd["q"], xd["k"], xd["v"], wd["q"], wd["k"], wd["v"],
                                    cf["q"], cf["k"], cf["v"], lad, betad, st_f, H, mask=mask,
                                    biases=None if bd is None else (bd["q"], bd["k"], bd["v"]),
                                    l2norm_qk=True, silu=silu)
        torch.cuda.synchronize()
        assert torch.equal(o_u, o_f), f"o differs at step {s}"
        assert torch.equal(st_u, st_f), f"state differs at step {s}"
        for n in "qkv":
            assert torch.equal(cu[n], cf[n]), f"cache {n} differs at step {s}"


def test_fused_matches_oracle(oracle):
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv, W, steps = 2, 3, 64, 128, 4, 3
    say("[case] fused decode vs oracle (conv, bf16 rounding, step)")
    s0 = D.np_state(B, H, dk, dv, 0.2, seed=7)
    state = to_dev(s0, dev=dev)
    ref_state = s0.astype(np.float64)
    cd = ref_c = None
    for s in range(steps):
        x, w, c, _, la, beta = _inputs(B, H, dk, dv, W, "bf16", seed=70 + s)
        if cd is None:
            cd = {n: to_dev(c[n], "bf16", dev) for n in "qkv"}
            ref_c = {n: c[n].astype(np.float64) for n in "qkv"}
        mask = np.array([1, 0 if s == 1 else 1], np.uint8)
        o = kda.decode_step_fused(*(to_dev(x[n], "bf16", dev) for n in "qkv"),
                                  *(to_dev(w[n], dev=dev) for n in "qkv"),
                                  cd["q"], cd["k"], cd["v"], to_dev(la, dev=dev), to_dev(beta, dev=dev),
                                  state, H, mask=to_dev(mask, dev=dev), l2norm_qk=True)
        y = {}
        for n in "qkv":
            yn, ref_c[n] = oracle.c_short_conv(x[n][:, None, :], w[n], None, mask[:, None], ref_c[n])
            y[n] = D.round_bf16(yn[:, 0].astype(np.float32))      # the conv output as stored
        ref_o, ref_state = oracle.c_decode_step(y["q"].reshape(B, H, dk), y["k"].reshape(B, H, dk),
                                                y["v"].reshape(B, H, dv), la, beta, ref_state,
                                                mask=mask, l2norm_qk=True)
        check(f"fused o step{s}", host(o), ref_o, "bf16")
        for n in "qkv":
            assert np.array_equal(host(cd[n]), ref_c[n]), f"cache {n} step {s}"
    check("fused state", host(state), ref_state, "bf16")


def test_fused_state_slots():
    """Sequence b updates slot[b] of the pool and nothing else; a slot outside the pool
    behaves like a masked sequence."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv, W, S = 4, 2, 128, 128, 4, 9
    say("[case] fused decode state slots")
    x, w, c, _, la, beta = _inputs(B, H, dk, dv, W, "bf16", seed=91)
    slot = np.array([7, 2, -1, 4], np.int32)
    pool = to_dev(np.concatenate([D.np_state(1, H, dk, dv, 0.2, seed=100 + i) for i in range(S)]), dev=dev)
    before = pool.clone()
    xd = {n: to_dev(x[n], "bf16", dev) for n in "qkv"}
    wd = {n: to_dev(w[n], dev=dev) for n in "qkv"}
    cf = {n: to_dev(c[n], "bf16", dev) for n in "qkv"}
    cu = {n: cf[n].clone() for n in "qkv"}
    lad, betad = to_dev(la, dev=dev), to_dev(beta, dev=dev)
    o_f = kda.decode_step_fused(xd["q"], xd["k"], xd["v"], wd["q"], wd["k"], wd["v"], cf["q"], cf["k"],
                                cf["v"], lad, betad, pool, H, slot=to_dev(slot, dev=dev), l2norm_qk=True)
    # reference: gather the used slots, run the unfused step with the bad slot masked, scatter
    valid = slot >= 0
    gathered = torch.stack([before[int(s)] if s >= 0 else torch.zeros_like(before[0]) for s in slot])
    mask = to_dev(valid.astype(np.uint8), dev=dev)
    o_u = _unfused(kda, xd, wd, cu, None, lad, betad, gathered, mask, H, False)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_u)
    assert torch.count_nonzero(o_f[2]) == 0
    for b in range(B):
        if valid[b]:
            assert torch.equal(pool[int(slot[b])], gathered[b])
    untouched = [i for i in range(S) if i not in set(slot[valid].tolist())]
    for i in untouched:
        assert torch.equal(pool[i], before[i]), f"slot {i} changed"
    for n in "qkv":
        assert torch.equal(cf[n], cu[n])


def test_fused_step_in_graph_replays():
    """The fused step captured once in a graph and replayed step after step (new inputs
    copied into the captured buffers eagerly between replays, with a synchronisation each
    time) gives every step the eager result bit for bit."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv, W, steps = 4, 4, 128, 128, 4, 4
    say("[case] fused decode graph replay")
    x0, w, c, _, la0, beta0 = _inputs(B, H, dk, dv, W, "bf16", seed=120)
    wd = {n: to_dev(w[n], dev=dev) for n in "qkv"}
    s0 = to_dev(D.np_state(B, H, dk, dv, 0.2, seed=12), dev=dev)
    # captured buffers
    xg = {n: to_dev(x0[n], "bf16", dev) for n in "qkv"}
    cg = {n: to_dev(c[n], "bf16", dev) for n in "qkv"}
    lag, betag, stg = to_dev(la0, dev=dev), to_dev(beta0, dev=dev), s0.clone()
    og = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)
    ce = {n: cg[n].clone() for n in "qkv"}                 # eager copies
    ste = s0.clone()

    def step(x, cch, la, beta, st, out):
        kda.decode_step_fused(x["q"], x["k"], x["v"], wd["q"], wd["k"], wd["v"], cch["q"], cch["k"],
                              cch["v"], la, beta, st, H, l2norm_qk=True, out=out)

    # warm up on a side stream on scratch copies, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(xg, {n: cg[n].clone() for n in "qkv"}, lag, betag, stg.clone(), torch.empty_like(og))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(xg, cg, lag, betag, stg, og)
    torch.cuda.synchronize()
    # capture does not run the step: reset the captured state and caches to the start
    stg.copy_(s0)
    for n in "qkv":
        cg[n].copy_(ce[n])
    torch.cuda.synchronize()
    for s in range(steps):
        x, _, _, _, la, beta = _inputs(B, H, dk, dv, W, "bf16", seed=130 + s)
        for n in "qkv":
            xg[n].copy_(to_dev(x[n], "bf16", dev))
        lag.copy_(to_dev(la, dev=dev))
        betag.copy_(to_dev(beta, dev=dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oe = torch.empty_like(og)
        step({n: to_dev(x[n], "bf16", dev) for n in "qkv"}, ce, to_dev(la, dev=dev), to_dev(beta, dev=dev), ste, oe)
        torch.cuda.synchronize()
        assert torch.equal(og, oe), f"o differs at replay {s}"
        assert torch.equal(stg, ste), f"state differs at replay {s}"
        for n in "qkv":
            assert torch.equal(cg[n], ce[n]), f"cache {n} differs at replay {s}"
