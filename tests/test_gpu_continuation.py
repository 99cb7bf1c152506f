"""Cached continuation with padding on the GPU (Transformers issue report on Kimi Linear:
padding in a cached continuation must advance neither the convolution state nor the
recurrent state; the baseline is always the unpadded run, checked on the current outputs
and on a following probe token).

Per sequence: a cached prefix (conv caches and recurrent state produced by the prefill path),
then a continuation left- or right-padded with zero inputs, a 0/1 mask, and random
non-neutral gates at the padded positions.  Pipeline: raw x -> short conv (cache) -> KDA
prefill with in-kernel L2 normalisation of q, k -> probe token via conv(T=1) + decode step.
"""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, metrics, say, to_dev

pytestmark = pytest.mark.gpu


def _raw(n, T, Dm, seed, tid):
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed * 1000 + tid)
    return torch.randn(n, T, Dm, device="cuda:0", generator=g).to(torch.bfloat16)


def _gates(n, T, H, dk, seed):
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    la = -torch.nn.functional.softplus(torch.randn(n, T, H, dk, device="cuda:0", generator=g))
    beta = torch.sigmoid(torch.randn(n, T, H, device="cuda:0", generator=g))
    return la.contiguous(), beta.contiguous()


def _pipeline(x, w, caches, la, beta, H, dk, dv, mask=None, state=None, chunk=64):
    """conv(q,k,v) with the given caches (updated in place) -> prefill; returns (y dict, o, S)."""
    from linear_attention_recurrence_kda_amd import kda
    ys = {n: kda.short_conv(x[n], w[n], None, mask, caches[n]) for n in ("q", "k", "v")}
    B, T = x["q"].shape[:2]
    o, s = kda.chunk_prefill(ys["q"].view(B, T, H, dk), ys["k"].view(B, T, H, dk), ys["v"].view(B, T, H, dv),
                             la, beta, mask=mask, initial_state=state, chunk_size=chunk, l2norm_qk=True)
    return ys, o, s


def _probe(xp, w, caches, la, beta, state, H, dk, dv):
    from linear_attention_recurrence_kda_amd import kda
    ys = {n: kda.short_conv(xp[n], w[n], None, None, caches[n]) for n in ("q", "k", "v")}
    B = xp["q"].shape[0]
    return kda.decode_step(ys["q"].view(B, H, dk), ys["k"].view(B, H, dk), ys["v"].view(B, H, dv),
                           la, beta, state, l2norm_qk=True)


def _run_case(oracle, n_seq, H, dk, dv, prefix_max, cont_max, Tpad, seed, oracle_checks):
    import torch
    dev = device()
    prefixes, conts, sides = D.continuation_lengths(n_seq, seed, prefix_max, 3, cont_max)
    say(f"[case] continuation n={n_seq} H={H} prefixes={prefixes} conts={conts} Tpad={Tpad}")
    dims = {"q": H * dk, "k": H * dk, "v": H * dv}
    gw = torch.Generator(device=dev)
    gw.manual_seed(seed)
    w = {n: (torch.rand(d, 4, device=dev, generator=gw) - 0.5).contiguous() for n, d in dims.items()}

    # ---- cached prefixes through the prefill path
    caches, states, prefix_inputs = [], [], []
    for b in range(n_seq):
        P = prefixes[b]
        x = {n: _raw(1, P, d, seed + b, i) for i, (n, d) in enumerate(dims.items())}
        la, beta = _gates(1, P, H, dk, 100 + seed + b)
        c = {n: torch.zeros(1, 3, d, dtype=torch.bfloat16, device=dev) for n, d in dims.items()}
        ys, _, s = _pipeline(x, w, c, la, beta, H, dk, dv)
        caches.append(c)
        states.append(s)
        prefix_inputs.append((x, la, beta, ys))
    torch.cuda.synchronize()

    # ---- continuation: valid tokens, then the padded batch
    mask_np = D.padded_layout(conts, Tpad, sides)
    mask = to_dev(mask_np, dev=dev)
    xv = [{n: _raw(1, conts[b], d, 500 + seed + b, i) for i, (n, d) in enumerate(dims.items())} for b in range(n_seq)]
    gv = [_gates(1, conts[b], H, dk, 600 + seed + b) for b in range(n_seq)]
    la_pad, beta_pad = _gates(n_seq, Tpad, H, dk, 700 + seed)          # non-neutral gates at pads
    x_pad = {n: torch.zeros(n_seq, Tpad, d, dtype=torch.bfloat16, device=dev) for n, d in dims.items()}
    pos = []
    for b in range(n_seq):
        idx = torch.from_numpy(np.nonzero(mask_np[b])[0]).to(dev)
        pos.append(idx)
        for n in dims:
            x_pad[n][b, idx] = xv[b][n][0]
        la_pad[b, idx] = gv[b][0][0]
        beta_pad[b, idx] = gv[b][1][0]

    def clone(cs):
        return [{n: c[n].clone() for n in c} for c in cs]

    def stack(cs):
        return {n: torch.cat([c[n] for c in cs], 0).contiguous() for n in dims}

    s0 = torch.cat(states, 0).contiguous()
    pad_caches = stack(clone(caches))
    ys_pad, o_pad, s_pad = _pipeline(x_pad, w, pad_caches, la_pad, beta_pad, H, dk, dv, mask=mask, state=s0.clone())
    naive_caches = stack(clone(caches))
    _, o_naive, s_naive = _pipeline(x_pad, w, naive_caches, la_pad, beta_pad, H, dk, dv, mask=None, state=s0.clone())

    base_caches = clone(caches)
    o_base, s_base, ys_base = [], [], []
    for b in range(n_seq):
        ysb, ob, sb = _pipeline(xv[b], w, base_caches[b], gv[b][0], gv[b][1], H, dk, dv, state=states[b].clone())
        o_base.append(ob)
        s_base.append(sb)
        ys_base.append(ysb)
    torch.cuda.synchronize()

    # ---- current outputs, states and conv caches: padded == unpadded
    worst_left = 0.0
    for b in range(n_seq):
        check(f"cont o seq{b} ({sides[b]})", host(o_pad[b, pos[b]]), host(o_base[b][0]), "bf16")
        for n in dims:
            assert torch.equal(ys_pad[n][b, pos[b]], ys_base[b][n][0]), f"conv output {n} seq{b}"
            assert torch.equal(pad_caches[n][b], base_caches[b][n][0]), f"conv cache {n} seq{b}"
        assert torch.count_nonzero(o_pad[b][mask[b] == 0]) == 0
        if sides[b] == "left":
            worst_left = max(worst_left, metrics(host(o_naive[b, pos[b]]), host(o_base[b][0]))[0])
    check("cont state", host(s_pad), host(torch.cat(s_base, 0)), "bf16")
    s_after = s_pad.clone()                    # the probe below advances s_pad in place

    # ---- probe token after the continuation
    xp = {n: _raw(n_seq, 1, d, 900 + seed, i) for i, (n, d) in enumerate(dims.items())}
    lp, bp = _gates(n_seq, 1, H, dk, 901 + seed)
    lp, bp = lp[:, 0].contiguous(), bp[:, 0].contiguous()
    probe_pad = _probe(xp, w, pad_caches, lp, bp, s_pad, H, dk, dv)
    probe_base = _probe(xp, w, stack(base_caches), lp, bp, torch.cat(s_base, 0).contiguous(), H, dk, dv)
    probe_naive = _probe(xp, w, naive_caches, lp, bp, s_naive, H, dk, dv)
    torch.cuda.synchronize()
    check("cont probe", host(probe_pad), host(probe_base), "bf16")

    # ---- positive control: ignoring the mask must visibly change the result
    naive_probe = metrics(host(probe_naive), host(probe_base))[0]
    say(f"[control] naive padding: left-pad valid-output max diff {worst_left:.3f}, probe max diff {naive_probe:.3f}")
    assert naive_probe > 0.02
    if "left" in sides:
        assert worst_left > 0.02

    # ---- parity of sampled heads against the oracle, stage by stage
    for (b, hh) in oracle_checks:
        x, la, beta, ys = prefix_inputs[b]
        yq, yk, yv = (host(ys[n])[0] for n in ("q", "k", "v"))
        sl = lambda y, d: y.reshape(-1, H, d)[:, hh:hh + 1][None]
        _, ref_s = oracle.c_prefill(sl(yq, dk), sl(yk, dk), sl(yv, dv), host(la[:, :, hh:hh + 1]),
                                    host(beta[:, :, hh:hh + 1]), l2norm_qk=True)
        check(f"prefix state seq{b} h{hh}", host(states[b][:, hh:hh + 1]), ref_s, "bf16")
        yq, yk, yv = (host(ys_pad[n])[b] for n in ("q", "k", "v"))
        ref_o, ref_s2 = oracle.c_prefill(sl(yq, dk), sl(yk, dk), sl(yv, dv), host(la_pad[b:b + 1, :, hh:hh + 1]),
                                         host(beta_pad[b:b + 1, :, hh:hh + 1]), mask=mask_np[b:b + 1],
                                         init_state=host(states[b][:, hh:hh + 1]), l2norm_qk=True)
        check(f"cont o seq{b} h{hh} vs oracle", host(o_pad[b:b + 1, :, hh:hh + 1]), ref_o, "bf16")
        check(f"cont state seq{b} h{hh} vs oracle", host(s_after[b:b + 1, hh:hh + 1]), ref_s2, "bf16")
        # conv stage against the oracle (same raw inputs and cache)
        xr = host(x_pad["q"][b:b + 1])
        ref_y, _ = oracle.c_short_conv(xr, host(w["q"]), None, mask_np[b:b + 1], host(caches[b]["q"]))
        check(f"cont conv q seq{b} vs oracle", host(ys_pad["q"][b:b + 1]), ref_y, "bf16")


def test_continuation_small(oracle):
    _run_case(oracle, n_seq=4, H=4, dk=64, dv=64, prefix_max=300, cont_max=64, Tpad=64, seed=1,
              oracle_checks=[(0, 0), (1, 3)])


def test_continuation_full_config(oracle):
    """8 sequences, cached prefixes U{1..8192}, continuations U{3..512} padded to 512
    (even sequences left-padded, odd right-padded), H=32, dk=dv=128, bf16."""
    _run_case(oracle, n_seq=8, H=32, dk=128, dv=128, prefix_max=8192, cont_max=512, Tpad=512, seed=0,
              oracle_checks=[(0, 0), (1, 31)])


def test_left_padding_from_empty_state_is_harmless_even_naively(oracle):
    """The issue report notes that left padding from an empty state did not show the defect:
    with zero conv history and zero state, leading zero-input pads leave everything at zero."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    say("[case] empty-state left padding")
    H, dk, dv, T, L = 2, 64, 64, 40, 25
    dims = {"q": H * dk, "k": H * dk, "v": H * dv}
    gw = torch.Generator(device=dev)
    gw.manual_seed(3)
    w = {n: (torch.rand(d, 4, device=dev, generator=gw) - 0.5).contiguous() for n, d in dims.items()}
    x = {n: torch.zeros(1, T, d, dtype=torch.bfloat16, device=dev) for n, d in dims.items()}
    for i, n in enumerate(dims):
        x[n][0, T - L:] = _raw(1, L, dims[n], 11, i)[0]
    la, beta = _gates(1, T, H, dk, 12)
    c1 = {n: torch.zeros(1, 3, d, dtype=torch.bfloat16, device=dev) for n, d in dims.items()}
    c2 = {n: torch.zeros(1, 3, d, dtype=torch.bfloat16, device=dev) for n, d in dims.items()}
    _, o_naive, s_naive = _pipeline(x, w, c1, la, beta, H, dk, dv)
    xs = {n: x[n][:, T - L:].contiguous() for n in dims}
    _, o_ref, s_ref = _pipeline(xs, w, c2, la[:, T - L:].contiguous(), beta[:, T - L:].contiguous(), H, dk, dv)
    torch.cuda.synchronize()
    check("empty-state left pad o", host(o_naive[:, T - L:]), host(o_ref), "bf16")
    check("empty-state left pad state", host(s_naive), host(s_ref), "bf16")
