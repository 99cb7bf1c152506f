"""GPU parity of kda_decode_step against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _step_inputs(B, H, dk, dv, dtype, seed, decay="default"):
    g = D.np_kda_inputs(B, 1, H, dk, dv, dtype, seed=seed, decay=decay)
    return {n: x[:, 0] for n, x in g.items()}


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_steps_match_oracle(oracle, dk, dv, dtype):
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, steps = 3, 2, 6
    say(f"[case] decode dk={dk} dv={dv} {dtype}")
    s0 = D.np_state(B, H, dk, dv, 0.3, seed=1)
    state = to_dev(s0, dev=dev)
    ref_state = s0.astype(np.float64)
    for s in range(steps):
        inp = _step_inputs(B, H, dk, dv, dtype, seed=100 + s)
        mask = np.array([1, 1 if s % 2 else 0, 1], np.uint8)
        o = kda.decode_step(*(to_dev(inp[n], dtype if n in "qkv" else None, dev) for n in ("q", "k", "v")),
                            to_dev(inp["log_alpha"], dev=dev), to_dev(inp["beta"], dev=dev), state,
                            mask=to_dev(mask, dev=dev))
        ref_o, ref_state = oracle.c_decode_step(**inp, state=ref_state, mask=mask)
        check(f"decode o step{s}", host(o), ref_o, dtype)
    check("decode state", host(state), ref_state, dtype)


def test_masked_decode_leaves_state_bitwise(oracle):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv = 2, 4, 128, 128
    say("[case] decode mask=0 is a no-op")
    inp = _step_inputs(B, H, dk, dv, "bf16", seed=5)
    inp["q"][0] = np.nan                                  # garbage at the masked row never leaks
    inp["log_alpha"][0] = -3.0
    state = to_dev(D.np_state(B, H, dk, dv, 0.1, seed=5), dev=dev)
    before = state.clone()
    o = kda.decode_step(*(to_dev(inp[n], "bf16" if n in "qkv" else None, dev) for n in ("q", "k", "v")),
                        to_dev(inp["log_alpha"], dev=dev), to_dev(inp["beta"], dev=dev), state,
                        mask=to_dev(np.array([0, 1], np.uint8), dev=dev))
    torch.cuda.synchronize()
    assert torch.equal(state[0], before[0])
    assert torch.count_nonzero(o[0]) == 0
    assert not torch.equal(state[1], before[1])


def test_decode_l2norm_flag(oracle):
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv = 2, 3, 64, 64
    say("[case] decode l2norm flag")
    inp = _step_inputs(B, H, dk, dv, "fp32", seed=7)
    inp["q"] = inp["q"] * 3.0
    inp["k"] = inp["k"] * 0.25
    s0 = D.np_state(B, H, dk, dv, 0.2, seed=7)
    state = to_dev(s0, dev=dev)
    o = kda.decode_step(*(to_dev(inp[n], "fp32", dev) for n in ("q", "k", "v")),
                        to_dev(inp["log_alpha"], dev=dev), to_dev(inp["beta"], dev=dev), state, l2norm_qk=True)
    ref_o, ref_s = oracle.c_decode_step(**inp, state=s0, l2norm_qk=True)
    check("decode l2norm o", host(o), ref_o, "fp32")
    check("decode l2norm state", host(state), ref_s, "fp32")


def test_decode_full_size_sampled(oracle):
    """The batched decode workload at full size (256 sequences x 32 heads, 128x128 fp32 states),
    in the launch configuration the benchmark times; sampled (b,h) pairs against the oracle."""
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, H, dk, dv = 256, 32, 128, 128
    say("[case] decode full size 256x32x128x128, 3 steps")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    state = 0.02 * torch.randn(B, H, dk, dv, device=dev, generator=g)
    picks = [(0, 0), (17, 5), (128, 31), (255, 30), (200, 16)]
    ref = {bh: state[bh].double().cpu().numpy() for bh in picks}
    for s in range(3):
        x = D.torch_kda_inputs(B, 1, H, dk, dv, dev, "bf16", seed=10 + s)
        step = {n: t[:, 0].contiguous() for n, t in x.items()}
        o = kda.decode_step(step["q"], step["k"], step["v"], step["log_alpha"], step["beta"], state)
        for (b, h) in picks:
            one = {n: host(step[n][b:b + 1, h:h + 1]) for n in step}
            ro, rs = oracle.c_decode_step(**one, state=ref[(b, h)][None, None])
            ref[(b, h)] = rs[0, 0]
            check(f"decode full o b{b}h{h} step{s}", host(o[b, h]), ro[0, 0], "bf16")
    for (b, h) in picks:
        check(f"decode full state b{b}h{h}", host(state[b, h]), ref[(b, h)], "bf16")
