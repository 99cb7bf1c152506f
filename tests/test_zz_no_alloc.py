"""kda_chunk_prefill_noalloc (the prefill for callers that cannot allocate: its workspace is
the library's per-GPU scratch array) against kda_chunk_prefill with a caller workspace:
same kernels, so the results must be equal bit for bit, and they are checked against the
oracle too.  Two calls in a row, the second smaller, share the array."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _case(B, T, H, dk, dv, chunk, dtype, seed, masked):
    inp = D.np_kda_inputs(B, T, H, dk, dv, dtype, seed=seed)
    s0 = D.np_state(B, H, dk, dv, 0.05, seed=seed)
    mask = None
    if masked:
        mask = np.ones((B, T), np.uint8)
        mask[0, : T // 5] = 0
    return inp, s0, mask


def test_noalloc_equals_workspace_call_twice(oracle):
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lim = int(kda.load().kda_noalloc_scratch_bytes())
    for i, (B, T, H, dk, dv, chunk, dtype, masked) in enumerate(
            [(2, 777, 8, 128, 128, 64, "bf16", True), (1, 130, 3, 64, 128, 32, "fp32", False)]):
        need = kda.prefill_workspace_size(B, T, H, dk, dv, chunk, kda.KDA_BF16 if dtype == "bf16" else kda.KDA_F32)
        assert 0 < need <= lim
        say(f"[case] noalloc call {i}: B={B} T={T} H={H} dk={dk} dv={dv} chunk={chunk} {dtype} "
            f"workspace {need} of {lim} bytes")
        inp, s0, mask = _case(B, T, H, dk, dv, chunk, dtype, 80 + i, masked)
        args = [to_dev(inp[n], dtype, dev) for n in ("q", "k", "v")] + \
               [to_dev(inp["log_alpha"], dev=dev), to_dev(inp["beta"], dev=dev)]
        md = None if mask is None else to_dev(mask, dev=dev)
        sd = to_dev(s0, dev=dev)
        o_ref, s_ref = kda.chunk_prefill(*args, mask=md, initial_state=sd, chunk_size=chunk, l2norm_qk=True)
        o_na, s_na = kda.chunk_prefill_noalloc(*args, mask=md, initial_state=sd, chunk_size=chunk, l2norm_qk=True)
        torch.cuda.synchronize()
        assert torch.equal(o_ref, o_na), f"call {i}: o differs from the workspace call"
        assert torch.equal(s_ref, s_na), f"call {i}: final state differs from the workspace call"
        ro, rs = oracle.c_prefill(**inp, mask=mask, init_state=s0, l2norm_qk=True)
        check(f"noalloc call {i} o", host(o_na), ro, dtype)
        check(f"noalloc call {i} state", host(s_na), rs, dtype)


def test_noalloc_rejects_workspace_beyond_scratch():
    import torch
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    lim = int(kda.load().kda_noalloc_scratch_bytes())
    B, H, dk, dv = 1, 32, 128, 128
    T = 64
    while kda.prefill_workspace_size(B, T, H, dk, dv, 64, kda.KDA_BF16) <= lim:
        T *= 2
    say(f"[case] noalloc rejects T={T} (workspace above {lim} bytes)")
    q = torch.zeros(B, T, H, dk, dtype=torch.bfloat16, device=dev)
    la = torch.zeros(B, T, H, dk, device=dev)
    beta = torch.zeros(B, T, H, device=dev)
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_prefill_noalloc(q, q, q, la, beta)
    assert e.value.status == -3
