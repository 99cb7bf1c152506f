"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/kda.h declares, and rejects bad arguments with the documented status
before making any HIP call (so no device is touched)."""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_kda_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x10000)          # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10004)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    return kda.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert declared_symbols() == sorted(kda.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 4
    for code in (0, -1, -2, -3, -4):
        assert lib.kda_status_string(code).decode().startswith(kda.STATUS[code])
    assert lib.kda_status_string(17) == b"unknown kda_status"
    assert lib.kda_last_hip_error() == 0


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, mask=None, state=FAKE, o=FAKE,
             B=2, H=2, dk=128, dv=128, dtype=0, flags=0)
    a.update(kw)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["la"], a["beta"], a["mask"], a["state"],
                               a["o"], a["B"], a["H"], a["dk"], a["dv"], a["dtype"], a["flags"], None)


def test_decode_validation(lib):
    assert _decode(lib, dk=7) == UNSUPPORTED
    assert _decode(lib, dv=256) == UNSUPPORTED
    assert _decode(lib, dtype=5) == INVALID
    assert _decode(lib, B=-1) == INVALID
    assert _decode(lib, flags=8) == INVALID
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, state=None) == INVALID
    assert _decode(lib, state=MISALIGNED) == INVALID
    assert _decode(lib, o=ctypes.c_void_p(0x10001)) == INVALID
    assert _decode(lib, B=0) == OK          # nothing to do, nothing launched
    assert _decode(lib, H=0, q=None) == OK


def _fused(lib, **kw):
    a = dict(xq=FAKE, xk=FAKE, xv=FAKE, wq=FAKE, wk=FAKE, wv=FAKE, bq=None, bk=None, bv=None,
             cq=FAKE, ck=FAKE, cv=FAKE, la=FAKE, beta=FAKE, mask=None, state=FAKE, slot=None, o=FAKE,
             B=2, H=2, S=2, dk=128, dv=128, W=4, dtype=0, flags=0)
    a.update(kw)
    return lib.kda_decode_step_fused(a["xq"], a["xk"], a["xv"], a["wq"], a["wk"], a["wv"], a["bq"],
                                     a["bk"], a["bv"], a["cq"], a["ck"], a["cv"], a["la"], a["beta"],
                                     a["mask"], a["state"], a["slot"], a["o"], a["B"], a["H"], a["S"],
                                     a["dk"], a["dv"], a["W"], a["dtype"], a["flags"], None)


def test_fused_decode_validation(lib):
    assert _fused(lib, dk=48) == UNSUPPORTED
    assert _fused(lib, W=5) == UNSUPPORTED
    assert _fused(lib, W=1) == UNSUPPORTED
    assert _fused(lib, dtype=3) == INVALID
    assert _fused(lib, flags=8) == INVALID
    assert _fused(lib, S=-1) == INVALID
    assert _fused(lib, S=1) == INVALID              # no slot array: sequence b needs slot b < S
    assert _fused(lib, xv=None) == INVALID
    assert _fused(lib, cv=None) == INVALID
    assert _fused(lib, state=MISALIGNED) == INVALID
    assert _fused(lib, slot=ctypes.c_void_p(0x10002)) == INVALID
    assert _fused(lib, B=0) == OK                   # nothing to do, nothing launched
    assert _fused(lib, H=0, xq=None) == OK


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, mask=None, s0=None, o=FAKE, sT=FAKE,
             B=1, T=64, H=2, dk=128, dv=128, chunk=64, dtype=0, flags=0, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.kda_chunk_prefill(a["q"], a["k"], a["v"], a["la"], a["beta"], a["mask"], a["s0"],
                                 a["o"], a["sT"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                 a["chunk"], a["dtype"], a["flags"], a["ws"], a["wsb"], None)


def test_prefill_validation(lib):
    assert _prefill(lib, chunk=48) == UNSUPPORTED
    assert _prefill(lib, chunk=512) == UNSUPPORTED
    assert _prefill(lib, chunk=0) == UNSUPPORTED
    assert _prefill(lib, dk=100) == UNSUPPORTED
    assert _prefill(lib, H=65536) == UNSUPPORTED
    assert _prefill(lib, B=65536) == UNSUPPORTED
    # launch extents in threads fit 32 bits: H x chunks workgroups of 256 threads (< 2^24),
    # and the scan's B*H rows rounded up to 8 times 8 tiles of 512 threads (B*H <= 2^20 - 8)
    assert _prefill(lib, T=1 << 30, H=256, chunk=64) == UNSUPPORTED
    # (no workspace given: a supported size stops at the workspace check, before any HIP call)
    assert _prefill(lib, T=64 * ((1 << 19) - 1), H=32, ws=None) == WORKSPACE
    assert _prefill(lib, T=64 * (1 << 19), H=32, ws=None) == UNSUPPORTED
    assert lib.kda_chunk_prefill_workspace_size(1, 64 * ((1 << 19) - 1), 32, 128, 128, 64, 0) > 0
    assert lib.kda_chunk_prefill_workspace_size(1, 64 * (1 << 19), 32, 128, 128, 64, 0) == 0
    assert _prefill(lib, B=32767, H=32, ws=None) == WORKSPACE
    assert _prefill(lib, B=32768, H=32, ws=None) == UNSUPPORTED
    assert _prefill(lib, T=-3) == INVALID
    assert _prefill(lib, dtype=2) == INVALID
    assert _prefill(lib, flags=2) == INVALID            # SILU belongs to the short conv
    assert _prefill(lib, flags=16) == INVALID           # no such flag
    assert _prefill(lib, flags=8, ws=None) == WORKSPACE  # KDA_FLAG_SERIAL_SCAN is accepted
    assert _prefill(lib, v=None) == INVALID
    assert _prefill(lib, sT=None) == INVALID
    assert _prefill(lib, s0=ctypes.c_void_p(0x10002)) == INVALID
    assert _prefill(lib, la=MISALIGNED) == INVALID
    # the per-head gate is read element by element: 4-byte alignment passes (the call then
    # stops at the short workspace, before any launch)
    assert _prefill(lib, la=MISALIGNED, flags=4, wsb=16) == WORKSPACE
    assert _prefill(lib, la=ctypes.c_void_p(0x10002), flags=4) == INVALID
    assert _prefill(lib, v=MISALIGNED) == INVALID
    assert _prefill(lib, o=ctypes.c_void_p(0x10001)) == INVALID
    assert _prefill(lib, wsb=16) == WORKSPACE
    assert _prefill(lib, ws=None) == WORKSPACE
    assert _prefill(lib, B=0, ws=None, wsb=0) == OK


def test_workspace_size_query(lib):
    f = lib.kda_chunk_prefill_workspace_size
    assert f(1, 0, 32, 128, 128, 64, 0) == 0
    assert f(1, 64, 32, 128, 128, 48, 0) == 0            # unsupported chunk
    assert f(1, 64, 32, 100, 128, 64, 0) == 0            # unsupported head size
    one = f(1, 64, 1, 128, 128, 64, 0)
    per_chunk = f(1, 128, 1, 128, 128, 64, 0) - one       # a fixed tail plus a size per chunk
    assert one > 0 and one % 16 == 0 and per_chunk > 0 and per_chunk % 16 == 0
    assert f(1, 65, 1, 128, 128, 64, 0) == one + per_chunk   # ragged tail takes a whole chunk
    assert f(4, 4096, 32, 128, 128, 64, 0) == one + (4 * 32 * 64 - 1) * per_chunk
    assert f(1, 64, 1, 128, 128, 64, 1) > one            # fp32 inputs keep residual parts
    for big in (128, 256):                               # outside the supported chunks
        assert f(4, 4096, 32, 128, 128, big, 0) == 0
    assert f(1, 64, 1, 128, 128, 512, 0) == 0


def _varlen(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, cu=FAKE, s0=None, o=FAKE, sT=FAKE, slot=None,
             nslot=0, ck=None, nck=0, every=0, N=3, T=200, H=2, dk=128, dv=128, chunk=64, dtype=0, flags=0,
             ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.kda_chunk_prefill_varlen(a["q"], a["k"], a["v"], a["la"], a["beta"], a["cu"], a["s0"],
                                        a["o"], a["sT"], a["slot"], a["nslot"], a["ck"], a["nck"], a["every"],
                                        a["N"], a["T"],
                                        a["H"], a["dk"], a["dv"],
                                        a["chunk"], a["dtype"], a["flags"], a["ws"], a["wsb"], None)


def test_prefill_states_validation(lib):
    """kda_chunk_prefill_states: the batch prefill's checks plus those of the state
    checkpoints (a positive multiple of chunk, a 4-byte aligned array, a capacity >= 0); each
    valid case stops at the short workspace, before any HIP call."""
    def call(**kw):
        a = dict(ck=FAKE, nck=4, every=64, B=1, T=256, H=2, chunk=64, wsb=64, flags=0)
        a.update(kw)
        return lib.kda_chunk_prefill_states(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                                            a["ck"], a["nck"], a["every"], a["B"], a["T"], a["H"],
                                            128, 128, a["chunk"], 0, a["flags"], FAKE, a["wsb"], None)
    assert call() == WORKSPACE
    assert call(ck=None) == WORKSPACE                   # no checkpoints: the plain prefill
    assert call(every=0) == INVALID
    assert call(every=96) == INVALID
    assert call(every=48, chunk=32) == INVALID
    assert call(every=96, chunk=32) == WORKSPACE
    assert call(nck=-1) == INVALID
    assert call(ck=ctypes.c_void_p(0x10002)) == INVALID
    assert call(chunk=128) == UNSUPPORTED
    assert call(flags=2) == INVALID
    assert call(B=0) == OK


def test_prefill_varlen_validation(lib):
    assert _varlen(lib, chunk=48) == UNSUPPORTED
    assert _varlen(lib, dv=8) == UNSUPPORTED
    assert _varlen(lib, N=65536) == UNSUPPORTED
    # H x (ceil(T / chunk) + N) chunk workgroups of 256 threads must stay below 2^24
    assert lib.kda_chunk_prefill_varlen_workspace_size(1000, 64 * ((1 << 19) - 1000), 32, 128, 128, 64, 0) == 0
    assert _varlen(lib, T=(1 << 29) - 64 * 1000, N=1000, H=256, chunk=64) == UNSUPPORTED
    assert _varlen(lib, N=-1) == INVALID
    assert _varlen(lib, T=-1) == INVALID
    assert _varlen(lib, flags=2) == INVALID
    assert _varlen(lib, cu=None) == INVALID               # the offsets are required
    assert _varlen(lib, cu=ctypes.c_void_p(0x10002)) == INVALID
    assert _varlen(lib, q=MISALIGNED) == INVALID
    assert _varlen(lib, sT=None) == INVALID
    assert _varlen(lib, beta=None) == INVALID
    # state checkpoints: an interval that is a positive multiple of chunk, a 4-byte aligned
    # array and a capacity >= 0 (each valid case stops at the short workspace, before a launch)
    assert _varlen(lib, ck=FAKE, nck=4, every=0) == INVALID
    assert _varlen(lib, ck=FAKE, nck=4, every=96) == INVALID
    assert _varlen(lib, ck=FAKE, nck=-1, every=128) == INVALID
    assert _varlen(lib, ck=ctypes.c_void_p(0x10002), nck=4, every=128) == INVALID
    assert _varlen(lib, ck=FAKE, nck=4, every=128, wsb=64) == WORKSPACE
    assert _varlen(lib, ck=None, nck=-5, every=-1, wsb=64) == WORKSPACE   # ignored without an array
    assert _varlen(lib, slot=ctypes.c_void_p(0x10002), nslot=4) == INVALID
    assert _varlen(lib, slot=FAKE, nslot=-1) == INVALID
    assert _varlen(lib, slot=FAKE, nslot=8, wsb=64) == WORKSPACE   # a valid slot pool
    assert _varlen(lib, wsb=64) == WORKSPACE
    assert _varlen(lib, ws=None) == WORKSPACE
    assert _varlen(lib, N=0, cu=None, ws=None, wsb=0) == OK   # no sequence: nothing to do


def test_varlen_workspace_size_query(lib):
    f = lib.kda_chunk_prefill_varlen_workspace_size
    g = lib.kda_chunk_prefill_workspace_size
    assert f(0, 100, 32, 128, 128, 64, 0) == 0
    assert f(2, 100, 32, 128, 128, 48, 0) == 0             # unsupported chunk
    assert f(-1, 100, 32, 128, 128, 64, 0) == 0
    assert f(65536, 100, 1, 128, 128, 64, 0) == 0
    # room for ceil(T / chunk) + N chunks per head, plus the chunk table; T = 0 still needs
    # the table (empty sequences copy their state through the scan)
    per_chunk = g(1, 128, 1, 128, 128, 64, 0) - g(1, 64, 1, 128, 128, 64, 0)
    assert f(3, 0, 1, 128, 128, 64, 0) > 3 * per_chunk
    for N, T in ((1, 64), (4, 1000), (17, 4096)):
        nc = -(-T // 64) + N
        base = f(N, T, 2, 128, 128, 64, 0)
        assert base % 16 == 0
        assert base >= 2 * nc * per_chunk
        # one more chunk per head, and 8 more bytes of chunk table (kept 16-byte aligned)
        assert 0 <= f(N, T + 64, 2, 128, 128, 64, 0) - (base + 2 * per_chunk) <= 16
        assert f(N, T, 3, 128, 128, 64, 0) == base + nc * per_chunk


def _conv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, bias=None, mask=None, cache=FAKE, y=FAKE, B=2, T=8, D=64, W=4,
             dtype=0, flags=0)
    a.update(kw)
    return lib.kda_short_conv(a["x"], a["w"], a["bias"], a["mask"], a["cache"], a["y"], a["B"],
                              a["T"], a["D"], a["W"], a["dtype"], a["flags"], None)


def test_conv_validation(lib):
    assert _conv(lib, W=5) == UNSUPPORTED
    assert _conv(lib, W=1) == UNSUPPORTED
    assert _conv(lib, D=12) == UNSUPPORTED
    assert _conv(lib, D=0) == INVALID
    assert _conv(lib, flags=1) == INVALID               # L2NORM belongs to the recurrence
    assert _conv(lib, w=None) == INVALID
    assert _conv(lib, x=None) == INVALID
    assert _conv(lib, cache=MISALIGNED) == INVALID
    assert _conv(lib, T=0) == OK
    assert _conv(lib, B=0) == OK


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.short_conv(x, torch.zeros(8, 4))
    q = torch.zeros(8, 2, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.chunk_prefill_varlen(q, q, q, torch.zeros(8, 2, 16), torch.zeros(8, 2),
                                 torch.tensor([0, 8], dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.chunk_prefill(q[None], q[None], q[None], torch.zeros(1, 8, 2, 16), torch.zeros(1, 8, 2))


def test_checkpoint_count():
    """Entries of the packed prefill's state checkpoints: floor(length / interval) per
    sequence (host-side helper of the binding)."""
    pytest.importorskip("torch")
    assert kda.num_checkpoints([0, 5, 70, 70, 200], 32) == 0 + 2 + 0 + 4
    assert kda.num_checkpoints([0, 64, 128], 64) == 2
    assert kda.num_checkpoints([0], 16) == 0


def test_noalloc_validation(lib):
    """kda_chunk_prefill_noalloc checks its arguments as kda_chunk_prefill does, and rejects a
    call whose workspace would not fit the scratch array, all before any HIP call."""
    lim = lib.kda_noalloc_scratch_bytes()
    assert lim == 256 << 20

    def call(**kw):
        a = dict(B=1, T=4096, H=4, dk=128, dv=128, chunk=64, dtype=0, flags=0, q=FAKE, o=FAKE)
        a.update(kw)
        return lib.kda_chunk_prefill_noalloc(a["q"], FAKE, FAKE, FAKE, FAKE, None, None, a["o"], FAKE,
                                             a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"],
                                             a["dtype"], a["flags"], None)
    assert call(dk=7) == UNSUPPORTED
    assert call(q=MISALIGNED) == INVALID
    assert call(flags=16) == INVALID
    assert call(o=None) == INVALID
    big = 1
    while lib.kda_chunk_prefill_workspace_size(1, big, 32, 128, 128, 64, 0) <= lim:
        big *= 2
    assert call(T=big, H=32) == WORKSPACE
    assert call(B=0) == OK                   # nothing to do: no HIP call either


def test_large_chunks_are_rejected(lib):
    """chunk 128 and 256 are outside the supported set: the size queries return 0 and the
    calls return KDA_ERR_UNSUPPORTED before any HIP call (batch, packed and no-alloc)."""
    for chunk in (128, 256, 48, 0, -64):
        assert lib.kda_chunk_prefill_workspace_size(1, 1024, 4, 128, 128, chunk, 0) == 0
        assert lib.kda_chunk_prefill_varlen_workspace_size(2, 1024, 4, 128, 128, chunk, 0) == 0
        st = lib.kda_chunk_prefill(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                                   1, 1024, 4, 128, 128, chunk, 0, 0, FAKE, 1 << 30, None)
        assert st == UNSUPPORTED, (chunk, st)
        st = lib.kda_chunk_prefill_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                                           1, 1024, 4, 128, 128, chunk, 0, 0, None)
        assert st == UNSUPPORTED, (chunk, st)
    for chunk in (16, 32, 64):
        assert lib.kda_chunk_prefill_workspace_size(1, 1024, 4, 128, 128, chunk, 0) > 0


def test_backward_validation(lib):
    """kda_chunk_prefill_backward rejects bad arguments before any HIP call: flags other than
    the per-head gate and the q/k norm, unsupported head sizes, missing or misaligned
    pointers, a short workspace."""
    assert lib.kda_chunk_prefill_backward_workspace_size(1, 0, 4, 128, 128, 0, 0, 0) == 0
    assert lib.kda_chunk_prefill_backward_workspace_size(1, 16, 4, 24, 128, 0, 0, 0) == 0
    assert lib.kda_chunk_prefill_backward_workspace_size(1, 16, 4, 64, 64, 7, 0, 0) == 0
    bf = lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 0, 0)
    f32 = lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 1, 0, 0)
    assert 0 < bf < f32
    # with the chunk-end states given, the forward's workspace, outputs and states drop out
    bf_s = lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 0, 1)
    fwd = lib.kda_chunk_prefill_workspace_size(2, 130, 3, 64, 32, 64, 0)
    assert 0 < bf_s <= bf - fwd - 2 * 130 * 3 * 32 * 2 - 2 * 3 * 64 * 32 * 4 - 2 * 2 * 3 * 64 * 32 * 4
    # the chunk operands alone (scan fragments, P^T, G, M, dP, dG, dS1, dU, U): 2 * 3 * 3 chunks
    assert bf > 2 * 3 * 3 * (3 * 64 * 64 * 2 + 64 * 64 * 4 + 4 * 64 * 64 * 4 + 64 * 32 * 4 * 3)

    def call(**kw):
        a = dict(B=1, T=33, H=2, dk=64, dv=64, dtype=0, flags=0, q=FAKE, dq=FAKE, s0=None, dinit=FAKE,
                 ws=FAKE, wsb=1 << 30, cs=None)
        a.update(kw)
        return lib.kda_chunk_prefill_backward(a["q"], FAKE, FAKE, FAKE, FAKE, None, a["s0"], a["cs"], FAKE, None,
                                              a["dq"], FAKE, FAKE, FAKE, FAKE, a["dinit"],
                                              a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dtype"],
                                              a["flags"], a["ws"], a["wsb"], None)
    assert call(flags=1, ws=None) == WORKSPACE   # the q/k L2 norm: accepted
    assert call(flags=5, ws=None) == WORKSPACE
    assert call(flags=2) == INVALID           # SILU belongs to the short conv
    assert call(flags=8) == INVALID
    assert call(flags=4, ws=None) == WORKSPACE   # the per-head gate: accepted
    # the per-head gate needs its per-channel gradient in the workspace (the sum comes after)
    assert (lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 4, 0)
            == lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 0, 0) + 2 * 130 * 3 * 64 * 4)
    # the q/k norm adds the two row scales per token and head (rounded up to 256 bytes)
    assert (lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 1, 0)
            == lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 0, 0) + 6400)
    assert lib.kda_chunk_prefill_backward_workspace_size(2, 130, 3, 64, 32, 0, 2, 0) == 0
    assert call(dk=48) == UNSUPPORTED
    assert call(dtype=5) == INVALID
    assert call(T=-1) == INVALID
    assert call(q=None) == INVALID
    assert call(q=MISALIGNED) == INVALID      # 16-byte alignment for the vector loads
    assert call(dq=MISALIGNED) == INVALID
    assert call(s0=MISALIGNED) == INVALID
    assert call(dinit=None) == INVALID
    assert call(cs=MISALIGNED) == INVALID     # chunk-end states: 16-byte vector loads
    assert call(cs=ctypes.c_void_p(0x10008)) == INVALID
    assert call(cs=FAKE, ws=None) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(ws=ctypes.c_void_p(0x10010)) == WORKSPACE   # 256-byte alignment
    assert call(H=0) == OK                   # nothing to do: no HIP call either
    # launch extents in threads fit 32 bits: B*H*ceil(T/64) <= 2^22 - 8 for the channel-slice grid
    assert lib.kda_chunk_prefill_backward_workspace_size(64, 64 * 1023, 64, 128, 128, 0, 0, 0) > 0
    assert lib.kda_chunk_prefill_backward_workspace_size(64, 64 * 1024, 64, 128, 128, 0, 0, 0) == 0
    assert lib.kda_chunk_prefill_backward_workspace_size(64, 64 * 1024, 64, 128, 128, 0, 0, 1) == 0
    assert call(B=64, T=64 * 1023, H=64, ws=None) == WORKSPACE
    assert call(B=64, T=64 * 1024, H=64, ws=None) == UNSUPPORTED


def test_varlen_backward_validation(lib):
    """kda_chunk_prefill_varlen_backward: the backward's checks plus cu_seqlens, and a
    workspace of ceil(T/64) + N chunk slots per head (with the states given, that of a batch
    row of as many chunks plus the sequence and chunk tables)."""
    size = lib.kda_chunk_prefill_varlen_backward_workspace_size
    bsize = lib.kda_chunk_prefill_backward_workspace_size
    # 3 sequences, 130 tokens: 3 + 3 = 6 slots per head, as a 384-token batch row; tables of
    # 3 x 16 and 6 x 8 bytes, each rounded up to 256
    assert size(3, 130, 2, 64, 64, 0, 0, 1) == bsize(1, 384, 2, 64, 64, 0, 0, 1) + 256 + 256
    assert size(3, 130, 2, 64, 64, 1, 4, 1) == bsize(1, 384, 2, 64, 64, 1, 0, 1) + 512 + 130 * 2 * 64 * 4
    # without the states, the packed forward's workspace, outputs and checkpoints come in
    assert size(3, 130, 2, 64, 64, 0, 0, 0) > size(3, 130, 2, 64, 64, 0, 0, 1) + \
        lib.kda_chunk_prefill_varlen_workspace_size(3, 130, 2, 64, 64, 64, 0)
    assert size(3, 0, 2, 64, 64, 0, 0, 1) > 0              # the sequence table: d_init = d_final
    assert size(3, 130, 2, 64, 64, 0, 1, 1) == size(3, 130, 2, 64, 64, 0, 0, 1) + 2304   # q/k norm scales
    assert size(3, 130, 2, 64, 64, 0, 2, 0) == 0           # SILU: not a backward flag
    assert size(3, 130, 2, 48, 64, 0, 0, 0) == 0
    assert size(70000, 130, 2, 64, 64, 0, 0, 0) == 0       # N <= 65535
    # launch extents: H (ceil(T/64) + N) <= 2^22 - 8
    assert size(15, 64 * 65520, 64, 128, 128, 0, 0, 1) > 0
    assert size(15, 64 * 65521, 64, 128, 128, 0, 0, 1) == 0
    cu = FAKE

    def call(**kw):
        a = dict(N=2, T=100, H=2, dk=64, dv=64, dtype=0, flags=0, q=FAKE, dq=FAKE, s0=None, dinit=FAKE,
                 ws=FAKE, wsb=1 << 30, cs=None, ns=0, cu=cu)
        a.update(kw)
        return lib.kda_chunk_prefill_varlen_backward(a["q"], FAKE, FAKE, FAKE, FAKE, a["cu"], a["s0"], a["cs"],
                                                     a["ns"], FAKE, None, a["dq"], FAKE, FAKE, FAKE, FAKE,
                                                     a["dinit"], a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                                     a["dtype"], a["flags"], a["ws"], a["wsb"], None)
    assert call(flags=1, ws=None) == WORKSPACE
    assert call(flags=2) == INVALID
    assert call(flags=4, ws=None) == WORKSPACE
    assert call(cu=None) == INVALID
    assert call(cu=ctypes.c_void_p(0x10002)) == INVALID      # int32 offsets
    assert call(cs=FAKE, ns=-1) == INVALID
    assert call(cs=MISALIGNED, ns=1) == INVALID
    assert call(cs=FAKE, ns=1, ws=None) == WORKSPACE
    assert call(q=None) == INVALID
    assert call(dq=MISALIGNED) == INVALID
    assert call(dinit=None) == INVALID
    assert call(s0=MISALIGNED) == INVALID
    assert call(dk=48) == UNSUPPORTED
    assert call(N=-1) == INVALID
    assert call(N=70000) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(N=0) == OK                      # nothing to do
    assert call(H=0) == OK
    assert call(N=15, T=64 * 65521, H=64, dk=128, dv=128, ws=None) == UNSUPPORTED


def test_segmented_workspace_size(lib):
    """A batch prefill that may run as a segmented scan (bf16, dv = 128, B*H < 64, at least 128
    chunks) needs, after the chunks and the 16 KB sink (rounded up to 256 bytes), one fp32
    dk x dv entry state and one int per (b, h, segment); otherwise only chunks and sink."""
    def size(B, T, H, dk=128, dv=128, chunk=64, dtype=0):
        return lib.kda_chunk_prefill_workspace_size(B, T, H, dk, dv, chunk, dtype)
    per_chunk = (size(1, 64, 1) - 16384)                    # one (b, h) chunk
    assert per_chunk > 0
    plain = lambda B, T, H: B * H * ((T + 63) // 64) * per_chunk + 16384
    assert size(1, 8128, 2) == plain(1, 8128, 2)            # 127 chunks: one chain
    for B, T, H, G in ((1, 8192, 2, 2), (1, 16421, 2, 4), (1, 131072, 32, 2), (2, 8192, 4, 2)):
        base = plain(B, T, H)
        want = (base + 255) // 256 * 256 + B * H * G * (128 * 128 * 4 + 4)
        assert size(B, T, H) == want, (B, T, H)
    assert size(1, 8192, 64) == plain(1, 8192, 64)          # 64 (b, h) pairs: never segmented
    assert size(1, 8192, 2, dv=64) == (lambda pc: 2 * 128 * pc + 16384)(size(1, 64, 1, dv=64) - 16384)
    fp = size(1, 8192, 2, dtype=1)                          # fp32: never segmented
    assert fp == 2 * 128 * (size(1, 64, 1, dtype=1) - 16384) + 16384


def test_segmented_varlen_workspace_size(lib):
    """The packed prefill reserves, when it may segment (bf16, dv = 128, fewer than 64
    (sequence, head) pairs, at least 128 chunks in the bound), one fp32 dk x dv entry state
    and one int for each of its at most H * min(chunks / 64, N * Gmax) (sequence, head,
    segment) jobs after its chunk table (Gmax: the most segments H heads allow)."""
    def size(N, T, H, dk=128, dv=128, dtype=0):
        return lib.kda_chunk_prefill_varlen_workspace_size(N, T, H, dk, dv, 64, dtype)
    def a16(x):
        return (x + 15) // 16 * 16
    per_chunk = lib.kda_chunk_prefill_workspace_size(1, 64, 1, 128, 128, 64, 0) - 16384
    def base(N, T, H):
        nc = (T + 63) // 64 + N
        return H * nc * per_chunk + 16384 + a16(nc * 8) + N * 16 + a16((N + 1) * 4)
    def gmax(H):
        g = 1
        while H * g < 64:
            g *= 2
        return g
    for N, T, H in ((3, 8000, 2), (6, 17766, 2), (1, 1 << 20, 32), (1, 131072, 32)):
        nc = (T + 63) // 64 + N
        jobs = H * min(nc // 64, N * gmax(H))
        want = (base(N, T, H) + 255) // 256 * 256 + jobs * (128 * 128 * 4 + 4)
        assert nc >= 128 and size(N, T, H) == want, (N, T, H)
    assert size(32, 131072, 32) == base(32, 131072, 32)    # 1024 (sequence, head) pairs: never
    assert size(2, 8000, 64) == base(2, 8000, 64)          # 64 heads: never segmented
    assert size(2, 64 * 100, 2) == base(2, 64 * 100, 2)    # 102 chunks: too short
