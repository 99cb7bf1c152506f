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
    assert lib.kda_abi_version() == 1
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
    # the chunk-local grid holds H x chunks workgroups: at most 2^31 - 1
    assert _prefill(lib, T=1 << 30, H=256, chunk=64) == UNSUPPORTED
    assert _prefill(lib, T=-3) == INVALID
    assert _prefill(lib, dtype=2) == INVALID
    assert _prefill(lib, flags=2) == INVALID            # SILU belongs to the short conv
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
    for big in (128, 256):                               # run as 64-token chunks: same workspace
        assert f(4, 4096, 32, 128, 128, big, 0) == f(4, 4096, 32, 128, 128, 64, 0)
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


def test_prefill_varlen_validation(lib):
    assert _varlen(lib, chunk=48) == UNSUPPORTED
    assert _varlen(lib, dv=8) == UNSUPPORTED
    assert _varlen(lib, N=65536) == UNSUPPORTED
    # H x (ceil(T / chunk) + N) chunk workgroups must stay below 2^31
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
