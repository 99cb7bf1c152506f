"""Thin Python binding over libkda.so (C ABI in include/kda.h).

Argument marshalling only: shapes/dtypes are checked, pointers and the current
HIP stream are passed through, and every step of the computation runs in the
library's gfx950 kernels.  PyTorch provides device memory and streams.  There
is no fallback: if libkda.so is missing or the tensors are not on the GPU, the
call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
KDA_FLAG_L2NORM_QK, KDA_FLAG_SILU, KDA_FLAG_SCALAR_GATE, KDA_FLAG_SERIAL_SCAN = 1, 2, 4, 8
STATUS = {0: "KDA_OK", -1: "KDA_ERR_INVALID_ARG", -2: "KDA_ERR_UNSUPPORTED",
          -3: "KDA_ERR_WORKSPACE", -4: "KDA_ERR_HIP"}
EXPORTS = ("kda_abi_version", "kda_status_string", "kda_last_hip_error",
           "kda_chunk_prefill_workspace_size", "kda_chunk_prefill", "kda_decode_step",
           "kda_short_conv", "kda_decode_step_fused", "kda_chunk_prefill_varlen_workspace_size",
           "kda_chunk_prefill_varlen", "kda_chunk_prefill_noalloc", "kda_noalloc_scratch_bytes",
           "kda_chunk_prefill_backward_workspace_size", "kda_chunk_prefill_backward",
           "kda_chunk_prefill_states", "kda_chunk_prefill_varlen_backward_workspace_size",
           "kda_chunk_prefill_varlen_backward")

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        msg = f"{fn} returned {STATUS.get(status, status)}"
        if status == -4:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


def load():
    """Load libkda.so (raises if it has not been built) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, up = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i, u, sz = ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.kda_abi_version.restype = i
    lib.kda_abi_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i]
    lib.kda_last_hip_error.restype = i
    lib.kda_last_hip_error.argtypes = []
    lib.kda_chunk_prefill_workspace_size.restype = sz
    lib.kda_chunk_prefill_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_chunk_prefill.restype = i
    lib.kda_chunk_prefill.argtypes = [vp, vp, vp, fp, fp, up, fp, vp, fp,
                                      i, i, i, i, i, i, i, u, vp, sz, vp]
    lib.kda_decode_step.restype = i
    lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, up, fp, vp, i, i, i, i, i, u, vp]
    lib.kda_short_conv.restype = i
    lib.kda_short_conv.argtypes = [vp, fp, fp, up, vp, vp, i, i, i, i, i, u, vp]
    lib.kda_decode_step_fused.restype = i
    lib.kda_decode_step_fused.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, fp, vp, vp, vp, fp, fp, up,
                                          fp, vp, vp, i, i, i, i, i, i, i, u, vp]
    lib.kda_chunk_prefill_varlen_workspace_size.restype = sz
    lib.kda_chunk_prefill_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.kda_chunk_prefill_varlen.restype = i
    lib.kda_chunk_prefill_varlen.argtypes = [vp, vp, vp, fp, fp, vp, fp, vp, fp, vp, i, fp, i, i,
                                             i, i, i, i, i, i, i, u, vp, sz, vp]
    lib.kda_chunk_prefill_noalloc.restype = i
    lib.kda_chunk_prefill_noalloc.argtypes = [vp, vp, vp, fp, fp, up, fp, vp, fp,
                                              i, i, i, i, i, i, i, u, vp]
    lib.kda_noalloc_scratch_bytes.restype = sz
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_chunk_prefill_backward_workspace_size.restype = sz
    lib.kda_chunk_prefill_backward_workspace_size.argtypes = [i, i, i, i, i, i, u, i]
    lib.kda_chunk_prefill_backward.restype = i
    lib.kda_chunk_prefill_backward.argtypes = [vp, vp, vp, fp, fp, up, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp,
                                               i, i, i, i, i, i, u, vp, sz, vp]
    lib.kda_chunk_prefill_states.restype = i
    lib.kda_chunk_prefill_states.argtypes = [vp, vp, vp, fp, fp, up, fp, vp, fp, fp, i, i,
                                             i, i, i, i, i, i, i, u, vp, sz, vp]
    lib.kda_chunk_prefill_varlen_backward_workspace_size.restype = sz
    lib.kda_chunk_prefill_varlen_backward_workspace_size.argtypes = [i, i, i, i, i, i, u, i]
    lib.kda_chunk_prefill_varlen_backward.restype = i
    lib.kda_chunk_prefill_varlen_backward.argtypes = [vp, vp, vp, fp, fp, vp, fp, fp, i, vp, fp, fp, fp, fp, fp,
                                                      fp, fp, i, i, i, i, i, i, u, vp, sz, vp]
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise KdaError(fn, status, load().kda_last_hip_error() if status == -4 else 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _req(t, name, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libkda has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def prefill_workspace_size(B, T, H, dk, dv, chunk, dtype_code) -> int:
    return int(load().kda_chunk_prefill_workspace_size(B, T, H, dk, dv, chunk, dtype_code))


def chunk_prefill(q, k, v, log_alpha, beta, mask=None, initial_state=None, chunk_size=64,
                  l2norm_qk=False, out=None, final_state=None, workspace=None, scalar_gate=False,
                  serial_scan=False):
    """KDA prefill.  q,k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32), log_alpha [B,T,H,dk] fp32,
    beta [B,T,H] fp32, mask [B,T] uint8/bool or None, initial_state [B,H,dk,dv] fp32 or None.
    serial_scan: KDA_FLAG_SERIAL_SCAN (each (b, h) scanned as one chain, never in segments).
    Returns (o [B,T,H,dv] in q's dtype, final_state [B,H,dk,dv] fp32)."""
    o, fin, _ = _prefill_batch(q, k, v, log_alpha, beta, mask, initial_state, chunk_size, l2norm_qk,
                               out, final_state, workspace, scalar_gate, None, 0, serial_scan)
    return o, fin


def chunk_prefill_states(q, k, v, log_alpha, beta, mask=None, initial_state=None, chunk_size=64,
                         state_interval=64, chunk_states=None, l2norm_qk=False, out=None,
                         final_state=None, workspace=None, scalar_gate=False):
    """kda_chunk_prefill_states: chunk_prefill that also returns the state after every
    state_interval tokens of each row, chunk_states [B * (T // state_interval), H, dk, dv] fp32
    (row b's j-th state at entry b * (T // state_interval) + j - 1; a given array with fewer
    entries receives those that fit).  With state_interval = 64
    these are the chunk-end states chunk_prefill_backward takes.  Returns (o, final_state,
    chunk_states)."""
    import torch
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if state_interval <= 0:
        raise ValueError("state_interval must be positive")
    n = B * (T // state_interval)
    if chunk_states is None:
        chunk_states = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
    _req(chunk_states, "chunk_states", torch.float32)
    if chunk_states.dim() != 4 or tuple(chunk_states.shape[1:]) != (H, dk, dv):
        raise ValueError(f"chunk_states must be [M,{H},{dk},{dv}], got {tuple(chunk_states.shape)}")
    return _prefill_batch(q, k, v, log_alpha, beta, mask, initial_state, chunk_size, l2norm_qk, out,
                          final_state, workspace, scalar_gate, chunk_states, int(state_interval))


def _prefill_batch(q, k, v, log_alpha, beta, mask, initial_state, chunk_size, l2norm_qk, out,
                   final_state, workspace, scalar_gate, chunk_states, state_interval, serial_scan=False):
    import torch
    lib = load()
    dt = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _req(q, "q")
    _req(k, "k", q.dtype, (B, T, H, dk))
    _req(v, "v", q.dtype, (B, T, H, dv))
    _req(log_alpha, "log_alpha", torch.float32, (B, T, H) if scalar_gate else (B, T, H, dk))
    _req(beta, "beta", torch.float32, (B, T, H))
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        _req(mask, "mask", torch.uint8, (B, T))
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, (B, H, dk, dv))
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _req(out, "out", q.dtype, (B, T, H, dv))
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    _req(final_state, "final_state", torch.float32, (B, H, dk, dv))
    need = prefill_workspace_size(B, T, H, dk, dv, chunk_size, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = ((KDA_FLAG_L2NORM_QK if l2norm_qk else 0) | (KDA_FLAG_SCALAR_GATE if scalar_gate else 0) |
             (KDA_FLAG_SERIAL_SCAN if serial_scan else 0))
    if chunk_states is None:
        st = lib.kda_chunk_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(mask),
                                   _ptr(initial_state), _ptr(out), _ptr(final_state),
                                   B, T, H, dk, dv, int(chunk_size), dt, flags,
                                   _ptr(workspace), wbytes, _stream())
        _check("kda_chunk_prefill", st)
    else:
        st = lib.kda_chunk_prefill_states(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(mask),
                                          _ptr(initial_state), _ptr(out), _ptr(final_state), _ptr(chunk_states),
                                          chunk_states.shape[0], state_interval,
                                          B, T, H, dk, dv, int(chunk_size), dt, flags,
                                          _ptr(workspace), wbytes, _stream())
        _check("kda_chunk_prefill_states", st)
    return out, final_state, chunk_states


def chunk_prefill_noalloc(q, k, v, log_alpha, beta, mask=None, initial_state=None, chunk_size=64,
                          l2norm_qk=False, out=None, final_state=None, scalar_gate=False,
                          serial_scan=False):
    """kda_chunk_prefill_noalloc: chunk_prefill without a workspace (the library's per-GPU
    scratch array stands in for it).  out and final_state may be given so that the call
    itself allocates nothing; otherwise they are allocated here, before the C call."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _req(q, "q")
    _req(k, "k", q.dtype, (B, T, H, dk))
    _req(v, "v", q.dtype, (B, T, H, dv))
    _req(log_alpha, "log_alpha", torch.float32, (B, T, H) if scalar_gate else (B, T, H, dk))
    _req(beta, "beta", torch.float32, (B, T, H))
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        _req(mask, "mask", torch.uint8, (B, T))
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, (B, H, dk, dv))
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _req(out, "out", q.dtype, (B, T, H, dv))
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    _req(final_state, "final_state", torch.float32, (B, H, dk, dv))
    st = lib.kda_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(mask),
                                       _ptr(initial_state), _ptr(out), _ptr(final_state),
                                       B, T, H, dk, dv, int(chunk_size), dt,
                                       (KDA_FLAG_L2NORM_QK if l2norm_qk else 0) |
                                       (KDA_FLAG_SCALAR_GATE if scalar_gate else 0) |
                                       (KDA_FLAG_SERIAL_SCAN if serial_scan else 0), _stream())
    _check("kda_chunk_prefill_noalloc", st)
    return out, final_state


def _given(t):
    """A tensor passed as chunk_states reaches the library as a pointer; an empty one (no
    64-token boundary to hold a state) as NULL, so the workspace is sized from that."""
    return t is not None and t.data_ptr() != 0


def _bwd_flags(scalar_gate, l2norm_qk):
    return (KDA_FLAG_SCALAR_GATE if scalar_gate else 0) | (KDA_FLAG_L2NORM_QK if l2norm_qk else 0)


def backward_workspace_size(B, T, H, dk, dv, dtype_code, states_given=False, scalar_gate=False,
                            l2norm_qk=False):
    """Bytes of workspace kda_chunk_prefill_backward needs (less when the chunk-end states
    are given, more with the per-head gate or the q/k norm)."""
    return int(load().kda_chunk_prefill_backward_workspace_size(
        B, T, H, dk, dv, dtype_code, _bwd_flags(scalar_gate, l2norm_qk), int(bool(states_given))))


def chunk_prefill_backward(q, k, v, log_alpha, beta, d_o, d_final_state=None, mask=None,
                           initial_state=None, workspace=None, chunk_states=None, scalar_gate=False,
                           l2norm_qk=False):
    """Gradients of chunk_prefill for L = sum <d_o, o> + <d_final_state, final_state>.
    Inputs as for chunk_prefill (no flags); d_o [B,T,H,dv] in q's dtype, d_final_state
    [B,H,dk,dv] fp32 or None.  chunk_states: the states chunk_prefill_states wrote for the
    same inputs with state_interval = 64, or None (the forward then runs again inside the
    call).  scalar_gate: log_alpha is one gate per (token, head), [B,T,H], and so is its
    gradient.  l2norm_qk: the forward normalised q and k (chunk_prefill's flag); dq and dk are
    then the gradients with respect to the raw q and k.  Returns a dict of fp32 tensors dq,
    dk, dv, dlog_alpha, dbeta (shapes of the inputs) and dinit_state [B,H,dk,dv]."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _req(q, "q")
    _req(k, "k", q.dtype, (B, T, H, dk))
    _req(v, "v", q.dtype, (B, T, H, dv))
    _req(d_o, "d_o", q.dtype, (B, T, H, dv))
    _req(log_alpha, "log_alpha", torch.float32, (B, T, H) if scalar_gate else (B, T, H, dk))
    _req(beta, "beta", torch.float32, (B, T, H))
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        _req(mask, "mask", torch.uint8, (B, T))
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, (B, H, dk, dv))
    if d_final_state is not None:
        _req(d_final_state, "d_final_state", torch.float32, (B, H, dk, dv))
    if chunk_states is not None:
        _req(chunk_states, "chunk_states", torch.float32, (B * (T // 64), H, dk, dv))
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"dq": torch.empty(B, T, H, dk, **f32), "dk": torch.empty(B, T, H, dk, **f32),
         "dv": torch.empty(B, T, H, dv, **f32),
         "dlog_alpha": torch.empty(*((B, T, H) if scalar_gate else (B, T, H, dk)), **f32),
         "dbeta": torch.empty(B, T, H, **f32), "dinit_state": torch.empty(B, H, dk, dv, **f32)}
    flags = _bwd_flags(scalar_gate, l2norm_qk)
    need = int(lib.kda_chunk_prefill_backward_workspace_size(B, T, H, dk, dv, dt, flags, int(_given(chunk_states))))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(mask),
                                        _ptr(initial_state), _ptr(chunk_states), _ptr(d_o), _ptr(d_final_state),
                                        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]),
                                        _ptr(g["dbeta"]), _ptr(g["dinit_state"]), B, T, H, dk, dv, dt, flags,
                                        _ptr(workspace), wbytes, _stream())
    _check("kda_chunk_prefill_backward", st)
    return g


def prefill_varlen_workspace_size(N, T, H, dk, dv, chunk, dtype_code) -> int:
    return int(load().kda_chunk_prefill_varlen_workspace_size(N, T, H, dk, dv, chunk, dtype_code))


def num_checkpoints(cu_seqlens, state_interval) -> int:
    """Entries of the state checkpoints of a packed prefill: sum over the sequences of
    floor(length / state_interval).  cu_seqlens may be a list or a tensor (a GPU tensor is
    copied to the host, which synchronises)."""
    import torch
    cu = torch.as_tensor(cu_seqlens).to("cpu", torch.int64)
    return int(((cu[1:] - cu[:-1]).clamp_min(0) // int(state_interval)).sum())


def chunk_prefill_varlen(q, k, v, log_alpha, beta, cu_seqlens, initial_state=None, chunk_size=64,
                         l2norm_qk=False, out=None, final_state=None, workspace=None, scalar_gate=False,
                         state_interval=0, chunk_states=None, slot=None, serial_scan=False):
    """KDA prefill of N sequences packed end to end.  q,k [T,H,dk], v [T,H,dv] (bf16 or fp32),
    log_alpha [T,H,dk] fp32 ([T,H] with scalar_gate), beta [T,H] fp32, cu_seqlens [N+1] int32
    on the GPU (sequence i = tokens cu_seqlens[i] .. cu_seqlens[i+1]-1), initial_state
    [N,H,dk,dv] fp32 or None.  Returns (o [T,H,dv] in q's dtype, final_state [N,H,dk,dv] fp32).
    With state_interval > 0 it also saves each sequence's state after every state_interval
    tokens (a multiple of chunk_size) and returns (o, final_state, chunk_states [M,H,dk,dv]),
    sequence by sequence in order; chunk_states is allocated when not given (M from
    cu_seqlens, copied to the host).  With slot ([N] int32 on the GPU), initial_state and
    final_state are a pool [S,H,dk,dv] (pass the same tensor to update it in place) and
    sequence i uses entry slot[i]; final_state must then be given.  serial_scan:
    KDA_FLAG_SERIAL_SCAN (every sequence scanned as one chain, never in segments)."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    T, H, dk = q.shape
    dv = v.shape[-1]
    _req(q, "q")
    _req(k, "k", q.dtype, (T, H, dk))
    _req(v, "v", q.dtype, (T, H, dv))
    _req(log_alpha, "log_alpha", torch.float32, (T, H) if scalar_gate else (T, H, dk))
    _req(beta, "beta", torch.float32, (T, H))
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    n_slots = 0
    if slot is not None:
        _req(slot, "slot", torch.int32, (N,))
        if final_state is None:
            raise ValueError("with slot, final_state (the state pool) must be given")
        n_slots = final_state.shape[0]
    rows = n_slots if slot is not None else N
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, (rows, H, dk, dv))
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    _req(out, "out", q.dtype, (T, H, dv))
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _req(final_state, "final_state", torch.float32, (rows, H, dk, dv))
    n_states = 0
    if state_interval:
        if chunk_states is None:
            m = num_checkpoints(cu_seqlens, state_interval)
            chunk_states = torch.empty((m, H, dk, dv), dtype=torch.float32, device=q.device)
        _req(chunk_states, "chunk_states", torch.float32)
        if chunk_states.dim() != 4 or tuple(chunk_states.shape[1:]) != (H, dk, dv):
            raise ValueError(f"chunk_states must be [M,{H},{dk},{dv}], got {tuple(chunk_states.shape)}")
        n_states = chunk_states.shape[0]
    elif chunk_states is not None:
        raise ValueError("chunk_states needs state_interval > 0")
    need = prefill_varlen_workspace_size(N, T, H, dk, dv, chunk_size, dt)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                      _ptr(cu_seqlens), _ptr(initial_state), _ptr(out), _ptr(final_state),
                                      _ptr(slot), n_slots,
                                      _ptr(chunk_states) if state_interval else None, n_states,
                                      int(state_interval),
                                      N, T, H, dk, dv, int(chunk_size), dt,
                                      (KDA_FLAG_L2NORM_QK if l2norm_qk else 0) |
                                      (KDA_FLAG_SCALAR_GATE if scalar_gate else 0) |
                                      (KDA_FLAG_SERIAL_SCAN if serial_scan else 0),
                                      _ptr(workspace), wbytes, _stream())
    _check("kda_chunk_prefill_varlen", st)
    if state_interval:
        return out, final_state, chunk_states
    return out, final_state


def varlen_backward_workspace_size(N, T, H, dk, dv, dtype_code, states_given=False, scalar_gate=False,
                                   l2norm_qk=False):
    """Bytes of workspace kda_chunk_prefill_varlen_backward needs."""
    return int(load().kda_chunk_prefill_varlen_backward_workspace_size(
        N, T, H, dk, dv, dtype_code, _bwd_flags(scalar_gate, l2norm_qk), int(bool(states_given))))


def chunk_prefill_varlen_backward(q, k, v, log_alpha, beta, cu_seqlens, d_o, d_final_state=None,
                                  initial_state=None, chunk_states=None, workspace=None, scalar_gate=False,
                                  l2norm_qk=False):
    """Gradients of chunk_prefill_varlen (no slots) for
    L = sum <d_o, o> + sum_i <d_final_state[i], final_state[i]>.  Inputs as for
    chunk_prefill_varlen: q,k [T,H,dk], v [T,H,dv], log_alpha [T,H,dk] ([T,H] with
    scalar_gate), beta [T,H], cu_seqlens [N+1] int32 on the GPU, initial_state [N,H,dk,dv] or
    None; d_o [T,H,dv] in q's dtype, d_final_state [N,H,dk,dv] fp32 or None.  chunk_states:
    the checkpoints chunk_prefill_varlen wrote for the same inputs with state_interval = 64
    ([M,H,dk,dv]), or None (the forward then runs again inside the call).  scalar_gate and
    l2norm_qk as for chunk_prefill_backward.  Returns a dict of fp32 tensors dq, dk, dv,
    dlog_alpha, dbeta (shapes of the inputs) and dinit_state [N,H,dk,dv]."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    T, H, dk = q.shape
    dv = v.shape[-1]
    _req(q, "q")
    _req(k, "k", q.dtype, (T, H, dk))
    _req(v, "v", q.dtype, (T, H, dv))
    _req(d_o, "d_o", q.dtype, (T, H, dv))
    _req(log_alpha, "log_alpha", torch.float32, (T, H) if scalar_gate else (T, H, dk))
    _req(beta, "beta", torch.float32, (T, H))
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, (N, H, dk, dv))
    if d_final_state is not None:
        _req(d_final_state, "d_final_state", torch.float32, (N, H, dk, dv))
    n_states = 0
    if chunk_states is not None:
        _req(chunk_states, "chunk_states", torch.float32)
        if chunk_states.dim() != 4 or tuple(chunk_states.shape[1:]) != (H, dk, dv):
            raise ValueError(f"chunk_states must be [M,{H},{dk},{dv}], got {tuple(chunk_states.shape)}")
        n_states = chunk_states.shape[0]
    f32 = dict(dtype=torch.float32, device=q.device)
    g = {"dq": torch.empty(T, H, dk, **f32), "dk": torch.empty(T, H, dk, **f32),
         "dv": torch.empty(T, H, dv, **f32),
         "dlog_alpha": torch.empty(*((T, H) if scalar_gate else (T, H, dk)), **f32),
         "dbeta": torch.empty(T, H, **f32), "dinit_state": torch.empty(N, H, dk, dv, **f32)}
    flags = _bwd_flags(scalar_gate, l2norm_qk)
    need = int(lib.kda_chunk_prefill_varlen_backward_workspace_size(N, T, H, dk, dv, dt, flags,
                                                                    int(_given(chunk_states))))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_prefill_varlen_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                               _ptr(cu_seqlens), _ptr(initial_state), _ptr(chunk_states),
                                               n_states, _ptr(d_o), _ptr(d_final_state), _ptr(g["dq"]),
                                               _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]),
                                               _ptr(g["dbeta"]), _ptr(g["dinit_state"]), N, T, H, dk, dv, dt,
                                               flags, _ptr(workspace), wbytes, _stream())
    _check("kda_chunk_prefill_varlen_backward", st)
    return g


def decode_step(q, k, v, log_alpha, beta, state, mask=None, l2norm_qk=False, out=None,
                scalar_gate=False):
    """One decode step.  q,k [B,H,dk], v [B,H,dv], log_alpha [B,H,dk], beta [B,H],
    state [B,H,dk,dv] fp32 updated in place, mask [B] or None.  Returns o [B,H,dv]."""
    import torch
    lib = load()
    dt = _dtype_code(q)
    B, H, dk = q.shape
    dv = v.shape[-1]
    _req(q, "q")
    _req(k, "k", q.dtype, (B, H, dk))
    _req(v, "v", q.dtype, (B, H, dv))
    _req(log_alpha, "log_alpha", torch.float32, (B, H) if scalar_gate else (B, H, dk))
    _req(beta, "beta", torch.float32, (B, H))
    _req(state, "state", torch.float32, (B, H, dk, dv))
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        _req(mask, "mask", torch.uint8, (B,))
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    _req(out, "out", q.dtype, (B, H, dv))
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(mask),
                             _ptr(state), _ptr(out), B, H, dk, dv, dt,
                             (KDA_FLAG_L2NORM_QK if l2norm_qk else 0) |
                             (KDA_FLAG_SCALAR_GATE if scalar_gate else 0), _stream())
    _check("kda_decode_step", st)
    return out


def decode_step_fused(xq, xk, xv, wq, wk, wv, cache_q, cache_k, cache_v, log_alpha, beta,
                      state, H, mask=None, slot=None, biases=None, l2norm_qk=False, silu=False,
                      out=None, scalar_gate=False):
    """One fused decode step: the three short convs at T = 1 (caches updated in place), the
    optional q/k L2 norm and the state update, in one launch.  xq, xk [B,H*dk], xv [B,H*dv]
    raw inputs; wq, wk [H*dk,W], wv [H*dv,W] fp32; caches [B,W-1,H*d] (x's dtype);
    log_alpha [B,H,dk], beta [B,H]; state [S,H,dk,dv] fp32 pool updated in place at slot[b]
    (slot [B] int32, or None for slot b); mask [B] or None; biases (bq, bk, bv) or None.
    Returns o [B,H,dv]."""
    import torch
    lib = load()
    dt = _dtype_code(xq)
    B = xq.shape[0]
    dk, dv = xq.shape[1] // H, xv.shape[1] // H
    W = wq.shape[1]
    S = state.shape[0]
    _req(xq, "xq", shape=(B, H * dk))
    _req(xk, "xk", xq.dtype, (B, H * dk))
    _req(xv, "xv", xq.dtype, (B, H * dv))
    _req(wq, "wq", torch.float32, (H * dk, W))
    _req(wk, "wk", torch.float32, (H * dk, W))
    _req(wv, "wv", torch.float32, (H * dv, W))
    _req(cache_q, "cache_q", xq.dtype, (B, W - 1, H * dk))
    _req(cache_k, "cache_k", xq.dtype, (B, W - 1, H * dk))
    _req(cache_v, "cache_v", xq.dtype, (B, W - 1, H * dv))
    _req(log_alpha, "log_alpha", torch.float32, (B, H) if scalar_gate else (B, H, dk))
    _req(beta, "beta", torch.float32, (B, H))
    _req(state, "state", torch.float32, (S, H, dk, dv))
    bq = bk = bv = None
    if biases is not None:
        bq, bk, bv = biases
        _req(bq, "bq", torch.float32, (H * dk,))
        _req(bk, "bk", torch.float32, (H * dk,))
        _req(bv, "bv", torch.float32, (H * dv,))
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        _req(mask, "mask", torch.uint8, (B,))
    if slot is not None:
        _req(slot, "slot", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, H, dv), dtype=xq.dtype, device=xq.device)
    _req(out, "out", xq.dtype, (B, H, dv))
    flags = ((KDA_FLAG_L2NORM_QK if l2norm_qk else 0) | (KDA_FLAG_SILU if silu else 0) |
             (KDA_FLAG_SCALAR_GATE if scalar_gate else 0))
    st = lib.kda_decode_step_fused(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv),
                                   _ptr(bq), _ptr(bk), _ptr(bv), _ptr(cache_q), _ptr(cache_k),
                                   _ptr(cache_v), _ptr(log_alpha), _ptr(beta), _ptr(mask),
                                   _ptr(state), _ptr(slot), _ptr(out), B, H, S, dk, dv, W, dt,
                                   flags, _stream())
    _check("kda_decode_step_fused", st)
    return out


def short_conv(x, weight, bias=None, mask=None, conv_cache=None, silu=False, out=None):
    """Masked depthwise causal conv.  x [B,T,D], weight [D,W] fp32, bias [D] or None,
    mask [B,T] or None, conv_cache [B,W-1,D] (x's dtype, updated in place) or None.
    Returns y [B,T,D]."""
    import torch
    lib = load()
    dt = _dtype_code(x)
    B, T, D = x.shape
    W = weight.shape[1]
    _req(x, "x")
    _req(weight, "weight", torch.float32, (D, W))
    if bias is not None:
        _req(bias, "bias", torch.float32, (D,))
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.to(torch.uint8)
        _req(mask, "mask", torch.uint8, (B, T))
    if conv_cache is not None:
        _req(conv_cache, "conv_cache", x.dtype, (B, W - 1, D))
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", x.dtype, (B, T, D))
    st = lib.kda_short_conv(_ptr(x), _ptr(weight), _ptr(bias), _ptr(mask), _ptr(conv_cache),
                            _ptr(out), B, T, D, W, dt, KDA_FLAG_SILU if silu else 0, _stream())
    _check("kda_short_conv", st)
    return out
