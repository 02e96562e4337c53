"""Kimi Delta Attention on MI355X: Python binding of the C-ABI library libkda.so.

This module only marshals arguments: it allocates outputs with torch, passes
raw device pointers and the current HIP stream to the C entry points declared
in ``include/kda.h``, and turns status codes into exceptions.  Every step of
the computation runs in the HIP kernels; there is no CPU or PyTorch fallback,
and a missing library is an error.

    o, S_T, ckpt = prefill(q, k, v, g, beta, S0=None, checkpoint_every=0)
    o = decode_step(q, k, v, g, beta, S)        # S updated in place

    # speculative decoding: outputs of T draft tokens, then commit the accepted ones
    o = decode_multi(q, k, v, g, beta, S, update_state=False)          # [N,T,H,...] inputs
    decode_multi(q, k, v, g, beta, S, n_tokens=accepted, want_output=False)

    # packed sequences of different lengths: q [total_T,H,dk], offsets on the host
    o, S_T, ckpt = prefill_varlen(q, k, v, g, beta, cu_seqlens, S0=None, checkpoint_every=0)

    # the layer core: short convolution, L2 norm, sigmoid gates, output norm/gate
    o, S_T, ckpt, conv = prefill_layer(q, k, v, a, b, conv_w=w, silu=True, z=z, norm_w=nw)
    o = decode_layer_step(q1, k1, v1, a1, b1, S, conv_state=conv, conv_w=w, silu=True, z=z1)
    y = output_norm_gate(o, z, norm_w=nw)

    # the two bf16 prefill stages, separately (together: exactly prefill)
    ws = workspace(q, v)
    prefill_chunk_prep(q, k, v, g, beta, ws)
    o, S_T, ckpt = prefill_chunk_recur(ws, q, v, S0=None, checkpoint_every=0)

Shapes (dense, contiguous, on the GPU): prefill q, k, g [B,T,H,dk], v [B,T,H,dv],
beta [B,T,H], S0 [B,H,dk,dv]; decode q, k, g [N,H,dk], v [N,H,dv], beta [N,H],
S [N,H,dk,dv].  q, k, v share one dtype (bfloat16 or float32); g, beta and the
states are float32.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

from ._build import LIB as LIBRARY_PATH

__all__ = ["prefill", "prefill_noalloc", "prefill_chunk_prep", "prefill_chunk_recur", "workspace", "prefill_varlen",
           "decode_step", "decode_multi", "prefill_layer", "decode_layer_step", "output_norm_gate",
           "LayerOpts", "prefill_workspace", "varlen_workspace", "segment_tokens", "prefill_segment_prep",
           "prefill_segment_recur",
           "library", "KDAError", "HEADER_PATH", "LIBRARY_PATH", "declared_functions",
           "status_string", "CHUNK"]

HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "kda.h")
CHUNK = 64  # prefill chunk length; checkpoint intervals are multiples of it

KDA_FP32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_FP32, torch.bfloat16: KDA_BF16}

_lib = None
_lock = threading.Lock()


class LayerOpts(ctypes.Structure):
    """kda_layer_opts of include/kda.h."""
    _fields_ = [("conv_w", ctypes.c_void_p), ("conv_width", ctypes.c_int), ("conv_silu", ctypes.c_int),
                ("gate_z", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


class KDAError(RuntimeError):
    """A kda_* call returned a status other than KDA_OK."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s" % (where, status_string(code)))


def library() -> ctypes.CDLL:
    """Load libkda.so (built by ``__graft_entry__.build()``) and declare its ABI."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY_PATH):
                raise RuntimeError("libkda.so is not built (%s); run __graft_entry__.build()"
                                   % LIBRARY_PATH)
            lib = ctypes.CDLL(LIBRARY_PATH)
            vp, fp, ci, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            lib.kda_prefill_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
            lib.kda_prefill_workspace_size.restype = sz
            lib.kda_prefill_stage_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
            lib.kda_prefill_stage_workspace_size.restype = sz
            lib.kda_prefill_segment_tokens.argtypes = [ci, ci, ci, ci, ci, ci]
            lib.kda_prefill_segment_tokens.restype = ci
            lib.kda_prefill_segment_prep.argtypes = [vp, vp, vp, fp, fp, ci, ci, ci, ci, ci, ci, ci, ci,
                                                     vp, sz, vp]
            lib.kda_prefill_segment_prep.restype = ci
            lib.kda_prefill_segment_recur.argtypes = [vp, sz, fp, vp, fp, fp, ci, ci, ci, ci, ci, ci, ci,
                                                      ci, ci, vp]
            lib.kda_prefill_segment_recur.restype = ci
            lib.kda_prefill.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, ci,
                                        ci, ci, ci, ci, ci, ci, vp, sz, vp]
            lib.kda_prefill.restype = ci
            lib.kda_prefill_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, ci,
                                                ci, ci, ci, ci, ci, ci, vp]
            lib.kda_prefill_noalloc.restype = ci
            lib.kda_prefill_chunk_prep.argtypes = [vp, vp, vp, fp, fp, ci, ci, ci, ci, ci, ci,
                                                   vp, sz, vp]
            lib.kda_prefill_chunk_prep.restype = ci
            lib.kda_prefill_chunk_recur.argtypes = [vp, sz, fp, vp, fp, fp, ci, ci, ci, ci, ci, ci,
                                                    ci, vp]
            lib.kda_prefill_chunk_recur.restype = ci
            ip = ctypes.POINTER(ctypes.c_int)
            lib.kda_prefill_varlen_workspace_size.argtypes = [ip, ci, ci, ci, ci, ci]
            lib.kda_prefill_varlen_workspace_size.restype = sz
            lib.kda_prefill_varlen_num_checkpoints.argtypes = [ip, ci, ci]
            lib.kda_prefill_varlen_num_checkpoints.restype = ctypes.c_longlong
            lib.kda_prefill_varlen.argtypes = [vp, vp, vp, fp, fp, ip, ci, fp, vp, fp, fp, ci, ci, ci,
                                               ci, ci, vp, sz, vp]
            lib.kda_prefill_varlen.restype = ci
            lib.kda_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, ci, ci, ci, ci, ci, vp]
            lib.kda_decode_step.restype = ci
            lib.kda_decode_multi.argtypes = [vp, vp, vp, fp, fp, fp, vp, vp, ci, ci, ci, ci, ci, ci,
                                             ci, vp]
            lib.kda_decode_multi.restype = ci
            op = ctypes.POINTER(LayerOpts)
            lib.kda_prefill_layer.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, vp, fp, fp, ci, ci, ci, ci,
                                              ci, ci, ci, op, vp, sz, vp]
            lib.kda_prefill_layer.restype = ci
            lib.kda_decode_layer_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, ci, ci, ci, ci, ci, op, vp]
            lib.kda_decode_layer_step.restype = ci
            lib.kda_output_norm_gate.argtypes = [vp, vp, fp, ctypes.c_float, vp, ctypes.c_longlong, ci, ci,
                                                 vp]
            lib.kda_output_norm_gate.restype = ci
            lib.kda_status_string.argtypes = [ci]
            lib.kda_status_string.restype = ctypes.c_char_p
            lib.kda_version.argtypes = []
            lib.kda_version.restype = ci
            _lib = lib
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/kda.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def status_string(code: int) -> str:
    return library().kda_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tensor(name, t, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def prefill(q, k, v, g, beta, S0=None, checkpoint_every: int = 0, o=None, S_T=None, ckpt=None, ws=None):
    """Chunked KDA prefill (kda_prefill).  Returns (o, S_T, ckpt or None).

    ``o``, ``S_T``, ``ckpt`` and the workspace ``ws`` (``prefill_workspace``)
    may be passed in to reuse buffers; ``S_T`` may be the same tensor as
    ``S0``.  Checkpoint j is the state after token
    min((j+1) * checkpoint_every, T).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    dt = q.dtype
    for name, t, shp, ty in (("q", q, (B, T, H, dk), dt), ("k", k, (B, T, H, dk), dt),
                             ("v", v, (B, T, H, dv), dt), ("g", g, (B, T, H, dk), torch.float32),
                             ("beta", beta, (B, T, H), torch.float32)):
        _check_tensor(name, t, shp, ty)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32)
    n_ck = -(-T // checkpoint_every) if checkpoint_every > 0 else 0
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if n_ck and ckpt is None:
        ckpt = torch.empty((n_ck, B, H, dk, dv), dtype=torch.float32, device=dev)
    _check_tensor("o", o, (B, T, H, dv), dt)
    _check_tensor("S_T", S_T, (B, H, dk, dv), torch.float32)
    if n_ck:
        _check_tensor("ckpt", ckpt, (n_ck, B, H, dk, dv), torch.float32)
    lib = library()
    if ws is None:
        ws_bytes = lib.kda_prefill_workspace_size(B, T, H, dk, dv, _DTYPES[dt])
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    ws_bytes = _ws_bytes(ws)
    rc = lib.kda_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                         _ptr(S_T), _ptr(ckpt if n_ck else None), int(checkpoint_every),
                         B, T, H, dk, dv, _DTYPES[dt], _ptr(ws), ws_bytes, _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill")
    return o, S_T, (ckpt if n_ck else None)


def prefill_noalloc(q, k, v, g, beta, S0=None, checkpoint_every: int = 0, o=None, S_T=None, ckpt=None):
    """kda_prefill_noalloc: prefill() without a workspace (the library's static
    device scratch holds the records).  Returns (o, S_T, ckpt or None); pass
    o, S_T and ckpt to make the call allocate nothing at all."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    dt = q.dtype
    for name, t, shp, ty in (("q", q, (B, T, H, dk), dt), ("k", k, (B, T, H, dk), dt),
                             ("v", v, (B, T, H, dv), dt), ("g", g, (B, T, H, dk), torch.float32),
                             ("beta", beta, (B, T, H), torch.float32)):
        _check_tensor(name, t, shp, ty)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32)
    n_ck = -(-T // checkpoint_every) if checkpoint_every > 0 else 0
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if n_ck and ckpt is None:
        ckpt = torch.empty((n_ck, B, H, dk, dv), dtype=torch.float32, device=dev)
    _check_tensor("o", o, (B, T, H, dv), dt)
    _check_tensor("S_T", S_T, (B, H, dk, dv), torch.float32)
    if n_ck:
        _check_tensor("ckpt", ckpt, (n_ck, B, H, dk, dv), torch.float32)
    rc = library().kda_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                       _ptr(S_T), _ptr(ckpt if n_ck else None), int(checkpoint_every),
                                       B, T, H, dk, dv, _DTYPES[dt], _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_noalloc")
    return o, S_T, (ckpt if n_ck else None)


def workspace(q, v, t_len: int | None = None):
    """A device workspace for the bf16 stage entry points: the records of all T
    tokens of prefill inputs shaped like q [B,T,H,dk], v [B,T,H,dv]
    (kda_prefill_stage_workspace_size), or of a segment of t_len tokens.
    None when the size is 0."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    n = library().kda_prefill_stage_workspace_size(B, T if t_len is None else int(t_len), H, dk, dv,
                                                   _DTYPES[q.dtype])
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def prefill_workspace(q, v):
    """A device workspace of kda_prefill_workspace_size bytes: what prefill()
    and prefill_layer() need (the records of one segment)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    n = library().kda_prefill_workspace_size(B, T, H, dk, dv, _DTYPES[q.dtype])
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def varlen_workspace(q, v, cu_seqlens):
    """A device workspace for prefill_varlen on packed inputs shaped like q
    [total_T,H,dk], v [total_T,H,dv] with these host offsets."""
    TT, H, dk = q.shape
    cu, S = _cu_array(cu_seqlens)
    n = library().kda_prefill_varlen_workspace_size(cu, S, H, dk, v.shape[-1], _DTYPES[q.dtype])
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def segment_tokens(q, v) -> int:
    """The segment length prefill() uses for inputs shaped like q and v."""
    B, T, H, dk = q.shape
    return int(library().kda_prefill_segment_tokens(B, T, H, dk, v.shape[-1], _DTYPES[q.dtype]))


def prefill_segment_prep(q, k, v, g, beta, t_begin: int, t_len: int, ws):
    """Stage 1 over tokens [t_begin, t_begin + t_len) (kda_prefill_segment_prep);
    q, k, v, g, beta are the full [B,T,H,...] tensors, ws holds the segment's
    records (``workspace(q, v, t_len)``)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt != torch.bfloat16:
        raise ValueError("the prefill stages take bfloat16 q, k, v")
    for name, t, shp, ty in (("q", q, (B, T, H, dk), dt), ("k", k, (B, T, H, dk), dt),
                             ("v", v, (B, T, H, dv), dt), ("g", g, (B, T, H, dk), torch.float32),
                             ("beta", beta, (B, T, H), torch.float32)):
        _check_tensor(name, t, shp, ty)
    rc = library().kda_prefill_segment_prep(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B, T, H, dk, dv,
                                            _DTYPES[dt], int(t_begin), int(t_len), _ptr(ws), _ws_bytes(ws),
                                            _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_segment_prep")


def prefill_segment_recur(ws, q, v, t_begin: int, t_len: int, S0=None, checkpoint_every: int = 0, o=None,
                          S_T=None, ckpt=None):
    """Stage 2 over tokens [t_begin, t_begin + t_len) (kda_prefill_segment_recur)
    from S0, the state before t_begin; o and ckpt are the full tensors, of
    which the segment's part is written.  Returns (o, S_T, ckpt or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt != torch.bfloat16:
        raise ValueError("the prefill stages take bfloat16 q, k, v")
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32)
    n_ck = -(-T // checkpoint_every) if checkpoint_every > 0 else 0
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if n_ck and ckpt is None:
        ckpt = torch.empty((n_ck, B, H, dk, dv), dtype=torch.float32, device=dev)
    _check_tensor("o", o, (B, T, H, dv), dt)
    _check_tensor("S_T", S_T, (B, H, dk, dv), torch.float32)
    if n_ck:
        _check_tensor("ckpt", ckpt, (n_ck, B, H, dk, dv), torch.float32)
    rc = library().kda_prefill_segment_recur(_ptr(ws), _ws_bytes(ws), _ptr(S0), _ptr(o), _ptr(S_T),
                                             _ptr(ckpt if n_ck else None), int(checkpoint_every), B, T, H, dk,
                                             dv, _DTYPES[dt], int(t_begin), int(t_len), _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_segment_recur")
    return o, S_T, (ckpt if n_ck else None)


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def prefill_chunk_prep(q, k, v, g, beta, ws):
    """Stage 1 of the bf16 prefill (kda_prefill_chunk_prep): per-chunk operand
    records into ``ws`` (from ``workspace(q, v)``)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    for name, t, shp, ty in (("q", q, (B, T, H, dk), dt), ("k", k, (B, T, H, dk), dt),
                             ("v", v, (B, T, H, dv), dt), ("g", g, (B, T, H, dk), torch.float32),
                             ("beta", beta, (B, T, H), torch.float32)):
        _check_tensor(name, t, shp, ty)
    rc = library().kda_prefill_chunk_prep(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          B, T, H, dk, dv, _DTYPES[dt], _ptr(ws), _ws_bytes(ws),
                                          _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_chunk_prep")


def prefill_chunk_recur(ws, q, v, S0=None, checkpoint_every: int = 0, o=None, S_T=None, ckpt=None):
    """Stage 2 of the bf16 prefill (kda_prefill_chunk_recur) over the records
    in ``ws``; q and v only give the sizes and dtype.  Returns (o, S_T, ckpt or
    None) like prefill()."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32)
    n_ck = -(-T // checkpoint_every) if checkpoint_every > 0 else 0
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if n_ck and ckpt is None:
        ckpt = torch.empty((n_ck, B, H, dk, dv), dtype=torch.float32, device=dev)
    _check_tensor("o", o, (B, T, H, dv), dt)
    _check_tensor("S_T", S_T, (B, H, dk, dv), torch.float32)
    if n_ck:
        _check_tensor("ckpt", ckpt, (n_ck, B, H, dk, dv), torch.float32)
    rc = library().kda_prefill_chunk_recur(_ptr(ws), _ws_bytes(ws), _ptr(S0), _ptr(o), _ptr(S_T),
                                           _ptr(ckpt if n_ck else None), int(checkpoint_every),
                                           B, T, H, dk, dv, _DTYPES[dt], _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_chunk_recur")
    return o, S_T, (ckpt if n_ck else None)


def _cu_array(cu_seqlens):
    """Host int32 copy of the sequence offsets and a ctypes pointer to it."""
    if isinstance(cu_seqlens, torch.Tensor):
        if cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be on the host (list, numpy array or CPU tensor)")
        vals = [int(x) for x in cu_seqlens.tolist()]
    else:
        vals = [int(x) for x in cu_seqlens]
    if not vals:
        raise ValueError("cu_seqlens needs num_seqs + 1 >= 1 entries")
    arr = (ctypes.c_int * len(vals))(*vals)
    return arr, len(vals) - 1


def prefill_varlen(q, k, v, g, beta, cu_seqlens, S0=None, checkpoint_every: int = 0, o=None, S_T=None,
                   ckpt=None, ws=None):
    """Prefill of packed sequences (kda_prefill_varlen).  q, k, g [total_T,H,dk],
    v [total_T,H,dv], beta [total_T,H] (bf16 q/k/v); cu_seqlens: host offsets
    [num_seqs+1].  Returns (o [total_T,H,dv], S_T [num_seqs,H,dk,dv], ckpt or
    None), where sequence i's checkpoints are consecutive entries of ckpt.
    ws: a workspace of varlen_workspace_bytes(...) bytes to reuse, or None."""
    TT, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    for name, t, shp, ty in (("q", q, (TT, H, dk), dt), ("k", k, (TT, H, dk), dt),
                             ("v", v, (TT, H, dv), dt), ("g", g, (TT, H, dk), torch.float32),
                             ("beta", beta, (TT, H), torch.float32)):
        _check_tensor(name, t, shp, ty)
    cu, S = _cu_array(cu_seqlens)
    if cu[S] != TT:
        raise ValueError("cu_seqlens[-1] = %d but the tensors hold %d tokens" % (cu[S], TT))
    if S0 is not None:
        _check_tensor("S0", S0, (S, H, dk, dv), torch.float32)
    lib = library()
    n_ck = lib.kda_prefill_varlen_num_checkpoints(cu, S, int(checkpoint_every))
    if n_ck < 0:
        raise KDAError(2 if checkpoint_every >= 0 and checkpoint_every % CHUNK == 0 else 5,
                       "kda_prefill_varlen_num_checkpoints")
    dev = q.device
    if o is None:
        o = torch.empty((TT, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((S, H, dk, dv), dtype=torch.float32, device=dev)
    if n_ck and ckpt is None:
        ckpt = torch.empty((n_ck, H, dk, dv), dtype=torch.float32, device=dev)
    _check_tensor("o", o, (TT, H, dv), dt)
    _check_tensor("S_T", S_T, (S, H, dk, dv), torch.float32)
    if n_ck:
        _check_tensor("ckpt", ckpt, (n_ck, H, dk, dv), torch.float32)
    if ws is None:
        ws_bytes = lib.kda_prefill_varlen_workspace_size(cu, S, H, dk, dv, _DTYPES[dt])
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    ws_bytes = _ws_bytes(ws)
    rc = lib.kda_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu, S, _ptr(S0),
                                _ptr(o), _ptr(S_T), _ptr(ckpt if n_ck else None), int(checkpoint_every),
                                H, dk, dv, _DTYPES[dt], _ptr(ws), ws_bytes, _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_varlen")
    return o, S_T, (ckpt if n_ck else None)


def decode_step(q, k, v, g, beta, S, o=None):
    """One decode token (kda_decode_step); S [N,H,dk,dv] is updated in place.
    Returns o [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    dt = q.dtype
    for name, t, shp, ty in (("q", q, (N, H, dk), dt), ("k", k, (N, H, dk), dt),
                             ("v", v, (N, H, dv), dt), ("g", g, (N, H, dk), torch.float32),
                             ("beta", beta, (N, H), torch.float32),
                             ("S", S, (N, H, dk, dv), torch.float32)):
        _check_tensor(name, t, shp, ty)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=q.device)
    _check_tensor("o", o, (N, H, dv), dt)
    rc = library().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S),
                                   _ptr(o), N, H, dk, dv, _DTYPES[dt], _stream())
    if rc != 0:
        raise KDAError(rc, "kda_decode_step")
    return o


def decode_multi(q, k, v, g, beta, S, n_tokens=None, update_state: bool = True, o=None,
                 want_output: bool = True):
    """Several tokens per sequence (kda_decode_multi): q, k, g [N,T,H,dk],
    v [N,T,H,dv], beta [N,T,H], S [N,H,dk,dv].  n_tokens: None or an int32
    GPU tensor [N] limiting each sequence's tokens; update_state=False leaves
    S untouched.  Returns o [N,T,H,dv] (None when want_output is False)."""
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    for name, t, shp, ty in (("q", q, (N, T, H, dk), dt), ("k", k, (N, T, H, dk), dt),
                             ("v", v, (N, T, H, dv), dt), ("g", g, (N, T, H, dk), torch.float32),
                             ("beta", beta, (N, T, H), torch.float32),
                             ("S", S, (N, H, dk, dv), torch.float32)):
        _check_tensor(name, t, shp, ty)
    if n_tokens is not None:
        _check_tensor("n_tokens", n_tokens, (N,), torch.int32)
    if want_output and o is None:
        o = torch.empty((N, T, H, dv), dtype=dt, device=q.device)
    if not want_output:
        o = None
    if o is not None:
        _check_tensor("o", o, (N, T, H, dv), dt)
    rc = library().kda_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S), _ptr(o),
                                    _ptr(n_tokens), int(bool(update_state)), N, T, H, dk, dv,
                                    _DTYPES[dt], _stream())
    if rc != 0:
        raise KDAError(rc, "kda_decode_multi")
    return o


def _layer_opts(conv_w, silu, z, norm_w, eps, H, dk, dv, z_shape, dt):
    """Check the optional layer tensors and fill a LayerOpts."""
    opts = LayerOpts()
    if conv_w is not None:
        if conv_w.dim() != 3 or conv_w.shape[0] != H or conv_w.shape[2] != 2 * dk + dv:
            raise ValueError("conv_w must be [H, W, 2dk+dv], got %s" % (tuple(conv_w.shape),))
        _check_tensor("conv_w", conv_w, tuple(conv_w.shape), torch.float32)
        opts.conv_w = conv_w.data_ptr()
        opts.conv_width = int(conv_w.shape[1])
        opts.conv_silu = 1 if silu else 0
    if z is not None:
        _check_tensor("z", z, z_shape, dt)
        opts.gate_z = z.data_ptr()
        if norm_w is not None:
            _check_tensor("norm_w", norm_w, (dv,), torch.float32)
            opts.norm_w = norm_w.data_ptr()
        opts.norm_eps = float(eps)
    return opts


def prefill_layer(q, k, v, a, b, conv_w=None, conv_state=None, silu: bool = False, S0=None,
                  checkpoint_every: int = 0, z=None, norm_w=None, eps: float = 1e-6, o=None, S_T=None,
                  ckpt=None, conv_state_out=None, ws=None):
    """The layer core over whole sequences (kda_prefill_layer, bf16): raw q, k, v
    [B,T,H,d], decay-gate logits a [B,T,H,dk], write-gate logits b [B,T,H];
    conv_w [H,W,2dk+dv] float32 or None; conv_state [B,H,2dk+dv,W-1] float32 or
    None (zeros); z [B,T,H,dv] output-gate logits or None.  Returns (o, S_T,
    ckpt or None, conv_state_out or None)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt != torch.bfloat16:
        raise ValueError("prefill_layer takes bfloat16 q, k, v")
    for name, t, shp, ty in (("q", q, (B, T, H, dk), dt), ("k", k, (B, T, H, dk), dt),
                             ("v", v, (B, T, H, dv), dt), ("a", a, (B, T, H, dk), torch.float32),
                             ("b", b, (B, T, H), torch.float32)):
        _check_tensor(name, t, shp, ty)
    opts = _layer_opts(conv_w, silu, z, norm_w, eps, H, dk, dv, (B, T, H, dv), dt)
    W = int(conv_w.shape[1]) if conv_w is not None else 1
    dev = q.device
    cs_shape = (B, H, 2 * dk + dv, W - 1)
    if conv_state is not None and W > 1:
        _check_tensor("conv_state", conv_state, cs_shape, torch.float32)
    if W > 1 and conv_state_out is None:
        conv_state_out = torch.empty(cs_shape, dtype=torch.float32, device=dev)
    if S0 is not None:
        _check_tensor("S0", S0, (B, H, dk, dv), torch.float32)
    n_ck = -(-T // checkpoint_every) if checkpoint_every > 0 else 0
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if n_ck and ckpt is None:
        ckpt = torch.empty((n_ck, B, H, dk, dv), dtype=torch.float32, device=dev)
    if ws is None:
        ws = prefill_workspace(q, v)
    rc = library().kda_prefill_layer(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                     _ptr(conv_state if W > 1 else None),
                                     _ptr(conv_state_out if W > 1 else None), _ptr(S0), _ptr(o), _ptr(S_T),
                                     _ptr(ckpt if n_ck else None), int(checkpoint_every), B, T, H, dk, dv,
                                     _DTYPES[dt], ctypes.byref(opts), _ptr(ws), _ws_bytes(ws), _stream())
    if rc != 0:
        raise KDAError(rc, "kda_prefill_layer")
    return o, S_T, (ckpt if n_ck else None), (conv_state_out if W > 1 else None)


def decode_layer_step(q, k, v, a, b, S, conv_state=None, conv_w=None, silu: bool = False, z=None,
                      norm_w=None, eps: float = 1e-6, o=None):
    """One decode token of the layer (kda_decode_layer_step): raw q, k, a [N,H,dk],
    v [N,H,dv], b [N,H]; S [N,H,dk,dv] and conv_state [N,H,2dk+dv,W-1] updated
    in place.  Returns o [N,H,dv] (normalized and gated when z is given)."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    for name, t, shp, ty in (("q", q, (N, H, dk), dt), ("k", k, (N, H, dk), dt), ("v", v, (N, H, dv), dt),
                             ("a", a, (N, H, dk), torch.float32), ("b", b, (N, H), torch.float32),
                             ("S", S, (N, H, dk, dv), torch.float32)):
        _check_tensor(name, t, shp, ty)
    opts = _layer_opts(conv_w, silu, z, norm_w, eps, H, dk, dv, (N, H, dv), dt)
    W = int(conv_w.shape[1]) if conv_w is not None else 1
    if W > 1:
        if conv_state is None:
            raise ValueError("a convolution wider than 1 needs conv_state")
        _check_tensor("conv_state", conv_state, (N, H, 2 * dk + dv, W - 1), torch.float32)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=q.device)
    _check_tensor("o", o, (N, H, dv), dt)
    rc = library().kda_decode_layer_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                         _ptr(conv_state if W > 1 else None), _ptr(S), _ptr(o), N, H, dk, dv,
                                         _DTYPES[dt], ctypes.byref(opts), _stream())
    if rc != 0:
        raise KDAError(rc, "kda_decode_layer_step")
    return o


def output_norm_gate(o, z, norm_w=None, eps: float = 1e-6, y=None):
    """y = o * w / sqrt(mean(o^2) + eps) * sigmoid(z) over the last dim
    (kda_output_norm_gate); y may be o."""
    dt = o.dtype
    if dt not in _DTYPES:
        raise ValueError("o must be bfloat16 or float32")
    dv = o.shape[-1]
    _check_tensor("o", o, tuple(o.shape), dt)
    _check_tensor("z", z, tuple(o.shape), dt)
    if norm_w is not None:
        _check_tensor("norm_w", norm_w, (dv,), torch.float32)
    if y is None:
        y = torch.empty_like(o)
    _check_tensor("y", y, tuple(o.shape), dt)
    rows = o.numel() // dv if dv else 0
    rc = library().kda_output_norm_gate(_ptr(o), _ptr(z), _ptr(norm_w), float(eps), _ptr(y), rows, dv,
                                        _DTYPES[dt], _stream())
    if rc != 0:
        raise KDAError(rc, "kda_output_norm_gate")
    return y
