"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
shares no code with the HIP path: the arithmetic lives in ``kda_oracle.c``
(plain C, fp64, token by token), built here with gcc.

The recurrence it implements is the gated delta rule with a diagonal forget
gate that the SemiAnalysis Kimi K3 primer derives (bayesiansapien wiki page,
section 1 "KDA is DeltaNet plus per-channel decay"):
``S_t = (I - b_t k_t k_t^T) Diag(exp g_t) S_{t-1} + b_t k_t v_t^T``,
``o_t = S_t^T q_t``.  Each public function converts its inputs to contiguous
fp64 arrays, calls the C routine, and returns new fp64 arrays.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms and special cases that the pages and the mathematics fix (linear
attention, Gated DeltaNet, exact retrieval, pure decay, an independent chunked
solve, a hand-worked example in ``tests/golden/``) and by mutation tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None
_lock = threading.Lock()

# No -ffast-math and no FMA contraction: the oracle's arithmetic is the plain
# sequence of fp64 operations written in kda_oracle.c.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
          "-Wall", "-Wextra", "-Werror"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source into a shared library with gcc."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load_library(path: str) -> ctypes.CDLL:
    """Load an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ci = ctypes.c_int
    lib.kda_oracle_prefill_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, ci,
                                           ci, ci, ci, ci, ci, ci]
    lib.kda_oracle_prefill_f64.restype = ci
    lib.kda_oracle_decode_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, ci, ci, ci, ci, ci]
    lib.kda_oracle_decode_f64.restype = ci
    return lib


def _library():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _lib = load_library(_LIB_PATH)
    return _lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    """Threads the oracle uses by default: the cores this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def prefill(q, k, v, g, beta, S0=None, ckpt_every: int = 0, threads: int | None = None,
            lib=None):
    """Token-by-token recurrence over a whole sequence.

    Shapes: q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; S0 [B,H,dk,dv] or
    None (zero state).  Returns (o [B,T,H,dv], S_T [B,H,dk,dv], ckpt) where
    ckpt is [ceil(T/N),B,H,dk,dv] (state after tokens N, 2N, ..., and T) when
    ``ckpt_every`` = N > 0, else None.  All results are fp64.
    """
    lib = lib or _library()
    q, k, v, g, beta, S0 = map(_f64, (q, k, v, g, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape, "q, k, g must be [B,T,H,dk]"
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    ck = None
    if ckpt_every > 0:
        n_ck = -(-T // ckpt_every)
        ck = np.zeros((n_ck, B, H, dk, dv))
    rc = lib.kda_oracle_prefill_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                    _ptr(o), _ptr(S_T), _ptr(ck), int(ckpt_every),
                                    B, T, H, dk, dv, int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_prefill_f64 failed with code %d" % rc)
    return o, S_T, ck


def decode_step(q, k, v, g, beta, S, threads: int | None = None, lib=None):
    """One token of the recurrence for N independent sequences.

    Shapes: q, k, g [N,H,dk]; v [N,H,dv]; beta [N,H]; S [N,H,dk,dv].  The
    input S is not modified.  Returns (o [N,H,dv], S_new [N,H,dk,dv]), fp64.
    """
    lib = lib or _library()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    S_new = np.array(S, dtype=np.float64, order="C", copy=True)
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert S_new.shape == (N, H, dk, dv) and beta.shape == (N, H)
    o = np.zeros((N, H, dv))
    rc = lib.kda_oracle_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S_new),
                                   _ptr(o), N, H, dk, dv, int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("kda_oracle_decode_f64 failed with code %d" % rc)
    return o, S_new
