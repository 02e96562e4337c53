"""Pins for the fp64 oracle: what the pages and the mathematics fix.

Each ``pin_*`` function takes an oracle library handle (``None`` = the built
oracle) and raises AssertionError if the oracle disagrees with a result that
is known independently of it.  ``tests/test_oracle_pins.py`` runs them on the
oracle; ``tests/test_oracle_mutants.py`` runs them on copies of the oracle with
planted mistakes and requires every mistake to be caught.

Sources of the expected values (Kimi K3 primer, bayesiansapien wiki page):
  * section 1 names the lineage linear attention -> DeltaNet -> Gated DeltaNet
    -> KDA; the special cases below reduce KDA to each ancestor;
  * section 2 gives the chunked two-kernel form (decay cumsum, decayed Q/K,
    (I+L)^-1 by Neumann, causal mask, chunk recurrence), reproduced
    independently in ``chunked_reference.py``;
  * ``golden/worked_example_T2_d2.json`` is a hand-worked example.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from chunked_reference import chunked_prefill

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(seed, B=1, T=9, H=2, dk=5, dv=3, g_lo=-0.6, g_hi=0.0, s0=True):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = _unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    g = r.uniform(g_lo, g_hi, (B, T, H, dk))
    beta = r.uniform(0.05, 1.0, (B, T, H))
    S0 = r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    err = np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
    assert err <= tol, "%s: scaled max error %.3e > %.1e" % (what, err, tol)


# -- hand-worked example ----------------------------------------------------

def pin_golden_worked_example(lib=None):
    """Two tokens computed by hand in exact fractions (tests/golden)."""
    with open(os.path.join(GOLDEN, "worked_example_T2_d2.json")) as f:
        ex = json.load(f)
    g = np.log(np.array(ex["g_is_log_of"]))[None, :, None, :]
    k = np.array(ex["k"])[None, :, None, :]
    v = np.array(ex["v"])[None, :, None, :]
    q = np.array(ex["q"])[None, :, None, :]
    beta = np.array(ex["beta"])[None, :, None]
    S0 = np.array(ex["S0"])[None, None]
    o, S_T, ck = oracle.prefill(q, k, v, g, beta, S0, ckpt_every=1, lib=lib)
    tol = ex["tolerance"]
    _close(o[0, :, 0], ex["o"], tol, "golden o")
    _close(S_T[0, 0], ex["S_T"], tol, "golden S_T")
    _close(ck[0, 0, 0], ex["S_1"], tol, "golden state after token 1")
    # The same two tokens through the one-token decode entry point.
    S = S0
    for t in range(2):
        o_t, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S, lib=lib)
        _close(o_t[0, 0], ex["o"][t], tol, "golden decode o_%d" % (t + 1))
    _close(S[0, 0], ex["S_T"], tol, "golden decode S_T")


# -- lineage special cases (section 1) --------------------------------------

def pin_matrix_form(lib=None):
    """The update written as dk x dk matrices, token by token:
    S_t = (I - b k k^T) Diag(exp g) S_{t-1} + b k v^T, o_t = S_t^T q_t."""
    q, k, v, g, beta, S0 = _rand_case(1, B=2, T=7, H=2, dk=5, dv=3, g_lo=-0.8, g_hi=0.3)
    beta = beta * 1.9  # exercise beta beyond 1 as well
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    B, T, H, dk = q.shape
    for b in range(B):
        for h in range(H):
            S = S0[b, h].copy()
            for t in range(T):
                kk = k[b, t, h][:, None]
                P = np.eye(dk) - beta[b, t, h] * (kk @ kk.T)
                S = P @ np.diag(np.exp(g[b, t, h])) @ S + beta[b, t, h] * kk @ v[b, t, h][None, :]
                _close(o[b, t, h], S.T @ q[b, t, h], 1e-12, "matrix form o")
            _close(S_T[b, h], S, 1e-12, "matrix form S_T")


def pin_linear_attention_orthonormal(lib=None):
    """alpha = 1, beta = 1, S0 = 0 and mutually orthonormal keys: the erase
    term never fires, so o_t is exactly linear attention sum_{s<=t}(q_t.k_s) v_s."""
    r = _rng(2)
    T = dk = 8
    dv = 5
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm.T[None, :, None, :]                      # rows are orthonormal keys
    q = r.standard_normal((1, T, 1, dk))
    v = r.standard_normal((1, T, 1, dv))
    g = np.zeros((1, T, 1, dk))
    beta = np.ones((1, T, 1))
    o, _, _ = oracle.prefill(q, k, v, g, beta, None, lib=lib)
    for t in range(T):
        ref = sum(np.dot(q[0, t, 0], k[0, s, 0]) * v[0, s, 0] for s in range(t + 1))
        _close(o[0, t, 0], ref, 1e-12, "orthonormal linear attention")


def pin_linear_attention_limit(lib=None):
    """alpha = 1, S0 = 0, beta = eps: o_t / eps -> sum_{s<=t}(q_t.k_s) v_s
    with an O(eps) remainder, for arbitrary (non-orthogonal) keys."""
    r = _rng(3)
    T, dk, dv, eps = 12, 6, 4, 1e-7
    q = r.standard_normal((1, T, 1, dk))
    k = _unit(r.standard_normal((1, T, 1, dk)))
    v = r.standard_normal((1, T, 1, dv))
    o, _, _ = oracle.prefill(q, k, v, np.zeros((1, T, 1, dk)), np.full((1, T, 1), eps), None,
                             lib=lib)
    for t in range(T):
        ref = sum(np.dot(q[0, t, 0], k[0, s, 0]) * v[0, s, 0] for s in range(t + 1))
        _close(o[0, t, 0] / eps, ref, 1e-5, "linear attention limit")


def pin_pure_decay(lib=None):
    """beta = 0: nothing is erased or written, S_t = Diag(exp sum_{s<=t} g_s) S0."""
    q, k, v, g, beta, S0 = _rand_case(4, B=1, T=10, H=3, dk=4, dv=6, g_lo=-0.9, g_hi=0.4)
    beta = np.zeros_like(beta)
    o, S_T, ck = oracle.prefill(q, k, v, g, beta, S0, ckpt_every=4, lib=lib)
    Gcum = np.cumsum(g, axis=1)
    for h in range(3):
        for t in range(10):
            S_t = np.exp(Gcum[0, t, h])[:, None] * S0[0, h]
            _close(o[0, t, h], S_t.T @ q[0, t, h], 1e-12, "pure decay o")
        _close(S_T[0, h], np.exp(Gcum[0, -1, h])[:, None] * S0[0, h], 1e-12, "pure decay S_T")
        for j, t_end in enumerate((4, 8, 10)):
            _close(ck[j, 0, h], np.exp(Gcum[0, t_end - 1, h])[:, None] * S0[0, h], 1e-12,
                   "pure decay checkpoint %d" % j)


def pin_retrieval_q_equals_k(lib=None):
    """beta = 1 and unit keys: S_t^T k_t = v_t for any decay and history
    (the delta rule replaces the value stored under k_t), so q_t = k_t gives o_t = v_t."""
    q, k, v, g, beta, S0 = _rand_case(5, B=1, T=11, H=2, dk=6, dv=4, g_lo=-1.0, g_hi=0.5)
    beta = np.ones_like(beta)
    o, _, _ = oracle.prefill(k, k, v, g, beta, S0, lib=lib)
    _close(o, v, 1e-12, "q = k retrieval")


def pin_orthonormal_full_retrieval(lib=None):
    """alpha = 1, beta = 1, orthonormal keys: every stored pair survives later
    writes, S_T^T k_s = v_s for all s, from any S0."""
    r = _rng(6)
    T = dk = 7
    dv = 3
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = Qm.T[None, :, None, :]
    q = r.standard_normal((1, T, 1, dk))
    v = r.standard_normal((1, T, 1, dv))
    S0 = r.standard_normal((1, 1, dk, dv))
    _, S_T, _ = oracle.prefill(q, k, v, np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), S0, lib=lib)
    for s in range(T):
        _close(S_T[0, 0].T @ k[0, s, 0], v[0, s, 0], 1e-12, "orthonormal retrieval")


def pin_scalar_gate_is_gated_deltanet(lib=None):
    """A decay that is equal across channels is Gated DeltaNet: the scalar gate
    commutes with the erase, S_t = a_t (I - b k k^T) S_{t-1} + b k v^T.  Checked
    against that scalar recurrence (decay applied after the erase)."""
    q, k, v, g1, beta, S0 = _rand_case(7, B=1, T=13, H=2, dk=5, dv=4)
    a = _rng(70).uniform(-0.7, 0.0, (1, 13, 2))
    g = np.repeat(a[..., None], 5, axis=-1)
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    for h in range(2):
        S = S0[0, h].copy()
        for t in range(13):
            kk = k[0, t, h]
            S = np.exp(a[0, t, h]) * (S - beta[0, t, h] * np.outer(kk, kk @ S)) \
                + beta[0, t, h] * np.outer(kk, v[0, t, h])
            _close(o[0, t, h], S.T @ q[0, t, h], 1e-12, "scalar gate o")
        _close(S_T[0, h], S, 1e-12, "scalar gate S_T")


# -- the chunked method (section 2) ------------------------------------------

def pin_chunked_forms(lib=None):
    """The chunk-parallel form (exact triangular solve, and the Neumann product
    for the inverse) equals the recurrence for chunk sizes 1, 3, 16, 64 and T,
    with a ragged last chunk."""
    q, k, v, g, beta, S0 = _rand_case(8, B=1, T=70, H=2, dk=6, dv=5, g_lo=-0.3, g_hi=0.0)
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    for C in (1, 3, 16, 64, 70):
        for method in ("solve", "neumann"):
            oc, Sc = chunked_prefill(q, k, v, g, beta, S0, C=C, method=method)
            _close(o, oc, 1e-10, "chunked o (C=%d, %s)" % (C, method))
            _close(S_T, Sc, 1e-10, "chunked S_T (C=%d, %s)" % (C, method))


# -- invariants of any correct implementation --------------------------------

def pin_layout_independence(lib=None):
    """Each (batch, head) is an independent chain: running the [B,T,H] tensors
    together equals running every (b, h) slice alone."""
    q, k, v, g, beta, S0 = _rand_case(9, B=2, T=6, H=3, dk=4, dv=5)
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    for b in range(2):
        for h in range(3):
            sl = np.s_[b:b + 1, :, h:h + 1]
            o1, S1, _ = oracle.prefill(q[sl], k[sl], v[sl], g[sl], beta[b:b + 1, :, h:h + 1],
                                       S0[b:b + 1, h:h + 1], lib=lib)
            _close(o[sl], o1, 1e-13, "slice o")
            _close(S_T[b, h], S1[0, 0], 1e-13, "slice S_T")


def pin_split_resume_and_checkpoints(lib=None):
    """Prefill of T1 tokens, resumed from its final state for T2 more tokens,
    equals one prefill of T1 + T2; checkpoint j equals the state after token
    min(j N, T)."""
    q, k, v, g, beta, S0 = _rand_case(10, B=2, T=23, H=2, dk=4, dv=3)
    o, S_T, ck = oracle.prefill(q, k, v, g, beta, S0, ckpt_every=5, lib=lib)
    assert ck.shape[0] == 5
    T1 = 9
    o1, S1, _ = oracle.prefill(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0,
                               lib=lib)
    o2, S2, _ = oracle.prefill(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], S1,
                               lib=lib)
    _close(o, np.concatenate([o1, o2], axis=1), 1e-12, "split o")
    _close(S_T, S2, 1e-12, "split S_T")
    for j in range(5):
        t_end = min(5 * (j + 1), 23)
        _, Sj, _ = oracle.prefill(q[:, :t_end], k[:, :t_end], v[:, :t_end], g[:, :t_end],
                                  beta[:, :t_end], S0, lib=lib)
        _close(ck[j], Sj, 1e-12, "checkpoint %d" % j)


def pin_decode_equals_prefill(lib=None):
    """T one-token decode steps from S0 equal one prefill of length T."""
    q, k, v, g, beta, S0 = _rand_case(11, B=3, T=8, H=2, dk=5, dv=4)
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    S = S0
    for t in range(8):
        o_t, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S, lib=lib)
        _close(o_t, o[:, t], 1e-12, "decode o step %d" % t)
    _close(S, S_T, 1e-12, "decode final state")


def pin_linearity_in_values_and_state(lib=None):
    """For fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear."""
    q, k, v, g, beta, S0 = _rand_case(12, B=1, T=10, H=2, dk=4, dv=4)
    r = _rng(120)
    v2 = r.standard_normal(v.shape)
    S02 = r.standard_normal(S0.shape)
    c = -0.7
    oa, Sa, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    ob, Sb, _ = oracle.prefill(q, k, v2, g, beta, S02, lib=lib)
    oc, Sc, _ = oracle.prefill(q, k, v + c * v2, g, beta, S0 + c * S02, lib=lib)
    _close(oc, oa + c * ob, 1e-12, "linearity o")
    _close(Sc, Sa + c * Sb, 1e-12, "linearity S_T")


def pin_value_column_permutation(lib=None):
    """Value channels are independent: permuting the dv columns of v and S0
    permutes the columns of o and S_T the same way."""
    q, k, v, g, beta, S0 = _rand_case(13, B=1, T=9, H=2, dk=4, dv=6)
    perm = np.array([3, 0, 5, 1, 4, 2])
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    op, Sp, _ = oracle.prefill(q, k, v[..., perm], g, beta, S0[..., perm], lib=lib)
    _close(op, o[..., perm], 1e-13, "permuted o")
    _close(Sp, S_T[..., perm], 1e-13, "permuted S_T")


def pin_rectangular_state(lib=None):
    """dk != dv: the chunked form and the matrix form agree with the oracle
    when the state is not square (catches swapped dk/dv strides)."""
    q, k, v, g, beta, S0 = _rand_case(14, B=1, T=19, H=2, dk=3, dv=7)
    o, S_T, _ = oracle.prefill(q, k, v, g, beta, S0, lib=lib)
    oc, Sc = chunked_prefill(q, k, v, g, beta, S0, C=8)
    _close(o, oc, 1e-10, "rectangular o")
    _close(S_T, Sc, 1e-10, "rectangular S_T")


PINS = [
    pin_golden_worked_example,
    pin_matrix_form,
    pin_linear_attention_orthonormal,
    pin_linear_attention_limit,
    pin_pure_decay,
    pin_retrieval_q_equals_k,
    pin_orthonormal_full_retrieval,
    pin_scalar_gate_is_gated_deltanet,
    pin_chunked_forms,
    pin_layout_independence,
    pin_split_resume_and_checkpoints,
    pin_decode_equals_prefill,
    pin_linearity_in_values_and_state,
    pin_value_column_permutation,
    pin_rectangular_state,
]
