"""The C ABI on the CPU: libkda.so loads, exports every function include/kda.h
declares, and rejects invalid arguments on the host with the documented status
codes.  No case here reaches a kernel launch (every call fails validation or is
a documented no-op), so nothing touches a device."""
import ctypes

import pytest

import kimi_delta_attention_chunked_amd as kda

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WS, ALIAS, HIP = range(9)
BF16, FP32 = 1, 0

# Fake, well-aligned "device" addresses, 1 GiB apart: validation only compares
# them, nothing dereferences them.
GiB = 1 << 30


def P(i):
    return ctypes.c_void_p((i + 1) * GiB)


@pytest.fixture(scope="module")
def lib():
    return kda.library()


def test_exports_every_declared_function(lib):
    names = kda.declared_functions()
    assert set(names) >= {"kda_prefill", "kda_prefill_chunk_prep", "kda_prefill_chunk_recur",
                          "kda_prefill_segment_prep", "kda_prefill_segment_recur",
                          "kda_prefill_segment_tokens", "kda_prefill_stage_workspace_size",
                          "kda_prefill_varlen", "kda_prefill_varlen_workspace_size",
                          "kda_prefill_varlen_num_checkpoints", "kda_decode_step",
                          "kda_prefill_workspace_size", "kda_decode_multi", "kda_status_string",
                          "kda_version", "kda_prefill_noalloc"}
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_version() == 100
    for code in range(9):
        s = kda.status_string(code)
        assert s.startswith("KDA_"), s
    assert kda.status_string(99) == "KDA_ERR_UNKNOWN"


def test_workspace_size(lib):
    # bf16: one operand record per (batch, head, 64-token chunk); fp32: none.
    assert lib.kda_prefill_stage_workspace_size(1, 32768, 32, 128, 128, BF16) == 32 * 512 * 72704
    assert lib.kda_prefill_stage_workspace_size(2, 100, 3, 64, 64, BF16) == 2 * 3 * 2 * 39936
    assert lib.kda_prefill_stage_workspace_size(1, 256, 2, 64, 64, FP32) == 0
    # kda_prefill: the fewest segments whose records stay within 232 MiB
    # (1136 bytes per token-head at dk = 128, 624 at dk = 64), of equal
    # whole-chunk lengths, at least 384 tokens: 32768 tokens of 32 heads allow
    # 6656 per segment, so 5 segments of 6592 (103 chunks; the last 6400)
    assert lib.kda_prefill_segment_tokens(1, 32768, 32, 128, 128, BF16) == 6592
    assert lib.kda_prefill_workspace_size(1, 32768, 32, 128, 128, BF16) == 32 * 103 * 72704
    assert lib.kda_prefill_segment_tokens(1, 32768, 16, 128, 128, BF16) == 10944  # 3 of at most 13376
    assert lib.kda_prefill_segment_tokens(1, 10000, 32, 128, 128, BF16) == 5056   # two nearly equal halves
    assert lib.kda_prefill_segment_tokens(1, 10 ** 6, 32, 128, 128, BF16) == 6656  # at the bound
    assert lib.kda_prefill_segment_tokens(1, 142000, 32, 128, 128, BF16) == 6464  # 22 of at most 6656
    assert lib.kda_prefill_segment_tokens(1, 5000, 32, 128, 128, BF16) == 5000   # shorter than a segment
    assert lib.kda_prefill_segment_tokens(4, 32768, 32, 128, 128, BF16) == 1664   # 20 of at most 1664
    assert lib.kda_prefill_segment_tokens(8, 32768, 32, 128, 128, BF16) == 832    # 40 of at most 832
    assert lib.kda_prefill_segment_tokens(16, 8192, 32, 128, 128, BF16) == 384   # 22 of at most 384
    assert lib.kda_prefill_segment_tokens(32, 8192, 32, 128, 128, BF16) == 8192  # segments would be < 384
    assert lib.kda_prefill_segment_tokens(1, 32768, 32, 64, 64, BF16) == 10944  # 3 of at most 12160
    assert lib.kda_prefill_workspace_size(2, 100, 3, 64, 64, BF16) == 2 * 3 * 2 * 39936
    assert lib.kda_prefill_workspace_size(1, 256, 2, 64, 64, FP32) == 0
    assert lib.kda_prefill_workspace_size(1, 0, 2, 128, 128, BF16) == 0
    assert lib.kda_prefill_workspace_size(-1, 64, 2, 128, 128, BF16) == 0


WS_NEED = 2 * 4 * 72704  # B=1, H=2, T=256, dk=128


def prefill(lib, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), S0=None, o=P(5), S_T=P(6), ckpt=None,
            ckpt_every=0, B=1, T=256, H=2, dk=128, dv=128, dt=BF16, ws=P(10), ws_bytes=WS_NEED):
    return lib.kda_prefill(q, k, v, g, beta, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv, dt,
                           ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE),
    (dict(B=-1), SHAPE), (dict(T=-1), SHAPE), (dict(H=-2), SHAPE), (dict(dk=0), SHAPE),
    (dict(ckpt_every=-64), SHAPE),
    (dict(dk=96, dv=96), UNSUP), (dict(dk=64, dv=128), UNSUP), (dict(dt=FP32, dk=96, dv=96), UNSUP),
    (dict(ckpt_every=100, ckpt=P(7)), UNSUP),
    (dict(S_T=None), NULL), (dict(q=None), NULL), (dict(beta=None), NULL), (dict(o=None), NULL),
    (dict(ckpt_every=64), NULL),
    (dict(q=ctypes.c_void_p(GiB + 8)), ALIGN), (dict(S0=ctypes.c_void_p(9 * GiB + 4)), ALIGN),
    (dict(o=ctypes.c_void_p(GiB + 4096)), ALIAS),            # o inside q
    (dict(S0=P(8), S_T=ctypes.c_void_p(9 * GiB + 256)), ALIAS),  # partial S_T/S0 overlap
    (dict(ckpt_every=64, ckpt=ctypes.c_void_p(7 * GiB + 16)), ALIAS),  # ckpt inside S_T
    (dict(ws_bytes=WS_NEED - 1), WS), (dict(ws=None), NULL),
    (dict(ws=ctypes.c_void_p(GiB + 65536)), ALIAS),          # workspace overlaps q
    (dict(ws=ctypes.c_void_p(11 * GiB + 8)), ALIGN),
    (dict(H=1 << 22, T=1 << 16), SHAPE),                     # 2^32 chunk workgroups
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(B=0, q=None, S_T=None)])
def test_prefill_empty_batch_is_noop(lib, kw):
    assert prefill(lib, **kw) == OK


def prefill_noalloc(lib, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), S0=None, o=P(5), S_T=P(6), ckpt=None,
                    ckpt_every=0, B=1, T=256, H=2, dk=128, dv=128, dt=BF16):
    return lib.kda_prefill_noalloc(q, k, v, g, beta, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE), (dict(B=-1), SHAPE), (dict(dk=96, dv=96), UNSUP),
    (dict(ckpt_every=100, ckpt=P(7)), UNSUP), (dict(S_T=None), NULL), (dict(ckpt_every=64), NULL),
    (dict(q=ctypes.c_void_p(GiB + 8)), ALIGN), (dict(o=ctypes.c_void_p(GiB + 4096)), ALIAS),
    # one 64-token chunk of all B*H heads must fit the 64 MiB static scratch
    (dict(H=924, T=64), WS), (dict(B=2, H=462, T=64), WS), (dict(H=1681, T=64, dk=64, dv=64), WS),
])
def test_prefill_noalloc_rejects(lib, kw, code):
    assert prefill_noalloc(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(B=0, q=None, S_T=None)])
def test_prefill_noalloc_empty_batch_is_noop(lib, kw):
    assert prefill_noalloc(lib, **kw) == OK


def prep(lib, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), B=1, T=256, H=2, dk=128, dv=128, dt=BF16,
         ws=P(10), ws_bytes=WS_NEED):
    return lib.kda_prefill_chunk_prep(q, k, v, g, beta, B, T, H, dk, dv, dt, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), DTYPE), (dict(dt=FP32), UNSUP), (dict(T=-1), SHAPE), (dict(dk=96, dv=96), UNSUP),
    (dict(q=None), NULL), (dict(beta=None), NULL), (dict(ws=None), NULL),
    (dict(ws_bytes=WS_NEED - 1), WS), (dict(g=ctypes.c_void_p(4 * GiB + 4)), ALIGN),
    (dict(ws=ctypes.c_void_p(GiB + 4096)), ALIAS),            # workspace overlaps q
    (dict(H=1 << 22, T=1 << 16), SHAPE),
])
def test_prefill_chunk_prep_rejects(lib, kw, code):
    assert prep(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(T=0), dict(B=0), dict(H=0), dict(T=0, q=None, ws=None)])
def test_prefill_chunk_prep_empty_is_noop(lib, kw):
    assert prep(lib, **kw) == OK


def recur(lib, ws=P(10), ws_bytes=WS_NEED, S0=None, o=P(5), S_T=P(6), ckpt=None, ckpt_every=0, B=1,
          T=256, H=2, dk=128, dv=128, dt=BF16):
    return lib.kda_prefill_chunk_recur(ws, ws_bytes, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv,
                                       dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), DTYPE), (dict(dt=FP32), UNSUP), (dict(B=-1), SHAPE), (dict(dk=64, dv=128), UNSUP),
    (dict(ckpt_every=100, ckpt=P(7)), UNSUP),
    (dict(S_T=None), NULL), (dict(o=None), NULL), (dict(ws=None), NULL),
    (dict(ckpt_every=64), NULL), (dict(ws_bytes=WS_NEED - 1), WS),
    (dict(o=ctypes.c_void_p(5 * GiB + 8)), ALIGN),
    (dict(o=ctypes.c_void_p(11 * GiB + 1024)), ALIAS),        # o inside the workspace
    (dict(S0=P(8), S_T=ctypes.c_void_p(9 * GiB + 256)), ALIAS),
])
def test_prefill_chunk_recur_rejects(lib, kw, code):
    assert recur(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(B=0, S_T=None, ws=None)])
def test_prefill_chunk_recur_empty_batch_is_noop(lib, kw):
    assert recur(lib, **kw) == OK


def CU(*vals):
    return (ctypes.c_int * len(vals))(*vals)


def test_varlen_workspace_and_checkpoint_counts(lib):
    cu = CU(0, 100, 100, 300)  # lengths 100, 0, 200 -> 2 + 0 + 4 chunks
    assert lib.kda_prefill_varlen_workspace_size(cu, 3, 2, 128, 128, BF16) == 2 * 6 * 72704 + 3 * 256
    assert lib.kda_prefill_varlen_workspace_size(cu, 3, 2, 64, 64, BF16) == 2 * 6 * 39936 + 3 * 256
    # 16 sequences of 2048 tokens, 32 heads: 512 chunks, whose records exceed
    # 232 MiB; segments of at most 104 chunks -> 5 segments of 103 (the last 100)
    cu16 = (ctypes.c_int * 17)(*[2048 * i for i in range(17)])
    assert lib.kda_prefill_varlen_workspace_size(cu16, 16, 32, 128, 128, BF16) == 32 * 103 * 72704 + 3 * 256
    # more heads, shorter segments, down to 6 chunks; below that, one segment
    assert lib.kda_prefill_varlen_workspace_size(cu16, 16, 256, 128, 128, BF16) == 256 * 13 * 72704 + 3 * 256
    assert lib.kda_prefill_varlen_workspace_size(cu16, 16, 512, 128, 128, BF16) == 512 * 6 * 72704 + 3 * 256
    assert lib.kda_prefill_varlen_workspace_size(cu16, 16, 1024, 128, 128, BF16) == 1024 * 512 * 72704 + 3 * 256
    assert lib.kda_prefill_varlen_workspace_size(cu, 3, 2, 128, 128, FP32) == 0
    assert lib.kda_prefill_varlen_workspace_size(CU(0, 5, 3), 2, 2, 128, 128, BF16) == 0
    assert lib.kda_prefill_varlen_num_checkpoints(cu, 3, 64) == 2 + 0 + 4
    assert lib.kda_prefill_varlen_num_checkpoints(cu, 3, 128) == 1 + 0 + 2
    assert lib.kda_prefill_varlen_num_checkpoints(cu, 3, 0) == 0
    assert lib.kda_prefill_varlen_num_checkpoints(cu, 3, 100) == -1
    assert lib.kda_prefill_varlen_num_checkpoints(CU(1, 5), 1, 64) == -1


VL_CU = CU(0, 100, 100, 300)
VL_WS = 2 * 6 * 72704 + 3 * 256


def varlen(lib, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), cu=VL_CU, S=3, S0=None, o=P(5), S_T=P(6),
           ckpt=None, ckpt_every=0, H=2, dk=128, dv=128, dt=BF16, ws=P(10), ws_bytes=VL_WS):
    return lib.kda_prefill_varlen(q, k, v, g, beta, cu, S, S0, o, S_T, ckpt, ckpt_every, H, dk, dv, dt,
                                  ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=4), DTYPE), (dict(dt=FP32), UNSUP), (dict(H=-1), SHAPE), (dict(S=-1), SHAPE),
    (dict(dk=96, dv=96), UNSUP), (dict(ckpt_every=96, ckpt=P(7)), UNSUP),
    (dict(cu=None), NULL), (dict(cu=CU(1, 100, 100, 300)), SHAPE), (dict(cu=CU(0, 100, 90, 300)), SHAPE),
    (dict(S_T=None), NULL), (dict(q=None), NULL), (dict(o=None), NULL), (dict(ws=None), NULL),
    (dict(ckpt_every=64), NULL), (dict(ws_bytes=VL_WS - 1), WS),
    (dict(v=ctypes.c_void_p(3 * GiB + 2)), ALIGN),
    (dict(o=ctypes.c_void_p(GiB + 512)), ALIAS),              # o inside q
    (dict(ws=ctypes.c_void_p(6 * GiB + 64)), ALIAS),          # workspace overlaps o
    (dict(H=1 << 29, cu=CU(0, 1 << 16)), SHAPE),              # 2^29 heads x 1024 chunks
])
def test_prefill_varlen_rejects(lib, kw, code):
    if "S" not in kw and "cu" in kw and kw["cu"] is not None:
        kw["S"] = len(kw["cu"]) - 1
    assert varlen(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(S=0, cu=CU(0)), dict(H=0), dict(S=0, cu=CU(0), q=None, S_T=None, ws=None)])
def test_prefill_varlen_empty_is_noop(lib, kw):
    assert varlen(lib, **kw) == OK


def decode(lib, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), S=P(5), o=P(6), N=64, H=32, dk=128,
           dv=128, dt=BF16):
    return lib.kda_decode_step(q, k, v, g, beta, S, o, N, H, dk, dv, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), DTYPE), (dict(N=-1), SHAPE), (dict(dv=0), SHAPE),
    (dict(dk=32, dv=32), UNSUP), (dict(dk=128, dv=64), UNSUP),
    (dict(S=None), NULL), (dict(o=None), NULL), (dict(g=None), NULL),
    (dict(k=ctypes.c_void_p(2 * GiB + 2)), ALIGN),
    (dict(o=ctypes.c_void_p(5 * GiB + 1024)), ALIAS),        # o inside S
    (dict(S=ctypes.c_void_p(GiB + 64)), ALIAS),              # S overlaps q
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(N=0), dict(H=0), dict(N=0, S=None)])
def test_decode_empty_is_noop(lib, kw):
    assert decode(lib, **kw) == OK


def multi(lib, q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), S=P(5), o=P(6), ntok=None, update=1, N=8, T=4,
          H=32, dk=128, dv=128, dt=BF16):
    return lib.kda_decode_multi(q, k, v, g, beta, S, o, ntok, update, N, T, H, dk, dv, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=2), DTYPE), (dict(T=-1), SHAPE), (dict(N=-3), SHAPE), (dict(update=2), SHAPE),
    (dict(T=17), UNSUP), (dict(dk=96, dv=96), UNSUP),
    (dict(S=None), NULL), (dict(beta=None), NULL),
    (dict(ntok=ctypes.c_void_p(7 * GiB + 4)), ALIGN), (dict(o=ctypes.c_void_p(6 * GiB + 2)), ALIGN),
    (dict(o=ctypes.c_void_p(6 * GiB + 4096)), ALIAS),        # o inside S
    (dict(S=ctypes.c_void_p(GiB + 256)), ALIAS),             # S overlaps q
])
def test_decode_multi_rejects(lib, kw, code):
    assert multi(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(N=0), dict(T=0), dict(H=0), dict(o=None, update=0),
                                dict(N=0, q=None, S=None)])
def test_decode_multi_noop(lib, kw):
    assert multi(lib, **kw) == OK



# ---- layer entry points ----
def _opts(conv_w=None, W=0, silu=0, z=None, norm_w=None, eps=1e-6):
    o = kda.LayerOpts()
    o.conv_w = conv_w.value if conv_w is not None else None
    o.conv_width = W
    o.conv_silu = silu
    o.gate_z = z.value if z is not None else None
    o.norm_w = norm_w.value if norm_w is not None else None
    o.norm_eps = eps
    return o


def prefill_layer(lib, q=P(0), k=P(1), v=P(2), a=P(3), b=P(4), conv_in=None, conv_out=None, S0=None,
                  o=P(5), S_T=P(6), ckpt=None, ckpt_every=0, B=1, T=256, H=2, dk=128, dv=128, dt=BF16,
                  opts=None, ws=P(10), ws_bytes=WS_NEED):
    return lib.kda_prefill_layer(q, k, v, a, b, conv_in, conv_out, S0, o, S_T, ckpt, ckpt_every, B, T, H,
                                 dk, dv, dt, ctypes.byref(opts) if opts is not None else None, ws, ws_bytes,
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=FP32), UNSUP), (dict(dt=5), DTYPE), (dict(dk=96, dv=96), UNSUP), (dict(T=-1), SHAPE),
    (dict(opts=_opts(conv_w=P(11), W=5)), UNSUP), (dict(opts=_opts(conv_w=P(11), W=0)), UNSUP),
    (dict(opts=_opts(conv_w=P(11), W=3, silu=2)), SHAPE),
    (dict(opts=_opts(z=P(12), eps=-1.0)), SHAPE),
    (dict(opts=_opts(conv_w=ctypes.c_void_p(11 * GiB + 4), W=3)), ALIGN),
    (dict(a=None), NULL), (dict(S_T=None), NULL),
    # conv_out overlapping conv_in, and conv_out inside q
    (dict(opts=_opts(conv_w=P(11), W=4), conv_in=P(13), conv_out=ctypes.c_void_p(14 * GiB + 64)), ALIAS),
    (dict(opts=_opts(conv_w=P(11), W=4), conv_out=ctypes.c_void_p(GiB + 4096)), ALIAS),
    # o overlapping the output-gate logits
    (dict(opts=_opts(z=ctypes.c_void_p(6 * GiB + 4096))), ALIAS),
    (dict(ws_bytes=WS_NEED - 1), WS),
])
def test_prefill_layer_rejects(lib, kw, code):
    assert prefill_layer(lib, **kw) == code


def test_prefill_layer_noop(lib):
    assert prefill_layer(lib, B=0) == OK
    assert prefill_layer(lib, H=0, opts=_opts(conv_w=P(11), W=4)) == OK


def decode_layer(lib, q=P(0), k=P(1), v=P(2), a=P(3), b=P(4), conv_state=None, S=P(6), o=P(5), N=4, H=2,
                 dk=128, dv=128, dt=BF16, opts=None):
    return lib.kda_decode_layer_step(q, k, v, a, b, conv_state, S, o, N, H, dk, dv, dt,
                                     ctypes.byref(opts) if opts is not None else None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), DTYPE), (dict(N=-1), SHAPE), (dict(dk=64, dv=128), UNSUP),
    (dict(opts=_opts(conv_w=P(11), W=3)), NULL),                      # W > 1 needs conv_state
    (dict(opts=_opts(conv_w=P(11), W=9), conv_state=P(13)), UNSUP),
    (dict(b=None), NULL),
    (dict(opts=_opts(conv_w=P(11), W=3), conv_state=ctypes.c_void_p(7 * GiB + 8)), ALIGN),
    (dict(opts=_opts(conv_w=P(11), W=3), conv_state=ctypes.c_void_p(GiB + 1024)), ALIAS),
    (dict(o=ctypes.c_void_p(7 * GiB + 1024)), ALIAS),                   # o inside S
])
def test_decode_layer_rejects(lib, kw, code):
    assert decode_layer(lib, **kw) == code


def test_decode_layer_noop(lib):
    assert decode_layer(lib, N=0, opts=_opts(conv_w=P(11), W=4)) == OK


@pytest.mark.parametrize("args,code", [
    ((P(0), P(1), None, 1e-6, P(2), 10, 128, 7), DTYPE),
    ((P(0), P(1), None, 1e-6, P(2), -1, 128, BF16), SHAPE),
    ((P(0), P(1), None, -1.0, P(2), 10, 128, BF16), SHAPE),
    ((P(0), P(1), None, 1e-6, P(2), 10, 96, BF16), UNSUP),
    ((P(0), None, None, 1e-6, P(2), 10, 128, BF16), NULL),
    ((P(0), P(1), None, 1e-6, ctypes.c_void_p(2 * GiB + 256), 10, 128, BF16), ALIAS),  # y inside z
    ((P(0), P(1), None, 1e-6, ctypes.c_void_p(GiB + 512), 10, 128, BF16), ALIAS),      # y partly on o
    ((P(0), P(1), ctypes.c_void_p(3 * GiB + 4), 1e-6, P(2), 10, 128, BF16), ALIGN),
    ((P(0), P(1), None, 1e-6, P(2), 0, 128, BF16), OK),
])
def test_output_norm_gate_rejects(lib, args, code):
    o, z, w, eps, y, rows, dv, dt = args
    assert lib.kda_output_norm_gate(o, z, w, eps, y, rows, dv, dt, None) == code


# ---- segment stages ----
SEG_WS = 2 * 2 * 72704  # B=1, H=2, 128 tokens, dk=128


@pytest.mark.parametrize("t_begin,t_len,ws_bytes,code", [
    (32, 64, SEG_WS, UNSUP),        # not on a chunk boundary
    (-64, 64, SEG_WS, SHAPE),
    (192, 128, SEG_WS, SHAPE),      # past T = 256
    (64, -1, SEG_WS, SHAPE),
    (64, 128, SEG_WS - 1, WS),      # workspace below the segment's records
    (64, 0, 0, OK),                 # empty segment: nothing to prepare
])
def test_segment_prep_rejects(lib, t_begin, t_len, ws_bytes, code):
    rc = lib.kda_prefill_segment_prep(P(0), P(1), P(2), P(3), P(4), 1, 256, 2, 128, 128, BF16, t_begin, t_len,
                                      P(10), ws_bytes, None)
    assert rc == code


@pytest.mark.parametrize("t_begin,t_len,ws_bytes,code", [
    (32, 64, SEG_WS, UNSUP), (192, 128, SEG_WS, SHAPE), (64, 128, SEG_WS - 1, WS),
])
def test_segment_recur_rejects(lib, t_begin, t_len, ws_bytes, code):
    rc = lib.kda_prefill_segment_recur(P(10), ws_bytes, None, P(5), P(6), None, 0, 1, 256, 2, 128, 128, BF16,
                                       t_begin, t_len, None)
    assert rc == code
