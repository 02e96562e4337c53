"""bench.py's host-side accounting on the CPU: the per-token byte and FLOP
models the roofline uses, the per-chunk record size it charges to the two
kernels (against the library's own workspace size), and the segment list it
times (against the library's segment rule).  Nothing here touches a device."""
import ctypes

import pytest

import bench
import kimi_delta_attention_chunked_amd as kda

BF16 = 1


def test_compulsory_bytes_per_token_head():
    # q, k, v, o in the input dtype, g per channel and beta in fp32: 1540 bytes
    # per token-head at dk = dv = 128 in bf16, 1284 at 64 in fp32.
    assert bench.prefill_min_bytes(1, 1, 1, 128, 2, False, 0) - 4 * 128 * 128 == 1540
    assert bench.prefill_min_bytes(1, 1, 1, 64, 4, False, 0) - 4 * 64 * 64 == 1284
    # states: S_T always, S0 when given, one per checkpoint
    base = bench.prefill_min_bytes(2, 10, 3, 128, 2, False, 0)
    assert bench.prefill_min_bytes(2, 10, 3, 128, 2, True, 0) - base == 2 * 3 * 4 * 128 * 128
    assert bench.prefill_min_bytes(2, 10, 3, 128, 2, False, 5) - base == 5 * 2 * 3 * 4 * 128 * 128


def test_pages_counts_per_chunk():
    # 12C^3 + 8C^2 D + 6CD^2 FLOPs and 8C^2 + 22CD bytes per chunk, at C = 64, D = 128
    C, D = 64, 128
    assert bench.prefill_flops_per_token_head(D) * C == 12 * C ** 3 + 8 * C * C * D + 6 * C * D * D
    assert bench.prefill_flops_per_token_head(D) == 212992
    assert bench.pages_bytes_per_chunk(D) == 8 * C * C + 22 * C * D == 212992
    assert bench.pages_bytes_per_chunk(D) // C == 3328


@pytest.mark.parametrize("D", [64, 128])
def test_record_bytes_match_library(D):
    lib = kda.library()
    lib.kda_prefill_stage_workspace_size.restype = ctypes.c_size_t
    per_chunk = lib.kda_prefill_stage_workspace_size(1, 64, 1, D, D, BF16)
    assert per_chunk == bench.RECORD_BYTES[D]


def test_kernel_traffic_counts_records_once_each_way():
    B, T, H, D = 1, 32768, 32, 128
    lib = kda.library()
    L = lib.kda_prefill_segment_tokens(B, T, H, D, D, BF16)
    segs = [(t0, min(L, T - t0)) for t0 in range(0, T, L)]
    assert len(segs) == 5 and sum(tl for _, tl in segs) == T
    t = bench.kernel_traffic_bytes(B, T, H, D, segs)
    rec = B * H * (T // 64) * bench.RECORD_BYTES[D]
    tok = B * T * H
    assert t[bench.PREP_KERNEL] == tok * (3 * D * 2 + 4 * D + 4) + rec
    # the recurrence: records, o, and the state written per segment and read back by the next
    assert t[bench.RECUR_KERNEL] == rec + tok * D * 2 + B * H * D * D * 4 * 9
    # records add 2 x 1136 bytes per token-head to the 1540 compulsory ones
    assert rec // tok == 1136
