/* Host-side validation of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every call below is rejected on the host or is
 * a documented no-op, so no kernel is launched and no device is needed.  Fake
 * "device" pointers are only compared, never dereferenced; host arrays
 * (cu_seqlens, the layer options) are real and exactly as long as documented,
 * so an out-of-bounds read by the library is reported by the sanitizer.
 * Exit status 0 when every status code is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "kda.h"

static int failures = 0;
#define GiB ((uintptr_t)1 << 30)
#define P(i) ((void *)(((uintptr_t)(i) + 1) * GiB))
#define F(i) ((float *)P(i))

static void expect(const char *what, int got, int want) {
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

int main(void) {
    const size_t ws = (size_t)2 * 4 * 72704;
    /* kda_prefill */
    expect("prefill ok-noop B=0", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 0, 256, 2, 128,
                                              128, KDA_BF16, P(10), ws, NULL), KDA_OK);
    expect("prefill dtype", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, 256, 2, 128, 128,
                                         (kda_dtype)7, P(10), ws, NULL), KDA_ERR_DTYPE);
    expect("prefill shape", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, -1, 2, 128, 128,
                                         KDA_BF16, P(10), ws, NULL), KDA_ERR_SHAPE);
    expect("prefill unsupported", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, 256, 2, 96,
                                               96, KDA_BF16, P(10), ws, NULL), KDA_ERR_UNSUPPORTED);
    expect("prefill null", kda_prefill(NULL, P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, 256, 2, 128, 128,
                                        KDA_BF16, P(10), ws, NULL), KDA_ERR_NULL);
    expect("prefill align", kda_prefill((char *)P(0) + 8, P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, 256, 2,
                                         128, 128, KDA_BF16, P(10), ws, NULL), KDA_ERR_ALIGN);
    expect("prefill alias", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, (char *)P(0) + 4096, F(6), NULL, 0, 1, 256,
                                         2, 128, 128, KDA_BF16, P(10), ws, NULL), KDA_ERR_ALIAS);
    expect("prefill workspace", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, 256, 2, 128,
                                             128, KDA_BF16, P(10), ws - 1, NULL), KDA_ERR_WORKSPACE);
    expect("prefill grid overflow", kda_prefill(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL, 0, 1, 1 << 16,
                                                 1 << 22, 128, 128, KDA_BF16, P(10), ws, NULL), KDA_ERR_SHAPE);
    /* kda_prefill_noalloc */
    expect("noalloc heads beyond the scratch", kda_prefill_noalloc(P(0), P(1), P(2), F(3), F(4), NULL, P(5), F(6), NULL,
                                                                   0, 1, 64, 924, 128, 128, KDA_BF16, NULL),
           KDA_ERR_WORKSPACE);
    expect("noalloc null", kda_prefill_noalloc(P(0), P(1), P(2), F(3), F(4), NULL, P(5), NULL, NULL, 0, 1, 64, 2, 128,
                                               128, KDA_BF16, NULL), KDA_ERR_NULL);
    /* workspace sizes and segment lengths (pure host arithmetic) */
    expect("workspace size", kda_prefill_workspace_size(1, 32768, 32, 128, 128, KDA_BF16) == (size_t)32 * 103 * 72704,
           1);
    expect("segment tokens", kda_prefill_segment_tokens(1, 32768, 32, 128, 128, KDA_BF16), 6592);
    expect("stage workspace", kda_prefill_stage_workspace_size(2, 100, 3, 64, 64, KDA_BF16) == (size_t)2 * 3 * 2 * 39936,
           1);
    /* stage entry points */
    expect("chunk prep dtype", kda_prefill_chunk_prep(P(0), P(1), P(2), F(3), F(4), 1, 256, 2, 128, 128, KDA_FP32, P(10),
                                                      ws, NULL), KDA_ERR_UNSUPPORTED);
    expect("chunk recur ws", kda_prefill_chunk_recur(P(10), ws - 1, NULL, P(5), F(6), NULL, 0, 1, 256, 2, 128, 128,
                                                     KDA_BF16, NULL), KDA_ERR_WORKSPACE);
    expect("segment prep begin", kda_prefill_segment_prep(P(0), P(1), P(2), F(3), F(4), 1, 256, 2, 128, 128, KDA_BF16,
                                                          32, 64, P(10), ws, NULL), KDA_ERR_UNSUPPORTED);
    expect("segment recur range", kda_prefill_segment_recur(P(10), ws, NULL, P(5), F(6), NULL, 0, 1, 256, 2, 128, 128,
                                                            KDA_BF16, 192, 128, NULL), KDA_ERR_SHAPE);
    /* packed prompts: host offsets, exactly num_seqs + 1 entries each */
    {
        int *cu = malloc(6 * sizeof(int));
        const int vals[6] = {0, 100, 100, 300, 301, 640};
        for (int i = 0; i < 6; ++i) cu[i] = vals[i];
        expect("varlen checkpoints", (int)kda_prefill_varlen_num_checkpoints(cu, 5, 128), 1 + 0 + 2 + 1 + 3);
        expect("varlen checkpoints interval", (int)kda_prefill_varlen_num_checkpoints(cu, 5, 100), -1);
        expect("varlen workspace > 0", kda_prefill_varlen_workspace_size(cu, 5, 4, 128, 128, KDA_BF16) > 0, 1);
        expect("varlen null o", kda_prefill_varlen(P(0), P(1), P(2), F(3), F(4), cu, 5, NULL, NULL, F(6), NULL, 0, 4,
                                                   128, 128, KDA_BF16, P(10), 1 << 30, NULL), KDA_ERR_NULL);
        cu[3] = 50; /* decreasing */
        expect("varlen decreasing", kda_prefill_varlen(P(0), P(1), P(2), F(3), F(4), cu, 5, NULL, P(5), F(6), NULL, 0, 4,
                                                       128, 128, KDA_BF16, P(10), 1 << 30, NULL), KDA_ERR_SHAPE);
        expect("varlen workspace of bad offsets", (int)kda_prefill_varlen_workspace_size(cu, 5, 4, 128, 128, KDA_BF16), 0);
        free(cu);
        int *one = malloc(sizeof(int));
        one[0] = 0;
        expect("varlen no sequences", kda_prefill_varlen(P(0), P(1), P(2), F(3), F(4), one, 0, NULL, P(5), F(6), NULL, 0,
                                                         4, 128, 128, KDA_BF16, P(10), 1 << 30, NULL), KDA_OK);
        free(one);
    }
    /* decode */
    expect("decode dtype", kda_decode_step(P(0), P(1), P(2), F(3), F(4), F(5), P(6), 4, 2, 128, 128, (kda_dtype)3, NULL),
           KDA_ERR_DTYPE);
    expect("decode alias", kda_decode_step(P(0), P(1), P(2), F(3), F(4), F(5), P(0), 4, 2, 128, 128, KDA_BF16, NULL),
           KDA_ERR_ALIAS);
    expect("decode noop", kda_decode_step(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 2, 128, 128, KDA_BF16, NULL),
           KDA_OK);
    expect("decode multi T", kda_decode_multi(P(0), P(1), P(2), F(3), F(4), F(5), P(6), NULL, 1, 4, 17, 2, 128, 128,
                                              KDA_BF16, NULL), KDA_ERR_UNSUPPORTED);
    /* layer entry points with a real options struct */
    {
        kda_layer_opts *opts = malloc(sizeof(kda_layer_opts));
        opts->conv_w = F(20);
        opts->conv_width = 5;
        opts->conv_silu = 1;
        opts->gate_z = NULL;
        opts->norm_w = NULL;
        opts->norm_eps = 1e-6f;
        expect("layer conv width", kda_prefill_layer(P(0), P(1), P(2), F(3), F(4), NULL, NULL, NULL, P(5), F(6), NULL, 0,
                                                     1, 256, 2, 128, 128, KDA_BF16, opts, P(10), 1 << 30, NULL),
               KDA_ERR_UNSUPPORTED);
        opts->conv_width = 4;
        expect("layer decode null state", kda_decode_layer_step(P(0), P(1), P(2), F(3), F(4), NULL, F(6), P(7), 4, 2,
                                                                128, 128, KDA_BF16, opts, NULL), KDA_ERR_NULL);
        free(opts);
    }
    expect("norm gate dv", kda_output_norm_gate(P(0), P(1), NULL, 1e-6f, P(2), 10, 96, KDA_BF16, NULL),
           KDA_ERR_UNSUPPORTED);
    for (int c = 0; c < 10; ++c)
        if (!kda_status_string((kda_status)c)) ++failures;
    if (failures) {
        fprintf(stderr, "%d unexpected status codes\n", failures);
        return 1;
    }
    printf("abi validation under sanitizers: ok\n");
    return 0;
}
