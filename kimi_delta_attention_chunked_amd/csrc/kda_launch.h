// kda_launch.h -- internal launchers behind the C ABI (not installed).
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

// The layer steps around the recurrence (short causal convolution of q, k, v,
// L2 norm of q and k, decay and write strength from sigmoid gates), applied
// while the inputs are loaded.  conv_w: [H, W, 2dk+dv] taps (tap j multiplies
// token t - (W-1) + j; channels q, then k, then v) or nullptr for no
// convolution; conv_in / conv_out: [seqs, H, 2dk+dv, W-1] inputs before the
// first token (oldest first) / after the last one, either may be nullptr.
struct LayerArgs {
    const float* conv_w;
    const float* conv_in;
    float* conv_out;
    int W;
    int silu;
};

// bf16 chunked prefill, stage 1: per-chunk operand records into ws (one
// record per (batch, head, 64-token chunk)) for tokens [t0, t0 + tlen) of B
// sequences of T tokens (tlen < 0: to the end); t0 is a multiple of 64.
hipError_t launch_prefill_prep(int dk, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, int B, int T, int H, void* ws, hipStream_t stream,
                               int t0 = 0, int tlen = -1);

// bf16 chunked prefill, stage 2: the chunk-to-chunk recurrence over the
// records of tokens [t0, t0 + tlen), from S0 (the state before t0).
hipError_t launch_prefill_recur(int dk, const void* ws, const float* S0, void* o, float* S_T, float* ckpt,
                                int ckpt_every, int B, int T, int H, hipStream_t stream, int t0 = 0,
                                int tlen = -1);

// Device workspace the prefill needs (per-chunk operand records of the bf16 path).
size_t prefill_workspace_bytes(int dt, int dk, int B, int T, int H);

// Bound on the records of one prefill segment (all heads).  The recurrence
// reads a segment's records back from the Infinity Cache only while they fit
// it with some margin: segments of 235 MiB of records were seen to fall out of
// it on some workspace buffers (the recurrence then ran 1.5x slower), segments
// of 229 MiB never were.
constexpr size_t kSegmentRecordBytes = 232ull << 20;

// bf16 prefill of S packed sequences (token offsets cu_seqlens_host[0..S], on
// the host; total_chunks = sum of ceil(len / 64)).  The offsets are passed to a
// small kernel as arguments, which writes them into
// the workspace, which holds varlen_workspace_bytes(...) bytes.
size_t varlen_workspace_bytes(int dk, int S, long long total_chunks, int H);
hipError_t launch_prefill_varlen(int dk, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int* cu_seqlens_host, int S, long long total_chunks,
                                 int H, const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every,
                                 void* ws, hipStream_t stream);

// bf16 layer prefill: stage 1 with the layer steps (a: decay-gate logits in
// place of g, b: write-gate logits in place of beta), then stage 2.  When
// conv_out is given and T == 0 it receives conv_in (zeros without one).
hipError_t launch_prefill_layer(int dk, const void* q, const void* k, const void* v, const float* a,
                                const float* b, const LayerArgs& la, int B, int T, int H, const float* S0,
                                void* o, float* S_T, float* ckpt, int ckpt_every, void* ws, hipStream_t stream,
                                int t0 = 0, int tlen = -1);

// y = o * w / sqrt(mean(o^2) + eps) * sigmoid(z) per row of dv (w == nullptr: ones); y may be o.
hipError_t launch_output_norm_gate(int dt, const void* o, const void* z, const float* w, float eps, void* y,
                                   long long rows, int dv, hipStream_t stream);

// out[i] = in[i] (in == nullptr: 0) for i < n.
hipError_t launch_fill_copy(const float* in, float* out, long long n, hipStream_t stream);

// One decode token of the layer: conv_state ([N, H, 2dk+dv, W-1]) and S in
// place; with z, o is normalized and gated.
hipError_t launch_decode_layer(int dt, int dk, const void* q, const void* k, const void* v, const float* a,
                               const float* b, const LayerArgs& la, float* conv_state, float* S, const void* z,
                               const float* norm_w, float eps, void* o, int N, int H, hipStream_t stream);

// Chunked prefill with fp32 q/k/v/o (fp32 MFMA operands); dk = 64 or 128.
hipError_t launch_prefill_f32(int dk, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* S0, void* o,
                              float* S_T, float* ckpt, int ckpt_every, int B, int T, int H,
                              hipStream_t stream);

// One decode token for N*H independent heads, state updated in place.
hipError_t launch_decode(int dt, int dk, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* S, void* o, int N, int H,
                         hipStream_t stream);

// Up to 16 tokens per sequence from the state S ([N,T,H,.] inputs, o may be
// NULL); ntok (device, [N]) limits each sequence's tokens, NULL = all T;
// update = 0 leaves S untouched.
hipError_t launch_decode_multi(int dt, int dk, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, float* S, void* o, const int* ntok, int N, int T, int H,
                               int update, hipStream_t stream);

}  // namespace kda
