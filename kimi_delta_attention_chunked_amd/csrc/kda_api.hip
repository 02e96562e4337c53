// kda_api.hip -- the C ABI declared in include/kda.h: host-side validation,
// then the kernel launches on the caller's stream.  No allocation, no host
// synchronisation; the only global state is the per-device address of
// kda_prefill_noalloc's static scratch.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

constexpr int kChunk = 64;  // prefill chunk length; checkpoints fall on chunk ends

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

struct Range {
    const void* p;
    size_t n;
};

// Any output range intersecting any input range, or two outputs intersecting.
// `allowed_same` names one (output, input) pair that may be the identical range.
bool bad_alias(const Range* outs, int n_out, const Range* ins, int n_in, const void* same_out,
               const void* same_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j) {
            if (!overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) continue;
            if (outs[i].p == same_out && ins[j].p == same_in && same_out == same_in &&
                outs[i].n == ins[j].n)
                continue;
            return true;
        }
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return true;
    }
    return false;
}

bool supported_head(int dk, int dv) { return dk == dv && (dk == 64 || dk == 128); }

// The integer an enum argument carries, read from its bytes: C callers may pass
// any int, and in C++ reading an enum object whose value lies outside the
// enumeration's range is undefined, so the value is validated as an int.
static_assert(sizeof(kda_dtype) == sizeof(int) && sizeof(kda_status) == sizeof(int), "enum ABI");
template <class E>
int enum_bits(const E* e) {
    int x;
    memcpy(&x, e, sizeof x);
    return x;
}

}  // namespace

// Layer options: a missing struct means no convolution and no output step.
static kda_status check_layer_opts(const kda_layer_opts* opts, int H, int dk, int dv, kda::LayerArgs* la,
                                   size_t* taps_bytes) {
    *la = kda::LayerArgs{};
    *taps_bytes = 0;
    if (!opts) return KDA_OK;
    if (opts->conv_w) {
        if (opts->conv_width < 1 || opts->conv_width > 4) return KDA_ERR_UNSUPPORTED;
        if (opts->conv_silu != 0 && opts->conv_silu != 1) return KDA_ERR_SHAPE;
        if (!aligned16(opts->conv_w)) return KDA_ERR_ALIGN;
        la->conv_w = opts->conv_w;
        la->W = opts->conv_width;
        la->silu = opts->conv_silu;
        *taps_bytes = (size_t)H * opts->conv_width * (2 * dk + dv) * sizeof(float);
    }
    if (opts->gate_z && !(opts->norm_eps >= 0.f && opts->norm_eps <= 3.0e38f)) return KDA_ERR_SHAPE;
    if (!aligned16(opts->gate_z) || !aligned16(opts->norm_w)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

extern "C" {

const char* kda_status_string(kda_status s_arg) {
    switch (enum_bits(&s_arg)) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is negative or out of range";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown dtype";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a pointer is not 16-byte aligned";
        case KDA_ERR_UNSUPPORTED:
            return "KDA_ERR_UNSUPPORTED: needs dk == dv in {64, 128}, "
                   "ckpt_every a multiple of 64";
        case KDA_ERR_WORKSPACE:
            return "KDA_ERR_WORKSPACE: workspace too small (kda_prefill_noalloc: one chunk of all B*H heads "
                   "exceeds its static scratch)";
        case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
    }
    return "KDA_ERR_UNKNOWN";
}

int kda_version(void) { return 100; }

static kda_status check_prefill_sizes(int dt, int B, int T, int H, int dk, int dv, int ckpt_every);
static int segment_tokens_impl(int B, int T, int H, int dk);

kda_status kda_prefill_layer(const void* q, const void* k, const void* v, const float* a, const float* b,
                             const float* conv_in, float* conv_out, const float* S0, void* o, float* S_T,
                             float* ckpt, int ckpt_every, int B, int T, int H, int dk, int dv, kda_dtype dt_arg,
                             const kda_layer_opts* opts, void* workspace, size_t workspace_bytes, void* stream) {
    const int dt = enum_bits(&dt_arg);
    kda_status st = check_prefill_sizes(dt, B, T, H, dk, dv, ckpt_every);
    if (st != KDA_OK) return st;
    if (dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    kda::LayerArgs la;
    size_t taps_bytes;
    if ((st = check_layer_opts(opts, H, dk, dv, &la, &taps_bytes)) != KDA_OK) return st;
    if (B == 0 || H == 0) return KDA_OK;
    if (!S_T) return KDA_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !a || !b || !o)) return KDA_ERR_NULL;
    const int n_ck = ckpt_every > 0 ? (T + ckpt_every - 1) / ckpt_every : 0;
    if (n_ck > 0 && !ckpt) return KDA_ERR_NULL;
    const void* z = opts ? opts->gate_z : nullptr;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) ||
        !aligned16(conv_in) || !aligned16(conv_out) || !aligned16(S0) || !aligned16(o) ||
        !aligned16(S_T) || !aligned16(ckpt) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const size_t ws_need = kda_prefill_workspace_size(B, T, H, dk, dv, (kda_dtype)dt);  // dt checked above
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE;
    if (ws_need > 0 && !workspace) return KDA_ERR_NULL;
    const int W = la.conv_w ? la.W : 1;
    if (W == 1) conv_in = nullptr, conv_out = nullptr;  // a width-1 convolution carries no state
    la.conv_in = conv_in;
    la.conv_out = conv_out;

    const size_t es = 2;
    const size_t tok = (size_t)B * T * H;
    const size_t stb = (size_t)B * H * dk * dv * sizeof(float);
    const size_t csb = (size_t)B * H * (2 * dk + dv) * (W - 1) * sizeof(float);
    const Range ins[] = {{q, tok * dk * es}, {k, tok * dk * es}, {v, tok * dv * es},
                         {a, tok * dk * sizeof(float)}, {b, tok * sizeof(float)}, {S0, S0 ? stb : 0},
                         {conv_in, conv_in ? csb : 0}, {la.conv_w, taps_bytes},
                         {z, z ? tok * dv * es : 0}, {opts ? opts->norm_w : nullptr, dv * sizeof(float)}};
    const Range outs[] = {{o, tok * dv * es}, {S_T, stb}, {ckpt, n_ck > 0 ? (size_t)n_ck * stb : 0},
                          {workspace, ws_need}, {conv_out, conv_out ? csb : 0}};
    if (bad_alias(outs, 5, ins, 10, S_T, S0)) return KDA_ERR_ALIAS;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    const int L = segment_tokens_impl(B, T, H, dk);
    for (int t0 = 0; e == hipSuccess; t0 += L) {
        const int tl = T - t0 < L ? T - t0 : L;
        kda::LayerArgs seg = la;
        if (t0 + L < T) seg.conv_out = nullptr;  // the carried state is the last segment's
        e = kda::launch_prefill_layer(dk, q, k, v, a, b, seg, B, T, H, t0 == 0 ? S0 : S_T, o, S_T,
                                      n_ck > 0 ? ckpt : nullptr, n_ck > 0 ? ckpt_every : 0, workspace, s, t0, tl);
        if (t0 + L >= T) break;
    }
    if (e == hipSuccess && z && T > 0)
        e = kda::launch_output_norm_gate(1, o, z, opts->norm_w, opts->norm_eps, o, (long long)tok, dv, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_layer_step(const void* q, const void* k, const void* v, const float* a, const float* b,
                                 float* conv_state, float* S, void* o, int N, int H, int dk, int dv,
                                 kda_dtype dt_arg, const kda_layer_opts* opts, void* stream) {
    const int dt = enum_bits(&dt_arg);
    if (dt != KDA_FP32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (!supported_head(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_SHAPE;
    kda::LayerArgs la;
    size_t taps_bytes;
    kda_status st = check_layer_opts(opts, H, dk, dv, &la, &taps_bytes);
    if (st != KDA_OK) return st;
    if (N == 0 || H == 0) return KDA_OK;
    const int W = la.conv_w ? la.W : 1;
    if (!q || !k || !v || !a || !b || !S || !o || (W > 1 && !conv_state)) return KDA_ERR_NULL;
    if (W == 1) conv_state = nullptr;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) ||
        !aligned16(conv_state) || !aligned16(S) || !aligned16(o))
        return KDA_ERR_ALIGN;
    const void* z = opts ? opts->gate_z : nullptr;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t nh = (size_t)N * H;
    const Range ins[] = {{q, nh * dk * es}, {k, nh * dk * es}, {v, nh * dv * es},
                         {a, nh * dk * sizeof(float)}, {b, nh * sizeof(float)}, {la.conv_w, taps_bytes},
                         {z, z ? nh * dv * es : 0}, {opts ? opts->norm_w : nullptr, dv * sizeof(float)}};
    const Range outs[] = {{o, nh * dv * es}, {S, nh * dk * dv * sizeof(float)},
                          {conv_state, conv_state ? nh * (2 * dk + dv) * (W - 1) * sizeof(float) : 0}};
    if (bad_alias(outs, 3, ins, 8, nullptr, nullptr)) return KDA_ERR_ALIAS;
    const hipError_t e = kda::launch_decode_layer(dt == KDA_BF16 ? 1 : 0, dk, q, k, v, a, b, la, conv_state, S, z,
                                                  opts ? opts->norm_w : nullptr, opts ? opts->norm_eps : 0.f, o,
                                                  N, H, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_output_norm_gate(const void* o, const void* z, const float* norm_w, float eps, void* y,
                                long long rows, int dv, kda_dtype dt_arg, void* stream) {
    const int dt = enum_bits(&dt_arg);
    if (dt != KDA_FP32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (rows < 0 || dv <= 0 || !(eps >= 0.f && eps <= 3.0e38f)) return KDA_ERR_SHAPE;
    if (dv != 64 && dv != 128) return KDA_ERR_UNSUPPORTED;
    if (rows == 0) return KDA_OK;
    if (!o || !z || !y) return KDA_ERR_NULL;
    if (!aligned16(o) || !aligned16(z) || !aligned16(y) || !aligned16(norm_w)) return KDA_ERR_ALIGN;
    const size_t n = (size_t)rows * dv * (dt == KDA_BF16 ? 2 : 4);
    const Range ins[] = {{o, n}, {z, n}, {norm_w, norm_w ? dv * sizeof(float) : 0}};
    const Range outs[] = {{y, n}};
    if (bad_alias(outs, 1, ins, 3, y, o)) return KDA_ERR_ALIAS;
    const hipError_t e = kda::launch_output_norm_gate(dt == KDA_BF16 ? 1 : 0, o, z, norm_w, eps, y, rows, dv,
                                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Segment length of the bf16 prefill.  A segment's records (all B*H heads)
// should stay within kSegmentRecordBytes (232 MiB), so that the recurrence
// reads them back from the 256 MB Infinity Cache instead of HBM; the inputs
// they are made from are read with the streaming hint and do not stay in that
// cache.  The length is the whole sequence split into the fewest segments
// under that bound, rounded up to whole chunks, so that the last segment is
// not a short remainder.  Below 384 tokens per segment the per-segment
// start-up costs more than the cache saves, and the whole length is one
// segment.
static int segment_tokens_impl(int B, int T, int H, int dk) {
    const size_t rec = kda::prefill_workspace_bytes(1, dk, 1, kChunk, 1);  // one record
    if (rec == 0 || B <= 0 || H <= 0 || T <= 0) return T;
    const size_t per_token = (size_t)B * H * (rec / kChunk);
    const long long Lmax = (long long)(kda::kSegmentRecordBytes / per_token) / kChunk * kChunk;
    if (Lmax < 384 || Lmax >= T) return T;
    const long long n = (T + Lmax - 1) / Lmax;                              // segments
    const long long L = ((T + n - 1) / n + kChunk - 1) / kChunk * kChunk;  // <= Lmax
    return (int)L;
}

int kda_prefill_segment_tokens(int B, int T, int H, int dk, int dv, kda_dtype dt_arg) {
    const int dt = enum_bits(&dt_arg);
    if (B < 0 || T < 0 || H < 0 || dk != dv || dt != KDA_BF16) return T < 0 ? 0 : T;
    return segment_tokens_impl(B, T, H, dk);
}

size_t kda_prefill_stage_workspace_size(int B, int T, int H, int dk, int dv, kda_dtype dt_arg) {
    const int dt = enum_bits(&dt_arg);
    if (B < 0 || T < 0 || H < 0 || dk != dv || (dt != KDA_FP32 && dt != KDA_BF16)) return 0;
    return kda::prefill_workspace_bytes(dt == KDA_BF16 ? 1 : 0, dk, B, T, H);
}

size_t kda_prefill_workspace_size(int B, int T, int H, int dk, int dv, kda_dtype dt_arg) {
    const int dt = enum_bits(&dt_arg);
    if (B < 0 || T < 0 || H < 0 || dk != dv || (dt != KDA_FP32 && dt != KDA_BF16)) return 0;
    if (dt != KDA_BF16) return 0;
    return kda::prefill_workspace_bytes(1, dk, B, segment_tokens_impl(B, T, H, dk), H);
}

// Sizes, dtype and checkpoint interval shared by the prefill entry points.
static kda_status check_prefill_sizes(int dt, int B, int T, int H, int dk, int dv, int ckpt_every) {
    if (dt != KDA_FP32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || ckpt_every < 0) return KDA_ERR_SHAPE;
    if (!supported_head(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (ckpt_every % kChunk != 0) return KDA_ERR_UNSUPPORTED;
    // Grids: B*H*(dv/16) workgroups for the recurrence, B*H*ceil(T/64) for the
    // chunk preparation; token indices B*T; all must fit a signed 32-bit int.
    const int64_t chunks = ((int64_t)T + kChunk - 1) / kChunk;
    if ((int64_t)B * H * (dv / 16) > INT32_MAX || (int64_t)B * T > INT32_MAX ||
        (int64_t)B * H * chunks > INT32_MAX)
        return KDA_ERR_SHAPE;
    return KDA_OK;
}

// Validation shared by kda_prefill and kda_prefill_noalloc: sizes, pointers,
// alignment and aliasing of the caller's tensors and of the workspace range
// [workspace, workspace + ws_bytes) (none for the static scratch).  *n_ck
// receives the number of checkpoints.  KDA_OK with *noop set: nothing to do.
static kda_status prefill_checks(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every, int B, int T,
                                 int H, int dk, int dv, int dt, const void* workspace, size_t ws_bytes,
                                 int* n_ck, bool* noop) {
    *noop = false;
    kda_status st = check_prefill_sizes(dt, B, T, H, dk, dv, ckpt_every);
    if (st != KDA_OK) return st;
    if (B == 0 || H == 0) {
        *noop = true;
        return KDA_OK;
    }
    if (!S_T) return KDA_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    *n_ck = ckpt_every > 0 ? (T + ckpt_every - 1) / ckpt_every : 0;
    if (*n_ck > 0 && !ckpt) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(S0) || !aligned16(o) || !aligned16(S_T) || !aligned16(ckpt) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t tok = (size_t)B * T * H;
    const size_t stb = (size_t)B * H * dk * dv * sizeof(float);
    const Range ins[] = {{q, tok * dk * es}, {k, tok * dk * es}, {v, tok * dv * es},
                         {g, tok * dk * sizeof(float)}, {beta, tok * sizeof(float)}, {S0, S0 ? stb : 0}};
    const Range outs[] = {{o, tok * dv * es}, {S_T, stb}, {ckpt, *n_ck > 0 ? (size_t)*n_ck * stb : 0},
                          {workspace, ws_bytes}};
    if (bad_alias(outs, 4, ins, 6, S_T, S0)) return KDA_ERR_ALIAS;
    return KDA_OK;
}

// The bf16 prefill in segments of L tokens through one workspace; the state
// carries over in S_T.  fp32: the fused kernel (no workspace).
static hipError_t run_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every, int n_ck, int B,
                              int T, int H, int dk, int dt, void* workspace, int L, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (dt == KDA_BF16) {
        for (int t0 = 0; e == hipSuccess; t0 += L) {
            const int tl = T - t0 < L ? T - t0 : L;
            e = kda::launch_prefill_prep(dk, q, k, v, g, beta, B, T, H, workspace, s, t0, tl);
            if (e == hipSuccess)
                e = kda::launch_prefill_recur(dk, workspace, t0 == 0 ? S0 : S_T, o, S_T,
                                              n_ck > 0 ? ckpt : nullptr, n_ck > 0 ? ckpt_every : 0, B, T, H,
                                              s, t0, tl);
            if (t0 + L >= T) break;
        }
    } else {
        e = kda::launch_prefill_f32(dk, q, k, v, g, beta, S0, o, S_T, n_ck > 0 ? ckpt : nullptr,
                                    n_ck > 0 ? ckpt_every : 0, B, T, H, s);
    }
    return e;
}

kda_status kda_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every, int B, int T,
                       int H, int dk, int dv, kda_dtype dt_arg, void* workspace, size_t workspace_bytes,
                       void* stream) {
    const int dt = enum_bits(&dt_arg);
    kda_status st = check_prefill_sizes(dt, B, T, H, dk, dv, ckpt_every);
    if (st != KDA_OK) return st;
    const size_t ws_need = kda_prefill_workspace_size(B, T, H, dk, dv, (kda_dtype)dt);  // dt checked above
    int n_ck = 0;
    bool noop;
    st = prefill_checks(q, k, v, g, beta, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv, dt, workspace, ws_need,
                        &n_ck, &noop);
    if (st != KDA_OK || noop) return st;
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE;
    if (ws_need > 0 && !workspace) return KDA_ERR_NULL;
    const hipError_t e = run_prefill(q, k, v, g, beta, S0, o, S_T, ckpt, ckpt_every, n_ck, B, T, H, dk, dt,
                                     workspace, segment_tokens_impl(B, T, H, dk), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ---- kda_prefill_noalloc: the prefill with its records in static device memory ----
//
// The scratch array holds one segment's operand records.  In host code its
// name is only a stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and is
// the only thing passed to kernels.
constexpr size_t kNoallocScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device; nullptr until first looked up

// Device address of `scratch` on device dev.
hipError_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (r != hipSuccess) return r;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

// Segment length when one segment's records must fit the static scratch: the
// fewest segments under that bound, of equal whole-chunk lengths; 0 when not
// even one chunk of all B * H heads fits.
static int noalloc_segment_tokens(int B, int T, int H, int dk) {
    const size_t rec = kda::prefill_workspace_bytes(1, dk, 1, kChunk, 1);
    if (rec == 0 || B <= 0 || H <= 0 || T <= 0) return T;
    const size_t per_chunk = (size_t)B * H * rec;
    const long long cmax = (long long)(kNoallocScratchBytes / per_chunk);
    if (cmax == 0) return 0;
    const long long chunks = ((long long)T + kChunk - 1) / kChunk;
    if (cmax >= chunks) return T;
    const long long n = (chunks + cmax - 1) / cmax;
    return (int)(((chunks + n - 1) / n) * kChunk);
}

kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every, int B, int T,
                               int H, int dk, int dv, kda_dtype dt_arg, void* stream) {
    const int dt = enum_bits(&dt_arg);
    int n_ck = 0;
    bool noop;
    kda_status st = prefill_checks(q, k, v, g, beta, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv, dt, nullptr,
                                   0, &n_ck, &noop);
    if (st != KDA_OK || noop) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int L = T;
    void* ws = nullptr;
    if (dt == KDA_BF16 && T > 0) {
        L = noalloc_segment_tokens(B, T, H, dk);
        if (L == 0) return KDA_ERR_WORKSPACE;  // one chunk of every head exceeds the scratch
        int dev = -1;
        if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return KDA_ERR_HIP;
        if (scratch_address(dev, &ws) != hipSuccess) return KDA_ERR_HIP;
    }
    const hipError_t e = run_prefill(q, k, v, g, beta, S0, o, S_T, ckpt, ckpt_every, n_ck, B, T, H, dk, dt, ws, L, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Tokens [t_begin, t_begin + t_len) of every sequence: t_begin a multiple of
// the chunk length, the range inside [0, T].
static kda_status check_segment(int T, int t_begin, int t_len) {
    if (t_begin < 0 || t_len < 0 || (int64_t)t_begin + t_len > T) return KDA_ERR_SHAPE;
    if (t_begin % kChunk != 0) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

static kda_status segment_prep(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               int B, int T, int H, int dk, int dv, int dt, int t_begin, int t_len,
                               void* workspace, size_t workspace_bytes, void* stream) {
    kda_status st = check_prefill_sizes(dt, B, T, H, dk, dv, 0);
    if (st != KDA_OK) return st;
    if (dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((st = check_segment(T, t_begin, t_len)) != KDA_OK) return st;
    if (B == 0 || H == 0 || t_len == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !workspace) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const size_t ws_need = kda_prefill_stage_workspace_size(B, t_len, H, dk, dv, (kda_dtype)dt);  // dt checked above
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE;
    const size_t tok = (size_t)B * T * H;
    const Range ins[] = {{q, tok * dk * 2}, {k, tok * dk * 2}, {v, tok * dv * 2},
                         {g, tok * dk * sizeof(float)}, {beta, tok * sizeof(float)}};
    const Range outs[] = {{workspace, ws_need}};
    if (bad_alias(outs, 1, ins, 5, nullptr, nullptr)) return KDA_ERR_ALIAS;
    const hipError_t e = kda::launch_prefill_prep(dk, q, k, v, g, beta, B, T, H, workspace,
                                                  static_cast<hipStream_t>(stream), t_begin, t_len);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static kda_status segment_recur(const void* workspace, size_t workspace_bytes, const float* S0, void* o,
                                float* S_T, float* ckpt, int ckpt_every, int B, int T, int H, int dk, int dv,
                                int dt, int t_begin, int t_len, void* stream) {
    kda_status st = check_prefill_sizes(dt, B, T, H, dk, dv, ckpt_every);
    if (st != KDA_OK) return st;
    if (dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((st = check_segment(T, t_begin, t_len)) != KDA_OK) return st;
    if (B == 0 || H == 0) return KDA_OK;
    if (!S_T) return KDA_ERR_NULL;
    if (t_len > 0 && (!o || !workspace)) return KDA_ERR_NULL;
    const int n_ck = ckpt_every > 0 ? (T + ckpt_every - 1) / ckpt_every : 0;
    if (n_ck > 0 && !ckpt) return KDA_ERR_NULL;
    if (!aligned16(workspace) || !aligned16(S0) || !aligned16(o) || !aligned16(S_T) || !aligned16(ckpt))
        return KDA_ERR_ALIGN;
    const size_t ws_need = kda_prefill_stage_workspace_size(B, t_len, H, dk, dv, (kda_dtype)dt);  // dt checked above
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE;
    const size_t tok = (size_t)B * T * H;
    const size_t stb = (size_t)B * H * dk * dv * sizeof(float);
    const Range ins[] = {{workspace, ws_need}, {S0, S0 ? stb : 0}};
    const Range outs[] = {{o, tok * dv * 2}, {S_T, stb}, {ckpt, n_ck > 0 ? (size_t)n_ck * stb : 0}};
    if (bad_alias(outs, 3, ins, 2, S_T, S0)) return KDA_ERR_ALIAS;
    const hipError_t e = kda::launch_prefill_recur(dk, workspace, S0, o, S_T, n_ck > 0 ? ckpt : nullptr,
                                                   n_ck > 0 ? ckpt_every : 0, B, T, H,
                                                   static_cast<hipStream_t>(stream), t_begin, t_len);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_prefill_chunk_prep(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, int B, int T, int H, int dk, int dv, kda_dtype dt_arg,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    const int dt = enum_bits(&dt_arg);
    return segment_prep(q, k, v, g, beta, B, T, H, dk, dv, dt, 0, T < 0 ? 0 : T, workspace, workspace_bytes,
                        stream);
}

kda_status kda_prefill_chunk_recur(const void* workspace, size_t workspace_bytes, const float* S0, void* o,
                                   float* S_T, float* ckpt, int ckpt_every, int B, int T, int H, int dk,
                                   int dv, kda_dtype dt_arg, void* stream) {
    const int dt = enum_bits(&dt_arg);
    return segment_recur(workspace, workspace_bytes, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv, dt, 0,
                         T < 0 ? 0 : T, stream);
}

kda_status kda_prefill_segment_prep(const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, int B, int T, int H, int dk, int dv, kda_dtype dt_arg,
                                    int t_begin, int t_len, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    const int dt = enum_bits(&dt_arg);
    return segment_prep(q, k, v, g, beta, B, T, H, dk, dv, dt, t_begin, t_len, workspace, workspace_bytes,
                        stream);
}

kda_status kda_prefill_segment_recur(const void* workspace, size_t workspace_bytes, const float* S0, void* o,
                                     float* S_T, float* ckpt, int ckpt_every, int B, int T, int H, int dk,
                                     int dv, kda_dtype dt_arg, int t_begin, int t_len, void* stream) {
    const int dt = enum_bits(&dt_arg);
    return segment_recur(workspace, workspace_bytes, S0, o, S_T, ckpt, ckpt_every, B, T, H, dk, dv, dt, t_begin,
                         t_len, stream);
}

// Packed-sequence offsets: cu[0] == 0, non-decreasing.  Totals of tokens,
// 64-token chunks and checkpoints (ceil(len / ckpt_every) per sequence).
static kda_status check_cu(const int* cu, int S, int ckpt_every, long long* tokens, long long* chunks,
                           long long* ckpts) {
    if (S < 0) return KDA_ERR_SHAPE;
    if (!cu) return KDA_ERR_NULL;
    if (cu[0] != 0) return KDA_ERR_SHAPE;
    long long nc = 0, nk = 0;
    for (int i = 0; i < S; ++i) {
        if (cu[i + 1] < cu[i]) return KDA_ERR_SHAPE;
        const long long len = (long long)cu[i + 1] - cu[i];
        nc += (len + kChunk - 1) / kChunk;
        if (ckpt_every > 0) nk += (len + ckpt_every - 1) / ckpt_every;
    }
    *tokens = cu[S];
    *chunks = nc;
    *ckpts = nk;
    return KDA_OK;
}

size_t kda_prefill_varlen_workspace_size(const int* cu_seqlens, int num_seqs, int H, int dk, int dv,
                                         kda_dtype dt_arg) {
    const int dt = enum_bits(&dt_arg);
    if (dt != KDA_BF16 || H < 0 || !supported_head(dk, dv)) return 0;
    long long tokens, chunks, ckpts;
    if (check_cu(cu_seqlens, num_seqs, 0, &tokens, &chunks, &ckpts) != KDA_OK) return 0;
    return kda::varlen_workspace_bytes(dk, num_seqs, chunks, H);
}

long long kda_prefill_varlen_num_checkpoints(const int* cu_seqlens, int num_seqs, int ckpt_every) {
    if (ckpt_every <= 0 || ckpt_every % kChunk != 0) return ckpt_every == 0 ? 0 : -1;
    long long tokens, chunks, ckpts;
    if (check_cu(cu_seqlens, num_seqs, ckpt_every, &tokens, &chunks, &ckpts) != KDA_OK) return -1;
    return ckpts;
}

kda_status kda_prefill_varlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              const int* cu_seqlens, int num_seqs, const float* S0, void* o, float* S_T,
                              float* ckpt, int ckpt_every, int H, int dk, int dv, kda_dtype dt_arg,
                              void* workspace, size_t workspace_bytes, void* stream) {
    const int dt = enum_bits(&dt_arg);
    if (dt != KDA_FP32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (num_seqs < 0 || H < 0 || dk <= 0 || dv <= 0 || ckpt_every < 0) return KDA_ERR_SHAPE;
    if (!supported_head(dk, dv) || dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (ckpt_every % kChunk != 0) return KDA_ERR_UNSUPPORTED;
    long long tokens, chunks, n_ck;
    const kda_status st = check_cu(cu_seqlens, num_seqs, ckpt_every, &tokens, &chunks, &n_ck);
    if (st != KDA_OK) return st;
    // Grids: H * chunks workgroups for the preparation, num_seqs * H * (dv/16)
    // for the recurrence; record and checkpoint indices stay in range too.
    if ((long long)H * chunks > INT32_MAX || (long long)num_seqs * H * (dv / 16) > INT32_MAX ||
        chunks > INT32_MAX || n_ck > INT32_MAX)
        return KDA_ERR_SHAPE;
    if (num_seqs == 0 || H == 0) return KDA_OK;
    if (!S_T) return KDA_ERR_NULL;
    if (tokens > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    if (n_ck > 0 && !ckpt) return KDA_ERR_NULL;
    if (!workspace) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(S0) || !aligned16(o) || !aligned16(S_T) || !aligned16(ckpt) || !aligned16(workspace))
        return KDA_ERR_ALIGN;
    const size_t ws_need = kda::varlen_workspace_bytes(dk, num_seqs, chunks, H);
    if (workspace_bytes < ws_need) return KDA_ERR_WORKSPACE;

    const size_t tok = (size_t)tokens * H;
    const size_t stb = (size_t)num_seqs * H * dk * dv * sizeof(float);
    const size_t ckb = (size_t)n_ck * H * dk * dv * sizeof(float);
    const Range ins[] = {{q, tok * dk * 2}, {k, tok * dk * 2}, {v, tok * dv * 2},
                         {g, tok * dk * sizeof(float)}, {beta, tok * sizeof(float)}, {S0, S0 ? stb : 0}};
    const Range outs[] = {{o, tok * dv * 2}, {S_T, stb}, {ckpt, ckb}, {workspace, ws_need}};
    if (bad_alias(outs, 4, ins, 6, S_T, S0)) return KDA_ERR_ALIAS;

    const hipError_t e = kda::launch_prefill_varlen(dk, q, k, v, g, beta, cu_seqlens, num_seqs, chunks, H, S0, o,
                                                    S_T, n_ck > 0 ? ckpt : nullptr, n_ck > 0 ? ckpt_every : 0,
                                                    workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           float* S, void* o, int N, int H, int dk, int dv, kda_dtype dt_arg, void* stream) {
    const int dt = enum_bits(&dt_arg);
    if (dt != KDA_FP32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
    if (!supported_head(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(S) || !aligned16(o))
        return KDA_ERR_ALIGN;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t nh = (size_t)N * H;
    const Range ins[] = {{q, nh * dk * es}, {k, nh * dk * es}, {v, nh * dv * es},
                         {g, nh * dk * sizeof(float)}, {beta, nh * sizeof(float)}};
    const Range outs[] = {{o, nh * dv * es}, {S, nh * dk * dv * sizeof(float)}};
    if (bad_alias(outs, 2, ins, 5, nullptr, nullptr)) return KDA_ERR_ALIAS;

    const hipError_t e = kda::launch_decode(dt == KDA_BF16 ? 1 : 0, dk, q, k, v, g, beta, S, o, N, H,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_multi(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            float* S, void* o, const int* n_tokens, int update_state, int N, int T, int H,
                            int dk, int dv, kda_dtype dt_arg, void* stream) {
    const int dt = enum_bits(&dt_arg);
    if (dt != KDA_FP32 && dt != KDA_BF16) return KDA_ERR_DTYPE;
    if (N < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || (update_state != 0 && update_state != 1))
        return KDA_ERR_SHAPE;
    if (!supported_head(dk, dv) || T > 16) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX || (int64_t)N * T * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0 || H == 0 || T == 0 || (!o && !update_state)) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S) return KDA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(S) || !aligned16(o) || !aligned16(n_tokens))
        return KDA_ERR_ALIGN;
    const size_t es = dt == KDA_BF16 ? 2 : 4;
    const size_t rows = (size_t)N * T * H;
    const Range ins[] = {{q, rows * dk * es}, {k, rows * dk * es}, {v, rows * dv * es},
                         {g, rows * dk * sizeof(float)}, {beta, rows * sizeof(float)},
                         {n_tokens, n_tokens ? (size_t)N * sizeof(int) : 0}};
    const Range outs[] = {{o, o ? rows * dv * es : 0}, {S, (size_t)N * H * dk * dv * sizeof(float)}};
    if (bad_alias(outs, 2, ins, 6, nullptr, nullptr)) return KDA_ERR_ALIAS;
    const hipError_t e = kda::launch_decode_multi(dt == KDA_BF16 ? 1 : 0, dk, q, k, v, g, beta, S, o, n_tokens, N,
                                                  T, H, update_state, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
