// kda_prefill.hip -- chunked KDA prefill for gfx950, bf16 operands: two kernels.
//
// Method (SemiAnalysis "Kimi K3" primer, bayesiansapien wiki page, section 2
// "FlashKDA's complexity"): split each sequence into chunks of C = 64 tokens;
// per chunk form the cumulative log-decay, the decayed queries and keys, the
// inverse of the unit-lower-triangular intra-chunk system (I + L) and the
// causal mask, then carry the dk x dv state from chunk to chunk.  With
// G_r = sum_{i<=r} g_i inside a chunk (per key channel) the token recurrence
// of section 1 is, exactly:
//
//   Qt = q e^{G},  Kt = k e^{G},  Kh = k e^{-G}                      (rows r)
//   A  = Diag(beta) strict_tril(Kt Kh^T),   Aqk = tril(Qt Kh^T)
//   [W | U'] = (I + A)^{-1} Diag(beta) [Kt | V]
//   U = U' - W S,   O = Qt S + Aqk U,   S <- Diag(e^{G_C}) S + Ke^T U
// with Ke = k e^{G_C - G}.  e^{-G} alone would overflow once a channel decays
// by more than e^-88 inside a chunk, so the Gram products are formed from
// factors taken relative to the decay R_b at the start of each 16-row block b
// (Kt_b' = k e^{G - R_b} <= 1, Kh_b' = k e^{R_b - G} <= e^{16-token decay}),
// with the per-channel factor e^{R_bi - R_bj} <= 1 between row blocks bi > bj;
// every exponential then spans at most 16 tokens or is at most 1.
//
// Kernel 1 (kda_chunk_prep) does everything that does not depend on S, for
// every (batch, head, chunk) of a range of tokens at once: 3296 independent
// workgroups for a 6592-token segment of 32 heads, so occupancy hides the
// latency of the decay prologue, the Gram products, the triangular solve and
// the substitution.  It writes one record per chunk into the caller's
// workspace, with every operand already in the MFMA fragment layout kernel 2
// consumes (lane-major slots), so kernel 2 never reshuffles data.  All
// operands are bf16 like the MFMA inputs, U' included (kernel 2 widens it to
// the fp32 accumulator U is formed in); e^{G_C} is fp32.
//
// Kernel 2 (kda_chunk_recur) is the only sequential part: one workgroup per
// (sequence, head, 16-wide value-column block).  One wave carries the 128 x 16
// fp32 state slice in registers through all chunks (U = U' - W S, then
// S <- e^{G_C} S + Ke^T U: 32 MFMAs per chunk); two waves compute the chunk's
// outputs from the state and U it hands over in LDS; two waves stream the
// records into an LDS ring with global->LDS DMA, two chunks ahead.
//
// The host runs the two kernels over segments of the sequences whose records
// fit the MI355X's 256 MB Infinity Cache, so kernel 2 reads them back from
// there (the inputs and outputs pass it by, with the streaming hint); the
// state passes from one segment to the next through S_T.
#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int C = 64;     // chunk length (tokens)
constexpr int BV = 16;    // value columns per MFMA tile / state slice
constexpr float LOG2E = 1.4426950408889634f;

typedef uint16_t bf16_t;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2v));
}
__device__ __forceinline__ bf16_t cvt1(float x) { return __builtin_bit_cast(bf16_t, (__bf16)x); }
__device__ __forceinline__ float lo_f(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ f32x4 mma(f32x4 c, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 frag_acc(f32x4 x, f32x4 y) {
    return __builtin_bit_cast(bf16x8, u32x4{cvt2(x[0], x[1]), cvt2(x[2], x[3]), cvt2(y[0], y[1]),
                                            cvt2(y[2], y[3])});
}
__device__ __forceinline__ bf16x8 frag_acc_lo(f32x4 x) {
    return __builtin_bit_cast(bf16x8, u32x4{cvt2(x[0], x[1]), cvt2(x[2], x[3]), 0u, 0u});
}
__device__ __forceinline__ bf16x8 as_frag(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS ops, not
// for its global loads/stores or LDS-DMA copies (__syncthreads() would drain
// all of them, which defeats prefetching).  DMA completion is awaited
// explicitly with s_waitcnt vmcnt before the barrier that publishes it.
// Streaming accesses (the nontemporal hint): the chunk inputs, read once, and
// the outputs, written once, then do not take the last-level cache from the
// operand records, which the recurrence reads back right after they are
// written.
template <class T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void st_stream(T x, T* p) { __builtin_nontemporal_store(x, p); }

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Transposing LDS read of 16-bit elements (gfx950 ds_read_b64_tr_b16).  In each
// group of 16 lanes, lane 4j + a passes the address of 4 consecutive elements
// (row t_j, columns 4a .. 4a+3 of a 16-column block); lane i then receives
// column i of the 4 x 16 block: its element j comes from row t_j.  With
// t_j = 4 consecutive rows this is a column slice in MFMA accumulator order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x2 ld_tr16(const uint16_t* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// s_waitcnt immediate: wait until at most n vector-memory ops of this wave are
// outstanding (expcnt and lgkmcnt unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Offset of element (r, c) in a [rows][ROWLEN] bf16 LDS tile whose 4-element
// chunks are XOR-swizzled with the row index: fragment reads of 16 rows hit
// 16 different chunks, so the tiles need no padding.
template <int ROWLEN>
__device__ __forceinline__ int swz(int r, int c) {
    constexpr int NCH = ROWLEN / 4;
    return r * ROWLEN + ((((c >> 2) ^ r) & (NCH - 1)) << 2) + (c & 3);
}

// Fragment of contraction block m (see kda_device.h) from row r of a swizzled
// tile: elements [32m + 4q, +4) and [32m + 16 + 4q, +4).
template <int ROWLEN>
__device__ __forceinline__ bf16x8 frag(const bf16_t* t, int r, int m, int q) {
    constexpr int NCH = ROWLEN / 4;
    const bf16_t* row = t + r * ROWLEN;
    const int x = r & (NCH - 1);
    const u32x2 a = *reinterpret_cast<const u32x2*>(row + (((8 * m + q) ^ x) << 2));
    const u32x2 b = *reinterpret_cast<const u32x2*>(row + (((8 * m + 4 + q) ^ x) << 2));
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// Per-chunk record written by kernel 1 and read by kernel 2.  Every field is a
// list of MFMA fragments [fragment][lane 0..63][16 bytes] (U': accumulator
// tiles, 8 bytes per lane; G: fp32 per channel), 1 KiB aligned so kernel 2 can
// copy it with 1 KiB-per-wave DMA pieces.
template <int DK>
struct Rec {
    static constexpr int KB = DK / 32;   // contraction blocks over key channels
    static constexpr int NDT = DK / 16;  // 16-row tiles of the state
    static constexpr int NCB = DK / 16;  // 16-column blocks of the value dim (dv = dk)
    static constexpr int OFF_W = 0;                          // -W, A fragments [t 4][m KB]
    static constexpr int OFF_KT = OFF_W + 4 * KB * 1024;     // Ke^T = (k e^{G_C - G})^T, A fragments [d NDT][m 2]
    static constexpr int OFF_G = OFF_KT + NDT * 2 * 1024;    // e^{G_C}, DK floats (1 KiB slot)
    static constexpr int OFF_UP = OFF_G + 1024;              // U', accumulator tiles [cb][t 4][lane][4] bf16
    static constexpr int OFF_Q = OFF_UP + NCB * 2048;        // Qt, A fragments [t 4][m KB]
    static constexpr int OFF_A = OFF_Q + 4 * KB * 1024;      // Aqk, A fragments (t, m2): 6 of them
    static constexpr int BYTES = OFF_A + 6 * 1024;
    static constexpr int CHAIN = OFF_UP + 2048;              // W, Ke^T, G and U' of one column block
};

// Contraction-slot channels of a fragment (see frag): slots 0-3 are channels
// 32m + 4q + 0..3, slots 4-7 are 32m + 16 + 4q + 0..3.  scale_frag multiplies
// the eight values by the per-channel factors fac[c] (all <= 1).
__device__ __forceinline__ bf16x8 scale_frag(bf16x8 f, const float* fac, int m, int q) {
    const u32x4 u = __builtin_bit_cast(u32x4, f);
    const f32x4 a = *reinterpret_cast<const f32x4*>(fac + 32 * m + 4 * q);
    const f32x4 b = *reinterpret_cast<const f32x4*>(fac + 32 * m + 16 + 4 * q);
    return __builtin_bit_cast(bf16x8, u32x4{cvt2(lo_f(u[0]) * a[0], hi_f(u[0]) * a[1]),
                                            cvt2(lo_f(u[1]) * a[2], hi_f(u[1]) * a[3]),
                                            cvt2(lo_f(u[2]) * b[0], hi_f(u[2]) * b[1]),
                                            cvt2(lo_f(u[3]) * b[2], hi_f(u[3]) * b[3])});
}

// Aqk fragment index of row tile t and contraction block m2 (m2 <= t / 2).
__device__ __forceinline__ int afrag(int t, int m2) { return t < 2 ? t : (t == 2 ? 2 + m2 : 4 + m2); }

// One 16x16 tile of X Y^T over DK channels: X rows 16 bi.., Y rows 16 bj...
// With fac given, channel c of the X side (SX) or the Y side is scaled by
// fac[c] first.
template <int DK>
__device__ __forceinline__ f32x4 gram_tile(const bf16_t* X, const bf16_t* Y, int bi, int bj, int i16, int q4,
                                           const float* fac = nullptr, bool SX = false) {
    constexpr int KB = DK / 32;
    bf16x8 xa[KB], yb[KB];
#pragma unroll
    for (int m = 0; m < KB; ++m) {
        xa[m] = frag<DK>(X, 16 * bi + i16, m, q4);
        yb[m] = frag<DK>(Y, 16 * bj + i16, m, q4);
        if (fac) {
            if (SX)
                xa[m] = scale_frag(xa[m], fac, m, q4);
            else
                yb[m] = scale_frag(yb[m], fac, m, q4);
        }
    }
    f32x4 acc = zero4();
#pragma unroll
    for (int m = 0; m < KB; ++m) acc = mma(acc, xa[m], yb[m]);
    return acc;
}

// Where the sequences of one prefill call live.
//   uniform: B sequences of T tokens ([B,T,H,.] tensors), N chunks each; the
//            record of (b, h, chunk n) is number (b H + h) N + n.
//   packed:  S sequences laid end to end ([total_T,H,.] tensors), sequence s
//            spanning tokens cu_seqlens[s] .. cu_seqlens[s+1]-1.  Device tables
//            give its first chunk cu_chunks[s] (of TC in total) and its first
//            checkpoint cu_ckpts[s]; the record of (head h, global chunk c) is
//            number h TC + c.
// Uniform batches may be processed in segments of tokens: tokens
// [tbase, tbase + T) of every sequence, N = ceil(T / 64) chunks, sequences
// tstride tokens apart, Tfull tokens long (checkpoints use absolute positions).
// Packed batches may be processed in segments of global chunks: chunks
// [c0, c0 + TC) of the S sequences, whose records are numbered h TC + c - c0;
// the recurrence then runs sequences p0 .. p0 + NS - 1, each over its chunks
// in the segment.
struct SeqMap {
    int B, T, N;
    int tbase, tstride, Tfull;
    int S, TC;
    const int* cu_seqlens;  // nullptr: uniform
    const int* cu_chunks;
    const int* cu_ckpts;
    int c0, p0, NS;
};

// Largest s < S with cu[s] <= x (cu non-decreasing, cu[0] = 0 <= x): the
// sequence that owns global chunk x, skipping empty sequences.
__device__ __forceinline__ int owner(const int* cu, int S, int x) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= x)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// ============================ kernel 1: chunk prep ============================

constexpr int NT1 = 512;  // 8 waves

// Per-channel decay factors, computed once the block references are known
// (R_b: log decay before row block b; G_C: over the whole chunk).
template <int DK>
struct PrepFac {
    float eR[4][DK];   // e^{R_b}
    float eGR[4][DK];  // e^{G_C - R_b}
    float F[6][DK];    // e^{R_bi - R_bj} for the block pairs bi > bj, in pair order
};

// The short convolution's staging: the inputs of the W-1 tokens before the
// chunk (fp32: a carried state need not be bf16) and the head's taps.
template <int DK>
struct PrepConv {
    float halo[3][3 * DK];
    float taps[4][3 * DK];  // [j][channel]
};

// The convolution staging is dead before the factors are written (every wave
// has passed the barrier that follows its convolution), so the two share space.
template <int DK, bool CONV>
union PrepLate {
    PrepFac<DK> fac;
    PrepConv<DK> conv;
};
template <int DK>
union PrepLate<DK, false> {
    PrepFac<DK> fac;
};

// Block pair index of (bi, bj), bi > bj: (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
__device__ __forceinline__ int pair_index(int bi, int bj) { return bi * (bi - 1) / 2 + bj; }

template <int DK, bool CONV>
struct alignas(16) PrepSmem {
    bf16_t Qt[C * DK];        // q e^G        (swizzled rows of DK)
    bf16_t Kt[C * DK];        // k e^G
    bf16_t Kh[C * DK];        // k e^-G
    bf16_t Aneg[C * C];       // -A in the strictly lower off-diagonal 16x16 blocks, else 0
    bf16_t DinvT[C * 16];     // (I + A_bb)^{-1} transposed: row 16 b + j holds column j of block b's inverse
    float DiagAT[4][16][16];  // diagonal blocks of A, transposed: [b][m][r] = A[16b+r][16b+m]
    float beta[C];
    PrepLate<DK, CONV> late;
};

// LY < 0: the recurrence's inputs as given.  LY >= 0: the layer steps, with a
// short convolution of width LY (0: none).
template <int DK, int LY>
__global__ void __launch_bounds__(NT1, 4)  // 2 workgroups (16 waves) per CU
kda_chunk_prep(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
               const float* __restrict__ g, const float* __restrict__ beta, uint8_t* __restrict__ ws,
               SeqMap map, int H, LayerArgs la) {
    typedef Rec<DK> RC;
    constexpr int NW1 = NT1 / 64;
    constexpr int KB = RC::KB;
    constexpr int NCT = DK / 16;      // 16-channel tiles of W
    constexpr int NCB = RC::NCB;      // 16-column tiles of V
    // Substitution tiles per wave: dk = 128 -> W tile w and V tile w;
    // dk = 64 -> waves 0-3 one W tile, waves 4-7 one V tile.
    constexpr int NTW = (NCT + NCB) / NW1;
    static_assert(NTW == 1 || NTW == 2, "tile split");
    __shared__ PrepSmem<DK, (LY > 0)> sm;

    // This workgroup's (head, chunk).  Heads vary fastest in dispatch order,
    // so the workgroups of one chunk's heads run together: they read whole
    // token rows of q, k, v and g between them, and share the cache lines of
    // beta ([.., H] per token).  Records stay in the recurrence's order.
    int h, n, len, seq;
    size_t tok0;  // first token of the sequence
    size_t ri;    // record index
    h = blockIdx.x % H;
    if (!map.cu_seqlens) {
        const int cr = blockIdx.x / H;  // chunk row: sequence seq, chunk n
        n = cr % map.N;
        seq = cr / map.N;
        tok0 = (size_t)seq * map.tstride + map.tbase;
        len = map.T;
        ri = ((size_t)seq * H + h) * map.N + n;
    } else {
        const int gl = blockIdx.x / H;  // chunk within the segment
        const int gc = map.c0 + gl;
        seq = owner(map.cu_chunks, map.S, gc);
        n = gc - map.cu_chunks[seq];
        tok0 = map.cu_seqlens[seq];
        len = map.cu_seqlens[seq + 1] - map.cu_seqlens[seq];
        ri = (size_t)h * map.TC + gl;
    }
    const int t0 = n * C, L = min(C, len - t0);
    [[maybe_unused]] const int tb = map.cu_seqlens ? 0 : map.tbase;  // tokens of the sequence before tok0
    uint8_t* rec = ws + ri * RC::BYTES;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, i16 = lane % 16, q4 = lane / 16;
    auto tok = [&](int r) { return (tok0 + t0 + r) * H + h; };
    // The value tile this wave solves for in the substitution (if any).
    const bool hasV = NTW == 2 || w >= NCT;
    const int vcb = NTW == 2 ? w : w - NCT;

    // ---- (a1, a2) cumulative log-decay (base 2) and decayed Q/K ----
    // Every lane holds NI rows of 4 channels (coalesced 8- and 16-byte vectors).
    // The layer steps (whose L2 norms want whole rows in a wave): wave w reads
    // rows 8w .. 8w+7 whole, lane (hr, c4) channels 4c4 .. 4c4+3 of rows
    // 8w + RPI i + hr; the prefix over rows is a scan across the lane groups of
    // a row set, a running sum over the lane's rows, then the totals of the
    // earlier waves (via LDS).
    constexpr int LPR = DK / 4;        // lanes per row
    constexpr int RPI = 64 / LPR;      // rows per load instruction
    constexpr int RW = C / NW1;        // rows per wave
    constexpr int NI = RW / RPI;       // rows per lane
    [[maybe_unused]] const int c4 = lane % LPR, hr = lane / LPR;
    uint32_t vr[NI][2];  // the chunk's values, staged through LDS for the substitution
    int vrow0, vrstep, vch;  // their rows (vrow0 + vrstep i) and first channel
    if constexpr (LY < 0) {
        // Wave w covers the 16-row block bw = w / 2 and the channel half w % 2:
        // lane (rg, cq) holds channels ch0 .. ch0+3 of rows r0 .. r0+NI-1.  The
        // decay within a block, relative to its start (the reference R_b), is
        // then a prefix within the wave: a running sum over the lane's rows,
        // then a scan across its row groups.  The tiles need nothing else, so
        // each wave writes them as soon as its own inputs arrive; only the
        // block totals, for the factors, pass through LDS.
        constexpr int LH = DK / 8;   // lanes per half row
        constexpr int RG = 64 / LH;  // row groups
        static_assert(16 / RG == NI, "rows per lane");
        const int bw = w / 2, cq = lane % LH, rg = lane / LH;
        const int ch0 = (w % 2) * (DK / 2) + 4 * cq;
        const int r0 = 16 * bw + NI * rg;
        vrow0 = r0;
        vrstep = 1;
        vch = ch0;
        u32x2 qv[NI], kv[NI];
        f32x4 gv[NI];
        const size_t e0 = tok(r0) * DK + ch0;
        const size_t es = (size_t)H * DK;
        auto load_row = [&](int j) {
            const size_t e = e0 + (size_t)j * es;
            qv[j] = ld_stream(reinterpret_cast<const u32x2*>(q + e));
            kv[j] = ld_stream(reinterpret_cast<const u32x2*>(k + e));
            const u32x2 vv = ld_stream(reinterpret_cast<const u32x2*>(v + e));
            vr[j][0] = vv[0];
            vr[j][1] = vv[1];
            gv[j] = ld_stream(reinterpret_cast<const f32x4*>(g + e));
        };
        if (L == C) {  // every chunk but a sequence's ragged last one
#pragma unroll
            for (int j = 0; j < NI; ++j) load_row(j);
        } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (r0 + j < L) {
                    load_row(j);
                } else {
                    qv[j] = kv[j] = u32x2{0u, 0u};
                    vr[j][0] = vr[j][1] = 0u;
                    gv[j] = zero4();
                }
            }
        }
        if (tid < C) sm.beta[tid] = tid < L ? beta[tok(tid)] : 0.f;
        // -A starts as zeros (the Gram phase writes its strictly lower
        // off-diagonal blocks), written once the loads are in flight.
        static_assert(sizeof(sm.Aneg) == NT1 * 16, "one 16-byte store per thread");
        reinterpret_cast<u32x4*>(sm.Aneg)[tid] = u32x4{0u, 0u, 0u, 0u};
        f32x4 P[NI];
        f32x4 run = zero4();
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            run += gv[j] * LOG2E;
            P[j] = run;
        }
        f32x4 x = run;  // inclusive scan of the lanes' sums over the row groups
#pragma unroll
        for (int d = LH; d < 64; d *= 2) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const float y = __shfl_up(x[cc], d, 64);
                if (lane >= d) x[cc] += y;
            }
        }
        const f32x4 off = x - run;  // the rows of the earlier row groups
        float* bsum = &sm.DiagAT[0][0][0];  // 4 x DK block totals, free until the Gram phase
        if (rg == RG - 1) *reinterpret_cast<f32x4*>(bsum + bw * DK + ch0) = x;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const f32x4 a = P[j] + off;  // G - R_b <= 0
            f32x4 e, f;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                e[cc] = __builtin_amdgcn_exp2f(a[cc]);
                f[cc] = __builtin_amdgcn_exp2f(-a[cc]);
            }
            const float q0 = lo_f(qv[j][0]), q1 = hi_f(qv[j][0]), q2 = lo_f(qv[j][1]), q3 = hi_f(qv[j][1]);
            const float k0 = lo_f(kv[j][0]), k1 = hi_f(kv[j][0]), k2 = lo_f(kv[j][1]), k3 = hi_f(kv[j][1]);
            const int o = swz<DK>(r0 + j, ch0);
            *reinterpret_cast<u32x2*>(&sm.Qt[o]) = u32x2{cvt2(q0 * e[0], q1 * e[1]), cvt2(q2 * e[2], q3 * e[3])};
            *reinterpret_cast<u32x2*>(&sm.Kt[o]) = u32x2{cvt2(k0 * e[0], k1 * e[1]), cvt2(k2 * e[2], k3 * e[3])};
            *reinterpret_cast<u32x2*>(&sm.Kh[o]) = u32x2{cvt2(k0 * f[0], k1 * f[1]), cvt2(k2 * f[2], k3 * f[3])};
        }
        lds_barrier();
        // The decay factors of the record and Gram steps, each exp2 taken once
        // per channel, from R_b (the block totals before block b) and G_C.
        for (int e = tid; e < 2 * DK; e += NT1) {
            const int c = e % DK;
            float R[5];
            R[0] = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b) R[b + 1] = R[b] + bsum[b * DK + c];
            if (e < DK) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    sm.late.fac.eR[b][c] = __builtin_amdgcn_exp2f(R[b]);
                    sm.late.fac.eGR[b][c] = __builtin_amdgcn_exp2f(R[4] - R[b]);
                }
                // G over the whole chunk (rows past the end add 0)
                reinterpret_cast<float*>(rec + RC::OFF_G)[c] = __builtin_amdgcn_exp2f(R[4]);
            } else {
#pragma unroll
                for (int bi = 1; bi < 4; ++bi) {
#pragma unroll
                    for (int bj = 0; bj < bi; ++bj)
                        sm.late.fac.F[pair_index(bi, bj)][c] = __builtin_amdgcn_exp2f(R[bi] - R[bj]);
                }
            }
        }
    } else {
        vrow0 = RW * w + hr;
        vrstep = RPI;
        vch = 4 * c4;
        u32x2 qv[NI], kv[NI];
        f32x4 gv[NI];
        {
            // Layer steps (primer section 3): q, k, v through the short causal
            // convolution (and SiLU), q and k divided by their L2 norm, then
            // rounded to bf16 like stored inputs; g = log sigmoid(a) from the
            // decay-gate logits, beta = sigmoid(b).
            constexpr int CH = 3 * DK;  // q, k and v channels (dv = dk)
            constexpr int W = LY > 0 ? LY : 1;
#pragma unroll
            for (int i = 0; i < NI; ++i) {  // every raw input row is read once
                const int r = RW * w + RPI * i + hr;
                if (r < L) {
                    qv[i] = ld_stream(reinterpret_cast<const u32x2*>(q + tok(r) * DK + 4 * c4));
                    kv[i] = ld_stream(reinterpret_cast<const u32x2*>(k + tok(r) * DK + 4 * c4));
                    const u32x2 vv = ld_stream(reinterpret_cast<const u32x2*>(v + tok(r) * DK + 4 * c4));
                    vr[i][0] = vv[0];
                    vr[i][1] = vv[1];
                    gv[i] = ld_stream(reinterpret_cast<const f32x4*>(g + tok(r) * DK + 4 * c4));  // gate logits
                } else {
                    qv[i] = kv[i] = u32x2{0u, 0u};
                    vr[i][0] = vr[i][1] = 0u;
                    gv[i] = zero4();
                }
            }
            // The convolution's halo (its W-1 inputs before the chunk: input
            // rows, or the carried state before the sequence's start) and its
            // taps, loaded together with the rows, before anything waits for
            // them: each thread holds at most one vector of each.
            [[maybe_unused]] u32x2 hraw{0u, 0u};  // halo from an input row (bf16)
            [[maybe_unused]] f32x4 hci = zero4();  // halo from the carried state
            [[maybe_unused]] int hsrc = 0;         // 0: zero, 1: hraw, 2: hci
            [[maybe_unused]] f32x4 tap = zero4();
            if constexpr (LY > 0) {
                static_assert((W - 1) * (CH / 4) <= NT1 && W * CH / 4 <= NT1, "one halo and one tap vector per thread");
                if (tid < (W - 1) * (CH / 4)) {
                    const int j = tid / (CH / 4), ch = 4 * (tid % (CH / 4));
                    const int ts = t0 - (W - 1) + j;  // token relative to tok0
                    if (tb + ts >= 0) {
                        const size_t row = (tok0 + ts) * H + h;
                        const bf16_t* src = ch < DK ? q + row * DK + ch : ch < 2 * DK ? k + row * DK + ch - DK
                                                                                      : v + row * DK + ch - 2 * DK;
                        hraw = *reinterpret_cast<const u32x2*>(src);
                        hsrc = 1;
                    } else if (la.conv_in) {
                        const float* ci = la.conv_in + (((size_t)seq * H + h) * CH + ch) * (W - 1) + (W - 1) + tb + ts;
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) hci[cc] = ci[(size_t)cc * (W - 1)];
                        hsrc = 2;
                    }
                }
                if (tid < W * CH / 4) tap = *reinterpret_cast<const f32x4*>(la.conv_w + (size_t)h * W * CH + 4 * tid);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (RW * w + RPI * i + hr < L) {
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) gv[i][cc] = log_sigmoid(gv[i][cc]);
                }
            }
            if (tid < C) sm.beta[tid] = tid < L ? sigmoid1(beta[tok(tid)]) : 0.f;
            if constexpr (LY > 0) {
                // Rows of other lanes feed a row's taps: stage the raw chunk in
                // the decayed-tile areas (written only after the decay scan), the
                // W-1 inputs before the chunk in `halo`, the taps in `taps`.
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int o = swz<DK>(RW * w + RPI * i + hr, 4 * c4);
                    *reinterpret_cast<u32x2*>(&sm.Qt[o]) = qv[i];
                    *reinterpret_cast<u32x2*>(&sm.Kt[o]) = kv[i];
                    *reinterpret_cast<u32x2*>(&sm.Kh[o]) = u32x2{vr[i][0], vr[i][1]};
                }
                if (tid < (W - 1) * (CH / 4)) {  // 4 channels per thread
                    const int j = tid / (CH / 4), ch = 4 * (tid % (CH / 4));
                    *reinterpret_cast<f32x4*>(&sm.late.conv.halo[j][ch]) =
                        hsrc == 1 ? f32x4{lo_f(hraw[0]), hi_f(hraw[0]), lo_f(hraw[1]), hi_f(hraw[1])}
                                  : hsrc == 2 ? hci : zero4();
                }
                if (tid < W * CH / 4) *reinterpret_cast<f32x4*>(&sm.late.conv.taps[0][0] + 4 * tid) = tap;
                lds_barrier();
            }
            // Per row: convolution, SiLU, L2 norms (over the row's LPR lanes,
            // all lanes taking part), bf16 like stored inputs.  Rows past the
            // end stay zero (their convolution need not be).
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int r = RW * w + RPI * i + hr;
                f32x4 xq = f32x4{lo_f(qv[i][0]), hi_f(qv[i][0]), lo_f(qv[i][1]), hi_f(qv[i][1])};
                f32x4 xk = f32x4{lo_f(kv[i][0]), hi_f(kv[i][0]), lo_f(kv[i][1]), hi_f(kv[i][1])};
                f32x4 xv = f32x4{lo_f(vr[i][0]), hi_f(vr[i][0]), lo_f(vr[i][1]), hi_f(vr[i][1])};
                if constexpr (LY > 0) {
                    // Every tap reads the staged chunk (the lane's own row too),
                    // so the raw registers are free from the staging on.
                    xq = xk = xv = zero4();
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        const int rr = r - (W - 1) + j;
                        f32x4 a4, b4, c4v;
                        if (rr >= 0) {
                            const int o = swz<DK>(rr, 4 * c4);
                            const u32x2 uq = *reinterpret_cast<const u32x2*>(&sm.Qt[o]);
                            const u32x2 uk = *reinterpret_cast<const u32x2*>(&sm.Kt[o]);
                            const u32x2 uv = *reinterpret_cast<const u32x2*>(&sm.Kh[o]);
                            a4 = f32x4{lo_f(uq[0]), hi_f(uq[0]), lo_f(uq[1]), hi_f(uq[1])};
                            b4 = f32x4{lo_f(uk[0]), hi_f(uk[0]), lo_f(uk[1]), hi_f(uk[1])};
                            c4v = f32x4{lo_f(uv[0]), hi_f(uv[0]), lo_f(uv[1]), hi_f(uv[1])};
                        } else {
                            const float* hl = sm.late.conv.halo[W - 1 + rr];
                            a4 = *reinterpret_cast<const f32x4*>(hl + 4 * c4);
                            b4 = *reinterpret_cast<const f32x4*>(hl + DK + 4 * c4);
                            c4v = *reinterpret_cast<const f32x4*>(hl + 2 * DK + 4 * c4);
                        }
                        xq += *reinterpret_cast<const f32x4*>(&sm.late.conv.taps[j][4 * c4]) * a4;
                        xk += *reinterpret_cast<const f32x4*>(&sm.late.conv.taps[j][DK + 4 * c4]) * b4;
                        xv += *reinterpret_cast<const f32x4*>(&sm.late.conv.taps[j][2 * DK + 4 * c4]) * c4v;
                        // One tap's reads at a time: holding all of them would
                        // exceed the register budget of two workgroups per CU.
                        asm volatile("" ::: "memory");
                    }
                }
                if (LY > 0 && la.silu) {
                    xq = silu4(xq);
                    xk = silu4(xk);
                    xv = silu4(xv);
                }
                float nq = xq[0] * xq[0] + xq[1] * xq[1] + xq[2] * xq[2] + xq[3] * xq[3];
                float nk = xk[0] * xk[0] + xk[1] * xk[1] + xk[2] * xk[2] + xk[3] * xk[3];
#pragma unroll
                for (int off = LPR / 2; off > 0; off >>= 1) {
                    nq += __shfl_xor(nq, off, 64);
                    nk += __shfl_xor(nk, off, 64);
                }
                // 1 / max(|x|, 1e-12) as min(rsqrt(|x|^2), 1e12): one hardware op
                const float iq = fminf(__builtin_amdgcn_rsqf(nq), 1e12f);
                const float ik = fminf(__builtin_amdgcn_rsqf(nk), 1e12f);
                const bool in = r < L;
                qv[i] = in ? u32x2{cvt2(xq[0] * iq, xq[1] * iq), cvt2(xq[2] * iq, xq[3] * iq)} : u32x2{0u, 0u};
                kv[i] = in ? u32x2{cvt2(xk[0] * ik, xk[1] * ik), cvt2(xk[2] * ik, xk[3] * ik)} : u32x2{0u, 0u};
                vr[i][0] = in ? cvt2(xv[0], xv[1]) : 0u;
                vr[i][1] = in ? cvt2(xv[2], xv[3]) : 0u;
            }
            // The convolution state after the sequence's last token: its last
            // W-1 inputs (from conv_in where the sequence is shorter).
            if (LY > 1 && la.conv_out && t0 + C >= len) {
                float* co = la.conv_out + ((size_t)seq * H + h) * CH * (W - 1);
                const float* ci = la.conv_in ? la.conv_in + ((size_t)seq * H + h) * CH * (W - 1) : nullptr;
                for (int e = tid; e < CH * (W - 1); e += NT1) {
                    const int ch = e / (W - 1), j = e % (W - 1);
                    const int ts = len - (W - 1) + j;  // relative to tok0
                    float x = 0.f;
                    if (tb + ts >= 0) {
                        const size_t row = (tok0 + ts) * H + h;
                        const bf16_t* src = ch < DK ? q + row * DK + ch : ch < 2 * DK ? k + row * DK + ch - DK
                                                                                      : v + row * DK + ch - 2 * DK;
                        x = __uint_as_float((uint32_t)*src << 16);
                    } else if (ci) {
                        x = ci[(size_t)ch * (W - 1) + (W - 1) + tb + ts];
                    }
                    co[e] = x;
                }
            }
        }
        // -A starts as zeros (the Gram phase writes its strictly lower
        // off-diagonal blocks), written once the loads are in flight.
        static_assert(sizeof(sm.Aneg) == NT1 * 16, "one 16-byte store per thread");
        reinterpret_cast<u32x4*>(sm.Aneg)[tid] = u32x4{0u, 0u, 0u, 0u};
        f32x4 G[NI];
        f32x4 run = zero4();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            f32x4 part;  // inclusive scan over the RPI rows of load i
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x = gv[i][j] * LOG2E;
#pragma unroll
                for (int d = LPR; d < 64; d *= 2) {
                    const float y = __shfl_up(x, d, 64);
                    if (lane >= d) x += y;
                }
                part[j] = x;
            }
            f32x4 tot;  // sum over the RPI rows: the last lane group's inclusive value
#pragma unroll
            for (int j = 0; j < 4; ++j) tot[j] = __shfl(part[j], (RPI - 1) * LPR + c4, 64);
            G[i] = run + part;
            run += tot;
        }
        // Totals of this wave's rows per channel -> LDS; prefix of earlier waves.
        float* wsum = &sm.DiagAT[0][0][0];  // DK x NW1 floats, free until the Gram phase
        if (hr == 0) *reinterpret_cast<f32x4*>(wsum + w * DK + 4 * c4) = run;
        lds_barrier();
        // Row block of this wave (16 rows = 2 waves) and its reference R_b:
        // the decay accumulated before the block, i.e. over the waves before
        // its first wave.
        static_assert(RW * 2 == 16, "two waves per 16-row block");
        const int bw = w / 2;
        f32x4 pre = zero4(), refb = zero4();
        for (int w2 = 0; w2 < w; ++w2) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(wsum + w2 * DK + 4 * c4);
            pre += t;
            if (w2 < 2 * bw) refb += t;
        }
        // The decay factors of the record and Gram steps, each exp2 taken once
        // per channel: R_b and G_C summed from the wave totals in the order
        // used for pre and refb (so the factors equal exp2 of those sums).
        for (int e = tid; e < 2 * DK; e += NT1) {
            const int c = e % DK;
            float R[5];
            R[0] = 0.f;
            float acc = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW1; ++w2) {
                acc += wsum[w2 * DK + c];
                if (w2 % 2 == 1) R[w2 / 2 + 1] = acc;
            }
            if (e < DK) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    sm.late.fac.eR[b][c] = __builtin_amdgcn_exp2f(R[b]);
                    sm.late.fac.eGR[b][c] = __builtin_amdgcn_exp2f(R[4] - R[b]);
                }
            } else {
#pragma unroll
                for (int bi = 1; bi < 4; ++bi) {
#pragma unroll
                    for (int bj = 0; bj < bi; ++bj)
                        sm.late.fac.F[pair_index(bi, bj)][c] = __builtin_amdgcn_exp2f(R[bi] - R[bj]);
                }
            }
        }
        if (w == NW1 - 1 && hr == 0) {
            const f32x4 gc = pre + run;  // G over the whole chunk (rows past the end add 0)
            *reinterpret_cast<f32x4*>(rec + RC::OFF_G + 16 * c4) =
                f32x4{__builtin_amdgcn_exp2f(gc[0]), __builtin_amdgcn_exp2f(gc[1]),
                      __builtin_amdgcn_exp2f(gc[2]), __builtin_amdgcn_exp2f(gc[3])};
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = RW * w + RPI * i + hr;
            const f32x4 a = G[i] + pre - refb;  // G - R_b <= 0
            f32x4 e, f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e[j] = __builtin_amdgcn_exp2f(a[j]);
                f[j] = __builtin_amdgcn_exp2f(-a[j]);
            }
            const float q0 = lo_f(qv[i][0]), q1 = hi_f(qv[i][0]), q2 = lo_f(qv[i][1]), q3 = hi_f(qv[i][1]);
            const float k0 = lo_f(kv[i][0]), k1 = hi_f(kv[i][0]), k2 = lo_f(kv[i][1]), k3 = hi_f(kv[i][1]);
            const int o = swz<DK>(r, 4 * c4);
            *reinterpret_cast<u32x2*>(&sm.Qt[o]) = u32x2{cvt2(q0 * e[0], q1 * e[1]), cvt2(q2 * e[2], q3 * e[3])};
            *reinterpret_cast<u32x2*>(&sm.Kt[o]) = u32x2{cvt2(k0 * e[0], k1 * e[1]), cvt2(k2 * e[2], k3 * e[3])};
            *reinterpret_cast<u32x2*>(&sm.Kh[o]) = u32x2{cvt2(k0 * f[0], k1 * f[1]), cvt2(k2 * f[2], k3 * f[3])};
        }
    }
    lds_barrier();

    // ---- Qt and Ke^T fragments to the record ----
    // Written by the six waves of the off-diagonal Gram pairs: waves 6 and 7
    // carry the diagonal blocks and their inverses, the longest Gram work.
    constexpr int NRF = 6;
    for (int f = w; f < 4 * KB && w < NRF; f += NRF) {
        const int t = f / KB, m = f % KB;
        // Qt = Qt_t' e^{R_t}: the stored rows are relative to their block.
        *reinterpret_cast<u32x4*>(rec + RC::OFF_Q + ((size_t)f * 64 + lane) * 16) = __builtin_bit_cast(
            u32x4, scale_frag(frag<DK>(sm.Qt, 16 * t + i16, m, q4), sm.late.fac.eR[t], m, q4));
    }
    // Ke^T = (k e^{G_C - G})^T as A fragments: lane (i16, q4) of fragment
    // (d, m2) holds channel 16d + i16 at tokens 32m2 + 4q4 + 0..3 and
    // 32m2 + 16 + 4q4 + 0..3; from the stored Kh' rows, Ke = Kh' e^{G_C - R_b}.
    // The channel's four consecutive tokens come from one transposing read:
    // as a source, lane (i16, q4) addresses token row tj of the four and the
    // four channels 4 ta .. 4 ta + 3 of the 16-channel block.
    const int tj = i16 >> 2, ta = i16 & 3;
    for (int f = w; f < 2 * RC::NDT && w < NRF; f += NRF) {
        const int d = f / 2, m2 = f % 2;
        const int c = 16 * d + i16;
        uint32_t u[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float sc = sm.late.fac.eGR[2 * m2 + hh][c];
            // Kh' at channel c, tokens 32 m2 + 16 hh + 4 q4 + 0..3
            const u32x2 x = ld_tr16(&sm.Kh[swz<DK>(32 * m2 + 16 * hh + 4 * q4 + tj, 16 * d + 4 * ta)]);
            u[2 * hh] = cvt2(lo_f(x[0]) * sc, hi_f(x[0]) * sc);
            u[2 * hh + 1] = cvt2(lo_f(x[1]) * sc, hi_f(x[1]) * sc);
        }
        *reinterpret_cast<u32x4*>(rec + RC::OFF_KT + ((size_t)f * 64 + lane) * 16) = u32x4{u[0], u[1], u[2], u[3]};
    }

    // ---- (a3, a4) Gram blocks ----
    // Aqk block (bi, bj), bj <= bi, is computed transposed, so lane (i16, q4)
    // holds row 16bi+i16, columns 16bj+4q4..+3: masked to the causal part and
    // written to the record as half an A fragment.
    auto aqk_store = [&](int bi, int bj, f32x4 acc) {
        const int r = 16 * bi + i16;
        f32x4 val;
#pragma unroll
        for (int i = 0; i < 4; ++i) val[i] = 16 * bj + 4 * q4 + i <= r ? acc[i] : 0.f;
        *reinterpret_cast<u32x2*>(rec + RC::OFF_A + ((size_t)afrag(bi, bj / 2) * 64 + lane) * 16 + (bj % 2) * 8) =
            u32x2{cvt2(val[0], val[1]), cvt2(val[2], val[3])};
    };
    if (w < 6) {
        // Off-diagonal pair p = w: (bi, bj) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
        // Kh's rows of block bj, scaled by e^{R_bi - R_bj}, serve both -A (bi, bj)
        // (as the second operand) and Aqk (bi, bj) (transposed, as the first).
        const int p = w;
        const int bi = p < 1 ? 1 : p < 3 ? 2 : 3;
        const int bj = p - (bi == 1 ? 0 : bi == 2 ? 1 : 3);
        bf16x8 kh[KB], kt[KB], qt[KB];
#pragma unroll
        for (int m = 0; m < KB; ++m) {
            kh[m] = scale_frag(frag<DK>(sm.Kh, 16 * bj + i16, m, q4), sm.late.fac.F[p], m, q4);
            kt[m] = frag<DK>(sm.Kt, 16 * bi + i16, m, q4);
            qt[m] = frag<DK>(sm.Qt, 16 * bi + i16, m, q4);
        }
        f32x4 acc = zero4(), accq = zero4();
#pragma unroll
        for (int m = 0; m < KB; ++m) {
            acc = mma(acc, kt[m], kh[m]);
            accq = mma(accq, kh[m], qt[m]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * bi + 4 * q4 + i;
            sm.Aneg[swz<C>(r, 16 * bj + i16)] = cvt1(-acc[i] * sm.beta[r]);
        }
        aqk_store(bi, bj, accq);
    } else {
        // Waves 6 and 7: diagonal blocks b0 = 2 (w - 6) and b0 + 1 of A (no
        // decay factor between rows of a block; transposed into DiagAT) and of
        // Aqk, one set of Kt, Kh, Qt fragments serving both, then those two
        // blocks' inverses (I + A_bb)^{-1} at once by fp32 forward substitution:
        // lane (j, q4) computes column j of block b0 + (q4 & 1)'s inverse (lane
        // groups 2 and 3 repeat groups 0 and 1 and store nothing).
        const int b0 = 2 * (w - 6);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int bb = b0 + h2;
            bf16x8 kt[KB], kh[KB], qt[KB];
#pragma unroll
            for (int m = 0; m < KB; ++m) {
                kt[m] = frag<DK>(sm.Kt, 16 * bb + i16, m, q4);
                kh[m] = frag<DK>(sm.Kh, 16 * bb + i16, m, q4);
                qt[m] = frag<DK>(sm.Qt, 16 * bb + i16, m, q4);
            }
            f32x4 acc = zero4(), accq = zero4();
#pragma unroll
            for (int m = 0; m < KB; ++m) {
                acc = mma(acc, kt[m], kh[m]);
                accq = mma(accq, kh[m], qt[m]);
            }
            f32x4 val;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q4 + i;
                val[i] = i16 < r ? acc[i] * sm.beta[16 * bb + r] : 0.f;
            }
            *reinterpret_cast<f32x4*>(&sm.DiagAT[bb][i16][4 * q4]) = val;
            aqk_store(bb, bb, accq);
        }
        // The Aqk fragment half above the diagonal, (b0, b0 + 1), is zero.
        *reinterpret_cast<u32x2*>(rec + RC::OFF_A + ((size_t)afrag(b0, b0 / 2) * 64 + lane) * 16 + 8) = u32x2{0u, 0u};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int bb = b0 + (q4 & 1);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == i16 ? 1.f : 0.f;
        // Column m of the block (rows 4u..4u+3; broadcast LDS reads within each
        // lane group), read one step ahead of its use.
        f32x4 col[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) col[0][u] = *reinterpret_cast<const f32x4*>(&sm.DiagAT[bb][0][4 * u]);
#pragma unroll
        for (int m = 0; m < 15; ++m) {
            if (m + 1 < 15) {
#pragma unroll
                for (int u = (m + 1) / 4; u < 4; ++u)
                    col[(m + 1) & 1][u] = *reinterpret_cast<const f32x4*>(&sm.DiagAT[bb][m + 1][4 * u]);
            }
            const float xm = x[m];
#pragma unroll
            for (int r = m + 1; r < 16; ++r) x[r] -= col[m & 1][r / 4][r % 4] * xm;
        }
        // Column i16 of the inverse, rows 0..15: one contiguous 32-byte row of DinvT.
        if (q4 < 2) {
            u32x4* dst = reinterpret_cast<u32x4*>(&sm.DinvT[(16 * bb + i16) * 16]);
            dst[0] = u32x4{cvt2(x[0], x[1]), cvt2(x[2], x[3]), cvt2(x[4], x[5]), cvt2(x[6], x[7])};
            dst[1] = u32x4{cvt2(x[8], x[9]), cvt2(x[10], x[11]), cvt2(x[12], x[13]), cvt2(x[14], x[15])};
        }
    }
    lds_barrier();

    // The values, staged row-major into the Qt tile (no longer needed) so each
    // substitution wave can read its 16-column tile.
    bf16_t* Vs = sm.Qt;
#pragma unroll
    for (int i = 0; i < NI; ++i)
        *reinterpret_cast<u32x2*>(&Vs[swz<DK>(vrow0 + vrstep * i, vch)]) = u32x2{vr[i][0], vr[i][1]};
    lds_barrier();

    // ---- (a4, a5) [W | U'] = (I + A)^{-1} Diag(beta) [Kt | V], 16-row block substitution ----
    // The wave's tiles advance stage by stage together so their dependent
    // MFMA chains overlap.  Tile 0 is a W tile unless this wave only owns V.
    const bool tile0V = NTW == 1 && hasV;
    const bool hasW = !tile0V;
    const int ct = w;  // W tile index (when the wave owns one)
    f32x4 Y[NTW][4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        // Row 16 bb + i16 of the block inverse, columns 4 q4 .. 4 q4 + 3 (one
        // transposing read of DinvT), then 4 zero columns: the contraction
        // block has 32 slots, 16 of them live.
        const u32x2 dv = ld_tr16(&sm.DinvT[(16 * bb + 4 * q4 + tj) * 16 + 4 * ta]);
        const bf16x8 dfr = as_frag(u32x4{dv[0], dv[1], 0u, 0u});
        const bf16x8 a0 = frag<C>(sm.Aneg, 16 * bb + i16, 0, q4);
        const bf16x8 a1 = frag<C>(sm.Aneg, 16 * bb + i16, 1, q4);
        // Kt = Kt_bb' e^{R_bb} for this lane's channel (the W tile's right-hand side).
        const float kscale = hasW ? sm.late.fac.eR[bb][16 * ct + i16] : 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NTW; ++s2) {
            const bool isV = s2 == 1 || tile0V;
            // Rows 16 bb + 4 q4 + 0..3 of the right-hand side's column (one transposing read).
            const int rs = 16 * bb + 4 * q4 + tj;
            const u32x2 xr = ld_tr16(isV ? &Vs[swz<DK>(rs, BV * vcb + 4 * ta)] : &sm.Kt[swz<DK>(rs, 16 * ct + 4 * ta)]);
            const f32x4 xs = f32x4{lo_f(xr[0]), hi_f(xr[0]), lo_f(xr[1]), hi_f(xr[1])};
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sm.beta[16 * bb + 4 * q4]);
            f32x4 rh;
#pragma unroll
            for (int i = 0; i < 4; ++i) rh[i] = b4[i] * (isV ? xs[i] : xs[i] * kscale);
            if (bb >= 1) rh = mma(rh, a0, bb == 1 ? frag_acc_lo(Y[s2][0]) : frag_acc(Y[s2][0], Y[s2][1]));
            if (bb == 3) rh = mma(rh, a1, frag_acc_lo(Y[s2][2]));
            const bf16x8 rf = frag_acc_lo(rh);
            Y[s2][bb] = mma(zero4(), dfr, rf);
            if (!isV) {
                // Transposed product: lane (i16, q4) gets W[16bb + i16][16ct + 4q4 .. +3],
                // half of the A fragment (row tile bb, contraction block ct / 2).
                const f32x4 yt = mma(zero4(), rf, dfr);
                *reinterpret_cast<u32x2*>(rec + RC::OFF_W + ((size_t)(bb * KB + ct / 2) * 64 + lane) * 16 + (ct % 2) * 8) =
                    u32x2{cvt2(-yt[0], -yt[1]), cvt2(-yt[2], -yt[3])};
            }
        }
    }
#pragma unroll
    for (int s2 = 0; s2 < NTW; ++s2) {
        if (s2 == 1 || tile0V) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                *reinterpret_cast<u32x2*>(rec + RC::OFF_UP + ((size_t)(vcb * 4 + bb) * 64 + lane) * 8) =
                    u32x2{cvt2(Y[s2][bb][0], Y[s2][bb][1]), cvt2(Y[s2][bb][2], Y[s2][bb][3])};
        }
    }
}

// ======================= kernel 2: chunk recurrence ==========================

// One workgroup per (batch, head, 16-wide value-column block), five waves with
// fixed roles, each running its own loop so that the compiler's wait-counter
// bookkeeping of one role never sees another role's memory traffic.
// Iteration n (one workgroup barrier each):
//   wave 0     carry:   chunk n from chain slot n % NSLOT; hands S_n and U_n (as
//                       MFMA B fragments) to hand slot n % 2
//   waves 1-2  output:  chunk n-1, token tiles {0,1} (wave 1) or {2,3} (wave 2);
//                       Qt and Aqk fragments come straight from the record into
//                       registers, one chunk ahead
//   waves 3-4  loader:  DMA the chain part of record n + NSLOT - 1 into its slot,
//                       then wait for record n + 1: NSLOT - 1 records in flight
// Every slot written in iteration n was last read in iteration n-1.  With the
// records in the Infinity Cache a record's DMA lands in about 2,000 cycles, so
// two records in flight cover it; a deeper ring (more DMA in flight beside the
// output waves' loads) measured slower at dk = 128 and at dk = 64.
constexpr int NT2 = 320;
constexpr int LDS_BYTES = 160 * 1024;

template <int DK>
struct RecurCfg {
    static constexpr int HAND = 2 * (DK / 32 + 2) * 64 * 16;  // two slots of S_n, U_n fragments
    static constexpr int SLOTS = (LDS_BYTES - HAND) / Rec<DK>::CHAIN;
    static constexpr int NSLOT = SLOTS > 3 ? 3 : SLOTS;
};

template <int DK>
struct alignas(16) RecurSmem {
    uint8_t chain[RecurCfg<DK>::NSLOT][Rec<DK>::CHAIN];  // W | Ke^T | G | U' of the workgroup's column block
    u32x4 hand[2][DK / 32 + 2][64];                       // [slot]: S_n (KB frags), U_n (2 frags)
};

template <int DK>
__global__ void __launch_bounds__(NT2, 1)
kda_chunk_recur(const uint8_t* __restrict__ ws, const float* S0, bf16_t* __restrict__ o,
                float* S_T, float* __restrict__ ckpt, int ckpt_every, SeqMap map, int H) {
    // S0 and S_T are not restrict-qualified: they may be the same array (a
    // later segment starts from the state the previous one left in S_T, and
    // callers may pass S_T == S0).
    typedef Rec<DK> RC;
    typedef RecurSmem<DK> SM;
    constexpr int DV = DK;
    constexpr int KB = RC::KB, NDT = RC::NDT;
    constexpr int NG = RC::NCB;                  // workgroups per head
    constexpr int NSLOT = RecurCfg<DK>::NSLOT;
    constexpr int AHEAD = NSLOT - 1;             // records in flight
    constexpr int CP = RC::CHAIN / 1024;         // 1 KiB DMA pieces of the chain part
    constexpr int CPA = (CP + 1) / 2, CPB = CP / 2;  // pieces per loader wave
    static_assert(NSLOT >= 3, "ring too shallow");
    static_assert(AHEAD * CPA <= 63, "vmcnt range");
    static_assert(sizeof(SM) <= LDS_BYTES, "LDS");
    __shared__ SM sm;

    // Workgroups are dispatched to the 8 XCDs round-robin (blockIdx % 8).  Unit
    // u (a sequence-head pair) gets its NG workgroups on XCD u % 8, so they
    // share that XCD's L2, and consecutive units spread over all XCDs, so
    // every XCD gets an equal share of every sequence (packed sequences of
    // very different lengths stay balanced).
    const int U = gridDim.x / NG;
    int lid = blockIdx.x;
    if (U % 8 == 0) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        lid = (x + 8 * (j / NG)) * NG + j % NG;
    }
    const int u = lid / NG, cb = lid % NG;  // u: (sequence, head) unit
    const int h = u % H;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, i16 = lane % 16, q4 = lane / 16;
    // The unit's chunks in this launch (N, covering T tokens from tok0), the
    // tokens of its sequence before them (tb), the sequence's length, its
    // records, its state (index su) and where that state starts from.
    int N, T, tb, Tlast, s = 0, su = u;
    bool from_S0 = true;  // else the state a previous segment left in S_T
    size_t tok0;
    const uint8_t* recs;
    if (!map.cu_seqlens) {
        N = map.N;
        T = map.T;
        tb = map.tbase;
        Tlast = map.Tfull;
        tok0 = (size_t)(u / H) * map.tstride + map.tbase;
        recs = ws + (size_t)u * map.N * RC::BYTES;
    } else {
        s = map.p0 + u / H;
        su = s * H + h;
        const int cs = map.cu_chunks[s], ce = map.cu_chunks[s + 1];
        const int lo = max(cs, map.c0), hi = min(ce, map.c0 + map.TC);  // its chunks in the segment
        Tlast = map.cu_seqlens[s + 1] - map.cu_seqlens[s];
        N = max(hi - lo, 0);
        tb = (lo - cs) * C;
        T = min(Tlast - tb, N * C);
        tok0 = (size_t)map.cu_seqlens[s] + tb;
        from_S0 = lo == cs;
        recs = ws + ((size_t)h * map.TC + (lo - map.c0)) * RC::BYTES;
    }
    // State unit index of checkpoint j (0-based) of this unit.
    auto ck_unit = [&](int j) -> size_t {
        if (!map.cu_seqlens) return (size_t)j * map.B * H + u;
        return ((size_t)map.cu_ckpts[s] + j) * H + h;
    };

    if (w == 0) {
        // ---- carry wave: (a6) U = U' - W S ; S <- e^{G_C} S + Ke^T U ----
        const size_t sbase = (size_t)su * DK * DV + BV * cb + i16;
        const float* Sin = from_S0 ? S0 : S_T;  // this workgroup alone reads and writes its slice
        f32x4 S[NDT];
#pragma unroll
        for (int d = 0; d < NDT; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[d][i] = Sin ? Sin[sbase + (size_t)(16 * d + 4 * q4 + i) * DV] : 0.f;
        lds_barrier();
        for (int n = 0; n < N; ++n) {
            const int t0 = n * C, L = min(C, T - t0);
            const uint8_t* rs = sm.chain[n % NSLOT];
            u32x4(*hand)[64] = sm.hand[n & 1];
            // Lane-derived LDS offsets are recomputed each chunk (cheap) instead
            // of being hoisted out of the loop and kept live.
            int ln = lane;
            asm volatile("" : "+v"(ln));
            // Operands are read in the order the products consume them (this
            // wave's LDS operations complete in issue order): U' and W for the
            // first product, e^{G_C}, then Ke^T for the second.  S_n goes to the
            // output waves' hand slot right after the W reads and U_n as soon as
            // it is formed, so that no LDS write is left for the end of the
            // iteration, where the barrier would wait for it.
            bf16x8 Wf[KB][4];
            f32x4 U[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x2 up = *reinterpret_cast<const u32x2*>(rs + RC::OFF_UP + (t * 64 + ln) * 8);
                U[t] = f32x4{lo_f(up[0]), hi_f(up[0]), lo_f(up[1]), hi_f(up[1])};
            }
#pragma unroll
            for (int m = 0; m < KB; ++m)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    Wf[m][t] = as_frag(*reinterpret_cast<const u32x4*>(rs + RC::OFF_W + ((t * KB + m) * 64 + ln) * 16));
            f32x4 gm[NDT];
#pragma unroll
            for (int d = 0; d < NDT; ++d) gm[d] = *reinterpret_cast<const f32x4*>(rs + RC::OFF_G + (16 * d + 4 * (ln / 16)) * 4);
            bf16x8 Sf[KB];
#pragma unroll
            for (int m = 0; m < KB; ++m) Sf[m] = frag_acc(S[2 * m], S[2 * m + 1]);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int m = 0; m < KB; ++m) hand[m][ln] = __builtin_bit_cast(u32x4, Sf[m]);
            asm volatile("" ::: "memory");
            bf16x8 Kf[2][NDT];
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int d = 0; d < NDT; ++d)
                    Kf[m2][d] = as_frag(*reinterpret_cast<const u32x4*>(rs + RC::OFF_KT + ((d * 2 + m2) * 64 + ln) * 16));
#pragma unroll
            for (int m = 0; m < KB; ++m)
#pragma unroll
                for (int t = 0; t < 4; ++t) U[t] = mma(U[t], Wf[m][t], Sf[m]);
            const bf16x8 Uf0 = frag_acc(U[0], U[1]), Uf1 = frag_acc(U[2], U[3]);
            hand[KB][ln] = __builtin_bit_cast(u32x4, Uf0);
            hand[KB + 1][ln] = __builtin_bit_cast(u32x4, Uf1);
#pragma unroll
            for (int d = 0; d < NDT; ++d) {
#pragma unroll
                for (int i = 0; i < 4; ++i) S[d][i] *= gm[d][i];
                S[d] = mma(S[d], Kf[0][d], Uf0);
            }
#pragma unroll
            for (int d = 0; d < NDT; ++d) S[d] = mma(S[d], Kf[1][d], Uf1);
            // (a7) periodic checkpoint.
            const int tend = tb + t0 + L;  // absolute position after the chunk
            if (ckpt_every > 0 && (tend % ckpt_every == 0 || tend == Tlast)) {
                float* dst = ckpt + ck_unit((tend - 1) / ckpt_every) * DK * DV + BV * cb + i16;
#pragma unroll
                for (int d = 0; d < NDT; ++d)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[(size_t)(16 * d + 4 * q4 + i) * DV] = S[d][i];
            }
            lds_barrier();
        }
        lds_barrier();
#pragma unroll
        for (int d = 0; d < NDT; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) S_T[sbase + (size_t)(16 * d + 4 * q4 + i) * DV] = S[d][i];
    } else if (w < 3) {
        // ---- output waves: O = Qt S_n + Aqk U_n for chunk n = iteration - 1 ----
        // Computed transposed (O^T = S_n^T Qt^T + U_n^T Aqk^T: the same fragments
        // with the operands swapped) so each lane holds four adjacent columns of
        // one token and stores them as one 8-byte word.
        auto out_loop = [&](auto tpc) {
            constexpr int TP = decltype(tpc)::value;   // token tiles 2TP, 2TP+1
            constexpr int NA = TP == 0 ? 2 : 4;        // Aqk fragments these tiles use
            constexpr int A0 = TP == 0 ? 0 : 2;        // ... starting at afrag(2TP, 0)
            constexpr int NQ = 2 * KB + NA;
            u32x4 F[2][NQ];                            // [buffer]: Qt frags (tile, m), then Aqk frags
            auto load = [&](int c, auto bufc) {
                constexpr int BF = decltype(bufc)::value;
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const uint8_t* rg = recs + (size_t)c * RC::BYTES;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int m = 0; m < KB; ++m)
                        F[BF][tt * KB + m] = *reinterpret_cast<const u32x4*>(rg + RC::OFF_Q + (((2 * TP + tt) * KB + m) * 64 + ln) * 16);
#pragma unroll
                for (int f = 0; f < NA; ++f)
                    F[BF][2 * KB + f] = *reinterpret_cast<const u32x4*>(rg + RC::OFF_A + ((A0 + f) * 64 + ln) * 16);
            };
            // One chunk from buffer BF.  Every chunk but the last is full, so
            // its step loads the next chunk and stores all rows unconditionally:
            // the vector-memory op counts are then the same on every path and
            // the wait for buffer BF leaves the next chunk's loads in flight.
            auto step = [&](int n, auto bufc, auto lastc) {
                constexpr int BF = decltype(bufc)::value;
                constexpr bool LAST = decltype(lastc)::value;
                if (!LAST) load(n + 1, std::integral_constant<int, 1 - BF>{});
                const int t0 = n * C, L = min(C, T - t0);
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int lj = ln % 16, lq4 = ln / 16;
                u32x4(*hand)[64] = sm.hand[n & 1];
                u32x4 Hf[KB + 2];
#pragma unroll
                for (int m = 0; m < KB; ++m) Hf[m] = hand[m][ln];
                Hf[KB] = hand[KB][ln];
                if (TP == 1) Hf[KB + 1] = hand[KB + 1][ln];
                bf16_t* orow = o + (tok0 + t0) * H * DV + (size_t)h * DV + BV * cb + 4 * lq4;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const int t = 2 * TP + tt;
                    f32x4 O = mma(zero4(), as_frag(Hf[KB]), as_frag(F[BF][2 * KB + afrag(t, 0) - A0]));
#pragma unroll
                    for (int m = 0; m < KB; ++m) O = mma(O, as_frag(Hf[m]), as_frag(F[BF][tt * KB + m]));
                    if (TP == 1) O = mma(O, as_frag(Hf[KB + 1]), as_frag(F[BF][2 * KB + afrag(t, 1) - A0]));
                    const int r = 16 * t + lj;
                    if (!LAST || r < L)
                        st_stream(u32x2{cvt2(O[0], O[1]), cvt2(O[2], O[3])}, reinterpret_cast<u32x2*>(orow + (size_t)r * H * DV));
                }
                lds_barrier();
            };
            typedef std::integral_constant<int, 0> B0;
            typedef std::integral_constant<int, 1> B1;
            typedef std::integral_constant<bool, false> Full;
            typedef std::integral_constant<bool, true> Last;
            if (N > 0) load(0, B0{});
            lds_barrier();
            lds_barrier();
            if (N == 1) {
                step(0, B0{}, Last{});
            } else if (N > 1) {
                step(0, B0{}, Full{});  // peeled: the loop is entered with buffer 1 pending behind one step's stores
                int n = 1;
                for (; n + 2 < N; n += 2) {
                    step(n, B1{}, Full{});
                    step(n + 1, B0{}, Full{});
                }
                if (n + 2 == N) {
                    step(n, B1{}, Full{});
                    step(n + 1, B0{}, Last{});
                } else {
                    step(n, B1{}, Last{});
                }
            }
        };
        if (w == 1)
            out_loop(std::integral_constant<int, 0>{});
        else
            out_loop(std::integral_constant<int, 1>{});
    } else {
        // ---- loader waves: wave 3 copies the even 1 KiB pieces, wave 4 the odd ----
        auto loader = [&](auto par) {
            constexpr int P = decltype(par)::value;
            constexpr int MINE = P == 0 ? CPA : CPB;
            auto dma = [&](int c) {
                const uint8_t* src = recs + (size_t)c * RC::BYTES;
                uint8_t* dst = sm.chain[c % NSLOT];
#pragma unroll
                for (int j = P; j < CP; j += 2) {
                    const int so = j * 1024 < RC::OFF_UP ? j * 1024 : RC::OFF_UP + cb * 2048 + (j * 1024 - RC::OFF_UP);
                    __builtin_amdgcn_global_load_lds((glb_void*)(src + so + lane * 16), (lds_void*)(dst + j * 1024), 16, 0, 0);
                }
            };
            // Prologue: records 0 .. AHEAD-1 in flight, wait for record 0.
            // Iteration n: issue record n + AHEAD, wait for record n + 1.  The
            // wait leaves the records issued after the awaited one in flight;
            // near the end fewer were issued, and the wait tightens to match.
            for (int c = 0; c < AHEAD; ++c)
                if (c < N) dma(c);
            auto wait_leaving = [&](int newer) {  // newer = records issued after the awaited one
                static_assert(AHEAD - 1 <= 5, "wait table");
                switch (newer) {
                    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * MINE)); break;
                    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * MINE)); break;
                    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * MINE)); break;
                    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * MINE)); break;
                    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1 * MINE)); break;
                    default: __builtin_amdgcn_s_waitcnt(0); break;
                }
            };
            // record 0 awaited; issued after it: records 1 .. min(AHEAD, N) - 1
            wait_leaving(max(0, min(AHEAD, N) - 1));
            lds_barrier();
            for (int n = 0; n <= N; ++n) {
                if (n + AHEAD < N) dma(n + AHEAD);
                // awaiting record n + 1; issued after it: n + 2 .. min(n + AHEAD, N - 1)
                wait_leaving(max(0, min(n + AHEAD, N - 1) - (n + 1)));
                lds_barrier();
            }
        };
        if (w == 3)
            loader(std::integral_constant<int, 0>{});
        else
            loader(std::integral_constant<int, 1>{});
    }
}

// The caller's host offsets reach the device as kernel arguments, up to
// CU_PER_LAUNCH values per launch: the launch copies them by value (also into
// a captured graph), so no host buffer has to outlive the call and the host
// never waits on a copy.
constexpr int CU_PER_LAUNCH = 960;
struct CuBlock {
    int first, count;
    int vals[CU_PER_LAUNCH];
};
__global__ void __launch_bounds__(256) kda_varlen_cu_write(int* __restrict__ dst, CuBlock blk) {
    for (int i = threadIdx.x; i < blk.count; i += blockDim.x) dst[blk.first + i] = blk.vals[i];
}

// Per-sequence chunk and checkpoint offsets of a packed batch (one workgroup,
// block-wide inclusive scans over 256 sequences at a time).
constexpr int NTT = 256;
__global__ void __launch_bounds__(NTT)
kda_varlen_tables(const int* __restrict__ cu_seqlens, int S, int ckpt_every, int* __restrict__ cu_chunks,
                  int* __restrict__ cu_ckpts) {
    __shared__ int sc[NTT], sk[NTT];
    const int tid = threadIdx.x;
    int carry_c = 0, carry_k = 0;
    if (tid == 0) {
        cu_chunks[0] = 0;
        cu_ckpts[0] = 0;
    }
    for (int base = 0; base < S; base += NTT) {
        const int i = base + tid;
        int nc = 0, nk = 0;
        if (i < S) {
            const int len = cu_seqlens[i + 1] - cu_seqlens[i];
            nc = (len + C - 1) / C;
            nk = ckpt_every > 0 ? (len + ckpt_every - 1) / ckpt_every : 0;
        }
        sc[tid] = nc;
        sk[tid] = nk;
        __syncthreads();
        for (int d = 1; d < NTT; d *= 2) {
            const int ac = tid >= d ? sc[tid - d] : 0, ak = tid >= d ? sk[tid - d] : 0;
            __syncthreads();
            sc[tid] += ac;
            sk[tid] += ak;
            __syncthreads();
        }
        if (i < S) {
            cu_chunks[i + 1] = carry_c + sc[tid];
            cu_ckpts[i + 1] = carry_k + sk[tid];
        }
        carry_c += sc[NTT - 1];
        carry_k += sk[NTT - 1];
        __syncthreads();
    }
}

template <int DK>
hipError_t launch_prep_t(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const SeqMap& map, int H, void* ws, hipStream_t stream, const LayerArgs* la = nullptr) {
    const long long wgs = map.cu_seqlens ? (long long)H * map.TC : (long long)map.B * H * map.N;
    if (wgs == 0) return hipSuccess;
    const int ly = !la ? -1 : la->conv_w ? la->W : 0;
    const LayerArgs args = la ? *la : LayerArgs{};
#define KDA_PREP(LYV)                                                                                      \
    hipLaunchKernelGGL((kda_chunk_prep<DK, LYV>), dim3((unsigned)wgs), dim3(NT1), 0, stream,               \
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),                      \
                       static_cast<const bf16_t*>(v), g, beta, static_cast<uint8_t*>(ws), map, H, args)
    switch (ly) {
        case -1: KDA_PREP(-1); break;
        case 0: KDA_PREP(0); break;
        case 1: KDA_PREP(1); break;
        case 2: KDA_PREP(2); break;
        case 3: KDA_PREP(3); break;
        case 4: KDA_PREP(4); break;
        default: return hipErrorInvalidValue;
    }
#undef KDA_PREP
    return hipGetLastError();
}

template <int DK>
hipError_t launch_recur_t(const void* ws, const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every,
                          const SeqMap& map, int H, hipStream_t stream) {
    const long long units = map.cu_seqlens ? (long long)map.NS * H : (long long)map.B * H;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_chunk_recur<DK>), dim3((unsigned)(units * (DK / BV))), dim3(NT2), 0, stream,
                       static_cast<const uint8_t*>(ws), S0, static_cast<bf16_t*>(o), S_T, ckpt, ckpt_every,
                       map, H);
    return hipGetLastError();
}

// Tokens [t0, t0 + tlen) of B sequences of T tokens.
SeqMap uniform_map(int B, int T, int t0 = 0, int tlen = -1) {
    if (tlen < 0) tlen = T - t0;
    SeqMap m{};
    m.B = B;
    m.T = tlen;
    m.N = (tlen + C - 1) / C;
    m.tbase = t0;
    m.tstride = T;
    m.Tfull = T;
    return m;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t record_bytes(int dk) { return dk == 128 ? Rec<128>::BYTES : dk == 64 ? Rec<64>::BYTES : 0; }

}  // namespace

size_t prefill_workspace_bytes(int dt, int dk, int B, int T, int H) {
    if (dt != 1) return 0;
    return (size_t)B * H * ((T + C - 1) / C) * record_bytes(dk);
}

// Chunks per segment of a packed prefill: like the uniform prefill's
// segments, the records of a segment (all H heads) stay within
// kSegmentRecordBytes, so that the recurrence reads them back from the
// Infinity Cache; segments are the fewest under that bound, of equal length,
// and at least 6 chunks (else all chunks are one segment).
long long varlen_segment_chunks(int dk, int H, long long total_chunks) {
    const size_t per_chunk = (size_t)H * record_bytes(dk);
    if (per_chunk == 0 || total_chunks <= 0) return total_chunks;
    const long long cmax = (long long)(kSegmentRecordBytes / per_chunk);
    if (cmax < 6 || cmax >= total_chunks) return total_chunks;
    const long long n = (total_chunks + cmax - 1) / cmax;
    return (total_chunks + n - 1) / n;
}

size_t varlen_workspace_bytes(int dk, int S, long long total_chunks, int H) {
    return align256((size_t)H * varlen_segment_chunks(dk, H, total_chunks) * record_bytes(dk)) +
           3 * align256((size_t)(S + 1) * sizeof(int));
}

hipError_t launch_prefill_prep(int dk, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, int B, int T, int H, void* ws, hipStream_t stream, int t0,
                               int tlen) {
    const SeqMap m = uniform_map(B, T, t0, tlen);
    if (dk == 128) return launch_prep_t<128>(q, k, v, g, beta, m, H, ws, stream);
    if (dk == 64) return launch_prep_t<64>(q, k, v, g, beta, m, H, ws, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_recur(int dk, const void* ws, const float* S0, void* o, float* S_T, float* ckpt,
                                int ckpt_every, int B, int T, int H, hipStream_t stream, int t0, int tlen) {
    const SeqMap m = uniform_map(B, T, t0, tlen);
    if (dk == 128) return launch_recur_t<128>(ws, S0, o, S_T, ckpt, ckpt_every, m, H, stream);
    if (dk == 64) return launch_recur_t<64>(ws, S0, o, S_T, ckpt, ckpt_every, m, H, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_layer(int dk, const void* q, const void* k, const void* v, const float* a,
                                const float* b, const LayerArgs& la, int B, int T, int H, const float* S0,
                                void* o, float* S_T, float* ckpt, int ckpt_every, void* ws, hipStream_t stream,
                                int t0, int tlen) {
    const SeqMap m = uniform_map(B, T, t0, tlen);
    hipError_t e = hipSuccess;
    if (T == 0 && la.conv_w && la.conv_out && la.W > 1)  // no token: the carried state passes through
        e = launch_fill_copy(la.conv_in, la.conv_out, (long long)B * H * 3 * dk * (la.W - 1), stream);
    if (e != hipSuccess) return e;
    if (dk == 128) {
        e = launch_prep_t<128>(q, k, v, a, b, m, H, ws, stream, &la);
        if (e == hipSuccess) e = launch_recur_t<128>(ws, S0, o, S_T, ckpt, ckpt_every, m, H, stream);
        return e;
    }
    if (dk == 64) {
        e = launch_prep_t<64>(q, k, v, a, b, m, H, ws, stream, &la);
        if (e == hipSuccess) e = launch_recur_t<64>(ws, S0, o, S_T, ckpt, ckpt_every, m, H, stream);
        return e;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_varlen(int dk, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int* cu_seqlens_host, int S, long long total_chunks,
                                 int H, const float* S0, void* o, float* S_T, float* ckpt, int ckpt_every,
                                 void* ws, hipStream_t stream) {
    // Workspace: one segment's records, then the three offset tables.
    const long long seg = varlen_segment_chunks(dk, H, total_chunks);
    uint8_t* base = static_cast<uint8_t*>(ws);
    const size_t tab = align256((size_t)(S + 1) * sizeof(int));
    int* d_cu = reinterpret_cast<int*>(base + align256((size_t)H * seg * record_bytes(dk)));
    int* d_chunks = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(d_cu) + tab);
    int* d_ckpts = reinterpret_cast<int*>(reinterpret_cast<uint8_t*>(d_chunks) + tab);
    hipError_t e = hipSuccess;
    for (int first = 0; first <= S; first += CU_PER_LAUNCH) {
        CuBlock blk;
        blk.first = first;
        blk.count = std::min(CU_PER_LAUNCH, S + 1 - first);
        for (int i = 0; i < blk.count; ++i) blk.vals[i] = cu_seqlens_host[first + i];
        hipLaunchKernelGGL(kda_varlen_cu_write, dim3(1), dim3(256), 0, stream, d_cu, blk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kda_varlen_tables, dim3(1), dim3(NTT), 0, stream, d_cu, S, ckpt_every, d_chunks, d_ckpts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    SeqMap m{};
    m.S = S;
    m.cu_seqlens = d_cu;
    m.cu_chunks = d_chunks;
    m.cu_ckpts = d_ckpts;
    auto chunks_of = [&](int i) { return ((long long)cu_seqlens_host[i + 1] - cu_seqlens_host[i] + C - 1) / C; };
    // Segment j covers global chunks [c_lo, c_hi).  Its sequences are those
    // with chunks in it, and the empty ones positioned in it (at the end of
    // all chunks: the last segment): a contiguous range [s_lo, s_hi], found
    // with one pass over the sequences for all segments.
    const long long nseg = total_chunks > 0 ? (total_chunks + seg - 1) / seg : 1;
    int s_lo = 0;
    long long cs_lo = 0;  // first chunk of sequence s_lo
    for (long long j = 0; j < nseg && e == hipSuccess; ++j) {
        const long long c_lo = j * seg, c_hi = std::min(total_chunks, c_lo + seg);
        const bool last = j == nseg - 1;
        while (s_lo < S) {  // sequences wholly before the segment
            const long long n = chunks_of(s_lo);
            if (n > 0 ? cs_lo + n > c_lo : cs_lo >= c_lo) break;
            cs_lo += n;
            ++s_lo;
        }
        int s_hi = s_lo - 1;
        long long cs = cs_lo;  // first chunk of sequence s_hi + 1
        while (s_hi + 1 < S && (last || cs < c_hi)) {  // sequences starting before the segment's end
            ++s_hi;
            cs += chunks_of(s_hi);
        }
        m.TC = (int)(c_hi - c_lo);
        m.c0 = (int)c_lo;
        m.p0 = s_lo;
        m.NS = s_hi - s_lo + 1;
        if (dk == 128) {
            e = launch_prep_t<128>(q, k, v, g, beta, m, H, ws, stream);
            if (e == hipSuccess) e = launch_recur_t<128>(ws, S0, o, S_T, ckpt, ckpt_every, m, H, stream);
        } else if (dk == 64) {
            e = launch_prep_t<64>(q, k, v, g, beta, m, H, ws, stream);
            if (e == hipSuccess) e = launch_recur_t<64>(ws, S0, o, S_T, ckpt, ckpt_every, m, H, stream);
        } else {
            e = hipErrorInvalidValue;
        }
    }
    return e;
}

}  // namespace kda
