// kda_device.h -- wavefront-level primitives for the gfx950 KDA kernels.
//
// MFMA tiles are 16 x 16 with fp32 accumulation.  One "fragment" is the 8
// contraction values a lane contributes to a 16 x 16 x 32 product:
//   bf16: one v_mfma_f32_16x16x32_bf16 (8 bf16 per lane)
//   fp32: eight v_mfma_f32_16x16x4_f32 (1 float per lane each)
// For both, lane l = 16 q + i supplies row (A) or column (B) i and contraction
// slots s = 0..7 of lane group q; A-lane (i, q) slot s meets B-lane (j, q) slot s.
//
// Contraction order.  Every product uses one fixed permutation of the 32
// contraction indices of block m:
//     slot (q, s)  <->  k = 32 m + 16 (s / 4) + 4 q + (s % 4)
// An accumulator tile holds rows 4 q + i (i = 0..3) of column j in lane (j, q),
// so tiles 2m and 2m+1 of an accumulator ARE the B fragment of contraction
// block m without moving data between lanes: a result can feed the next
// product straight from registers.  Fragments read from LDS use the same
// order: elements [4q, 4q+4) and [16+4q, 16+4q+4) of a 32-wide row segment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Gate functions of the layer steps, in fp32 with the hardware exp2/log2/rcp
// (about 1 ulp each).  sigmoid(x) = 1 / (1 + e^-x) saturates cleanly at both
// ends; log sigmoid(x) = min(x, 0) - log(1 + e^-|x|) never overflows.
__device__ __forceinline__ float sigmoid1(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}
__device__ __forceinline__ float log_sigmoid(float x) {
    const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * 1.4426950408889634f);
    return fminf(x, 0.f) - __builtin_amdgcn_logf(1.f + e) * 0.6931471805599453f;
}
__device__ __forceinline__ f32x4 silu4(f32x4 x) {
    return f32x4{x[0] * sigmoid1(x[0]), x[1] * sigmoid1(x[1]), x[2] * sigmoid1(x[2]), x[3] * sigmoid1(x[3])};
}

// Operand precision policy: bf16 operands on the bf16 MFMA.
struct OpBF16 {
    typedef uint16_t lds_t;  // bf16 bits in LDS
    typedef bf16x8 frag_t;

    __device__ static __forceinline__ lds_t cvt(float x) { return f2bf(x); }
    __device__ static __forceinline__ float to_f(lds_t x) { return bf2f(x); }

    // p points at element 32 m of a row whose contraction index is contiguous.
    __device__ static __forceinline__ frag_t load(const lds_t* p, int q) {
        u32x2 a = *reinterpret_cast<const u32x2*>(p + 4 * q);
        u32x2 b = *reinterpret_cast<const u32x2*>(p + 16 + 4 * q);
        u32x4 u = {a[0], a[1], b[0], b[1]};
        return __builtin_bit_cast(frag_t, u);
    }
    // Fragment of contraction block m from accumulator tiles 2m (x) and 2m+1 (y).
    __device__ static __forceinline__ frag_t from_acc(f32x4 x, f32x4 y) {
        u32x4 u = {pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]),
                   pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
        return __builtin_bit_cast(frag_t, u);
    }
    __device__ static __forceinline__ frag_t from_acc_lo(f32x4 x) {
        u32x4 u = {pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), 0u, 0u};
        return __builtin_bit_cast(frag_t, u);
    }
    __device__ static __forceinline__ f32x4 mma(f32x4 c, frag_t a, frag_t b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// Operand precision policy: fp32 operands on the fp32 MFMA (exact products).
struct OpF32 {
    typedef float lds_t;
    struct frag_t {
        f32x4 lo, hi;
    };

    __device__ static __forceinline__ lds_t cvt(float x) { return x; }
    __device__ static __forceinline__ float to_f(lds_t x) { return x; }

    __device__ static __forceinline__ frag_t load(const lds_t* p, int q) {
        frag_t f;
        f.lo = *reinterpret_cast<const f32x4*>(p + 4 * q);
        f.hi = *reinterpret_cast<const f32x4*>(p + 16 + 4 * q);
        return f;
    }
    __device__ static __forceinline__ frag_t from_acc(f32x4 x, f32x4 y) { return frag_t{x, y}; }
    __device__ static __forceinline__ frag_t from_acc_lo(f32x4 x) { return frag_t{x, zero4()}; }
    __device__ static __forceinline__ f32x4 mma(f32x4 c, frag_t a, frag_t b) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], c, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], c, 0, 0, 0);
        return c;
    }
};

// Element types of q, k, v and o in global memory.
struct InBF16 {
    typedef uint16_t elem_t;
    __device__ static __forceinline__ float to_f(elem_t x) { return bf2f(x); }
    __device__ static __forceinline__ elem_t from_f(float x) { return f2bf(x); }
};
struct InF32 {
    typedef float elem_t;
    __device__ static __forceinline__ float to_f(elem_t x) { return x; }
    __device__ static __forceinline__ elem_t from_f(float x) { return x; }
};

}  // namespace kda
