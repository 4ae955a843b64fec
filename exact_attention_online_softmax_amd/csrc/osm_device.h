// osm_device.h -- device helpers shared by the gfx950 kernels of libosm.
//
// Everything here runs on the GPU.  Exponentials are taken in base 2 with
// the hardware v_exp_f32 instruction ([P3] "Precision, and what can still
// go wrong": e^x = 2^(x log2 e), fold log2 e into the scale, keep the
// running maximum in scaled units).
//
//   [P3] "Online softmax" (zerotofrontier.app, efficient-attention chapter)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

constexpr float kLog2e = 1.44269502162933349609375f;     // fp32 nearest to log2(e)
constexpr float kLog2eLo = 1.925963033500011e-08f;       // log2(e) - kLog2e
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float t) { return __builtin_amdgcn_exp2f(t); }

// e^d for d <= 0 (or -inf), to about one fp32 rounding beyond the rounding
// already present in d.  d * log2(e) is carried as hi + lo: hi = fl(d*L),
// lo = the exact residual of that product plus d * (log2 e - L), so the
// fp32 rounding of the exponent does not reach the result.
// 2^(hi + lo) = 2^hi * (1 + lo ln2) to second order in |lo| <= 2^-16.
// Inputs below -200 are clamped (the result is 0 in fp32 either way), which
// also keeps -inf from producing inf - inf.
__device__ __forceinline__ float exp_acc(float d) {
    d = fmaxf(d, -200.0f);
    float hi = d * kLog2e;
    float lo = fmaf(d, kLog2e, -hi);
    lo = fmaf(d, kLog2eLo, lo);
    float e = fast_exp2(hi);
    return fmaf(e, lo * kLn2, e);
}

// Merge of two (m, l) summaries of disjoint pieces of a row ([P3] "Merging
// partial results"): bring both to the larger maximum, then add.  The empty
// piece (-inf, 0) is the identity and never produces exp(-inf - (-inf)).
__device__ __forceinline__ void merge_ml(float &m, float &l, float m2, float l2) {
    float mn = fmaxf(m, m2);
    if (mn == kNegInf) {
        m = kNegInf;
        l = 0.0f;
        return;
    }
    float a = (m == kNegInf) ? 0.0f : exp_acc(m - mn);
    float b = (m2 == kNegInf) ? 0.0f : exp_acc(m2 - mn);
    l = l * a + l2 * b;
    m = mn;
}

// Butterfly merge of per-lane (m, l) over the 64 lanes of a wavefront.
__device__ __forceinline__ void wave_merge_ml(float &m, float &l) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float m2 = __shfl_xor(m, off, 64);
        float l2 = __shfl_xor(l, off, 64);
        merge_ml(m, l, m2, l2);
    }
}

// bf16 helpers (bit-level; bf16 values widen to fp32 exactly).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// The same two conversions in one gfx950 instruction (v_cvt_pk_bf16_f32,
// round-to-nearest-even under the default rounding mode): bit-identical to
// pack_bf16x2 for every non-NaN input.  For epilogues that convert many
// accumulators at once.
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

}  // namespace osm
