// radamw_math.h -- the per-element arithmetic of the update, shared by the
// fused kernels (radamw_update.hip) and the staged baseline
// (radamw_staged.hip) so both round identically.
//
// Page abbreviation: FA-ja = RUDA docs page "実験的なデバイス上の融合 AdamW /
// AMSGrad"; the formula is the one of its section "この演算子を使用する理由".
// Device math is FP32 and the pages allow fusion and reassociation; the
// contractions are written out (fmaf) rather than left to the compiler, so
// that every kernel using these helpers produces the same bits.
#pragma once

#include "radamw_internal.h"

namespace radamw {

// g = stored / gradient_scale, negated when maximizing (sign folded into
// inv_scale on the host).
__device__ __forceinline__ float unscale(float x, const Coefs &c) { return x * c.inv_scale; }

// m = beta1 * m_old + (1 - beta1) * g
__device__ __forceinline__ float first_moment(float m_old, float g, const Coefs &c) {
    return __builtin_fmaf(c.beta1, m_old, c.one_minus_beta1 * g);
}

// v = beta2 * v_old + (1 - beta2) * g * g
__device__ __forceinline__ float second_moment(float v_old, float g, const Coefs &c) {
    return __builtin_fmaf(c.beta2, v_old, (c.one_minus_beta2 * g) * g);
}

// lr * (m / bc1) / (sqrt(v_used / bc2) + eps), with host-formed lr / bc1 and
// 1 / bc2; v_sqrt_f32 and v_rcp_f32 (about one ulp each).
__device__ __forceinline__ float step_delta(float m, float v_used, const Coefs &c) {
    const float denom = __builtin_amdgcn_sqrtf(v_used * c.inv_bc2) + c.eps;
    return (c.step_size * m) * __builtin_amdgcn_rcpf(denom);
}

// p * (1 - lr * weight_decay) - delta
__device__ __forceinline__ float apply_step(float p, float delta, const Coefs &c) {
    return __builtin_fmaf(p, c.decay, -delta);
}

}  // namespace radamw
