// dyt_math.hpp - float32 device math for the DyT kernels (gfx950).
//
// The layer needs t = tanh(u) and, in the backward, d = sech^2(u) = 1 - t^2
// for u = alpha * x. 1 - t*t cancels catastrophically once |u| grows (in
// float32 it loses 1e-6 relative accuracy near |u| = 2 and a whole bfloat16
// ulp near |u| = 6), so both quantities are built from e = exp(-2|u|):
//
//   tanh|u|  = (1 - e) / (1 + e)          sech^2 u = 4 e / (1 + e)^2
//
// which has no cancellation for |u| away from 0. Near 0, 1 - e cancels
// instead, so small |u| takes a short odd series for tanh (and 1 - t^2,
// which is then >= 0.87 and exact enough).
//
// Two variants, chosen by the storage dtype of x:
//   * accurate (float32 outputs): in the backward, e via Cody & Waite's
//     additive range reduction (W. J. Cody, W. Waite, "Software Manual for
//     the Elementary Functions", 1980) with the hardware 2^x on the reduced
//     argument and a Newton-refined reciprocal: about 3-5 float32 ulp on
//     sech^2 at every |u| (4e/(1+e)^2 does not cancel near 0 either). The
//     backward's t only feeds the float32 dgamma sums, judged at 1e-5, so
//     below |u| = 2^-5 it takes u - u^3/3 and above (1 - e)/(1 + e), whose
//     cancellation costs at most ~1e-6 relative just above 2^-5. The forward
//     needs t to 1e-6, well conditioned in e, so it takes e from the
//     hardware 2^x directly and the Taylor series of tanh through u^9 below
//     |u| = 0.35 (tanh_fwd_f32; coefficients 2^2n (2^2n - 1) B_2n / (2n)!,
//     B the Bernoulli numbers).
//   * fast (bfloat16 outputs): e straight from the hardware 2^x and 1/x
//     (about 1e-5 relative at |u| = 50, far below half a bfloat16 ulp);
//     in the forward tanh u ~= u below 2^-6 (relative error < 1e-4), in the
//     backward u - u^3/3 below 2^-5.
//
// IEEE behaviour is kept on purpose: u = +-inf gives t = +-1, d = 0; NaN
// propagates. Branches are selects evaluated after both sides are
// computed; NaN is never clamped away (v_min/v_max would drop it).
// float32 subnormals are not flushed (the library is built without
// fast-math or denormal flushing).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dyt {

// log2(e) and -2*log2(e), rounded to float32.
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kMinus2Log2e = -0x1.715476p+1f;
// ln 2 split into a float32 head and the float32 rounding of the remainder.
constexpr float kLn2Hi = 0x1.62e43p-1f;
constexpr float kLn2Lo = -0x1.05c61p-29f;

__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// copysign as one bitfield insert: magnitude bits of m, sign bit of s.
__device__ __forceinline__ float copy_sign(float m, float s) {
    return __builtin_copysignf(m, s);
}

constexpr float kAccurateSmall = 0.35f;
constexpr float kFastSmallBwd = 0x1p-5f;

// DYT_ACC_BWD_SERIES = 1 restores the longer small-|u| branch of the
// accurate backward (Taylor series of tanh through u^13 and sech^2 = 1 - t^2
// below |u| = 0.35) for comparison.
#ifndef DYT_ACC_BWD_SERIES
#define DYT_ACC_BWD_SERIES 0
#endif

// Taylor series of tanh(u)/u - 1 in s = u^2 (terms through s^6, u^13).
__device__ __forceinline__ float tanh_series_tail(float s) {
    float p = 0x1.d6d3d0p-9f;                  //  21844/6081075
    p = __builtin_fmaf(p, s, -0x1.226e36p-7f); // -1382/155925
    p = __builtin_fmaf(p, s, 0x1.664f48p-6f);  //  62/2835
    p = __builtin_fmaf(p, s, -0x1.ba1ba2p-5f); // -17/315
    p = __builtin_fmaf(p, s, 0x1.111112p-3f);  //  2/15
    p = __builtin_fmaf(p, s, -0x1.555556p-2f); // -1/3
    return p;
}

// Accurate tanh(u) and sech^2(u) (float32 outputs) for u = alpha * x.
// sech^2 has relative condition number 2|u tanh u| in u, so rounding u to
// float32 alone would cost ~|u| * 1.2e-7 relative error; the product is
// therefore carried as u + ul (ul = fma(alpha, x, -u), exact), and ul enters
// the reduced exponent argument. tanh is well conditioned and uses u only.
__device__ __forceinline__ void tanh_sech2_accurate(float x, float alpha, float& t, float& d) {
    const float u = alpha * x;
    const float ul = __builtin_fmaf(alpha, x, -u);
    const float a = __builtin_fabsf(u);
    // large |u|: e = exp(-2|u + ul|) = exp(z + zl), z = -2|u|,
    // zl = -2 sign(u) ul; Cody-Waite reduction
    float z = -2.0f * a;
    float zl = ul * copy_sign(2.0f, -u);
    const bool under = z < -104.0f;           // e rounds to 0; also u = +-inf
    z = under ? -104.0f : z;
    zl = under ? 0.0f : zl;                   // fma(inf, x, -inf) is NaN: drop it
    const float k = __builtin_rintf(z * kLog2e);
    float r = __builtin_fmaf(-k, kLn2Hi, z);
    r = r + zl;
    r = __builtin_fmaf(-k, kLn2Lo, r);
    const float e = __builtin_amdgcn_ldexpf(hw_exp2(r * kLog2e), (int)k);
    const float p = 1.0f + e;
    float rc = hw_rcp(p);
    rc = __builtin_fmaf(rc, __builtin_fmaf(-p, rc, 1.0f), rc);   // Newton step
    const float tl = (1.0f - e) * rc;
    const float dl = ((4.0f * e) * rc) * rc;
    // small |u|
    const float s = u * u;
#if DYT_ACC_BWD_SERIES
    const float ts = __builtin_fmaf(u * s, tanh_series_tail(s), u);
    const float ds = __builtin_fmaf(-ts, ts, 1.0f);
    const bool small = a < kAccurateSmall;
    t = small ? ts : copy_sign(tl, u);
    d = small ? ds : dl;
#else
    const float ts = __builtin_fmaf(u * s, -0x1.555556p-2f, u);
    t = (a < kFastSmallBwd) ? ts : copy_sign(tl, u);
    d = dl;
#endif
}

// Forward tanh for float32 outputs. y is checked at 1e-6 of |gamma t| +
// |beta|, and an error in e moves t = (1 - e)/(1 + e) by only
// sech^2(u)/2 times e's relative error, so the hardware 2^x of the rounded
// argument -2|u| log2(e) and one hardware reciprocal (each within one
// float32 ulp) suffice above |u| = 0.35; below, where 1 - e cancels, the odd
// series through u^9 (its truncation is under 3e-7 relative at 0.35).
// Modelled with 2^x and 1/x each off by one ulp either way, the worst
// relative error over |u| <= 12 is 4.1e-7. u = +-inf gives +-1; NaN
// propagates; subnormal u returns u.
__device__ __forceinline__ float tanh_fwd_f32(float u) {
    const float a = __builtin_fabsf(u);
    const float e = hw_exp2(a * kMinus2Log2e);
    const float r = hw_rcp(1.0f + e);
    const float tl = (1.0f - e) * r;
    const float s = u * u;
    float p = 0x1.664f48p-6f;                  //  62/2835
    p = __builtin_fmaf(p, s, -0x1.ba1ba2p-5f); // -17/315
    p = __builtin_fmaf(p, s, 0x1.111112p-3f);  //  2/15
    p = __builtin_fmaf(p, s, -0x1.555556p-2f); // -1/3
    const float ts = __builtin_fmaf(u * s, p, u);
    return (a < kAccurateSmall) ? ts : copy_sign(tl, u);
}

constexpr float kFastSmall = 0x1p-6f;

// Fast tanh(u) (bfloat16 outputs): e4 = 4 e^{-2|u|} from one hardware 2^x
// (the factor 4 rides in the exponent), t = (1 - e)/(1 + e).
__device__ __forceinline__ float tanh_fast(float u) {
    const float a = __builtin_fabsf(u);
    const float e4 = hw_exp2(__builtin_fmaf(a, kMinus2Log2e, 2.0f));
    const float r = hw_rcp(__builtin_fmaf(e4, 0.25f, 1.0f));
    const float tl = __builtin_fmaf(e4, -0.25f, 1.0f) * r;
    return (a < kFastSmall) ? u : copy_sign(tl, u);
}

// Fast tanh and sech^2 for the backward. t feeds the float32 dgamma sums,
// which are compared at 1e-5 relative, so small |u| keeps two series terms
// (u - u^3/3, relative error < 2e-7 below 2^-5) where 1 - e cancels.

__device__ __forceinline__ void tanh_sech2_fast(float u, float& t, float& d) {
    const float a = __builtin_fabsf(u);
    const float e4 = hw_exp2(__builtin_fmaf(a, kMinus2Log2e, 2.0f));
    const float r = hw_rcp(__builtin_fmaf(e4, 0.25f, 1.0f));
    const float tl = copy_sign(__builtin_fmaf(e4, -0.25f, 1.0f) * r, u);
    const float ts = __builtin_fmaf(u * (u * u), -0x1.555556p-2f, u);
    t = (a < kFastSmallBwd) ? ts : tl;
    d = (e4 * r) * r;
}

// ------------------------------------------------------------ storage types
// bfloat16 is carried as its raw 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

// IEEE binary16 is carried as its raw 16-bit pattern as well.
struct f16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v.bits << 16);
}
__device__ __forceinline__ float to_f32(f16_t v) {
    return (float)__builtin_bit_cast(_Float16, v.bits);
}

// float32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {lo, hi};
    const b2 r = __builtin_convertvector(v, b2);
    return __builtin_bit_cast(uint32_t, r);
}

// float32 -> float16 pair, round to nearest even, from the float32 values.
// The empty asm pins each value as a float32 register first: otherwise the
// compiler may contract the conversion with the fma or multiply producing it
// into a mixed-precision instruction (v_fma_mixlo_f16) that rounds the
// exact result once to float16, which differs in the last bit from rounding
// the float32 result in about 1 case in 16,000.
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    asm volatile("" : "+v"(lo), "+v"(hi));
    const f2 v = {lo, hi};
    const h2 r = __builtin_convertvector(v, h2);
    return __builtin_bit_cast(uint32_t, r);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    return bf16_t{(uint16_t)(pack2_bf16(v, 0.0f) & 0xffffu)};
}
// Through pack2_f16 (see there) like the 16-byte path.
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) {
    return f16_t{(uint16_t)(pack2_f16(v, 0.0f) & 0xffffu)};
}

}  // namespace dyt
