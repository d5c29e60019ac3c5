// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "common.h"

namespace g2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define G2_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// two values into one 32-bit word, a in the low half (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ void unpack8f(uint4 u, float (&o)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o[2 * k] = __uint_as_float(w[k] << 16);
        o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}

// activation element access for the two storage types
template <class T> struct Act;
template <> struct Act<float> {
    __device__ static float ld(const float* p, int64_t i) { return p[i]; }
    __device__ static void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Act<bf16_t> {
    __device__ static float ld(const bf16_t* p, int64_t i) { return bf2f(p[i]); }
    __device__ static void st(bf16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
};

// tanh approximation of GELU, 0.5 u (1 + tanh z) with z = sqrt(2/pi) (u + 0.044715 u^3),
// evaluated through the identity 0.5 (1 + tanh z) = 1 / (1 + exp(-2 z)): one exp and
// one reciprocal, no cancellation near zero. Its derivative uses
// 1 - tanh(z)^2 = 4 s (1 - s) with s = 1 / (1 + exp(-2 z)).
__device__ __forceinline__ float gelu_sig(float u) {
    const float k0x2 = 1.5957691216057308f, k1 = 0.044715f;  // 2 sqrt(2/pi)
    return __builtin_amdgcn_rcpf(1.0f + __expf(-k0x2 * (u + k1 * u * u * u)));
}
// GELU and its derivative at u from the same exponential; the forward stores the
// derivative for the backward, which then needs no exponential of its own
__device__ __forceinline__ void gelu_tanh_and_grad(float u, float& g, float& dg) {
    const float k0 = 0.7978845608028654f, k1 = 0.044715f;
    const float sg = gelu_sig(u);
    g = u * sg;
    dg = sg + 2.0f * u * sg * (1.0f - sg) * k0 * (1.0f + 3.0f * k1 * u * u);
}

// The exact GELU u Phi(u), Phi(u) = 0.5 (1 + erf(u / sqrt 2)), and its derivative
// Phi(u) + u phi(u) with phi(u) = exp(-u^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ void gelu_erf_and_grad(float u, float& g, float& dg) {
    const float Phi = 0.5f * (1.0f + erff(u * 0.70710678118654752f));
    g = u * Phi;
    dg = Phi + u * 0.39894228040143268f * __expf(-0.5f * u * u);
}

// Two gfx950 LDS transpose loads (ds_read_b64_tr_b16) 'gap' bytes apart, packed
// into one 8 x bf16 MFMA operand. In each 16-lane group, lane j addresses row
// j/4 and 4 consecutive 16-bit columns 4(j%4)..; lane i of the group receives
// column i of the 4 rows. p points into LDS.
__device__ __forceinline__ bf16x8 lds_tr_pair(const char* p, int gap) {
#if defined(__HIP_DEVICE_COMPILE__)
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((G2_LDS s16x4*)p);
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((G2_LDS s16x4*)(p + gap));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
#else
    (void)p; (void)gap;
    return bf16x8{};
#endif
}

// Two gfx950 LDS transpose loads from independent addresses, packed as above.
__device__ __forceinline__ bf16x8 lds_tr2(const char* p0, const char* p1) {
#if defined(__HIP_DEVICE_COMPILE__)
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((G2_LDS s16x4*)p0);
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((G2_LDS s16x4*)p1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
#else
    (void)p0; (void)p1;
    return bf16x8{};
#endif
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace g2
