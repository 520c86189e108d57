// ss_device.h -- device helpers shared by the gfx950 selective-scan kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Read-only memory seen through the constant address space: wave-uniform loads from it are
// selected as scalar (SMEM) loads.  Only for data no kernel writes while the reader runs.
typedef const __attribute__((address_space(4))) float cfloat;
__device__ __forceinline__ cfloat* to_constant(const float* p) { return (cfloat*)(p); }

// bf16 is carried as its raw 16 bits; widening to f32 is exact (the bits are the high half).
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }

// f32 -> bf16, round to nearest even (NaN stays a quiet NaN).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// two f32 -> two bf16 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Load K consecutive elements p[t0 .. t0+K) as f32; elements at t >= L read as 0.
// `vec` promises that p is 16-byte aligned at every multiple-of-8 (bf16) / 4 (f32) offset,
// and t0 is a multiple of K.
template <int K>
__device__ __forceinline__ void load_seg(const bf16_t* __restrict__ p, int64_t t0, int64_t L,
                                         bool vec, float (&out)[K]) {
  static_assert(K % 8 == 0, "K must be a multiple of 8");
  if (vec && t0 + K <= L) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p + t0);
#pragma unroll
    for (int i = 0; i < K / 8; ++i) {
      const u32x4 v = __builtin_nontemporal_load(q + i);
      out[8 * i + 0] = bf16_lo(v.x);
      out[8 * i + 1] = bf16_hi(v.x);
      out[8 * i + 2] = bf16_lo(v.y);
      out[8 * i + 3] = bf16_hi(v.y);
      out[8 * i + 4] = bf16_lo(v.z);
      out[8 * i + 5] = bf16_hi(v.z);
      out[8 * i + 6] = bf16_lo(v.w);
      out[8 * i + 7] = bf16_hi(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = (t0 + j < L) ? to_f32(p[t0 + j]) : 0.f;
  }
}

template <int K>
__device__ __forceinline__ void load_seg(const float* __restrict__ p, int64_t t0, int64_t L,
                                         bool vec, float (&out)[K]) {
  static_assert(K % 4 == 0, "K must be a multiple of 4");
  if (vec && t0 + K <= L) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p + t0);
#pragma unroll
    for (int i = 0; i < K / 4; ++i) {
      const f32x4 v = __builtin_nontemporal_load(q + i);
      out[4 * i + 0] = v.x;
      out[4 * i + 1] = v.y;
      out[4 * i + 2] = v.z;
      out[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = (t0 + j < L) ? p[t0 + j] : 0.f;
  }
}

// Store K consecutive values to p[t0 .. t0+K), skipping t >= L.
template <int K>
__device__ __forceinline__ void store_seg(float* __restrict__ p, int64_t t0, int64_t L, bool vec,
                                          const float (&v)[K]) {
  if (vec && t0 + K <= L) {
    f32x4* q = reinterpret_cast<f32x4*>(p + t0);
#pragma unroll
    for (int i = 0; i < K / 4; ++i) {
      f32x4 w = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      __builtin_nontemporal_store(w, q + i);
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (t0 + j < L) p[t0 + j] = v[j];
  }
}

template <int K>
__device__ __forceinline__ void store_seg(bf16_t* __restrict__ p, int64_t t0, int64_t L, bool vec,
                                          const float (&v)[K]) {
  if (vec && t0 + K <= L) {
    u32x4* q = reinterpret_cast<u32x4*>(p + t0);
#pragma unroll
    for (int i = 0; i < K / 8; ++i) {
      u32x4 w;
      w.x = pk_bf16(v[8 * i + 0], v[8 * i + 1]);
      w.y = pk_bf16(v[8 * i + 2], v[8 * i + 3]);
      w.z = pk_bf16(v[8 * i + 4], v[8 * i + 5]);
      w.w = pk_bf16(v[8 * i + 6], v[8 * i + 7]);
      __builtin_nontemporal_store(w, q + i);
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (t0 + j < L) p[t0 + j].bits = (uint16_t)f32_to_bf16_bits(v[j]);
  }
}

__device__ __forceinline__ void store_one(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_one(bf16_t* p, float v) { p->bits = (uint16_t)f32_to_bf16_bits(v); }

// softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|) so that it neither
// overflows for large x nor loses the small result for very negative x.
__device__ __forceinline__ float softplus_f32(float x) {
  return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z)
__device__ __forceinline__ float silu_f32(float z) { return z / (1.f + __expf(-z)); }

constexpr float kLn2 = 0.6931471805599453f;

// softplus(x) = max(x, 0) + log1p(e), e = exp(-|x|) in (0, 1], from the hardware exp2/log2.
// log1p(e) = log(1 + e) with the rounding error of 1 + e added back: that error is exactly
// e - ((1 + e) - 1) because 1 >= e (Fast2Sum), and adding it undivided by 1 + e changes the
// result by less than 2^-24 of it.  When e < 2^-24, 1 + e rounds to 1 and the result is e.
// Measured on gfx950 over x in [-30, 30]: within 1.8e-6 relative of the float64 value, the
// worst case being the rounding of the exp2 argument for large |x|.
__device__ __forceinline__ float softplus_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float u = 1.0f + e;
  const float corr = e - (u - 1.0f);
  return fmaxf(x, 0.f) + fmaf(__builtin_amdgcn_logf(u), kLn2, corr);
}

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (z -> -inf gives -0).
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// phi(x) = (exp(x) - 1) / x, phi(0) = 1: the zero-order-hold input coefficient is dt phi(dt A)
// = (exp(dt A) - 1) / A.  For |x| < 1/2 the Taylor polynomial sum_k x^k / (k + 1)! to degree 7
// (truncation below 2e-8 relative); elsewhere (e - 1) * rx with e = exp(x) and rx = 1 / x from
// the caller (there e - 1 is at least 0.39 in size, so its rounding stays near f32's).
__device__ __forceinline__ float zoh_phi(float x, float e, float rx) {
  float q = 1.f / 40320.f;
  q = fmaf(q, x, 1.f / 5040.f);
  q = fmaf(q, x, 1.f / 720.f);
  q = fmaf(q, x, 1.f / 120.f);
  q = fmaf(q, x, 1.f / 24.f);
  q = fmaf(q, x, 1.f / 6.f);
  q = fmaf(q, x, 0.5f);
  q = fmaf(q, x, 1.f);
  return fabsf(x) < 0.5f ? q : (e - 1.f) * rx;
}

constexpr float kLn2f = 0.6931471805599453f;

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// v with lane `lane` (wave-uniform) replaced by x
__device__ __forceinline__ float writelane_f(float x, int lane, float v) {
  return (int)(threadIdx.x & 63) == lane ? x : v;
}

// DPP move within a row of 16 lanes; lanes whose source is outside the row are fixed up
// by the caller (their value here is unspecified).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

}  // namespace ss
