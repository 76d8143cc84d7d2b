// Shared device helpers for the gfx950 low-rank block kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is stored as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// float -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

// Element traits: 16 bytes of operand per lane and per MFMA fragment.
template <typename T>
struct Elem;

template <>
struct Elem<bf16_t> {
  static constexpr int VEC = 8;     // elements per 16 bytes
  static constexpr int FRAG_K = 32; // k covered by one 16-byte fragment (1 MFMA)
  __device__ static float load(const bf16_t* p) { return __uint_as_float(uint32_t(p->bits) << 16); }
  __device__ static void store(bf16_t* p, float v) { p->bits = (uint16_t)f32_to_bf16_bits(v); }
};

template <>
struct Elem<float> {
  static constexpr int VEC = 4;
  static constexpr int FRAG_K = 16;  // 4 MFMAs of k = 4
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};

// Unpack a 16-byte vector into floats.
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& v, float* out);

template <>
__device__ __forceinline__ void unpack16<bf16_t>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16_lo(v[i]);
    out[2 * i + 1] = bf16_hi(v[i]);
  }
}

template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}

template <typename T>
__device__ __forceinline__ u32x4 pack16(const float* in);

template <>
__device__ __forceinline__ u32x4 pack16<bf16_t>(const float* in) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
  return v;
}

template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* in) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(in[i]);
  return v;
}

// Logistic sigmoid. The bf16 path uses the hardware exp2 and reciprocal
// approximations (v_exp_f32, v_rcp_f32: relative errors near 1e-6 and one
// ulp, far below bf16 rounding; a correctly rounded reciprocal costs ten
// instructions where v_rcp_f32 costs one); the fp32 path uses the accurate
// library exp and a true division. exp(-z) = inf gives 0, as it should.
template <typename T>
__device__ __forceinline__ float sigmoid_f(float z);

template <>
__device__ __forceinline__ float sigmoid_f<bf16_t>(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

template <>
__device__ __forceinline__ float sigmoid_f<float>(float z) {
  return 1.0f / (1.0f + expf(-z));
}

}  // namespace lr
