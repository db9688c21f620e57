// Shared device helpers for the gfx950 MoE layer with zero-computation experts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moezc {

constexpr int kWave = 64;  // CDNA wavefront width

typedef uint16_t bf16_t;  // raw bf16 storage (upper half of an fp32)
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
// 16 bytes as a native vector (HIP's uint4 is a struct whose copies become
// memcpy through private memory, which keeps staging arrays out of registers)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// fp32 -> bf16, IEEE round to nearest, ties to even (a NaN stays a NaN):
// gfx950's v_cvt_pk_bf16_f32, which converts two values in one instruction
// (fp32 denormals are kept, so it rounds denormals like any other value).
__device__ inline bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// a to the low and b to the high half of one dword
__device__ inline uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// sigmoid(a) = 1 / (1 + e^-a) with the hardware exponential and reciprocal
// (v_exp_f32 on a * log2(e), v_rcp_f32: about one ulp each), and the SwiGLU
// product silu(a) * u = (a * sigmoid(a)) * u.  Saturates cleanly: e^-a = inf
// gives sigmoid 0.  Every bf16 SwiGLU epilogue uses this one definition, so
// the packed, row-major and FP8 paths round the same values.
__device__ inline float sigmoid_fast(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ inline float swiglu_fast(float a, float u) { return a * sigmoid_fast(a) * u; }

__device__ __host__ inline float bf16_to_f32(bf16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Element access for the two storage types of the layer.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static inline float load(const float* p, int64_t i) { return p[i]; }
  __device__ static inline void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static inline float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static inline void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Eight consecutive elements as fp32 (16-byte aligned for bf16, 32 for fp32).
__device__ inline void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ inline void load8(const bf16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ inline void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ inline void store8(bf16_t* p, const float (&v)[8]) {
  uint4 a;
  a.x = f32x2_to_bf16x2(v[0], v[1]);
  a.y = f32x2_to_bf16x2(v[2], v[3]);
  a.z = f32x2_to_bf16x2(v[4], v[5]);
  a.w = f32x2_to_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = a;
}

__device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moezc
