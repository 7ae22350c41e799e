// Device helpers shared by the gfx950 kernels of libjepa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jepa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Exact (erf) GELU.
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752440f));
}

// Token id -> grid coordinates, T-major: id = t*gh*gw + h*gw + w.
struct Thw { int t, h, w; };
__device__ __forceinline__ Thw decode_id(int id, int gh, int gw) {
  const int hw = gh * gw;
  Thw r;
  r.t = id / hw;
  const int rem = id - r.t * hw;
  r.h = rem / gw;
  r.w = rem - r.h * gw;
  return r;
}

}  // namespace jepa
