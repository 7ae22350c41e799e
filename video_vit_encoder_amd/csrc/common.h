// Device helpers shared by the gfx950 kernels of libjepa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jepa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
  // one v_cvt_pk_bf16_f32 (round to nearest even)
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
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

// t, h and w (each below 256) one per byte, and the coordinate on axis a (0 t, 1 h, 2 w)
// taken back by one bit-field extract.  Picking a field of Thw by a lane-varying axis with
// selects can be lowered to an indexed load from private (scratch) memory instead.
__device__ __forceinline__ uint32_t thw_pack(const Thw& g) {
  return static_cast<uint32_t>(g.t) | (static_cast<uint32_t>(g.h) << 8) | (static_cast<uint32_t>(g.w) << 16);
}
__device__ __forceinline__ int thw_coord(uint32_t pk, int a) {
  return static_cast<int>(__builtin_amdgcn_ubfe(pk, 8 * a, 8));
}

// HBM/L2 -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane p of the wave
// writes LDS bytes [lds + 16p, lds + 16p + 16) from base + voff.  Issued through inline
// asm so that the kernel, not the compiler, decides how many of these may still be in
// flight at each barrier (s_waitcnt vmcnt).  lds must be wave-uniform.
// Store of one row's 32 bf16 columns of a 32 x 32 MFMA block.  Lane l (h = l / 32) holds
// the packed columns 8 gq + 4 h .. + 3 in pk[gq]; lanes l and l + 32 hold the same row.
// v_permlane32_swap trades the upper half of one word with the lower half of the next, so
// that each lane ends up with 8 contiguous columns: 16 p + 8 h .. + 7 for p = 0, 1, and
// two 16-byte stores per lane write the row in 32-byte pieces (four 8-byte stores
// otherwise).  Both lanes of a pair must be active.
__device__ __forceinline__ void store_row32_bf16(uint16_t* dst /* row, column 0 */, const u32x2 (&pk)[4], int h) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const auto w0 = __builtin_amdgcn_permlane32_swap(pk[2 * p][0], pk[2 * p + 1][0], false, false);
    const auto w1 = __builtin_amdgcn_permlane32_swap(pk[2 * p][1], pk[2 * p + 1][1], false, false);
    const u32x4 w = {w0[0], w1[0], w0[1], w1[1]};
    *reinterpret_cast<u32x4*>(dst + 16 * p + 8 * h) = w;
  }
}

__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  // both operands live in SGPRs: make their uniformity explicit
  // (readfirstlane returns int: widen through uint32_t, never by sign extension)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b & 0xFFFFFFFFu)));
  const uint64_t bs = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(voff), "s"(reinterpret_cast<const void*>(bs))
               : "memory");
}

// XOR swizzles of 16-byte chunks in LDS tiles read by ds_read_b128 down a column of
// chunks: the chunk c of row r sits at chunk c ^ key(r).  The LDS serves such a read 16
// lanes (16 consecutive rows) at a time from 64 four-byte banks, so 16 consecutive rows
// must land in 16 different 16-byte bank groups (and any 8 consecutive rows in 8).
// 128-byte rows (two rows per bank sweep): rows of one parity take 8 different keys.
__device__ __forceinline__ int lds_key128(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }
// 64-byte rows (four rows per bank sweep): rows 4 apart take 4 different keys.
__device__ __forceinline__ int lds_key64(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p)));
}

}  // namespace jepa
