// Host-side launchers of the gfx950 kernels (internal to libjepa).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jepa {

// Geometry and convention of the 3-D RoPE for one call.
struct RopeSpec {
  int gt, gh, gw;    // token grid
  int layout;        // 0 tiled, 1 interleaved
  float theta;       // 10000
  int ref_grid;      // 0: integer positions, R > 1: interpolate h, w onto [0, R-1]
};

// Largest grid side the attention kernels keep RoPE tables for.
constexpr int kMaxGridSide = 64;

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C,
                            int M, int N, int K, int epi, int out_f32, hipStream_t s);
hipError_t launch_gemm_f32(const float* A, const float* W, const float* bias, float* C,
                           int M, int N, int K, int epi, hipStream_t s);
hipError_t launch_layernorm(const float* x, const float* w, const float* b, int M, int D,
                            float eps, void* out, int out_bf16, hipStream_t s);
hipError_t launch_rope3d(const void* x, void* y, int bf16, int B, int N, int n_head,
                         int head_dim, int64_t row_stride, const int32_t* ids,
                         const RopeSpec& r, hipStream_t s);
hipError_t launch_attention_bf16(const uint16_t* qkv, uint16_t* out, int B, int N, int n_head,
                                 int head_dim, const int32_t* ids, const RopeSpec& r,
                                 hipStream_t s);
hipError_t launch_attention_f32(const float* qkv, float* out, int B, int N, int n_head,
                                int head_dim, const int32_t* ids, const RopeSpec& r,
                                hipStream_t s);
// uint8 [B,T,H,W,3] -> normalised patch rows [B*N, 1536] (bf16 or fp32).
hipError_t launch_patchify(const uint8_t* clip, int B, int T, int H, int W, void* A, int bf16,
                           hipStream_t s);
// dst[i, :] = src[clamp(ids[i]), :] (fp32 -> bf16 or fp32), i < n.
hipError_t launch_gather_rows(const float* src, int n_src, int D, const int32_t* ids, int n,
                              void* dst, int bf16, hipStream_t s);
// dst[i, :] = vec[:] for i < n (fp32).
hipError_t launch_fill_rows(float* dst, const float* vec, int n, int D, hipStream_t s);
// dst[i] = a[i] + b[i] (fp32), i < n.
hipError_t launch_add_vec(float* dst, const float* a, const float* b, int n, hipStream_t s);

}  // namespace jepa
