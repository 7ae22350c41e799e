// LayerNorm over rows of an fp32 [M, D] matrix, one wavefront (or half of one) per row.
//
// [Notes §1]: eps = 1e-6.  The variance is centred (mean first, then the mean of the
// squared deviations), as the CPU backend of [Parity "Parity on a GPU"] does; both
// passes run over the row held in registers, so HBM sees one read and one write.
// Lane l of a row's LANES lanes owns the vector chunks l, l+LANES, l+2 LANES, ... of VEC
// floats each, so every access of those lanes is contiguous.  LANES is 64 (VEC = 4 when D is
// a multiple of 256, else 2 or 1), or 32 where that gives 16-byte chunks instead of 8-byte
// ones (D = 384, 640, 1408): two rows per wavefront, and one reduction step fewer.
// The final norm of a forward runs in place (out == x), so x and out may alias: neither
// is declared __restrict__.
#include "common.h"
#include "kernels.h"

namespace jepa {

template <int VPT, int VEC, int LANES, bool OUT_BF16>
__global__ __launch_bounds__(256)
void layernorm_kernel(const float* x, const float* __restrict__ w,
                      const float* __restrict__ b, int M, float eps, void* out) {
  static_assert(LANES == 64 || LANES == 32, "a row takes a wavefront or half of one");
  constexpr int D = VPT * LANES;
  constexpr int NV = VPT / VEC;
  const int lane = threadIdx.x & (LANES - 1);
  const int row = blockIdx.x * (256 / LANES) + threadIdx.x / LANES;
  // (a half wave that returns here leaves the other half's reductions intact: they
  // exchange only within their own LANES lanes)
  if (row >= M) return;
  const float* xr = x + static_cast<size_t>(row) * D;
  float v[VPT];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * LANES + lane) * VEC;
    if constexpr (VEC == 4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(xr + c);
      v[j * 4 + 0] = t[0]; v[j * 4 + 1] = t[1]; v[j * 4 + 2] = t[2]; v[j * 4 + 3] = t[3];
    } else if constexpr (VEC == 2) {
      const float2 t = *reinterpret_cast<const float2*>(xr + c);
      v[j * 2 + 0] = t.x; v[j * 2 + 1] = t.y;
    } else {
      v[j] = xr[c];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) s += v[i];
#pragma unroll
  for (int o = LANES / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  const float mean = s * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    v[i] -= mean;
    q += v[i] * v[i];
  }
#pragma unroll
  for (int o = LANES / 2; o > 0; o >>= 1) q += __shfl_xor(q, o);
  const float rstd = 1.0f / sqrtf(q * (1.0f / D) + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int c = (j * LANES + lane) * VEC;
    float y[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = v[j * VEC + e] * rstd * w[c + e] + b[c + e];
    if constexpr (OUT_BF16) {
      uint16_t* o = static_cast<uint16_t*>(out) + static_cast<size_t>(row) * D + c;
      if constexpr (VEC == 4) {
        u32x2 p;
        p[0] = pack_bf16x2(y[0], y[1]);
        p[1] = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<u32x2*>(o) = p;
      } else if constexpr (VEC == 2) {
        *reinterpret_cast<uint32_t*>(o) = pack_bf16x2(y[0], y[1]);
      } else {
        o[0] = f32_to_bf16(y[0]);
      }
    } else {
      float* o = static_cast<float*>(out) + static_cast<size_t>(row) * D + c;
      if constexpr (VEC == 4) {
        *reinterpret_cast<f32x4*>(o) = f32x4{y[0], y[1], y[2], y[3]};
      } else if constexpr (VEC == 2) {
        *reinterpret_cast<float2*>(o) = make_float2(y[0], y[1]);
      } else {
        o[0] = y[0];
      }
    }
  }
}

template <int VPT64>
static hipError_t ln_dispatch(const float* x, const float* w, const float* b, int M, float eps,
                              void* out, int out_bf16, hipStream_t s) {
  // D = 64 VPT64: half-wave rows where that turns 8-byte chunks into 16-byte ones
  constexpr int LANES = (VPT64 % 4 == 2) ? 32 : 64;
  constexpr int VPT = VPT64 * 64 / LANES;
  constexpr int VEC = (VPT % 4 == 0) ? 4 : ((VPT % 2 == 0) ? 2 : 1);
  constexpr int RPB = 256 / LANES;   // rows per workgroup
  const dim3 grid((M + RPB - 1) / RPB);
  if (out_bf16)
    layernorm_kernel<VPT, VEC, LANES, true><<<grid, 256, 0, s>>>(x, w, b, M, eps, out);
  else
    layernorm_kernel<VPT, VEC, LANES, false><<<grid, 256, 0, s>>>(x, w, b, M, eps, out);
  return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, const float* w, const float* b, int M, int D,
                            float eps, void* out, int out_bf16, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!layernorm_width_ok(D)) return hipErrorInvalidValue;
  switch (D / 64) {
    case 1: return ln_dispatch<1>(x, w, b, M, eps, out, out_bf16, s);
    case 2: return ln_dispatch<2>(x, w, b, M, eps, out, out_bf16, s);
    case 3: return ln_dispatch<3>(x, w, b, M, eps, out, out_bf16, s);
    case 4: return ln_dispatch<4>(x, w, b, M, eps, out, out_bf16, s);
    case 5: return ln_dispatch<5>(x, w, b, M, eps, out, out_bf16, s);
    case 6: return ln_dispatch<6>(x, w, b, M, eps, out, out_bf16, s);
    case 8: return ln_dispatch<8>(x, w, b, M, eps, out, out_bf16, s);
    case 10: return ln_dispatch<10>(x, w, b, M, eps, out, out_bf16, s);
    case 12: return ln_dispatch<12>(x, w, b, M, eps, out, out_bf16, s);
    case 16: return ln_dispatch<16>(x, w, b, M, eps, out, out_bf16, s);
    case 20: return ln_dispatch<20>(x, w, b, M, eps, out, out_bf16, s);
    case 22: return ln_dispatch<22>(x, w, b, M, eps, out, out_bf16, s);
    case 24: return ln_dispatch<24>(x, w, b, M, eps, out, out_bf16, s);
    case 32: return ln_dispatch<32>(x, w, b, M, eps, out, out_bf16, s);
    case 40: return ln_dispatch<40>(x, w, b, M, eps, out, out_bf16, s);
    case 48: return ln_dispatch<48>(x, w, b, M, eps, out, out_bf16, s);
    case 64: return ln_dispatch<64>(x, w, b, M, eps, out, out_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace jepa

namespace jepa {

// Mean over the N tokens of each clip ([Card] "Run it", --pool mean): x fp32 [B, N, D] ->
// out fp32 [B, D].  One workgroup of 1024 threads per (64 columns, clip): 16 row groups
// (n mod 16) accumulate in fp64, added in group order, so the result does not depend on
// the launch.
__global__ __launch_bounds__(1024)
void mean_pool_kernel(const float* __restrict__ x, int N, int D, float* __restrict__ out) {
  __shared__ double part[16][64];
  const int tid = threadIdx.x, g = tid >> 6, c = tid & 63;
  const int col = blockIdx.x * 64 + c, b = blockIdx.y;
  double acc = 0.0;
  if (col < D) {
    const float* xb = x + static_cast<size_t>(b) * N * D + col;
    for (int n = g; n < N; n += 16) acc += static_cast<double>(xb[static_cast<size_t>(n) * D]);
  }
  part[g][c] = acc;
  __syncthreads();
  if (g == 0 && col < D) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i][c];
    out[static_cast<size_t>(b) * D + col] = static_cast<float>(s / N);
  }
}

hipError_t launch_mean_pool(const float* x, int B, int N, int D, float* out, hipStream_t s) {
  if (B <= 0 || D <= 0) return hipSuccess;
  if (N <= 0) return hipErrorInvalidValue;
  const dim3 grid((D + 63) / 64, B);
  mean_pool_kernel<<<grid, 1024, 0, s>>>(x, N, D, out);
  return hipGetLastError();
}

}  // namespace jepa
