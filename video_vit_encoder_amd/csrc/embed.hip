// Token-row producers: normalised tubelet rows for the patch-embedding GEMM, and the
// predictor's row gather / mask-token fill.
#include "common.h"
#include "kernels.h"

namespace jepa {

// Patch rows ([Notes §2]: feature order C, T, H, W of the TUBx16x16x3 tubelet, TUB = 2
// for clips and 1 for the 2.1 image path; [Notes §4]: tokens T-major).  Pixels are
// normalised in the fused float32 form (px - 255*mean)/(255*std) with the ImageNet
// statistics ([Parity "Preprocessing parity"]).  One thread per (token, dt, dy): it reads
// the 16 pixels x 3 channels of one image row segment (48 contiguous bytes of THWC input)
// and writes the three 16-wide feature runs c*TUB*256 + dt*256 + dy*16 + [0, 16).  With
// ids, output row b*K + k is the tubelet of token ids[b*K + k] of clip b (the context
// tokens of the masked forward, [HFport "Usage"]); ids outside [0, N) are clamped.
template <bool BF16, int TUB>
__global__ __launch_bounds__(256)
void patchify_kernel(const uint8_t* __restrict__ clip, int B, int T, int H, int W,
                     void* __restrict__ out, const int32_t* __restrict__ ids, int K) {
  constexpr int FEAT = 3 * TUB * 256, TPT = TUB * 16;   // features, threads per token
  const int gt = T / TUB, gh = H / 16, gw = W / 16;
  const int per_clip = gt * gh * gw;
  const int rows = ids ? K : per_clip;   // output rows per clip
  const long long ntok = static_cast<long long>(B) * rows;
  const long long gid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= ntok * TPT) return;
  const long long tokg = gid / TPT;
  const int sub = static_cast<int>(gid - tokg * TPT), dt = sub >> 4, dy = sub & 15;
  const int b = static_cast<int>(tokg / rows);
  int n = static_cast<int>(tokg - static_cast<long long>(b) * rows);
  if (ids) n = min(max(ids[tokg], 0), per_clip - 1);
  const int tp = n / (gh * gw), rem = n - tp * gh * gw, hp = rem / gw, wp = rem - hp * gw;
  const int t = TUB * tp + dt, y = 16 * hp + dy, x0 = 16 * wp;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(
      clip + ((((static_cast<long long>(b) * T + t) * H + y) * W + x0) * 3));
  uint32_t raw[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) raw[i] = src[i];
  const float mu255[3] = {static_cast<float>(255.0 * 0.485), static_cast<float>(255.0 * 0.456),
                          static_cast<float>(255.0 * 0.406)};
  const float sd255[3] = {static_cast<float>(255.0 * 0.229), static_cast<float>(255.0 * 0.224),
                          static_cast<float>(255.0 * 0.225)};
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    float v[16];
#pragma unroll
    for (int dx = 0; dx < 16; ++dx) {
      const int byte = dx * 3 + c;
      const float px = static_cast<float>((raw[byte >> 2] >> (8 * (byte & 3))) & 0xFF);
      v[dx] = (px - mu255[c]) / sd255[c];
    }
    const long long o = tokg * FEAT + c * (TUB * 256) + dt * 256 + dy * 16;
    if constexpr (BF16) {
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + o);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 p;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = pack_bf16x2(v[q * 8 + 2 * e], v[q * 8 + 2 * e + 1]);
        dst[q] = p;
      }
    } else {
      f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(out) + o);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    }
  }
}

hipError_t launch_patchify(const uint8_t* clip, int B, int T, int H, int W, void* A, int bf16,
                           hipStream_t s, const int32_t* ids, int K) {
  const long long rows = ids ? static_cast<long long>(K) : static_cast<long long>(T / 2) * (H / 16) * (W / 16);
  const long long threads = static_cast<long long>(B) * rows * 32;
  if (threads <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (bf16)
    patchify_kernel<true, 2><<<grid, 256, 0, s>>>(clip, B, T, H, W, A, ids, K);
  else
    patchify_kernel<false, 2><<<grid, 256, 0, s>>>(clip, B, T, H, W, A, ids, K);
  return hipGetLastError();
}

hipError_t launch_patchify_image(const uint8_t* img, int B, int H, int W, void* A, int bf16,
                                 hipStream_t s) {
  const long long threads = static_cast<long long>(B) * (H / 16) * (W / 16) * 16;
  if (threads <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (bf16)
    patchify_kernel<true, 1><<<grid, 256, 0, s>>>(img, B, 1, H, W, A, nullptr, 0);
  else
    patchify_kernel<false, 1><<<grid, 256, 0, s>>>(img, B, 1, H, W, A, nullptr, 0);
  return hipGetLastError();
}

template <bool BF16>
__global__ __launch_bounds__(256)
void gather_rows_kernel(const float* __restrict__ src, int n_src, int D,
                        const int32_t* __restrict__ ids, int n, void* __restrict__ dst) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const int r = min(max(ids[i], 0), n_src - 1);
  const float* s = src + static_cast<size_t>(r) * D;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    if constexpr (BF16)
      static_cast<uint16_t*>(dst)[static_cast<size_t>(i) * D + c] = f32_to_bf16(s[c]);
    else
      static_cast<float*>(dst)[static_cast<size_t>(i) * D + c] = s[c];
  }
}

hipError_t launch_gather_rows(const float* src, int n_src, int D, const int32_t* ids, int n,
                              void* dst, int bf16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (bf16)
    gather_rows_kernel<true><<<n, 256, 0, s>>>(src, n_src, D, ids, n, dst);
  else
    gather_rows_kernel<false><<<n, 256, 0, s>>>(src, n_src, D, ids, n, dst);
  return hipGetLastError();
}

__global__ __launch_bounds__(256)
void fill_rows_kernel(float* __restrict__ dst, const float* __restrict__ vec, int n, int D) {
  const int i = blockIdx.x;
  if (i >= n) return;
  for (int c = threadIdx.x; c < D; c += blockDim.x) dst[static_cast<size_t>(i) * D + c] = vec[c];
}

hipError_t launch_fill_rows(float* dst, const float* vec, int n, int D, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_rows_kernel<<<n, 256, 0, s>>>(dst, vec, n, D);
  return hipGetLastError();
}

__global__ void add_vec_kernel(float* __restrict__ dst, const float* __restrict__ a,
                               const float* __restrict__ b, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = a[i] + b[i];
}

hipError_t launch_add_vec(float* dst, const float* a, const float* b, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  add_vec_kernel<<<(n + 255) / 256, 256, 0, s>>>(dst, a, b, n);
  return hipGetLastError();
}

}  // namespace jepa
