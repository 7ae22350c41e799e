// Linear layers C = epilogue(A W^T + bias) for libjepa.
//
// Weights are stored [out, in] row-major ([Notes §2] key map), so both operands are
// contiguous along K and map straight onto the MFMA operand layout.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, fp32 accumulation.  A workgroup owns a BM x BN
// output tile; its waves own WM x WN sub-tiles made of 32x32 MFMA blocks.  K advances
// 64 at a time: the next K-slab is fetched global -> registers while the current one is
// consumed from LDS.  LDS rows are 128 B (64 bf16); the 16-byte chunk c of row r lives
// at chunk c ^ (r & 7), so the 8 lanes that read one chunk column of 8 consecutive rows
// hit 8 different bank groups.
//
// fp32 path: a plain 64x64-tile FMA kernel (no MFMA), used by the fp32 encoder.
#include "common.h"
#include "kernels.h"

namespace jepa {

enum { EPI_STORE = 0, EPI_GELU = 1, EPI_RESIDUAL = 2 };

template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
void gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                      const float* __restrict__ bias, void* __restrict__ Cv, int M, int N, int K) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int BK = 64;
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int A_CH = BM * BK / 8 / NT;
  constexpr int B_CH = BN * BK / 8 / NT;
  static_assert(A_CH * NT * 8 == BM * BK && B_CH * NT * 8 == BN * BK, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  u32x4 ra[A_CH], rb[B_CH];
#define JEPA_GEMM_GLOAD(k0)                                                                    \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                         \
      const int id = tid + i * NT, row = id >> 3, c = id & 7;                                  \
      const int gm = min(m0 + row, M - 1);                                                     \
      ra[i] = *reinterpret_cast<const u32x4*>(A + static_cast<size_t>(gm) * K + (k0) + c * 8); \
    }                                                                                          \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                         \
      const int id = tid + i * NT, row = id >> 3, c = id & 7;                                  \
      rb[i] = *reinterpret_cast<const u32x4*>(W + static_cast<size_t>(n0 + row) * K + (k0) + c * 8); \
    }                                                                                          \
  } while (0)
#define JEPA_GEMM_SSTORE()                                                                     \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                         \
      const int id = tid + i * NT, row = id >> 3, c = id & 7;                                  \
      *reinterpret_cast<u32x4*>(As + row * BK + ((c ^ (row & 7)) << 3)) = ra[i];               \
    }                                                                                          \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                         \
      const int id = tid + i * NT, row = id >> 3, c = id & 7;                                  \
      *reinterpret_cast<u32x4*>(Bs + row * BK + ((c ^ (row & 7)) << 3)) = rb[i];               \
    }                                                                                          \
  } while (0)

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / BK;
  JEPA_GEMM_GLOAD(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    JEPA_GEMM_SSTORE();
    __syncthreads();
    if (kt + 1 < KT) JEPA_GEMM_GLOAD((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8 af[TI], bfr[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(As + row * BK + ((ch ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int row = wn * WN + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + row * BK + ((ch ^ (row & 7)) << 3));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
#undef JEPA_GEMM_GLOAD
#undef JEPA_GEMM_SSTORE

  // Epilogue.  32x32 accumulator layout: lane l, element r holds
  // row 8*(r/4) + 4*(l/32) + (r%4), column l%32 of the block.
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int col = n0 + wn * WN + j * 32 + (lane & 31);
    const float bv = bias ? bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) {
          float v = acc[i][j][r] + bv;
          const size_t off = static_cast<size_t>(row) * N + col;
          if (EPI == EPI_GELU) v = gelu_erf(v);
          if (EPI == EPI_RESIDUAL) {
            float* C = static_cast<float*>(Cv);
            C[off] += v;
          } else if (OUT_F32) {
            static_cast<float*>(Cv)[off] = v;
          } else {
            static_cast<uint16_t*>(Cv)[off] = f32_to_bf16(v);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
static hipError_t dispatch_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C,
                                int M, int N, int K, int epi, int out_f32, hipStream_t s) {
  const dim3 grid(((M + BM - 1) / BM) * (N / BN));
  const dim3 block((BM / WM) * (BN / WN) * 64);
  if (epi == EPI_RESIDUAL) {
    gemm_bf16_kernel<BM, BN, WM, WN, EPI_RESIDUAL, true><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K);
  } else if (epi == EPI_GELU) {
    if (out_f32)
      gemm_bf16_kernel<BM, BN, WM, WN, EPI_GELU, true><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K);
    else
      gemm_bf16_kernel<BM, BN, WM, WN, EPI_GELU, false><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K);
  } else {
    if (out_f32)
      gemm_bf16_kernel<BM, BN, WM, WN, EPI_STORE, true><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K);
    else
      gemm_bf16_kernel<BM, BN, WM, WN, EPI_STORE, false><<<grid, block, 0, s>>>(A, W, bias, C, M, N, K);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C,
                            int M, int N, int K, int epi, int out_f32, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  return dispatch_bf16<256, 128, 128, 64>(A, W, bias, C, M, N, K, epi, out_f32, s);
}

// ---------------------------------------------------------------- fp32 path

template <int EPI>
__global__ __launch_bounds__(256)
void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                     const float* __restrict__ bias, float* __restrict__ C, int M, int N, int K) {
  constexpr int T = 64, BK = 16;
  __shared__ float As[BK][T + 1];
  __shared__ float Bs[BK][T + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int e = threadIdx.x; e < T * BK; e += 256) {
      const int r = e / BK, c = e % BK;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + c;
      As[c][r] = (gm < M && gk < K) ? A[static_cast<size_t>(gm) * K + gk] : 0.f;
      Bs[c][r] = (gn < N && gk < K) ? W[static_cast<size_t>(gn) * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < BK; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      float v = acc[i][j] + (bias ? bias[col] : 0.f);
      const size_t off = static_cast<size_t>(row) * N + col;
      if (EPI == EPI_GELU) v = gelu_erf(v);
      if (EPI == EPI_RESIDUAL) C[off] += v;
      else C[off] = v;
    }
  }
}

hipError_t launch_gemm_f32(const float* A, const float* W, const float* bias, float* C,
                           int M, int N, int K, int epi, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const dim3 grid((N + 63) / 64, (M + 63) / 64);
  if (epi == EPI_RESIDUAL)
    gemm_f32_kernel<EPI_RESIDUAL><<<grid, 256, 0, s>>>(A, W, bias, C, M, N, K);
  else if (epi == EPI_GELU)
    gemm_f32_kernel<EPI_GELU><<<grid, 256, 0, s>>>(A, W, bias, C, M, N, K);
  else
    gemm_f32_kernel<EPI_STORE><<<grid, 256, 0, s>>>(A, W, bias, C, M, N, K);
  return hipGetLastError();
}

}  // namespace jepa
