// Stand-alone 3-D RoPE over head vectors ([Notes §4]).
//
// Head dim hd splits into d = 2*((hd/3)/2) dims per axis: [0,d) rotate with the frame
// position t, [d,2d) with h, [2d,3d) with w, the rest pass through.  Within an axis the
// adjacent pairs (x[2k], x[2k+1]) become (x0 cos a - x1 sin a, x1 cos b + x0 sin b):
// tiled ([Notes §4.1]) a = p*omega_{(2k) mod d/2}, b = p*omega_{(2k+1) mod d/2};
// interleaved ([Notes §4.2]) a = b = p*omega_k.  omega_k = theta^(-k/(d/2)).
// Interpolation ([Notes §4.3]): h' = h(R-1)/(gh-1), w' = w(R-1)/(gw-1), t unchanged.
//
// One wavefront per token: its 3*(d/2) distinct angles are formed in fp64 and their
// cos/sin rounded to fp32 once, then shared by every head of the token; each lane then
// rotates pairs, so a wave streams n_head*hd contiguous elements.  HBM-bound.
#include "common.h"
#include "kernels.h"

namespace jepa {

struct RopeOmega {
  double w[16];
};

// VEC: each lane moves 4 consecutive elements (two pairs) per access, 16 bytes (fp32) or 8
// (bf16), and issues the loads of up to 4 such chunks before rotating any, so that a wave
// keeps several kilobytes in flight (rows 16-byte aligned, head dim a multiple of 4);
// otherwise one pair per access.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256)
void rope3d_kernel(const void* __restrict__ xv, void* __restrict__ yv, long long n_tok, int N,
                   int n_head, int hd, long long row_stride, const int32_t* __restrict__ ids,
                   RopeSpec r, RopeOmega om) {
  __shared__ float tab[4][48][2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long tok = static_cast<long long>(blockIdx.x) * 4 + wave;
  const bool valid = tok < n_tok;
  const int d = 2 * ((hd / 3) / 2), m = d / 2;
  if (valid && lane < 3 * m) {
    const int n = static_cast<int>(tok % N);
    const int ntot = r.gt * r.gh * r.gw;
    int id = ids ? ids[n] : n;
    id = min(max(id, 0), ntot - 1);
    const Thw g = decode_id(id, r.gh, r.gw);
    const int a = lane / m, k = lane - a * m;
    double p;
    if (a == 0) {
      p = g.t;
    } else if (r.ref_grid > 0) {
      const int c = (a == 1) ? g.h : g.w, side = (a == 1) ? r.gh : r.gw;
      p = static_cast<double>(c) * (r.ref_grid - 1) / (side - 1);
    } else {
      p = (a == 1) ? g.h : g.w;
    }
    double sv, cv;
    sincos(p * om.w[k], &sv, &cv);
    tab[wave][lane][0] = static_cast<float>(cv);
    tab[wave][lane][1] = static_cast<float>(sv);
  }
  __syncthreads();
  if (!valid) return;
  const long long base = tok * row_stride;
  // rotation of the pair (x0, x1) at dims (j, j + 1) of a head, j even
  auto rot = [&](float& x0, float& x1, int j) __attribute__((always_inline)) {
    if (j < 3 * d) {
      const int a = j / d, jl = j - a * d;
      int i0, i1;
      if (r.layout == 0) {
        i0 = jl % m;
        i1 = (jl + 1) % m;
      } else {
        i0 = i1 = jl >> 1;
      }
      const float c0 = tab[wave][a * m + i0][0], s0 = tab[wave][a * m + i0][1];
      const float c1 = tab[wave][a * m + i1][0], s1 = tab[wave][a * m + i1][1];
      const float y0 = x0 * c0 - x1 * s0;
      const float y1 = x1 * c1 + x0 * s1;
      x0 = y0;
      x1 = y1;
    }
  };
  if constexpr (VEC) {
    // 4-element chunk c: elements 4c .. 4c + 3 of the token's row
    const int nch = n_head * hd / 4;
  auto load4 = [&](int c, float (&v)[4]) __attribute__((always_inline)) {
    const long long off = base + 4LL * c;
    if constexpr (BF16) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(xv) + off);
      v[0] = bf16_to_f32(static_cast<uint16_t>(w[0] & 0xFFFF));
      v[1] = bf16_to_f32(static_cast<uint16_t>(w[0] >> 16));
      v[2] = bf16_to_f32(static_cast<uint16_t>(w[1] & 0xFFFF));
      v[3] = bf16_to_f32(static_cast<uint16_t>(w[1] >> 16));
    } else {
      const f32x4 t = *reinterpret_cast<const f32x4*>(static_cast<const float*>(xv) + off);
      v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    }
  };
    for (int c0 = lane; c0 < nch; c0 += 4 * 64) {
      float v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + 64 * u < nch) load4(c0 + 64 * u, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u;
        if (c < nch) {
          const int e4 = 4 * c;
          const int j = e4 - (e4 / hd) * hd;
          rot(v[u][0], v[u][1], j);
          rot(v[u][2], v[u][3], j + 2);
          const long long off = base + 4LL * c;
          if constexpr (BF16) {
            u32x2 w;
            w[0] = pack_bf16x2(v[u][0], v[u][1]);
            w[1] = pack_bf16x2(v[u][2], v[u][3]);
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(yv) + off) = w;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(yv) + off) = f32x4{v[u][0], v[u][1], v[u][2], v[u][3]};
          }
        }
      }
    }
    return;
  }
  const int half = hd / 2;
  const int npairs = n_head * half;
  for (int pi = lane; pi < npairs; pi += 64) {
    const int e = pi / half;
    const int j = 2 * (pi - e * half);
    const long long off = base + static_cast<long long>(e) * hd + j;
    float x0, x1;
    if constexpr (BF16) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(xv) + off);
      x0 = bf16_to_f32(static_cast<uint16_t>(u & 0xFFFF));
      x1 = bf16_to_f32(static_cast<uint16_t>(u >> 16));
    } else {
      const float2 t = *reinterpret_cast<const float2*>(static_cast<const float*>(xv) + off);
      x0 = t.x;
      x1 = t.y;
    }
    float y0 = x0, y1 = x1;
    rot(y0, y1, j);
    if constexpr (BF16) {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(yv) + off) = pack_bf16x2(y0, y1);
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(yv) + off) = make_float2(y0, y1);
    }
  }
}

hipError_t launch_rope3d(const void* x, void* y, int bf16, int B, int N, int n_head,
                         int head_dim, int64_t row_stride, const int32_t* ids,
                         const RopeSpec& r, hipStream_t s) {
  const long long n_tok = static_cast<long long>(B) * N;
  if (n_tok <= 0) return hipSuccess;
  const int d = 2 * ((head_dim / 3) / 2), m = d / 2;
  RopeOmega om{};
  for (int k = 0; k < m && k < 16; ++k) om.w[k] = 1.0 / pow(static_cast<double>(r.theta), static_cast<double>(k) / m);
  const dim3 grid(static_cast<unsigned>((n_tok + 3) / 4));
  // 16-byte (fp32) or 8-byte (bf16) accesses need aligned rows and whole 4-element chunks
  const uintptr_t align = bf16 ? 8 : 16;
  const bool vec = head_dim % 4 == 0 && row_stride % 4 == 0 && reinterpret_cast<uintptr_t>(x) % align == 0 &&
                   reinterpret_cast<uintptr_t>(y) % align == 0;
  if (bf16) {
    if (vec) rope3d_kernel<true, true><<<grid, 256, 0, s>>>(x, y, n_tok, N, n_head, head_dim, row_stride, ids, r, om);
    else rope3d_kernel<true, false><<<grid, 256, 0, s>>>(x, y, n_tok, N, n_head, head_dim, row_stride, ids, r, om);
  } else {
    if (vec) rope3d_kernel<false, true><<<grid, 256, 0, s>>>(x, y, n_tok, N, n_head, head_dim, row_stride, ids, r, om);
    else rope3d_kernel<false, false><<<grid, 256, 0, s>>>(x, y, n_tok, N, n_head, head_dim, row_stride, ids, r, om);
  }
  return hipGetLastError();
}

// (cos, sin) table of one grid for the RoPE-by-table helpers of rope_tab.h: entry
// (axis, coord, k) = p_axis(coord) * omega_k with the angle formed in fp64 and its cos/sin
// rounded to fp32, as in rope3d_kernel.  Entries past the grid side or past d/2
// frequencies hold (1, 0).
__global__ __launch_bounds__(256)
void rope_table_kernel(float2* __restrict__ tab, RopeSpec r, RopeOmega om, int mf) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= kRopeTabEntries) return;
  const int k = e % kRopeMaxFreq, rest = e / kRopeMaxFreq;
  const int coord = rest % kMaxGridSide, axis = rest / kMaxGridSide;
  const int side = axis == 0 ? r.gt : (axis == 1 ? r.gh : r.gw);
  float2 v = make_float2(1.f, 0.f);
  if (k < mf && coord < side) {
    double p = coord;
    if (axis > 0 && r.ref_grid > 0) p = p * (r.ref_grid - 1) / (side - 1);
    double sv, cv;
    sincos(p * om.w[k], &sv, &cv);
    v = make_float2(static_cast<float>(cv), static_cast<float>(sv));
  }
  tab[e] = v;
}

hipError_t launch_rope_table(void* tab, const RopeSpec& r, int head_dim, hipStream_t s) {
  const int m = (2 * ((head_dim / 3) / 2)) / 2;
  if (m >= kRopeMaxFreq) return hipErrorInvalidValue;   // the last entry stays (1, 0)
  RopeOmega om{};
  for (int k = 0; k < m; ++k) om.w[k] = 1.0 / pow(static_cast<double>(r.theta), static_cast<double>(k) / m);
  rope_table_kernel<<<(kRopeTabEntries + 255) / 256, 256, 0, s>>>(static_cast<float2*>(tab), r, om, m);
  return hipGetLastError();
}

}  // namespace jepa
