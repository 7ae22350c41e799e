// Multi-head softmax attention with the 3-D RoPE applied to q and k as they are loaded.
//
// What is computed ([Notes §4]): for each clip and head, softmax(R(q) R(k)^T / sqrt(hd)) v
// over every token of the clip (no mask), with R the 3-D RoPE of the token's (t, h, w)
// position: d = 2*((hd/3)/2) dims per axis, adjacent pairs rotated, tiled ([Notes §4.1])
// or interleaved ([Notes §4.2]) frequency layout, optional interpolation ([Notes §4.3]).
// RoPE acts on q and k only, before the 1/sqrt(hd) scaling.
//
// bf16 kernel (gfx950 MFMA, fp32 softmax and accumulation):
//   * a workgroup owns 128 query rows of one (clip, head); each of its 4 wavefronts owns
//     32 of them and keeps them, rotated and pre-scaled by log2(e)/sqrt(hd), as bf16
//     MFMA operands in registers;
//   * keys/values stream through LDS 64 at a time; K is rotated on its way from HBM to
//     LDS (angles from per-axis cos/sin tables built in LDS at kernel start), V is
//     written transposed so it can serve as the A operand of the second product;
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16): in the 32x32 accumulator a lane holds 16
//     keys of one query, so the running max and sum are per lane plus one exchange with
//     the lane 32 away;
//   * O^T += V^T P^T: P^T leaves the first product already in the B-operand layout of
//     the second (the key <-> register-slot map is the same on both sides), and O^T keeps
//     one query per lane, so the online-softmax rescale is per lane too.
// fp32 kernel: one query per thread, plain FMA, for the fp32 encoder path.
#include "common.h"
#include "kernels.h"

namespace jepa {

struct RopeFreq {
  float w[16];
};

// cos/sin of every (axis, coordinate, frequency) the clip's grid can need, in LDS:
// tab[(axis*kMaxGridSide + coord) * MF + k] = (cos, sin) of p_axis(coord) * omega_k.
template <int MF>
__device__ void build_rope_tables(float2* tab, const RopeSpec& r, const RopeFreq& fr) {
  // stage the frequencies through LDS with constant indices (no private copy of `fr`)
  __shared__ float om[16];
#pragma unroll
  for (int k = 0; k < MF; ++k)
    if (threadIdx.x == k) om[k] = fr.w[k];
  __syncthreads();
  const int rows = r.gt + r.gh + r.gw;
  for (int e = threadIdx.x; e < rows * MF; e += blockDim.x) {
    const int row = e / MF, k = e - row * MF;
    int axis, coord;
    if (row < r.gt) {
      axis = 0; coord = row;
    } else if (row < r.gt + r.gh) {
      axis = 1; coord = row - r.gt;
    } else {
      axis = 2; coord = row - r.gt - r.gh;
    }
    float p = static_cast<float>(coord);
    if (axis > 0 && r.ref_grid > 0) {
      const int side = axis == 1 ? r.gh : r.gw;
      p = p * static_cast<float>(r.ref_grid - 1) / static_cast<float>(side - 1);
    }
    float sv, cv;
    sincosf(p * om[k], &sv, &cv);
    tab[(axis * kMaxGridSide + coord) * MF + k] = make_float2(cv, sv);
  }
}

// Rotate the NE consecutive dims [j0, j0 + NE) (j0 even) of one head vector held in x.
template <int HD, int NE>
__device__ __forceinline__ void rope_chunk(float* x, int j0, const Thw& g, int layout,
                                           const float2* tab) {
  constexpr int D3 = 2 * ((HD / 3) / 2);
  constexpr int MF = D3 / 2;
#pragma unroll
  for (int e = 0; e < NE; e += 2) {
    const int j = j0 + e;
    if (j < 3 * D3) {
      const int a = j / D3, jl = j - a * D3;
      const int coord = a == 0 ? g.t : (a == 1 ? g.h : g.w);
      int i0, i1;
      if (layout == 0) {
        i0 = jl % MF;
        i1 = (jl + 1) % MF;
      } else {
        i0 = i1 = jl >> 1;
      }
      const float2 cs0 = tab[(a * kMaxGridSide + coord) * MF + i0];
      const float2 cs1 = tab[(a * kMaxGridSide + coord) * MF + i1];
      const float x0 = x[e], x1 = x[e + 1];
      x[e] = x0 * cs0.x - x1 * cs0.y;
      x[e + 1] = x1 * cs1.x + x0 * cs1.y;
    }
  }
}

__device__ __forceinline__ int token_id(const int32_t* ids, int n, int ntot) {
  const int id = ids ? ids[n] : n;
  return min(max(id, 0), ntot - 1);
}

// ---------------------------------------------------------------- bf16 / MFMA

// Unsigned division by a runtime constant d >= 1 for n < 2^31 (round-up multiplier:
// q = (umulhi(n, mul) + n) >> sh with sh = ceil(log2 d), mul = floor(2^32 (2^sh - d) / d) + 1).
struct FastDiv {
  uint32_t d, mul, sh;
};

static FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0, 0};
  while ((1ull << f.sh) < d) ++f.sh;
  f.mul = static_cast<uint32_t>(((1ull << 32) * ((1ull << f.sh) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.mul) + n) >> f.sh;
}

// Grid coordinates of a (clamped) token id.
__device__ __forceinline__ Thw decode_fast(int id, const FastDiv& dhw, const FastDiv& dw) {
  Thw g;
  g.t = static_cast<int>(fdiv(static_cast<uint32_t>(id), dhw));
  const int rem = id - g.t * static_cast<int>(dhw.d);
  g.h = static_cast<int>(fdiv(static_cast<uint32_t>(rem), dw));
  g.w = rem - g.h * static_cast<int>(dw.d);
  return g;
}

// Table code of head dim j: (axis << 24) | (axis*kMaxGridSide*MF + frequency index), or
// -1 for a pass-through dim.  tiled: frequency j mod d/2 within the axis ([Notes §4.1]);
// interleaved: frequency (j within the axis) / 2 ([Notes §4.2]).
template <int HD>
__device__ __forceinline__ int rope_code(int j, int layout) {
  constexpr int D3 = 2 * ((HD / 3) / 2);
  constexpr int MF = D3 / 2;
  if (j >= 3 * D3) return -1;
  const int a = j / D3, jl = j - a * D3;
  return (a << 24) | (a * kMaxGridSide * MF + (layout == 0 ? jl % MF : jl >> 1));
}

// Rotation of one 8-dim chunk of a head vector held in x[8]; code[e] from rope_code.
// Both dims of a pair always share the axis (d is even).
template <int MF>
__device__ __forceinline__ void rope8(float* x, const int* code, const Thw& g, const float2* tab) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    if (code[e] < 0) continue;
    const int ax = code[e] >> 24;
    const int c = ax == 0 ? g.t : (ax == 1 ? g.h : g.w);
    const float2 cs0 = tab[(code[e] & 0xFFFFFF) + c * MF];
    const float2 cs1 = tab[(code[e + 1] & 0xFFFFFF) + c * MF];
    const float x0 = x[e], x1 = x[e + 1];
    x[e] = x0 * cs0.x - x1 * cs0.y;
    x[e + 1] = x1 * cs1.x + x0 * cs1.y;
  }
}

// Flash attention, bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 softmax and accumulators.
//   * a workgroup of 4 wavefronts owns 256 queries of one (clip, head); each wave keeps
//     two groups of 32, rotated once and pre-scaled by log2(e)/sqrt(hd), as bf16 MFMA B
//     operands in registers.  256 queries share every key tile, so rotating K on its way
//     into LDS costs little next to the MFMAs;
//   * keys and values stream through LDS 64 at a time, double-buffered: the next tile is
//     fetched into registers while the current one is consumed, then rotated (K) or
//     transposed (V) into the other buffer; one barrier per tile;
//   * S^T = K Q^T puts 16 keys of one query in each lane, so the online max and sum are
//     per lane plus one exchange with the lane 32 away;
//   * P^T leaves that MFMA already in the B-operand layout of O^T += V^T P^T, whose slot
//     s of k-step ks is key 16ks + 8(s/4) + 4(l/32) + s%4.  V^T is stored in LDS with the
//     keys of each 16-group in that order (quads 1 and 2 swapped), so every A operand is
//     one 16-byte LDS read.
template <int HD>
__global__ __launch_bounds__(256, 2)
void attn_bf16_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ out, int N,
                      int H, const int32_t* __restrict__ ids, RopeSpec r, RopeFreq fr,
                      float qscale, FastDiv dhw, FastDiv dw, int nqb) {
  constexpr int D3 = 2 * ((HD / 3) / 2);
  constexpr int MF = D3 / 2;
  constexpr int BQ = 256, BKV = 64, NT = 256;
  constexpr int CH = HD / 8;                 // 16-byte chunks per head row
  constexpr int KS = HD / 16;                // MFMA k-steps over the head dim
  constexpr int DT = HD / 32;                // 32-dim blocks of the output
  constexpr int KCH = BKV * CH / NT;         // K chunks per thread per tile (2 or 1)
  constexpr int VCH = (BKV / 2) * CH;        // V (2 keys x 8 dims) units per tile
  constexpr int VP = BKV + 8;                // padded V^T row (keys), 144 B for 64 keys
  static_assert(BKV * CH % NT == 0, "K tile mapping");

  __shared__ float2 tab[3 * kMaxGridSide * MF];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BKV * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][HD * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  // Work-groups are dealt to the 8 XCDs round-robin; renumber them so that the query
  // blocks of one (clip, head), which read the same keys and values, share an XCD's L2.
  int wg = blockIdx.x;
  if ((gridDim.x & 7) == 0) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
  const int qblk = wg % nqb, bh = wg / nqb;
  const int head = bh % H, b = bh / H;
  const int D = H * HD, ld = 3 * D;
  const int ntot = r.gt * r.gh * r.gw;
  const uint16_t* base = qkv + static_cast<size_t>(b) * N * ld + head * HD;

  build_rope_tables<MF>(tab, r, fr);

  // per-thread constants of the K chunks this thread rotates: chunk c = tid % CH
  const int kc = tid % CH;
  int kcode[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) kcode[e] = rope_code<HD>(kc * 8 + e, r.layout);
  __syncthreads();

  // ---- queries: two groups of 32 per wave, rotated, scaled, bf16 B operands
  bf16x8 qf[2][KS];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int q = qblk * BQ + wave * 64 + g * 32 + l32;
    const int qr = min(q, N - 1);
    int id = ids ? ids[qr] : qr;
    id = min(max(id, 0), ntot - 1);
    const Thw gq = decode_fast(id, dhw, dw);
    const uint16_t* src = base + static_cast<size_t>(qr) * ld;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int c = kk * 2 + hh;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src + c * 8);
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_to_f32(static_cast<uint16_t>(raw[e] & 0xFFFF));
        x[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(raw[e] >> 16));
      }
      int qcode[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qcode[e] = rope_code<HD>(c * 8 + e, r.layout);
      rope8<MF>(x, qcode, gq, tab);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[g][kk][e] = static_cast<__bf16>(x[e] * qscale);
    }
  }

  // ---- tile staging: global -> registers -> (rotate / transpose) -> LDS
  u32x4 kraw[KCH];
  int kid[KCH];
  u32x4 vraw0, vraw1;
  const int vkp = tid % (BKV / 2), vc = tid / (BKV / 2);   // V: key pair, dim chunk
  auto fetch = [&](int kb) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int key = (tid + i * NT) / CH;
      const int kr = min(kb + key, N - 1);
      int id = ids ? ids[kr] : kr;
      kid[i] = min(max(id, 0), ntot - 1);
      kraw[i] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(kr) * ld + D + kc * 8);
    }
    if (tid < VCH) {
      const int k0 = min(kb + 2 * vkp, N - 1), k1 = min(kb + 2 * vkp + 1, N - 1);
      vraw0 = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(k0) * ld + 2 * D + vc * 8);
      vraw1 = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(k1) * ld + 2 * D + vc * 8);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int key = (tid + i * NT) / CH;
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_to_f32(static_cast<uint16_t>(kraw[i][e] & 0xFFFF));
        x[2 * e + 1] = bf16_to_f32(static_cast<uint16_t>(kraw[i][e] >> 16));
      }
      rope8<MF>(x, kcode, decode_fast(kid[i], dhw, dw), tab);
      u32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      const int sw = (HD == 64) ? (kc ^ (key & 7)) : (kc ^ ((key >> 1) & 3));
      *reinterpret_cast<u32x4*>(&Ks[buf][key * HD + sw * 8]) = p;
    }
    if (tid < VCH) {
      // keys 2vkp, 2vkp+1 go to the pair slot of the quad-swapped order
      const int k2 = 2 * vkp;
      const int quad = (k2 >> 2) & 3;
      const int pos = (k2 & ~15) | (((quad == 1) ? 2 : (quad == 2) ? 1 : quad) << 2) | (k2 & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (vraw0[e] & 0xFFFFu) | (vraw1[e] << 16);
        const uint32_t hi = (vraw0[e] >> 16) | (vraw1[e] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(&Vt[buf][(vc * 8 + 2 * e) * VP + pos]) = lo;
        *reinterpret_cast<uint32_t*>(&Vt[buf][(vc * 8 + 2 * e + 1) * VP + pos]) = hi;
      }
    }
  };

  f32x16 o[2][DT];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[g][dt][i] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  const int ntiles = (N + BKV - 1) / BKV;
  fetch(0);
  stage(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int kb = t * BKV, buf = t & 1;
    if (t + 1 < ntiles) fetch(kb + BKV);
    const uint16_t* Kb = Ks[buf];
    const uint16_t* Vb = Vt[buf];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      // S^T = K Q^T for keys [kb, kb + 64): two 32-key blocks
      f32x16 sc[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[t2][i] = 0.f;
        const int key = t2 * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int c = kk * 2 + hh;
          const int sw = (HD == 64) ? (c ^ (key & 7)) : (c ^ ((key >> 1) & 3));
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + key * HD + sw * 8);
          sc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[g][kk], sc[t2], 0, 0, 0);
        }
      }
      // element i of sc[t2] is key kb + 32 t2 + 8(i/4) + 4 hh + i%4 of this lane's query
      if (kb + BKV > N) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb + t2 * 32 + 8 * (i >> 2) + 4 * hh + (i & 3) >= N) sc[t2][i] = -INFINITY;
      }
      float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(sc[0][i], sc[1][i]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[g], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
      m_run[g] = m_new;
      float ls = 0.f;
      bf16x8 pf[4];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(sc[t2][i] - m_new);
          ls += pv;
          pf[t2 * 2 + (i >> 3)][i & 7] = static_cast<__bf16>(pv);
        }
      l_run[g] = l_run[g] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[g][dt][i] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dim = dt * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vb + dim * VP + ks * 16 + hh * 8);
          o[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[g][dt], 0, 0, 0);
        }
      }
      // keep the two query groups apart: their score blocks are never live together
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t + 1 < ntiles) stage(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: element i of o[g][dt] is dim 32 dt + 8(i/4) + 4 hh + i%4
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int q = qblk * BQ + wave * 64 + g * 32 + l32;
    const float inv = 1.0f / (l_run[g] + __shfl_xor(l_run[g], 32));
    if (q < N) {
      uint16_t* dst = out + (static_cast<size_t>(b) * N + q) * D + head * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 pk;
          pk[0] = pack_bf16x2(o[g][dt][4 * g4] * inv, o[g][dt][4 * g4 + 1] * inv);
          pk[1] = pack_bf16x2(o[g][dt][4 * g4 + 2] * inv, o[g][dt][4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(dst + dt * 32 + 8 * g4 + 4 * hh) = pk;
        }
    }
  }
}

static RopeFreq make_freq(int head_dim, float theta) {
  RopeFreq f{};
  const int m = (2 * ((head_dim / 3) / 2)) / 2;
  for (int k = 0; k < m && k < 16; ++k)
    f.w[k] = static_cast<float>(1.0 / pow(static_cast<double>(theta), static_cast<double>(k) / m));
  return f;
}

hipError_t launch_attention_bf16(const uint16_t* qkv, uint16_t* out, int B, int N, int n_head,
                                 int head_dim, const int32_t* ids, const RopeSpec& r,
                                 hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  const RopeFreq fr = make_freq(head_dim, r.theta);
  const float qscale = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(head_dim)));
  const FastDiv dhw = make_fastdiv(static_cast<uint32_t>(r.gh * r.gw));
  const FastDiv dw = make_fastdiv(static_cast<uint32_t>(r.gw));
  const int nqb = (N + 255) / 256;
  const dim3 grid(nqb * n_head * B);
  if (head_dim == 64)
    attn_bf16_kernel<64><<<grid, 256, 0, s>>>(qkv, out, N, n_head, ids, r, fr, qscale, dhw, dw, nqb);
  else if (head_dim == 32)
    attn_bf16_kernel<32><<<grid, 256, 0, s>>>(qkv, out, N, n_head, ids, r, fr, qscale, dhw, dw, nqb);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 / FMA

template <int HD>
__global__ __launch_bounds__(64)
void attn_f32_kernel(const float* __restrict__ qkv, float* __restrict__ out, int N, int H,
                     const int32_t* __restrict__ ids, RopeSpec r, RopeFreq fr, float scale) {
  constexpr int D3 = 2 * ((HD / 3) / 2);
  constexpr int MF = D3 / 2;
  constexpr int BKV = 64;
  __shared__ float2 tab[3 * kMaxGridSide * MF];
  __shared__ float Ks[BKV][HD];
  __shared__ float Vs[BKV][HD];
  const int tid = threadIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int D = H * HD, ld = 3 * D;
  const int ntot = r.gt * r.gh * r.gw;
  const float* base = qkv + static_cast<size_t>(b) * N * ld + head * HD;
  build_rope_tables<MF>(tab, r, fr);
  __syncthreads();

  const int q = blockIdx.x * 64 + tid;
  const int qr = min(q, N - 1);
  float qv[HD], ov[HD];
  {
    const Thw g = decode_id(token_id(ids, qr, ntot), r.gh, r.gw);
#pragma unroll
    for (int j = 0; j < HD; ++j) qv[j] = base[static_cast<size_t>(qr) * ld + j];
    rope_chunk<HD, HD>(qv, 0, g, r.layout, tab);
#pragma unroll
    for (int j = 0; j < HD; ++j) {
      qv[j] *= scale;
      ov[j] = 0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int kb = 0; kb < N; kb += BKV) {
    __syncthreads();
    {
      const int kr = min(kb + tid, N - 1);
      const Thw g = decode_id(token_id(ids, kr, ntot), r.gh, r.gw);
      float kv[HD];
#pragma unroll
      for (int j = 0; j < HD; ++j) kv[j] = base[static_cast<size_t>(kr) * ld + D + j];
      rope_chunk<HD, HD>(kv, 0, g, r.layout, tab);
#pragma unroll
      for (int j = 0; j < HD; ++j) {
        Ks[tid][j] = kv[j];
        Vs[tid][j] = base[static_cast<size_t>(kr) * ld + 2 * D + j];
      }
    }
    __syncthreads();
    const int nk = min(BKV, N - kb);
    for (int k = 0; k < nk; ++k) {
      float sc = 0.f;
#pragma unroll
      for (int j = 0; j < HD; ++j) sc = fmaf(qv[j], Ks[k][j], sc);
      if (sc > m_run) {
        const float a = expf(m_run - sc);
        l_run *= a;
#pragma unroll
        for (int j = 0; j < HD; ++j) ov[j] *= a;
        m_run = sc;
      }
      const float p = expf(sc - m_run);
      l_run += p;
#pragma unroll
      for (int j = 0; j < HD; ++j) ov[j] = fmaf(p, Vs[k][j], ov[j]);
    }
  }
  if (q < N) {
    const float inv = 1.0f / l_run;
    float* dst = out + (static_cast<size_t>(b) * N + q) * D + head * HD;
#pragma unroll
    for (int j = 0; j < HD; ++j) dst[j] = ov[j] * inv;
  }
}

hipError_t launch_attention_f32(const float* qkv, float* out, int B, int N, int n_head,
                                int head_dim, const int32_t* ids, const RopeSpec& r,
                                hipStream_t s) {
  if (B <= 0 || N <= 0) return hipSuccess;
  const RopeFreq fr = make_freq(head_dim, r.theta);
  const float scale = static_cast<float>(1.0 / sqrt(static_cast<double>(head_dim)));
  const dim3 grid((N + 63) / 64, n_head, B);
  if (head_dim == 64)
    attn_f32_kernel<64><<<grid, 64, 0, s>>>(qkv, out, N, n_head, ids, r, fr, scale);
  else if (head_dim == 32)
    attn_f32_kernel<32><<<grid, 64, 0, s>>>(qkv, out, N, n_head, ids, r, fr, scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jepa
