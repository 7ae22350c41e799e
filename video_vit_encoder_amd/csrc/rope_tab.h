// 3-D RoPE applied from a per-axis cos/sin table, shared by the QKV projection epilogue
// and the attention input preparation of libjepa.
//
// [Notes §4]: head dim hd splits into d = 2*((hd/3)/2) dims per axis ([0,d) follow the
// frame position t, [d,2d) h, [2d,3d) w, the rest pass through).  The adjacent pair
// (x[j], x[j+1]) of an axis becomes (x0 cos a - x1 sin a, x1 cos b + x0 sin b) with
// a = p*omega_{idx(j)}, b = p*omega_{idx(j+1)}; tiled ([Notes §4.1]) idx(j) = j mod d/2,
// interleaved ([Notes §4.2]) idx(j) = j div 2 for j counted within the axis.
//
// The table holds (cos, sin) of p_axis(coord) * omega_k for every axis, grid coordinate
// and frequency: tab[(axis * kMaxGridSide + coord) * kRopeMaxFreq + k]; it is built once
// per forward (launch_rope_table), with the angles formed in fp64.
#pragma once

#include "common.h"
#include "kernels.h"

namespace jepa {

// Where a token row's RoPE position comes from.
struct RopeArgs {
  const float2* tab;    // table above
  const int32_t* ids;   // grid ids of the N tokens of a clip (NULL: 0..N-1), clamped
  int N;                // tokens per clip: row r is token r % N of clip r / N
  int layout;           // 0 tiled, 1 interleaved
  int ntot, gh, gw;     // grid size gt*gh*gw and its last two sides
  int ids_stride;       // ids of clip b start at ids + b * ids_stride (0: shared by all)
  int lead;             // without ids: rows n < lead of a clip take grid position (0, 0, 0),
                        // where every rotation is the identity, and row n >= lead is token
                        // n - lead (a leading CLS row)
};

// Grid coordinates of the token of row r.
__device__ __forceinline__ Thw rope_token(int r, const RopeArgs& ra, int* clip) {
  const int b = r / ra.N, n = r - b * ra.N;
  *clip = b;
  int id = ra.ids ? ra.ids[b * ra.ids_stride + n] : n - ra.lead;
  id = min(max(id, 0), ra.ntot - 1);
  return decode_id(id, ra.gh, ra.gw);
}

// Table coordinates of the pair at head dims (j0, j0 + 1), j0 even: whether it rotates,
// its axis and the frequency indices of its two dims.  A pass-through pair points at the
// last entry of an axis row, which the table holds as (cos, sin) = (1, 0) (frequencies
// stop below kRopeMaxFreq - 1), so reading it leaves the pair unchanged: readers may skip
// the rot test.
struct RopePairIdx {
  int rot, axis, i0, i1;
};
template <int HD>
__device__ __forceinline__ RopePairIdx rope_pair_idx(int j0, int layout) {
  constexpr int D3 = 2 * ((HD / 3) / 2), MF = D3 / 2;
  static_assert(MF < kRopeMaxFreq, "identity entry");
  RopePairIdx r;
  r.rot = j0 < 3 * D3;
  r.axis = (j0 >= D3) + (j0 >= 2 * D3);   // pass-through pairs land on axis 2
  // by compares rather than division: a rotated pair has jl in [0, D3 - 2], jl even
  const int jl = j0 - r.axis * D3;
  const int t0 = jl >= MF ? jl - MF : jl;               // jl mod MF
  const int t1 = jl + 1 >= MF ? jl + 1 - MF : jl + 1;   // (jl + 1) mod MF
  r.i0 = !r.rot ? kRopeMaxFreq - 1 : (layout == 0 ? t0 : jl >> 1);
  r.i1 = !r.rot ? kRopeMaxFreq - 1 : (layout == 0 ? t1 : jl >> 1);
  return r;
}

// Rotate (x0, x1) by the table rows of stride ts (coordinates per axis).
__device__ __forceinline__ void rope_apply(float& x0, float& x1, const RopePairIdx& p, const Thw& g,
                                           const float2* tab, int ts) {
  if (!p.rot) return;
  const int c = thw_coord(thw_pack(g), p.axis);
  const float2* row = tab + (p.axis * ts + c) * kRopeMaxFreq;
  const float2 cs0 = row[p.i0], cs1 = row[p.i1];
  const float y0 = x0 * cs0.x - x1 * cs0.y;
  const float y1 = x1 * cs1.x + x0 * cs1.y;
  x0 = y0;
  x1 = y1;
}

// Rotate the pair (x0, x1) at head dims (j0, j0 + 1), j0 even, of a token at g, from the
// full table.
template <int HD>
__device__ __forceinline__ void rope_pair(float& x0, float& x1, int j0, const Thw& g, int layout,
                                          const float2* __restrict__ tab) {
  rope_apply(x0, x1, rope_pair_idx<HD>(j0, layout), g, tab, kMaxGridSide);
}

// Position of key n inside a 16-key group of the transposed V layout: quads 1 and 2 of the
// group trade places (bits 2 and 3 of n swap), which is the key order the attention
// kernel's probability fragments come out in.  The map is its own inverse.
__device__ __forceinline__ int vt_pos(int n) {
  return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
}

}  // namespace jepa
