// Multi-head softmax attention with the 3-D RoPE on q and k.
//
// What is computed ([Notes §4]): for each clip and head, softmax(R(q) R(k)^T / sqrt(hd)) v
// over every token of the clip (no mask), with R the 3-D RoPE of the token's (t, h, w)
// position: d = 2*((hd/3)/2) dims per axis, adjacent pairs rotated, tiled ([Notes §4.1])
// or interleaved ([Notes §4.2]) frequency layout, optional interpolation ([Notes §4.3]).
// RoPE acts on q and k only, before the 1/sqrt(hd) scaling.
//
// bf16 path: the rotation happens once per token, where q and k are produced (the QKV
// projection's epilogue in the forwards, qkv_prepare_kernel for the stand-alone entry
// point), which also folds log2(e)/sqrt(hd) into q and writes v transposed; the flash
// kernel (attn_fwd_kernel) then only streams tiles and runs the two products and the
// online softmax.
// fp32 path: one query per thread, plain FMA, RoPE applied as q and k are loaded (tables
// in LDS), for the fp32 encoder.
#include "common.h"
#include "kernels.h"
#include "rope_tab.h"

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
      const int coord = thw_coord(thw_pack(g), a);
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

// grid id of row n: ids[n], else n - lead (rows below lead clamp to id 0, position
// (0, 0, 0), where the rotation is the identity)
__device__ __forceinline__ int token_id(const int32_t* ids, int n, int ntot, int lead) {
  const int id = ids ? ids[n] : n - lead;
  return min(max(id, 0), ntot - 1);
}

// ---------------------------------------------------------------- bf16 / MFMA

// max(x[l], x[l ^ 32]) in every lane l: v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second, so the two results hold, lane by lane,
// the value of the lane and of its partner in the other half (no LDS round trip).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int kMaxSplit = 8;   // most key pieces per query block

// Flash attention, bf16 MFMA (v_mfma_f32_32x32x16_bf16), fp32 softmax and accumulators,
// on inputs prepared once per token (the QKV projection's epilogue or qkv_prepare_kernel):
// q rotated and scaled by log2(e)/sqrt(hd), k rotated, v transposed per (clip, head) with
// the keys of each 16-group in vt_pos order.
//   * a workgroup of 8 wavefronts owns 256 NG queries of one (clip, head); each wave keeps
//     NG groups of 32 as bf16 MFMA B operands in registers, and every K or V fragment it
//     reads from LDS feeds the MFMAs of all its groups (NG = 2, except NG = 1 for clips
//     short enough that 512-query blocks would leave most compute units idle);
//   * the waves form two halves of four (one wave of each half per SIMD) that take turns
//     between workgroup barriers: in one phase half A runs the matrix products of a key
//     tile (P V of the previous tile, then S = K Q of this one) while half B runs the
//     softmax of the tile it multiplied in the phase before (max, exp2, bf16 rounding,
//     row sums), and the other way round in the next phase, so each SIMD's matrix core
//     and vector ALU are busy at the same time (the matrix phase runs at raised wave
//     priority, so its MFMAs issue ahead of the other wave's vector instructions);
//   * 64-key tiles of K and V^T stream through a ring of 4 LDS buffers, filled by
//     global_load_lds_dwordx4 two tiles ahead (no register staging, no VALU); tile t is
//     read in phases 2t .. 2t + 3, so its buffer is refilled with tile t + 4 from phase
//     2t + 4 on;
//   * S^T = K Q^T puts 16 keys of one query in each lane, so the row max and sum are per
//     lane plus one exchange with the lane 32 away;
//   * P^T leaves that MFMA already in the B-operand layout of O^T += V^T P^T: slot s of
//     k-step ks holds key 16ks + 8(s/4) + 4(l/32) + s%4, i.e. position vt_pos of the
//     16-group, the order V^T is stored in, so every A operand is one 16-byte LDS read;
//   * the score accumulators start at minus the running max, so the MFMA hands back
//     scores relative to it (log2 units); the running max moves only when a tile's max
//     exceeds it by more than 8: between moves the probabilities stay in (0, 256] and
//     neither the scores nor the output accumulators are touched before exp2.  The first
//     tile sets the max exactly, so the running sum never underflows;
//   * the row sum adds the fp32 probabilities with plain adds in four chains: beside the
//     other wave's MFMAs, v_dot2_f32_bf16 on the rounded pairs (one instruction per pair)
//     took longer than two adds.
// BC: the block-causal mask of [Parity] "LeVJEPA ViT-L/16 — CLS, block-causal attention,
// tubelet 1".  Rows [0, n_cls) are CLS rows that see every key; row r >= n_cls is a patch
// token of temporal slot s = (r - n_cls) / slot and sees the keys [n_cls, lim(r)), lim(r) =
// n_cls + (s + 1) * slot capped at N: no CLS key, every key of its own and the earlier
// slots.  The query blocks take the patch rows in order and the CLS rows after them,
// aligned so that the last block ends on the last row; a block then needs only the key
// tiles below the limit of its last row (the last block, which holds the CLS rows and the
// last slot, needs them all), so the work follows the mask's density.  Scores outside
// [lo, lim) become -inf in the tiles that straddle a limit.  The heaviest blocks start
// first.
template <int HD, bool BC, int NG, bool SPLIT>
__global__ __launch_bounds__(512, 1)
void attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int ld,
                     const uint16_t* __restrict__ vt, int Ns, uint16_t* __restrict__ out, int N,
                     int H, int nqb, int n_cls, int slot, int nsplit, int tps,
                     float* __restrict__ part) {
  constexpr int NW = 8, BQ = NW * 32 * NG, BKV = 64, S = 4;
  constexpr int KS = HD / 16;                   // MFMA k-steps over the head dim
  constexpr int DT = HD / 32;                   // 32-dim blocks of the output
  constexpr int KROW = HD * 2;                  // LDS bytes per K row (128 / 64)
  constexpr int K_BYTES = BKV * KROW, V_BYTES = HD * BKV * 2;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int K_RPI = 1024 / KROW;            // K rows per 1 KB DMA instruction
  constexpr int K_CPR = KROW / 16;              // 16-byte chunks per K row
  constexpr int K_INS = K_BYTES / 1024, V_INS = V_BYTES / 1024;  // DMA instructions per tile
  constexpr int LOADS = (K_INS + V_INS) / NW;   // per wave and tile
  constexpr float TAU = 8.0f;
  constexpr float kTwoTau = 256.0f;   // 2^TAU
  static_assert(LOADS * NW == K_INS + V_INS, "DMA split");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2;                   // 0: A, 1: B
  const int h = lane >> 5, l32 = lane & 31;
  // Work-groups are dealt to the 8 XCDs round-robin; renumber them so that the query
  // blocks of one (clip, head), which read the same keys and values, share an XCD's L2.
  int wg = blockIdx.x;
  if ((gridDim.x & 7) == 0) wg = (wg & 7) * (gridDim.x >> 3) + (wg >> 3);
  // SPLIT: the key pieces of one query block are neighbours in this order (the same XCD)
  const int piece = SPLIT ? wg % nsplit : 0;
  if (SPLIT) wg /= nsplit;
  int qblk = wg % nqb, bh = wg / nqb;
  if (BC) {
    // heaviest blocks first: on the XCD it lands on (blockIdx.x % 8), workgroup i takes
    // rank i / per of one of that XCD's `per` (clip, head) pairs, the latest query block
    // first, so every XCD starts its longest blocks first and keeps each pair's blocks in
    // its own L2
    const int HB = gridDim.x / nqb;
    if ((HB & 7) == 0) {
      const int per = HB >> 3, i = blockIdx.x >> 3;
      qblk = nqb - 1 - i / per;
      bh = (blockIdx.x & 7) * per + i % per;
    } else {
      qblk = nqb - 1 - static_cast<int>(blockIdx.x) / HB;
      bh = blockIdx.x % HB;
    }
  }
  const int head = bh % H, b = bh / H;
  const int D = H * HD;

  // query j of the block order and its row: j >= N - n_cls are the CLS rows (BC)
  const int jbase = (BC ? N - nqb * BQ : 0) + qblk * BQ;
  auto row_of = [&](int j) { return j < N - n_cls ? j + n_cls : j - (N - n_cls); };
  auto limit_of = [&](int r) { return r < n_cls ? N : min(N, n_cls + ((r - n_cls) / slot + 1) * slot); };
  int qrow[NG], lo[NG], lim[NG];
  bool qok[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int j = jbase + wave * (32 * NG) + g * 32 + l32;
    if (BC) {
      qok[g] = j >= 0;
      qrow[g] = row_of(max(j, 0));
      lo[g] = qrow[g] < n_cls ? 0 : n_cls;
      lim[g] = limit_of(qrow[g]);
    } else {
      qok[g] = j < N;
      qrow[g] = min(j, N - 1);
    }
  }

  // K rows are 128 B (hd 64) or 64 B (hd 32), V^T rows 128 B; chunk c of row r sits at
  // c ^ kkey(r) (K) or c ^ lds_key128(r) (V^T)
  auto kkey = [](int r) { return HD == 64 ? lds_key128(r) : lds_key64(r); };
  const int krow_l = lane / K_CPR, kslot_l = lane % K_CPR;
  const int vrow_l = lane >> 3, vslot_l = lane & 7;
  const uint32_t sbase = lds_addr(smem);
  const uint16_t* kbase = k + static_cast<size_t>(b) * N * ld + head * HD;
  const uint16_t* vbase = vt + static_cast<size_t>(b * H + head) * HD * Ns;
  int ntiles = (N + BKV - 1) / BKV;
  if (BC) {
    const int jl = jbase + BQ - 1;   // the block's last query, in [0, N)
    if (jl < N - n_cls) ntiles = (limit_of(row_of(jl)) + BKV - 1) / BKV;
  }
  // SPLIT: this piece's key tiles, tps from tile t0 on; below, t counts the piece's tiles
  // and key0 + t BKV is the first key of tile t
  const int t0 = SPLIT ? piece * tps : 0;
  if (SPLIT) ntiles = min(tps, ntiles - t0);
  const int key0 = t0 * BKV;

  // Tile t into buffer t % S: instruction i = qd*NW + wave of the tile fills 1 KB of K
  // (i < K_INS) or of V^T.  K rows past N repeat row N - 1 (their scores are masked); V^T
  // rows read 64 keys from position 64t on (the caller's buffer holds them: see
  // launch_attention_fwd); positions of keys past N are zeroed in LDS below.
  auto issue = [&](int t) {
    const uint32_t st = sbase + (t % S) * STAGE;
    const int kb = key0 + t * BKV;
#pragma unroll
    for (int qd = 0; qd < LOADS; ++qd) {
      const int ins = qd * NW + wave;
      if (ins < K_INS) {
        const int r = ins * K_RPI + krow_l;   // row in the tile
        const int key = min(kb + r, N - 1);
        dma16(kbase, static_cast<uint32_t>(key) * ld * 2 + ((kslot_l ^ kkey(r)) << 4), st + ins * 1024);
      } else {
        const int vi = ins - K_INS;
        const int dim = vi * 8 + vrow_l;
        dma16(vbase, (static_cast<uint32_t>(dim) * Ns + kb) * 2 + ((vslot_l ^ lds_key128(dim)) << 4),
              st + K_BYTES + vi * 1024);
      }
    }
  };

  // ---- queries: NG groups of 32 per wave, B operands (dims 16kk + 8h .. +8)
  bf16x8 qf[NG][KS];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint16_t* src = q + (static_cast<size_t>(b) * N + qrow[g]) * ld + head * HD;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[g][kk] = *reinterpret_cast<const bf16x8*>(src + (2 * kk + h) * 8);
  }
  // Let the query loads land here, before any tile DMA is issued: the compiler cannot see
  // the DMAs, so a wait it placed at the first use of a fragment inside the loop would
  // also wait for the tiles in flight.  The empty asm takes the fragments as outputs, so
  // nothing after it depends on the loads.
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(qf[g][kk]));

  f32x16 o[NG][DT];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[g][dt][i] = 0.f;
  float m_run[NG], l_run[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) m_run[g] = l_run[g] = 0.f;
  // Scores of the tile this wave multiplied last; after its softmax the same registers hold
  // the tile's bf16 probabilities (words 0-3 and 8-11 of each block, see probs below) until
  // the next P V reads them.
  f32x16 sc[NG][2];
  // -m_run[g] in all 16 slots: the C operand of each score chain's first MFMA, rewritten
  // only when the running max moves
  f32x16 negm[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[g][i] = 0.f;

  int issued = 0;
  for (; issued < 2 && issued < ntiles; ++issued) issue(issued);

  // Barrier k opens phase k.  Before an even barrier, tile k/2 (first read in phase k)
  // must have landed for every wave: at most the one tile issued after it may still be in
  // flight.  After it, tile k/2 + 2 goes into the buffer of tile k/2 - 2 (read for the last
  // time in phase k - 1), and a ragged last tile gets its V^T positions of keys past N
  // zeroed (P is 0 there, and the words read past the clip's keys need not be finite;
  // V^T of tile t is first read in phase 2t + 2, two barriers later).
  auto sync = [&](int kph) __attribute__((always_inline)) {
    const int t = kph >> 1;
    if ((kph & 1) == 0 && t < ntiles) {
      if (issued - 1 - t >= 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if ((kph & 1) == 0) {
      if (issued < ntiles) {
        issue(issued);
        ++issued;
      }
      if (t == ntiles - 1 && key0 + t * BKV + BKV > N) {
        unsigned char* st = smem + (t % S) * STAGE;
        const int kb = key0 + t * BKV;
        for (int e = tid; e < HD * BKV; e += NW * 64) {
          const int dim = e / BKV, pos = e - dim * BKV;
          if (kb + vt_pos(pos) >= N)
            *reinterpret_cast<uint16_t*>(st + K_BYTES + dim * 128 + (((pos >> 3) ^ lds_key128(dim)) << 4) + (pos & 7) * 2) = 0;
        }
      }
    }
  };
  // probabilities of k-step ks of group g: words 8 (ks % 2) .. + 3 of sc[g][ks / 2]
  auto pfrag = [&](int g, int ks) __attribute__((always_inline)) {
    const int b = 8 * (ks & 1);
    const u32x4 w = {__float_as_uint(sc[g][ks >> 1][b]), __float_as_uint(sc[g][ks >> 1][b + 1]),
                     __float_as_uint(sc[g][ks >> 1][b + 2]), __float_as_uint(sc[g][ks >> 1][b + 3])};
    return __builtin_bit_cast(bf16x8, w);
  };
  // O^T += V^T P^T for tile t (probabilities in sc)
  auto mma_pv = [&](int t) __attribute__((always_inline)) {
    const unsigned char* st = smem + (t % S) * STAGE;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int dim = dt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + K_BYTES + dim * 128 + (((2 * ks + h) ^ lds_key128(dim)) << 4));
#pragma unroll
        for (int g = 0; g < NG; ++g)
          o[g][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pfrag(g, ks), o[g][dt], 0, 0, 0);
      }
    }
  };
  // S^T = K Q^T for tile t: element i of sc[g][t2] is key 64t + 32 t2 + 8(i/4) + 4h + i%4
  // of query l32 of group g; the accumulators start at -m_run, so the product comes out
  // relative to the running max
  auto mma_qk = [&](int t) __attribute__((always_inline)) {
    const unsigned char* st = smem + (t % S) * STAGE;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int r = t2 * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + r * KROW + (((2 * kk + h) ^ kkey(r)) << 4));
#pragma unroll
        for (int g = 0; g < NG; ++g)
          sc[g][t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[g][kk], kk == 0 ? negm[g] : sc[g][t2], 0, 0, 0);
      }
    }
  };
  // Softmax of tile t's scores, the bf16 probabilities written over them, updating m_run,
  // l_run (and o on a rescale).
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int kb = key0 + t * BKV;
    auto mask = [&]() __attribute__((always_inline)) {
    if (BC) {
      bool straddle = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) straddle = straddle || kb + BKV > lim[g] || kb < lo[g];
      if (__ballot(straddle) != 0) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          // key k = kb + 4h + c (c the element's constant offset) is outside [lo, lim) iff
          // k - lo or lim - 1 - k is negative: the sign of their OR picks -inf or +inf as
          // the bound of a minimum, with no lane mask
          const int a = kb + 4 * h - lo[g], bb = lim[g] - 1 - kb - 4 * h;
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int c = t2 * 32 + 8 * (i >> 2) + (i & 3);
              const uint32_t sgn = static_cast<uint32_t>((a + c) | (bb - c)) & 0x80000000u;
              sc[g][t2][i] = fminf(sc[g][t2][i], __uint_as_float(sgn | 0x7f800000u));
            }
        }
      }
    } else if (kb + BKV > N) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (kb + t2 * 32 + 8 * (i >> 2) + 4 * h + (i & 3) >= N) sc[g][t2][i] = -INFINITY;
    }
    };
    mask();
    // P = exp2(S - m) rounded to bf16, with each lane's sum of its 32 fp32 values per group
    // in four chains of adds.
    float lt[NG][4];
    auto lsum = [&](int g) __attribute__((always_inline)) { return (lt[g][0] + lt[g][1]) + (lt[g][2] + lt[g][3]); };
    auto probs = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int c = 0; c < 4; ++c) lt[g][c] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // slot s of k-step ks = element 8 (ks % 2) + s of sc[g][ks / 2]; each pair is
          // converted as one bf16x2 word
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 8 * (ks & 1) + 2 * e;
            const f32x2 pp = {__builtin_amdgcn_exp2f(sc[g][ks >> 1][i]),
                              __builtin_amdgcn_exp2f(sc[g][ks >> 1][i + 1])};
            const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
            lt[g][2 * (e & 1)] += pp[0];
            lt[g][2 * (e & 1) + 1] += pp[1];
            w[e] = __builtin_bit_cast(uint32_t, pb);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[g][ks >> 1][8 * (ks & 1) + e] = __uint_as_float(w[e]);
        }
      }
    };
    // The running max moves only when a score of the tile exceeds it by more than TAU (a
    // factor 2^TAU), and the first tile sets it to the tile's exact max.  After the first
    // tile the probabilities are formed against the running max straight away: a lane
    // whose 32 values sum to at most 2^TAU has none above 2^TAU, so the max (a serial
    // chain in front of every exp2) is taken only when some lane's sum exceeds that, and
    // then exactly as for the first tile, with the probabilities formed again.
    bool exact = t == 0;
    if (!exact) {
      probs();
      bool big = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) big = big || lsum(g) > kTwoTau;
      exact = __ballot(big) != 0;
      if (exact) {
        // the probabilities replaced the scores: form them again (tile t's K stays in its
        // ring buffer until phase 2t + 4 refills it)
        mma_qk(t);
        mask();
      }
    }
    if (exact) {
      // Row max of the tile relative to the running max, one wave-uniform decision for
      // all the wave's groups.
      float mxs[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // a linear chain of 3-input maxima (v_max3_f32): half an op per score
        float mx = fmaxf(sc[g][0][0], sc[g][1][0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(fmaxf(mx, sc[g][0][i]), sc[g][1][i]);
        mxs[g] = max_halves(mx);
      }
      bool moved = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) moved = moved || mxs[g] > TAU;
      if (t == 0 || __ballot(moved) != 0) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float d = t == 0 ? mxs[g] : (mxs[g] > TAU ? mxs[g] : 0.f);
          const float alpha = t == 0 ? 0.f : __builtin_amdgcn_exp2f(-d);
          m_run[g] += d;
          l_run[g] *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) negm[g][i] = -m_run[g];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[g][dt][i] *= alpha;
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[g][t2][i] -= d;
        }
      }
      probs();
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) l_run[g] += lsum(g);
  };

  // Matrix phase of tile t: P V of tile t - 1 and K Q of tile t at raised wave priority.
  // The SIMD's arbiter otherwise favours the older waves (half A), so half B's MFMAs
  // would wait behind half A's softmax; with the matrix wave first, the other wave's
  // vector instructions fill the MFMA shadow.
  auto mma_phase = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (t > 0) mma_pv(t - 1);
    mma_qk(t);
    if (t > 0) {
      // Scheduling groups: each K or V^T fragment read feeds NG MFMAs; issue the reads LA
      // steps ahead of their MFMAs instead of one, so that their LDS latency passes behind
      // the matrix work (left alone, the scheduler waited on each read one step later).
      // (two steps for the block-causal kernel, whose range registers leave less room)
      constexpr int NRD = DT * 4 + 2 * KS, LA = BC ? 2 : 3;
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int i = 0; i < NRD - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NG, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NG * LA, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Phase k: half A multiplies tile k/2 for even k (P V of tile k/2 - 1, then K Q of tile
  // k/2) and runs the softmax of tile (k-1)/2 for odd k; half B does the same one phase
  // later.  Both halves pass the same 2 ntiles + 2 barriers.
  if (half == 0) {
    sync(0);
    mma_phase(0);
    sync(1);
    softmax(0);
    for (int t = 1; t < ntiles; ++t) {
      sync(2 * t);
      mma_phase(t);
      sync(2 * t + 1);
      softmax(t);
    }
    sync(2 * ntiles);
    mma_pv(ntiles - 1);
    sync(2 * ntiles + 1);
  } else {
    sync(0);
    sync(1);
    mma_phase(0);
    sync(2);
    softmax(0);
    for (int t = 1; t < ntiles; ++t) {
      sync(2 * t + 1);
      mma_phase(t);
      sync(2 * t + 2);
      softmax(t);
    }
    sync(2 * ntiles + 1);
    mma_pv(ntiles - 1);
  }

  // ---- normalise and store: element i of o[g][dt] is dim 32 dt + 8(i/4) + 4h + i%4
  auto store_out = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float inv = 1.0f / (l_run[g] + __shfl_xor(l_run[g], 32));
      if (qok[g]) {
        uint16_t* dst = out + (static_cast<size_t>(b) * N + qrow[g]) * D + head * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          u32x2 pk[4];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            pk[g4][0] = pack_bf16x2(o[g][dt][4 * g4] * inv, o[g][dt][4 * g4 + 1] * inv);
            pk[g4][1] = pack_bf16x2(o[g][dt][4 * g4 + 2] * inv, o[g][dt][4 * g4 + 3] * inv);
          }
          // lanes l and l + 32 hold the same query row (qok is the same for both)
          store_row32_bf16(dst + dt * 32, pk, h);
        }
      }
    }
  };
  if (!SPLIT) {
    store_out();
    return;
  }

  // ---- key pieces: each leaves its unnormalised state (o, and the lane's m_run, l_run) in
  // `part`, one record per (query block, piece, wave, group) in the lanes' register order;
  // attn_merge_kernel combines them after this launch.
  constexpr int REC = (DT * 16 + 2) * 64;       // floats per (wave, group) record
  float* r = part + ((static_cast<size_t>(bh * nqb + qblk) * nsplit + piece) * NW + wave) * (NG * REC);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    f32x4* po = reinterpret_cast<f32x4*>(r + g * REC);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v = {o[g][dt][4 * i4], o[g][dt][4 * i4 + 1], o[g][dt][4 * i4 + 2], o[g][dt][4 * i4 + 3]};
        po[(dt * 4 + i4) * 64 + lane] = v;
      }
    const f32x2 ml = {m_run[g], l_run[g]};
    reinterpret_cast<f32x2*>(r + g * REC + DT * 16 * 64)[lane] = ml;
  }
}

// The pieces of one (query block, wave, group) merged in piece order: the running states
// are brought to their largest max, summed, normalised and stored as the kernel above
// stores a block it took whole.  One 64-thread workgroup per (query block, wave, group),
// so that many waves keep record reads in flight; lane l plays the part of lane l of that
// wave.
template <int HD, int NG>
__global__ __launch_bounds__(64)
void attn_merge_kernel(const float* __restrict__ part, uint16_t* __restrict__ out, int N, int H,
                       int nqb, int nsplit) {
  constexpr int NW = 8, BQ = NW * 32 * NG, DT = HD / 32;
  constexpr int REC = (DT * 16 + 2) * 64;
  const int lane = threadIdx.x, h = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.x % NG, wave = (blockIdx.x / NG) % NW, unit = blockIdx.x / (NG * NW);
  const int qblk = unit % nqb, bh = unit / nqb;
  const int head = bh % H, b = bh / H;
  const int D = H * HD;
  auto rec = [&](int p, int g) __attribute__((always_inline)) {
    return part + ((static_cast<size_t>(unit) * nsplit + p) * NW + wave) * (NG * REC) + g * REC;
  };
  {
    const int j = qblk * BQ + wave * (32 * NG) + g * 32 + l32;
    // (loops unrolled over the largest piece count, so that mp stays in registers)
    float mp[kMaxSplit];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p)
      if (p < nsplit) {
        mp[p] = reinterpret_cast<const f32x2*>(rec(p, g) + DT * 16 * 64)[lane][0];
        mx = fmaxf(mx, mp[p]);
      }
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float l = 0.f;
#pragma unroll
    for (int p = 0; p < kMaxSplit; ++p) {
      if (p >= nsplit) break;
      const float w = __builtin_amdgcn_exp2f(mp[p] - mx);
      l = fmaf(reinterpret_cast<const f32x2*>(rec(p, g) + DT * 16 * 64)[lane][1], w, l);
      const f32x4* po = reinterpret_cast<const f32x4*>(rec(p, g));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 v = po[(dt * 4 + i4) * 64 + lane];
#pragma unroll
          for (int c = 0; c < 4; ++c) o[dt][4 * i4 + c] = fmaf(v[c], w, o[dt][4 * i4 + c]);
        }
    }
    // element i of o[dt] is dim 32 dt + 8(i/4) + 4h + i%4 of query j; lanes l and l + 32
    // hold the same query and split its row sum
    const float inv = 1.0f / (l + __shfl_xor(l, 32));
    if (j < N) {
      uint16_t* dst = out + (static_cast<size_t>(b) * N + j) * D + head * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x2 pk[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          pk[g4][0] = pack_bf16x2(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv);
          pk[g4][1] = pack_bf16x2(o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv);
        }
        store_row32_bf16(dst + dt * 32, pk, h);
      }
    }
  }
}

// How the bf16 kernel covers a clip of N tokens: NG query groups of 32 per wave (256 NG
// queries per workgroup), nqb query blocks, and the keys of each block in nsplit pieces
// of tps tiles.  Everything here follows from N and the head count, never from the
// batch, so a clip's result does not depend on the batch it comes in.
//   * Short clips (at most 1024 keys) take one group per wave: twice the workgroups for the
//     few (clip, head) pairs.
//   * From 4096 keys on, when one clip's (head, query block) pairs would leave compute
//     units idle in the last round (the 2048 + 6144-token predictor: 192 pairs on 256
//     units), the keys are cut into pieces if the estimated time of one clip, rounds of
//     the units times (tiles per piece + a piece's fixed cost), drops by a tenth or more.
//     A large batch of such clips then pays that fixed cost per piece.
struct AttnPlan {
  int ng, nqb, nsplit, tps;
};
constexpr int kAttnShortN = 1024;   // longest clip that takes 256-query workgroups
constexpr int kSplitMinN = 4096;    // shortest clip whose keys may be cut into pieces
constexpr int kSplitCUs = 256;      // compute units the pieces are counted against
constexpr int kPieceCost = 4;       // a piece's prologue, record and merge, in key tiles
static_assert(kSplitMinN > kAttnShortN, "clips in pieces take two query groups per wave");

static AttnPlan attn_plan(int N, int n_head, bool bc) {
  AttnPlan p;
  p.ng = (!bc && N <= kAttnShortN) ? 1 : 2;
  const int bq = 256 * p.ng, ntiles = (N + 63) / 64;
  p.nqb = (N + bq - 1) / bq;
  p.nsplit = 1;
  p.tps = ntiles;
  if (bc || N < kSplitMinN) return p;
  const long long pairs = static_cast<long long>(n_head) * p.nqb;
  auto cost = [&](int tps) {
    const long long wgs = pairs * ((ntiles + tps - 1) / tps);
    return (wgs + kSplitCUs - 1) / kSplitCUs * (tps + kPieceCost);
  };
  const long long whole = cost(ntiles);
  long long best = whole;
  for (int sp = 2; sp <= kMaxSplit; ++sp) {
    const int tps = (ntiles + sp - 1) / sp;
    const long long c = cost(tps);
    if (10 * c <= 9 * whole && c < best) {
      best = c;
      p.tps = tps;
      p.nsplit = (ntiles + tps - 1) / tps;
    }
  }
  return p;
}

size_t attention_split_bytes(int B, int N, int n_head, int head_dim) {
  if (B <= 0 || N <= 0 || n_head <= 0 || (head_dim != 64 && head_dim != 32)) return 0;
  const AttnPlan p = attn_plan(N, n_head, false);
  if (p.nsplit == 1) return 0;
  // one fp32 record of (o, m_run, l_run) per (query block, piece, wave, group, lane)
  const size_t units = static_cast<size_t>(B) * n_head * p.nqb;
  return units * p.nsplit * 8 * p.ng * static_cast<size_t>(head_dim / 2 + 2) * 64 * 4;
}

template <int HD, bool BC, int NG, bool SPLIT = false>
static hipError_t attn_launch(const uint16_t* q, const uint16_t* k, int ld, const uint16_t* vt, int Ns,
                              uint16_t* out, int B, int N, int n_head, int n_cls, int slot,
                              const AttnPlan& p, void* split_ws, hipStream_t s) {
  constexpr int LDS = 4 * (64 * HD * 2 + HD * 64 * 2);
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<HD, BC, NG, SPLIT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const size_t units = static_cast<size_t>(p.nqb) * n_head * B;
  if (units * p.nsplit * 8 * NG > 0x7fffffffu) return hipErrorInvalidValue;
  if ((p.nsplit > 1) != SPLIT) return hipErrorInvalidValue;
  float* part = static_cast<float*>(split_ws);
  if (SPLIT && (!part || reinterpret_cast<uintptr_t>(part) % 16)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(units * p.nsplit));
  attn_fwd_kernel<HD, BC, NG, SPLIT><<<grid, 512, LDS, s>>>(q, k, ld, vt, Ns, out, N, n_head, p.nqb,
                                                             n_cls, slot, p.nsplit, p.tps, part);
  if constexpr (SPLIT) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_merge_kernel<HD, NG><<<static_cast<unsigned>(units * 8 * NG), 64, 0, s>>>(part, out, N, n_head,
                                                                             p.nqb, p.nsplit);
  }
  return hipGetLastError();
}

hipError_t launch_attention_fwd(const uint16_t* q, const uint16_t* k, int ld, const uint16_t* vt,
                                int Ns, uint16_t* out, int B, int N, int n_head, int head_dim,
                                hipStream_t s, int n_cls, int slot, void* split_ws) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if ((head_dim != 64 && head_dim != 32) || Ns < vt_stride(N) || Ns % 16 || ld % 8) return hipErrorInvalidValue;
  // 32-bit DMA offsets: one clip's rows of q/k and one (clip, head)'s V^T rows
  if (static_cast<size_t>(N) * ld * 2 >= (size_t(1) << 31) ||
      static_cast<size_t>(head_dim) * Ns * 2 >= (size_t(1) << 31))
    return hipErrorInvalidValue;
  if (slot > 0) {
    // the first key tile must hold a key every query sees (key n_cls)
    if (n_cls < 0 || n_cls >= 64 || n_cls >= N) return hipErrorInvalidValue;
    const AttnPlan p = attn_plan(N, n_head, true);
    if (head_dim == 64) return attn_launch<64, true, 2>(q, k, ld, vt, Ns, out, B, N, n_head, n_cls, slot, p, nullptr, s);
    return attn_launch<32, true, 2>(q, k, ld, vt, Ns, out, B, N, n_head, n_cls, slot, p, nullptr, s);
  }
  const AttnPlan p = attn_plan(N, n_head, false);
  if (p.nsplit > 1) {   // (only from 4096 keys on, so with two query groups per wave)
    if (head_dim == 64) return attn_launch<64, false, 2, true>(q, k, ld, vt, Ns, out, B, N, n_head, 0, 0, p, split_ws, s);
    return attn_launch<32, false, 2, true>(q, k, ld, vt, Ns, out, B, N, n_head, 0, 0, p, split_ws, s);
  }
  if (p.ng == 1) {
    if (head_dim == 64) return attn_launch<64, false, 1>(q, k, ld, vt, Ns, out, B, N, n_head, 0, 0, p, split_ws, s);
    return attn_launch<32, false, 1>(q, k, ld, vt, Ns, out, B, N, n_head, 0, 0, p, split_ws, s);
  }
  if (head_dim == 64) return attn_launch<64, false, 2>(q, k, ld, vt, Ns, out, B, N, n_head, 0, 0, p, split_ws, s);
  return attn_launch<32, false, 2>(q, k, ld, vt, Ns, out, B, N, n_head, 0, 0, p, split_ws, s);
}

// Attention inputs from a projection already in memory (the stand-alone entry point): one
// workgroup per (64-row tile, section x head, clip) of qkv [B*N, 3D].  Four threads per
// row each take HD/4 consecutive columns (16-byte loads): q and k are rotated (q also
// scaled) into qk [B*N, 2D]; v goes through LDS and leaves transposed, each thread writing
// one 16-key group of one dim (the keys in vt_pos order, 32 contiguous bytes), so the four
// threads of a dim store 128 contiguous bytes.
template <int HD>
__global__ __launch_bounds__(256)
void qkv_prepare_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ qk,
                        uint16_t* __restrict__ vt, int Ns, int N, int H, RopeArgs ra, float qscale) {
  constexpr int EPT = HD / 4;               // columns per thread
  __shared__ uint16_t tile[64][HD + 2];
  const int D = H * HD;
  const int r0 = blockIdx.x * 64, b = blockIdx.z;
  const int sec = blockIdx.y / H, head = blockIdx.y - sec * H;
  const int t = threadIdx.x, rl = t >> 2, c0 = (t & 3) * EPT;
  const int n = r0 + rl;
  const int row = b * N + n;
  uint16_t raw[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) raw[i] = 0;
  if (n < N) {
    const uint16_t* src = qkv + static_cast<size_t>(row) * 3 * D + sec * D + head * HD + c0;
#pragma unroll
    for (int i = 0; i < EPT / 8; ++i) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + 8 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        raw[8 * i + 2 * e] = static_cast<uint16_t>(w[e] & 0xFFFF);
        raw[8 * i + 2 * e + 1] = static_cast<uint16_t>(w[e] >> 16);
      }
    }
  }
  if (sec < 2) {   // uniform over the workgroup
    if (n >= N) return;
    int clip;
    const Thw g = rope_token(row, ra, &clip);
    uint16_t* dst = qk + static_cast<size_t>(row) * 2 * D + sec * D + head * HD + c0;
#pragma unroll
    for (int i = 0; i < EPT / 8; ++i) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 8 * i + 2 * e;
        float x0 = bf16_to_f32(raw[j]), x1 = bf16_to_f32(raw[j + 1]);
        rope_pair<HD>(x0, x1, c0 + j, g, ra.layout, ra.tab);
        if (sec == 0) {
          x0 *= qscale;
          x1 *= qscale;
        }
        w[e] = pack_bf16x2(x0, x1);
      }
      *reinterpret_cast<u32x4*>(dst + 8 * i) = w;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) tile[rl][c0 + i] = raw[i];   // rows past N hold 0
  __syncthreads();
  for (int e = t; e < HD * 4; e += 256) {
    const int d = e >> 2, grp = e & 3;
    const int k0 = r0 + 16 * grp;
    if (k0 >= N) continue;     // k0 + 16 <= Ns: Ns is at least N rounded up to 16
    uint16_t w16[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) w16[vt_pos(k)] = tile[16 * grp + k][d];
    uint16_t* dst = vt + (static_cast<size_t>(b * H + head) * HD + d) * Ns + k0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = static_cast<uint32_t>(w16[8 * i + 2 * q]) | (static_cast<uint32_t>(w16[8 * i + 2 * q + 1]) << 16);
      *reinterpret_cast<u32x4*>(dst + 8 * i) = w;
    }
  }
}

hipError_t launch_qkv_prepare(const uint16_t* qkv, uint16_t* qk, uint16_t* vt, int Ns, int B,
                              int N, int n_head, int head_dim, const int32_t* ids,
                              const RopeSpec& r, const void* tab, float qscale, hipStream_t s,
                              int lead) {
  if (B <= 0 || N <= 0) return hipSuccess;
  if ((head_dim != 64 && head_dim != 32) || Ns < vt_stride(N) || Ns % 16) return hipErrorInvalidValue;
  if (static_cast<long long>(B) * N >= (1LL << 31)) return hipErrorInvalidValue;
  const int D = n_head * head_dim;
  // clips go to grid z, at most 65535 per launch
  for (int b0 = 0; b0 < B; b0 += 65535) {
    const int nb = min(B - b0, 65535);
    const RopeArgs ra{static_cast<const float2*>(tab), ids, N, r.layout, r.gt * r.gh * r.gw, r.gh, r.gw,
                      0, lead};
    const size_t rows = static_cast<size_t>(b0) * N;
    const dim3 grid((N + 63) / 64, 3 * n_head, nb);
    uint16_t* vtb = vt + static_cast<size_t>(b0) * D * Ns;
    if (head_dim == 64)
      qkv_prepare_kernel<64><<<grid, 256, 0, s>>>(qkv + rows * 3 * D, qk + rows * 2 * D, vtb, Ns, N, n_head,
                                                   ra, qscale);
    else
      qkv_prepare_kernel<32><<<grid, 256, 0, s>>>(qkv + rows * 3 * D, qk + rows * 2 * D, vtb, Ns, N, n_head,
                                                   ra, qscale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static RopeFreq make_freq(int head_dim, float theta) {
  RopeFreq f{};
  const int m = (2 * ((head_dim / 3) / 2)) / 2;
  for (int k = 0; k < m && k < 16; ++k)
    f.w[k] = static_cast<float>(1.0 / pow(static_cast<double>(theta), static_cast<double>(k) / m));
  return f;
}

// ---------------------------------------------------------------- fp32 / FMA

template <int HD>
__global__ __launch_bounds__(64)
void attn_f32_kernel(const float* __restrict__ qkv, float* __restrict__ out, int N, int H,
                     const int32_t* __restrict__ ids_all, int ids_stride, RopeSpec r, RopeFreq fr,
                     float scale, int n_cls, int slot) {
  constexpr int D3 = 2 * ((HD / 3) / 2);
  constexpr int MF = D3 / 2;
  constexpr int BKV = 64;
  __shared__ float2 tab[3 * kMaxGridSide * MF];
  __shared__ float Ks[BKV][HD];
  __shared__ float Vs[BKV][HD];
  const int tid = threadIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int32_t* ids = ids_all ? ids_all + static_cast<size_t>(b) * ids_stride : nullptr;
  const int D = H * HD, ld = 3 * D;
  const int ntot = r.gt * r.gh * r.gw;
  const float* base = qkv + static_cast<size_t>(b) * N * ld + head * HD;
  build_rope_tables<MF>(tab, r, fr);
  __syncthreads();

  const int q = blockIdx.x * 64 + tid;
  const int qr = min(q, N - 1);
  float qv[HD], ov[HD];
  {
    const Thw g = decode_id(token_id(ids, qr, ntot, n_cls), r.gh, r.gw);
#pragma unroll
    for (int j = 0; j < HD; ++j) qv[j] = base[static_cast<size_t>(qr) * ld + j];
    rope_chunk<HD, HD>(qv, 0, g, r.layout, tab);
#pragma unroll
    for (int j = 0; j < HD; ++j) {
      qv[j] *= scale;
      ov[j] = 0.f;
    }
  }
  // block-causal mask (slot > 0): a patch row sees the keys [n_cls, lim), a CLS row all
  int lo = 0, lim = N;
  if (slot > 0 && qr >= n_cls) {
    lo = n_cls;
    lim = min(N, n_cls + ((qr - n_cls) / slot + 1) * slot);
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int kb = 0; kb < N; kb += BKV) {
    __syncthreads();
    {
      const int kr = min(kb + tid, N - 1);
      const Thw g = decode_id(token_id(ids, kr, ntot, n_cls), r.gh, r.gw);
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
      if (kb + k < lo || kb + k >= lim) continue;
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
                                int head_dim, const int32_t* ids, int ids_stride,
                                const RopeSpec& r, hipStream_t s, int n_cls, int slot) {
  if (B <= 0 || N <= 0) return hipSuccess;
  const RopeFreq fr = make_freq(head_dim, r.theta);
  const float scale = static_cast<float>(1.0 / sqrt(static_cast<double>(head_dim)));
  const dim3 grid((N + 63) / 64, n_head, B);
  if (head_dim == 64)
    attn_f32_kernel<64><<<grid, 64, 0, s>>>(qkv, out, N, n_head, ids, ids_stride, r, fr, scale, n_cls, slot);
  else if (head_dim == 32)
    attn_f32_kernel<32><<<grid, 64, 0, s>>>(qkv, out, N, n_head, ids, ids_stride, r, fr, scale, n_cls, slot);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jepa

namespace jepa {

// ---------------------------------------------------------------- single-query pooling

// The cross-attention of the attentive-pool head ([Notes §2] "Attentive-pool head"): one
// learned query row q (projected, fp32 [D]) attends over the N tokens of each clip, with
// k and v fp32 (rows of leading dimension ld: k at kv, v at kv + D), softmax(q k^T /
// sqrt(hd)) v per head, heads concatenated, no output projection; the raw query q0 is the
// residual: y[b] = q0 + o[b].  k and v are separate row blocks of leading dimension ld.
// One workgroup of 1024 threads per (head, clip): scores in LDS (N floats), the block max
// and sum, then the weighted sum of v split over 1024 / 64 = 16 key groups (n mod 16) and
// added in group order, so the result does not depend on the launch.
template <int HD>
__global__ __launch_bounds__(1024)
void xattn_query_kernel(const float* __restrict__ q, const float* __restrict__ k,
                        const float* __restrict__ v, int ld, const float* __restrict__ q0,
                        float* __restrict__ y, int N, int D, float scale) {
  constexpr int NT = 1024, G = NT / 64;
  extern __shared__ float sc[];   // [N] scores, then probabilities
  __shared__ float red[NT];
  __shared__ float part[G][HD];
  const int tid = threadIdx.x, head = blockIdx.x, b = blockIdx.y;
  const float* qh = q + head * HD;
  const float* kb = k + static_cast<size_t>(b) * N * ld + head * HD;
  const float* vb = v + static_cast<size_t>(b) * N * ld + head * HD;
  float mx = -INFINITY;
  for (int n = tid; n < N; n += NT) {
    const f32x4* kr = reinterpret_cast<const f32x4*>(kb + static_cast<size_t>(n) * ld);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < HD / 4; ++c) {
      const f32x4 k4 = kr[c];
      s = fmaf(qh[4 * c], k4[0], s);
      s = fmaf(qh[4 * c + 1], k4[1], s);
      s = fmaf(qh[4 * c + 2], k4[2], s);
      s = fmaf(qh[4 * c + 3], k4[3], s);
    }
    s *= scale;
    sc[n] = s;
    mx = fmaxf(mx, s);
  }
  red[tid] = mx;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int n = tid; n < N; n += NT) {
    const float p = expf(sc[n] - mx);
    sc[n] = p;
    sum += p;
  }
  red[tid] = sum;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  sum = red[0];
  // o[d] over the keys n = g, g + G, ... of group g = tid / 64 (HD <= 64 lanes per group)
  const int g = tid >> 6, d = tid & 63;
  if (d < HD) {
    float acc = 0.f;
    for (int n = g; n < N; n += G) acc = fmaf(sc[n], vb[static_cast<size_t>(n) * ld + d], acc);
    part[g][d] = acc;
  }
  __syncthreads();
  if (tid < HD) {
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) o += part[i][tid];
    y[static_cast<size_t>(b) * D + head * HD + tid] = q0[head * HD + tid] + o / sum;
  }
}

hipError_t launch_xattn_query(const float* q, const float* k, const float* v, int ld,
                              const float* q0, float* y, int B, int N, int n_head, int head_dim,
                              hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (N <= 0 || N > kXattnMaxTokens || ld % 4) return hipErrorInvalidValue;
  const int D = n_head * head_dim;
  const float scale = static_cast<float>(1.0 / sqrt(static_cast<double>(head_dim)));
  const dim3 grid(n_head, B);
  const size_t lds = static_cast<size_t>(N) * 4;
  static bool configured = false;   // up to 64 KB of dynamic LDS for the scores
  if (!configured) {
    for (const void* f : {reinterpret_cast<const void*>(&xattn_query_kernel<64>),
                          reinterpret_cast<const void*>(&xattn_query_kernel<32>)}) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kXattnMaxTokens * 4);
      if (e != hipSuccess) return e;
    }
    configured = true;
  }
  if (head_dim == 64)
    xattn_query_kernel<64><<<grid, 1024, lds, s>>>(q, k, v, ld, q0, y, N, D, scale);
  else if (head_dim == 32)
    xattn_query_kernel<32><<<grid, 1024, lds, s>>>(q, k, v, ld, q0, y, N, D, scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jepa
