// Linear layers C = epilogue(A W^T + bias) for libjepa.
//
// Weights are stored [out, in] row-major ([Notes §2] key map), so both operands are
// contiguous along K and map straight onto the MFMA operand layout.
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * a workgroup of 8 wavefronts (2 per SIMD) computes 256 (rows of A) x 256, 192 or
//     128 (rows of W) output tiles, the width chosen by the rounds of the CUs its tiles
//     need times the rows a tile streams per K slab: the bytes a CU copies into LDS per
//     MFMA fall as the tile grows, and the slab copies (their LDS writes and their issue
//     beside the fragment reads), not the MFMAs or the copies' latency, set the pace of
//     the main loop; each wave owns a 128x64, 64x96 or 64x64 part of the tile as 32x32
//     blocks;
//   * the kernel is persistent: one workgroup per CU walks its tiles, and the 64-deep
//     K-slabs of all its tiles form one stream through a ring of 2 or 3 LDS buffers,
//     filled by global_load_lds_dwordx4 (HBM/L2 -> LDS, no register staging) up to
//     STAGES - 1 slabs ahead of the MFMAs, so the next tile's first slabs load while
//     the current tile's epilogue runs; one barrier per slab;
//   * LDS rows are 128 B; the 16-byte chunk c of row r lives at chunk c ^ key(r), with a
//     key that keeps 16 consecutive rows of one chunk column in 16 different bank groups.
//     A DMA instruction writes 64 consecutive 16-byte slots (8 rows), so lane p of it
//     fetches the global chunk that belongs in slot p;
//   * the MFMA takes the W fragment as its first operand, so each lane ends up holding
//     runs of 4 consecutive output columns of one output row: the epilogue (bias, GELU,
//     residual) reads and writes 8- or 16-byte vectors;
//   * tiles are dealt so that the 32 workgroups of one XCD (work-groups go to the 8
//     XCDs round-robin) work on neighbouring tiles at the same time.
//
// fp32 path: a plain 64x64-tile FMA kernel (no MFMA), used by the fp32 encoder.
#include "common.h"
#include "kernels.h"
#include "rope_tab.h"

namespace jepa {

enum { EPI_STORE = 0, EPI_GELU = 1, EPI_RESIDUAL = 2, EPI_QKV64 = 3, EPI_QKV32 = 4 };

// Arguments of the QKV epilogue (EPI_QKV64 / EPI_QKV32 for head dim 64 / 32): columns
// [0, D) are q, [D, 2D) k, [2D, 3D) v of D = H * hd.  q and k are rotated by the 3-D RoPE
// of the row's token ([Notes §4]) and q is scaled by qscale; both are stored in place.
// v goes to vt [clip][head][dim][Ns], key n of a clip at position vt_pos(n).
// The epilogue reads the RoPE table from LDS: rows (axis, coord < ts) of the full table
// are copied after the slab ring at kernel start, kLdsTabRow float2 apart.  The 32 lanes
// of a half-wave hold consecutive tokens, up to 32 distinct coordinates on the w axis; a
// row of kRopeMaxFreq float2 (32 dwords) would put coordinates two apart on the same
// banks, the padded row (34 dwords) spreads 32 of them over distinct bank pairs.
constexpr int kLdsTabRow = kRopeMaxFreq + 1;
// After the table and the bias slots: one int4 per rotation pair of a head (at most 32),
// {byte offset of its two table entries at coordinate 0, bit offset of its axis'
// coordinate in the packed t, h, w}, built at kernel start.
constexpr int kPairMapBytes = 32 * 16;
struct QkvEpi {
  uint16_t* vt;
  RopeArgs ra;
  int D, H, Ns, ts;
  float qscale;
};

// GELU with erf from Abramowitz & Stegun 7.1.26 (|error of erf| <= 1.5e-7, far below
// the bf16 rounding of the output): for x = |z| / sqrt(2), 1 - erf(x) = q(t) exp(-x^2)
// with t = 1 / (1 + p x) and q a degree-5 polynomial in t without constant term.  Since
// GELU(z) = z Phi(z) = max(z, 0) - |z| (1 - erf(x)) / 2 for either sign of z, the tail term
// is formed directly (no 1 - erf cancellation for negative z) in 12 vector instructions
// plus v_rcp_f32 and v_exp_f32.
__device__ __forceinline__ float gelu_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, az, 1.0f));
  float y = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  y = fmaf(y, t, 0.5f * 1.421413741f);
  y = fmaf(y, t, 0.5f * -0.284496736f);
  y = fmaf(y, t, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(z * (z * -0.72134752044448170368f));   // exp(-z^2 / 2)
  return fmaf(-az, y * t * e, fmaxf(z, 0.0f));
}


// One tile configuration: BM x BN output tiles, 64-deep K slabs through a ring of STAGES
// LDS buffers, WGM x WGN waves of WM x WN, each held as 32 x 32 MFMA blocks.
template <int BM_, int BN_, int STAGES_, int WGM_, int WGN_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, STAGES = STAGES_;
  static constexpr int WGM = WGM_, WGN = WGN_, NWAVES = WGM * WGN, NT = NWAVES * 64;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FI = WM / 32, FJ = WN / 32;        // 32x32 blocks per wave
  static constexpr int ROWB = BK * 2;                     // LDS bytes per tile row (128)
  static constexpr int RPI = 1024 / ROWB;                 // rows per 1 KB DMA instruction
  static constexpr int CPR = ROWB / 16;                   // 16-byte chunks per row
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NWAVES;  // DMA instructions per thread
  static constexpr int B_LOADS = B_BYTES / 1024 / NWAVES;
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static constexpr int LDS = STAGES * STAGE_BYTES;
  // 1 KB bias slots, one per tile in flight: tile i's slot is rewritten for tile
  // i + NBIAS, whose first slab is issued (NBIAS - 1) * K/64 >= STAGES slabs after tile
  // i's last one, i.e. after a barrier that follows tile i's epilogue, for every K.
  static constexpr int NBIAS = STAGES + 1;
  static constexpr int BIAS_BYTES = NBIAS * 1024;
  static constexpr int EXTRA = BIAS_BYTES;
  static_assert(A_LOADS * NWAVES * 1024 == A_BYTES && B_LOADS * NWAVES * 1024 == B_BYTES, "DMA split");
  static_assert(FI * 32 == WM && FJ * 32 == WN, "wave tile");
  static_assert(STAGES >= 2 && STAGES <= 4 && LDS + EXTRA <= 160 * 1024, "LDS ring");
  // the ping-pong groups (waves 0-3, 4-7) are the two row halves of the tile
  static_assert(BN <= 256, "bias slot of 1 KB");
  __device__ static int key(int r) { return lds_key128(r); }
};
// 256 x 256: FFN up-projection (N = 4096 gives whole rounds of 256 CUs)
using Cfg256x256 = GemmCfg<256, 256, 2, 2, 4>;
// 256 x 192: QKV projection at D = 1024 (N = 3072)
using Cfg256x192 = GemmCfg<256, 192, 2, 4, 2>;
// 256 x 128: every other width that is a multiple of 128
using Cfg256x128 = GemmCfg<256, 128, 3, 4, 2>;
// 256 x 128 with a 2-buffer ring: leaves LDS for the RoPE table of the QKV epilogue
using Cfg256x128q = GemmCfg<256, 128, 2, 4, 2>;
// 128 x 128 (waves of 64 x 32): for outputs whose 256-row tiling leaves CUs idle (few
// token rows, as in the masked forward, or narrow outputs such as N = 384)
using Cfg128x128 = GemmCfg<128, 128, 4, 2, 4>;
using Cfg128x128q = GemmCfg<128, 128, 3, 2, 4>;
// 128 x 64 (waves of 32 x 32): twice the 128 x 128 tiles where those would still leave
// CUs idle (the masked forward's 2048 rows at N = 1024)
using Cfg128x64 = GemmCfg<128, 64, 4, 4, 2>;

template <class C, int EPI, bool OUT_F32>
__global__ __launch_bounds__(C::NT)
void gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                      const float* __restrict__ bias, void* __restrict__ Cv, int M, int N, int K,
                      QkvEpi qe) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, STAGES = C::STAGES, NWAVES = C::NWAVES;
  constexpr int FI = C::FI, FJ = C::FJ, WM = C::WM, WN = C::WN;
  constexpr int A_LOADS = C::A_LOADS, B_LOADS = C::B_LOADS;
  constexpr int STAGE_BYTES = C::STAGE_BYTES, A_BYTES = C::A_BYTES, ROWB = C::ROWB;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: DMA LDS bases
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int h = lane >> 5, l32 = lane & 31;

  const int tiles_n = N / BN;
  const int tiles = ((M + BM - 1) / BM) * tiles_n;
  const int G = gridDim.x, b = blockIdx.x;
  const int n_my = (tiles - b + G - 1) / G;   // tiles b, b + G, b + 2G, ...
  const int KT = K / BK;
  const int total = n_my * KT;

  // Tile of round i.  Work-groups are dealt to the 8 XCDs round-robin (b % 8).  When the
  // grid fills every CU and the tile grid splits evenly, the SPX = G/8 workgroups of XCD x
  // work, round by round, on a block of SPX/8 row tiles x 8 column tiles of its share:
  // they share those rows of A and columns of W in the XCD's L2, and the rows stay
  // resident while the rounds walk the columns.  Otherwise: consecutive tiles per XCD
  // in full rounds, plain order in the last, partial round.
  const int tiles_m = (M + BM - 1) / BM;
  const int spx = G >> 3, btm = spx >> 3;           // workgroups per XCD, block rows
  const bool blocked = (G & 63) == 0 && btm > 0 && tiles_m % (8 * btm) == 0 && tiles_n % 8 == 0;
  auto tile_of = [&](int i, int& m0, int& n0) {
    int tm, tn;
    if (blocked) {
      const int x = b & 7, j = b >> 3;              // XCD, slot in it
      const int k = i * spx + j;                    // position in the XCD's sequence
      const int rows = tiles_m / 8;                 // row tiles per XCD
      const int nb = k / spx, w = k % spx;          // column block, slot in it
      const int grp = nb / (tiles_n / 8);           // which group of btm row tiles
      tm = x * rows + grp * btm + w / 8;
      tn = (nb % (tiles_n / 8)) * 8 + (w % 8);
    } else {
      int t = i * G + b;
      if ((G & 7) == 0 && (i + 1) * G <= tiles) t = i * G + (b & 7) * (G >> 3) + (b >> 3);
      tm = t / tiles_n;
      tn = t - tm * tiles_n;
    }
    m0 = tm * BM;
    n0 = tn * BN;
  };

  // DMA mapping: instruction q of wave w fills rows [8 g, 8 g + 8) of a tile,
  // g = q*NWAVES + w; lane p -> row 8 g + p/8, slot p%8 holding logical chunk
  // (p%8) ^ key(row).
  const int prow = lane / C::CPR, pslot = lane % C::CPR;
  const uint32_t smem_base = lds_addr(smem);

  // Issue state: the next slab to load (tile it_iss, slab kt_iss) and the byte offsets
  // of this lane's source rows in that tile, refreshed when the tile changes.  Rows of A
  // past M are clamped to row M - 1 (loaded, never stored).
  int it_iss = 0, kt_iss = 0, s_iss = 0, n0_iss = 0;
  uint32_t a_row[A_LOADS], b_row[B_LOADS];
  auto set_rows = [&](int it) {
    int m0, n0;
    tile_of(it, m0, n0);
    n0_iss = n0;
#pragma unroll
    for (int q = 0; q < A_LOADS; ++q) {
      const int r = (q * NWAVES + wave) * C::RPI + prow;
      a_row[q] = static_cast<uint32_t>(static_cast<size_t>(min(m0 + r, M - 1)) * K * 2) + ((pslot ^ C::key(r)) << 4);
    }
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
      const int r = (q * NWAVES + wave) * C::RPI + prow;
      b_row[q] = static_cast<uint32_t>(static_cast<size_t>(n0 + r) * K * 2) + ((pslot ^ C::key(r)) << 4);
    }
  };
  // LDS after the ring: [RoPE table of the QKV epilogue] [NBIAS 1 KB bias slots] [pair map
  // of the QKV epilogue].  The bias columns of tile i go to slot i % NBIAS by one DMA of
  // wave 0, issued just before the tile's first slab: every wait for that slab or a later
  // one in wave 0 covers it, and the barrier after that wait publishes it.  The slot is
  // rewritten for tile i + NBIAS only after barriers that follow tile i's epilogue in
  // every wave (see GemmCfg::NBIAS).
  const int tab_bytes = (EPI == EPI_QKV64 || EPI == EPI_QKV32) ? 3 * qe.ts * kLdsTabRow * 8 : 0;
  const uint32_t bias_base = smem_base + C::LDS + tab_bytes;
  const bool has_bias = bias != nullptr;
  // One slab's copies in three parts, so that the copies can be spread between MFMAs:
  // issue_begin (the tile's bias, before its first slab), issue_load(q) for q < LOADS (q <
  // A_LOADS: 1 KB of A, else 1 KB of W), issue_end (advance to the next slab).
  auto issue_begin = [&]() __attribute__((always_inline)) {
    if (kt_iss == 0 && has_bias && wave == 0)
      dma16(bias, static_cast<uint32_t>(n0_iss * 4 + min(lane, BN / 4 - 1) * 16),
            bias_base + (it_iss % C::NBIAS) * 1024);
  };
  auto issue_load = [&](int q) __attribute__((always_inline)) {
    const uint32_t st = smem_base + (s_iss % STAGES) * STAGE_BYTES;
    const uint32_t k0 = kt_iss * BK * 2;
    if (q < A_LOADS)
      dma16(A, a_row[q] + k0, st + (q * NWAVES + wave) * 1024);
    else
      dma16(W, b_row[q - A_LOADS] + k0, st + A_BYTES + ((q - A_LOADS) * NWAVES + wave) * 1024);
  };
  auto issue_end = [&]() __attribute__((always_inline)) {
    ++s_iss;
    if (++kt_iss == KT) {
      kt_iss = 0;
      if (++it_iss < n_my) set_rows(it_iss);
    }
  };
  auto issue_next = [&]() {
    issue_begin();
#pragma unroll
    for (int q = 0; q < C::LOADS; ++q) issue_load(q);
    issue_end();
  };

  // fragment rows of this lane inside the A / W tiles (32x32x16 operand: row l%32,
  // 8 consecutive k at chunk 2*step + l/32)
  int arow[FI], brow[FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i) arow[i] = wm * WM + i * 32 + l32;
#pragma unroll
  for (int j = 0; j < FJ; ++j) brow[j] = wn * WN + j * 32 + l32;

  // Operand fragments of slab s, k-step ks (16 deep), from LDS.
  auto load_frags = [&](int s_, int ks, bf16x8* af, bf16x8* bfr) __attribute__((always_inline)) {
    const unsigned char* st = smem + (s_ % STAGES) * STAGE_BYTES;
    const int ch = ks * 2 + h;
#pragma unroll
    for (int i = 0; i < FI; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(st + arow[i] * ROWB + ((ch ^ C::key(arow[i])) << 4));
#pragma unroll
    for (int j = 0; j < FJ; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8*>(st + A_BYTES + brow[j] * ROWB + ((ch ^ C::key(brow[j])) << 4));
  };
  // Wait until slab s_ has landed in LDS for every lane of the workgroup: the slabs
  // issued after it (at most STAGES - 2, fewer near the end) may stay in flight.
  constexpr int PF1 = 0;
  constexpr int PER = C::LOADS;
  auto wait_slab = [&](int s_) __attribute__((always_inline)) {
    const int ahead = min(s_iss - 1 - s_, STAGES - 2);
    if (ahead >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER + PF1) : "memory");
    else if (ahead == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER + PF1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PF1) : "memory");
    __syncthreads();
  };

  // Prologue: slabs 0 .. STAGES - 2 issued, slab 0 landed, slab STAGES - 1 issued, slab
  // 0's first fragments loaded.  In the loop, slab s + 1's barrier and first fragment
  // loads come before slab s's last k-step of MFMAs, so LDS latency hides behind MFMAs;
  // the DMA issued right after that barrier (slab s + STAGES) reuses the buffer of slab s,
  // whose reads all completed before the barrier.  Up to STAGES - 1 slabs are in flight
  // while a slab is consumed.
  constexpr int KSTEPS = BK / 16;
  // The RoPE table rows (axis, coord < ts) of the QKV epilogue are copied before the first
  // slab DMA, so the waits for these loads cannot hold up the ring; the prologue's barrier
  // publishes them.
  if constexpr (EPI == EPI_QKV64 || EPI == EPI_QKV32) {
    constexpr int HD = EPI == EPI_QKV64 ? 64 : 32;
    if (tid < HD / 2) {
      const RopePairIdx r = rope_pair_idx<HD>(2 * tid, qe.ra.layout);
      const int row0 = r.axis * qe.ts * kLdsTabRow;
      reinterpret_cast<int4*>(smem + C::LDS + tab_bytes + C::BIAS_BYTES)[tid] =
          make_int4((row0 + r.i0) * 8, (row0 + r.i1) * 8, 8 * r.axis, 0);
    }
    float2* tabs = reinterpret_cast<float2*>(smem + C::LDS);
    const int n = 3 * qe.ts * kRopeMaxFreq;
    for (int e = tid; e < n; e += C::NT) {
      const int row = e / kRopeMaxFreq, k = e - row * kRopeMaxFreq;   // row = axis * ts + coord
      const int a = row / qe.ts, c = row - a * qe.ts;
      tabs[row * kLdsTabRow + k] = qe.ra.tab[(a * kMaxGridSide + c) * kRopeMaxFreq + k];
    }
  }
  // bias of the tile's columns c .. c + 3 (c relative to the tile) for tile it; without a
  // bias the slots hold zeros (written here, published by the prologue's barrier)
  if (!has_bias)
    for (int e = tid; e < C::BIAS_BYTES / 4; e += C::NT) reinterpret_cast<float*>(smem + C::LDS + tab_bytes)[e] = 0.f;
  auto bias4 = [&](int it, int c) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(smem + C::LDS + tab_bytes + (it % C::NBIAS) * 1024 + c * 4);
  };
  if (total > 0) set_rows(0);
  // Epilogue of tile it from the accumulators acc (one wave's blocks).
  auto epilogue = [&](int it, f32x16 (&acc)[FI][FJ]) __attribute__((always_inline)) {
    // Epilogue of tile it.  acc[i][j] is the 32 (W rows) x 32 (A rows) block with lane
    // l, element e at W row 8*(e/4) + 4*(l/32) + e%4 and A row l%32: runs of four
    // consecutive output columns per lane.
    int m0, n0;
    tile_of(it, m0, n0);
    if constexpr (EPI == EPI_QKV64 || EPI == EPI_QKV32) {
      constexpr int HD = EPI == EPI_QKV64 ? 64 : 32;
      const unsigned char* tabs = smem + C::LDS;
      const int4* pmap = reinterpret_cast<const int4*>(smem + C::LDS + tab_bytes + C::BIAS_BYTES);
      uint32_t g[FI];   // the row's t, h, w packed by thw_pack
      int clip[FI], nn[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int row = min(m0 + wm * WM + i * 32 + l32, M - 1);
        g[i] = thw_pack(rope_token(row, qe.ra, &clip[i]));
        nn[i] = row - clip[i] * qe.ra.N;
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        // a 32-column block lies inside one third (q, k or v) and one head
        const int col0 = n0 + wn * WN + j * 32;
        const int sec = col0 / qe.D, cin = col0 - sec * qe.D;
        const int head = cin / HD, jb = cin - head * HD;
        // this lane's columns col0 + 8gq + 4h .. +3: bias and the pair map entries of
        // their two pairs
        f32x4 bv[4];
        int4 pm[4][2];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          bv[gq] = bias4(it, col0 + 8 * gq + 4 * h - n0);
          const int p0 = (jb + 8 * gq + 4 * h) >> 1;
          pm[gq][0] = pmap[p0];
          pm[gq][1] = pmap[p0 + 1];
        }
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          const int row = m0 + wm * WM + i * 32 + l32;
          if (row >= M) continue;
          if (sec < 2) {
            // all table reads of the row first, so their LDS latency overlaps
            float2 cs[4][2][2];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const int4& m = pm[gq][pp];
                const int c = static_cast<int>(__builtin_amdgcn_ubfe(g[i], m.z, 8)) * (kLdsTabRow * 8);
                // pass-through pairs read the (1, 0) entry
                cs[gq][pp][0] = *reinterpret_cast<const float2*>(tabs + m.x + c);
                cs[gq][pp][1] = *reinterpret_cast<const float2*>(tabs + m.y + c);
              }
            const float sc = sec == 0 ? qe.qscale : 1.0f;
            u32x2 pk[4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * gq + e] + bv[gq][e];
              float y[4];
#pragma unroll
              for (int pp = 0; pp < 2; ++pp) {
                const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
                const float2 c0 = cs[gq][pp][0], c1 = cs[gq][pp][1];
                y[2 * pp] = (x0 * c0.x - x1 * c0.y) * sc;
                y[2 * pp + 1] = (x1 * c1.x + x0 * c1.y) * sc;
              }
              pk[gq][0] = pack_bf16x2(y[0], y[1]);
              pk[gq][1] = pack_bf16x2(y[2], y[3]);
            }
            store_row32_bf16(static_cast<uint16_t*>(Cv) + static_cast<size_t>(row) * N + col0, pk, h);
          } else {
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int jj = jb + 8 * gq + 4 * h;
              uint16_t* dst = qe.vt + (static_cast<size_t>(clip[i] * qe.H + head) * HD + jj) * qe.Ns + vt_pos(nn[i]);
#pragma unroll
              for (int e = 0; e < 4; ++e) dst[static_cast<size_t>(e) * qe.Ns] = f32_to_bf16(acc[i][j][4 * gq + e] + bv[gq][e]);
            }
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int row = m0 + wm * WM + i * 32 + l32;
      if (row >= M) continue;
      // the residual of this lane's row is read with all loads in flight together
      f32x4 xr[EPI == EPI_RESIDUAL ? FJ : 1][4];
      if constexpr (EPI == EPI_RESIDUAL) {
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            xr[j][g] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(Cv) + static_cast<size_t>(row) * N +
                                                       n0 + wn * WN + j * 32 + 8 * g + 4 * h);
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        u32x2 pk[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = n0 + wn * WN + j * 32 + 8 * g + 4 * h;
          const f32x4 bv = bias4(it, col - n0);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[i][j][4 * g + e] + bv[e];
            if (EPI == EPI_GELU) v[e] = OUT_F32 ? gelu_erf(v[e]) : gelu_as(v[e]);
          }
          const size_t off = static_cast<size_t>(row) * N + col;
          if constexpr (EPI == EPI_RESIDUAL) {
            f32x4 c = xr[j][g];
            c[0] += v[0]; c[1] += v[1]; c[2] += v[2]; c[3] += v[3];
            *reinterpret_cast<f32x4*>(static_cast<float*>(Cv) + off) = c;
          } else if (OUT_F32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(Cv) + off) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            pk[g][0] = pack_bf16x2(v[0], v[1]);
            pk[g][1] = pack_bf16x2(v[2], v[3]);
          }
        }
        if constexpr (EPI != EPI_RESIDUAL && !OUT_F32)
          store_row32_bf16(static_cast<uint16_t*>(Cv) + static_cast<size_t>(row) * N + n0 + wn * WN + j * 32, pk, h);
      }
    }
  };
  auto zero_acc = [&](f32x16 (&acc)[FI][FJ]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  };

#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < total) issue_next();
  bf16x8 af[2][FI], bfr[2][FJ];
  if (total > 0) {
    wait_slab(0);
    // slab STAGES - 1 goes into the buffer no slab has used yet
    if (s_iss < total) issue_next();
    load_frags(0, 0, af[0], bfr[0]);
  }
  int s = 0;  // position in this workgroup's slab stream
  for (int it = 0; it < n_my; ++it) {
    f32x16 acc[FI][FJ];
    zero_acc(acc);

    for (int kt = 0; kt < KT; ++kt, ++s) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int cur = ks & 1, nxt = cur ^ 1;
        bool spread = false;
        if (ks + 1 < KSTEPS) {
          load_frags(s, ks + 1, af[nxt], bfr[nxt]);
        } else if (s + 1 < total) {
          wait_slab(s + 1);
          load_frags(s + 1, 0, af[nxt], bfr[nxt]);
          spread = s_iss < total;
          if (spread) issue_begin();
        }
        // After a slab's barrier every wave has LOADS copies to issue; issued in one burst
        // they queue at the address unit while the matrix core waits, so they go out one
        // per MFMA of this k-step instead (the rest, if any, after the last MFMA).
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int j = 0; j < FJ; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
            if (ks + 1 == KSTEPS && i * FJ + j < C::LOADS) {
              __builtin_amdgcn_sched_barrier(0);
              if (spread) issue_load(i * FJ + j);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        if (ks + 1 < KSTEPS) {
          // Scheduling groups: the next k-step's fragment reads go out between the first
          // two MFMAs of this k-step (half of them after each), so their LDS latency has
          // the rest of the k-step to pass.  Left to itself the scheduler moved most of
          // them behind the last MFMA, right before their use.
          constexpr int NR = FI + FJ, R = (NR + 1) / 2;
#pragma unroll
          for (int m = 0; m < FI * FJ; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
#pragma unroll
            for (int r = 0; r < R; ++r)
              if (R * m + r < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          }
        }
        if (spread) {
#pragma unroll
          for (int q = FI * FJ; q < C::LOADS; ++q) issue_load(q);
          issue_end();
        }
        if (ks + 1 == KSTEPS) {
          // the fragments loaded above for slab s + 1 move into slot 0
#pragma unroll
          for (int i = 0; i < FI; ++i) af[0][i] = af[nxt][i];
#pragma unroll
          for (int j = 0; j < FJ; ++j) bfr[0][j] = bfr[nxt][j];
        }
      }
    }

    epilogue(it, acc);
  }
}

static int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    hipDeviceProp_t p;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess)
      n = p.multiProcessorCount;
    if (n <= 0) n = 256;
  }
  return n;
}

template <class C, int EPI, bool OUT_F32>
static hipError_t gemm_launch(const uint16_t* A, const uint16_t* W, const float* bias, void* Cp,
                              int M, int N, int K, hipStream_t s, const QkvEpi& qe = QkvEpi{}) {
  constexpr bool QKV = EPI == EPI_QKV64 || EPI == EPI_QKV32;
  constexpr int MAX_LDS = 160 * 1024;
  static_assert(!QKV || C::LDS + 3 * kMaxGridSide * kLdsTabRow * 8 + kPairMapBytes + C::EXTRA <= MAX_LDS,
                "LDS for the RoPE table");
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_kernel<C, EPI, OUT_F32>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, MAX_LDS);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int lds = C::LDS + (QKV ? 3 * qe.ts * kLdsTabRow * 8 + kPairMapBytes : 0) + C::EXTRA;
  const int tiles = ((M + C::BM - 1) / C::BM) * (N / C::BN);
  const dim3 grid(min(tiles, num_cus()));
  gemm_bf16_kernel<C, EPI, OUT_F32><<<grid, C::NT, lds, s>>>(A, W, bias, Cp, M, N, K, qe);
  return hipGetLastError();
}

template <class C>
static hipError_t gemm_dispatch(const uint16_t* A, const uint16_t* W, const float* bias, void* Cp,
                                int M, int N, int K, int epi, int out_f32, hipStream_t s) {
  if (epi == EPI_RESIDUAL) return gemm_launch<C, EPI_RESIDUAL, true>(A, W, bias, Cp, M, N, K, s);
  if (epi == EPI_GELU)
    return out_f32 ? gemm_launch<C, EPI_GELU, true>(A, W, bias, Cp, M, N, K, s)
                   : gemm_launch<C, EPI_GELU, false>(A, W, bias, Cp, M, N, K, s);
  return out_f32 ? gemm_launch<C, EPI_STORE, true>(A, W, bias, Cp, M, N, K, s)
                 : gemm_launch<C, EPI_STORE, false>(A, W, bias, Cp, M, N, K, s);
}

// Width of the 256-row tile (256, 192 or 128, at most max_w): the one with the least
// estimated time, taken as the rounds of the CUs the tiles need times the rows a tile
// streams into LDS per K slab (256 + width), since the slab copies set the pace of the
// main loop; ties go to the wider tile.
static int tile_width(int M, int N, int max_w = 256) {
  const long long cus = num_cus();
  const long long tm = (M + 255) / 256;
  int best = 128;
  long long best_cost = -1;
  for (int w : {256, 192, 128}) {
    if (w > max_w || N % w) continue;
    const long long rounds = (tm * (N / w) + cus - 1) / cus;
    const long long cost = rounds * (256 + w);
    if (best_cost < 0 || cost < best_cost) {
      best = w;
      best_cost = cost;
    }
  }
  return best;
}

// Whether 128-row tiles are used: only when 256 x 128 tiles would be fewer than the CUs,
// and then by the same estimate as tile_width (rounds of the CUs times the rows a tile
// streams per slab), so that 9216 rows of N = 768 take one round of 216 tiles of 256 x 128
// rather than 1.7 rounds of 432 tiles of 128 x 128, while 2048 rows keep the small tiles.
// The tile shape does not change the order in which an output element sums over K.
static bool short_rows(int M, int N) {
  const long long cus = num_cus();
  const long long t256 = static_cast<long long>((M + 255) / 256) * (N / 128);
  if (t256 >= cus) return false;
  const long long t128 = static_cast<long long>((M + 127) / 128) * (N / 128);
  return (t128 + cus - 1) / cus * (128 + 128) < (t256 + cus - 1) / cus * (256 + 128);
}

static bool gemm_shape_ok(int M, int N, int K) {
  // N in whole 128-column tiles, K in whole slabs; the DMA addressing uses 32-bit byte
  // offsets
  return N % 128 == 0 && K % 64 == 0 && static_cast<size_t>(M) * K * 2 < (size_t(1) << 31) &&
         static_cast<size_t>(N) * K * 2 < (size_t(1) << 31);
}

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C,
                            int M, int N, int K, int epi, int out_f32, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!gemm_shape_ok(M, N, K)) return hipErrorInvalidValue;
  if (short_rows(M, N)) {
    // 128 x 64 tiles when they take fewer rounds x rows streamed per slab (128 + 64)
    const long long cus = num_cus(), tm = (M + 127) / 128;
    const long long r128 = (tm * (N / 128) + cus - 1) / cus, r64 = (tm * (N / 64) + cus - 1) / cus;
    if (r64 * (128 + 64) < r128 * (128 + 128))
      return gemm_dispatch<Cfg128x64>(A, W, bias, C, M, N, K, epi, out_f32, s);
    return gemm_dispatch<Cfg128x128>(A, W, bias, C, M, N, K, epi, out_f32, s);
  }
  const int tw = tile_width(M, N);
  if (tw == 256) return gemm_dispatch<Cfg256x256>(A, W, bias, C, M, N, K, epi, out_f32, s);
  if (tw == 192) return gemm_dispatch<Cfg256x192>(A, W, bias, C, M, N, K, epi, out_f32, s);
  return gemm_dispatch<Cfg256x128>(A, W, bias, C, M, N, K, epi, out_f32, s);
}

template <class C>
static hipError_t gemm_qkv_dispatch(const uint16_t* A, const uint16_t* W, const float* bias,
                                    uint16_t* Cp, int M, int N, int K, int head_dim,
                                    const QkvEpi& qe, hipStream_t s) {
  if (head_dim == 64) return gemm_launch<C, EPI_QKV64, false>(A, W, bias, Cp, M, N, K, s, qe);
  return gemm_launch<C, EPI_QKV32, false>(A, W, bias, Cp, M, N, K, s, qe);
}

hipError_t launch_gemm_bf16_qkv(const uint16_t* A, const uint16_t* W, const float* bias,
                                uint16_t* C, uint16_t* vt, int Ns, int M, int D, int K,
                                int head_dim, const int32_t* ids, int ids_stride, int N,
                                const RopeSpec& r, const void* tab, float qscale, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int Ncol = 3 * D;
  if (!gemm_shape_ok(M, Ncol, K) || (head_dim != 64 && head_dim != 32) || D % head_dim ||
      D % 32 || N <= 0 || M % N || Ns < N)
    return hipErrorInvalidValue;
  QkvEpi qe;
  qe.vt = vt;
  qe.ra = RopeArgs{static_cast<const float2*>(tab), ids, N, r.layout, r.gt * r.gh * r.gw, r.gh, r.gw,
                   ids_stride};
  qe.D = D;
  qe.H = D / head_dim;
  qe.Ns = Ns;
  qe.ts = max(r.gt, max(r.gh, r.gw));
  qe.qscale = qscale;
  if (qe.ts > kMaxGridSide) return hipErrorInvalidValue;
  if (short_rows(M, Ncol)) return gemm_qkv_dispatch<Cfg128x128q>(A, W, bias, C, M, Ncol, K, head_dim, qe, s);
  // the 256 x 256 tile leaves too few registers for the RoPE epilogue
  const int tw = tile_width(M, Ncol, 192);
  if (tw == 192) return gemm_qkv_dispatch<Cfg256x192>(A, W, bias, C, M, Ncol, K, head_dim, qe, s);
  return gemm_qkv_dispatch<Cfg256x128q>(A, W, bias, C, M, Ncol, K, head_dim, qe, s);
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

// C[m, n] = A[m, :] . W[n, :] + bias[n] (fp32) for a few rows of A: one wavefront per output,
// lanes stride over K (coalesced rows of W), four partial sums per lane added in order and
// a butterfly over the wave, so every output sums in a fixed order whatever M is.
__global__ __launch_bounds__(64)
void gemv_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                     const float* __restrict__ bias, float* __restrict__ C, int N, int K) {
  const int n = blockIdx.x, m = blockIdx.y, lane = threadIdx.x;
  const float* a = A + static_cast<size_t>(m) * K;
  const float* w = W + static_cast<size_t>(n) * K;
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  int k = lane;
  for (; k + 192 < K; k += 256) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fmaf(a[k + 64 * i], w[k + 64 * i], p[i]);
  }
  for (int i = 0; k < K; k += 64, ++i) p[i & 3] = fmaf(a[k], w[k], p[i & 3]);
  float s = (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) C[static_cast<size_t>(m) * N + n] = s + (bias ? bias[n] : 0.f);
}

hipError_t launch_gemv_f32(const float* A, const float* W, const float* bias, float* C, int M,
                           int N, int K, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M > 65535) return hipErrorInvalidValue;
  gemv_f32_kernel<<<dim3(N, M), 64, 0, s>>>(A, W, bias, C, N, K);
  return hipGetLastError();
}

}  // namespace jepa
