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
// Frequencies per axis the RoPE tables hold (d/2 <= 16, i.e. head dims up to 96).
constexpr int kRopeMaxFreq = 16;
// Entries of a RoPE table (float2 each): 3 axes x kMaxGridSide coordinates x kRopeMaxFreq.
constexpr int kRopeTabEntries = 3 * kMaxGridSide * kRopeMaxFreq;

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* W, const float* bias, void* C,
                            int M, int N, int K, int epi, int out_f32, hipStream_t s);
hipError_t launch_gemm_f32(const float* A, const float* W, const float* bias, float* C,
                           int M, int N, int K, int epi, hipStream_t s);
// C = A W^T + bias (fp32) with one wavefront per output, for few rows (M <= 65535).
hipError_t launch_gemv_f32(const float* A, const float* W, const float* bias, float* C, int M,
                           int N, int K, hipStream_t s);
hipError_t launch_layernorm(const float* x, const float* w, const float* b, int M, int D,
                            float eps, void* out, int out_bf16, hipStream_t s);
// Row lengths the LayerNorm kernel is instantiated for: D = 64 * vpt with vpt in this list
// (D = 1408, vpt 22, is the ViT-g width).
inline bool layernorm_width_ok(int D) {
  if (D <= 0 || D % 64) return false;
  switch (D / 64) {
    case 1: case 2: case 3: case 4: case 5: case 6: case 8: case 10: case 12: case 16:
    case 20: case 22: case 24: case 32: case 40: case 48: case 64:
      return true;
    default:
      return false;
  }
}
hipError_t launch_rope3d(const void* x, void* y, int bf16, int B, int N, int n_head,
                         int head_dim, int64_t row_stride, const int32_t* ids,
                         const RopeSpec& r, hipStream_t s);
// (cos, sin) table of the grid for head dim head_dim (layout in rope_tab.h).
hipError_t launch_rope_table(void* tab, const RopeSpec& r, int head_dim, hipStream_t s);
// QKV projection (bf16) whose epilogue rotates q and k, scales q by qscale and writes v
// transposed: q, k into C [M, 3D] (columns [0, 2D)), v into vt [B][H][hd][Ns].
hipError_t launch_gemm_bf16_qkv(const uint16_t* A, const uint16_t* W, const float* bias,
                                uint16_t* C, uint16_t* vt, int Ns, int M, int D, int K,
                                int head_dim, const int32_t* ids, int ids_stride, int N,
                                const RopeSpec& r, const void* tab, float qscale, hipStream_t s);
// The same preparation from a projection already in memory: qkv [M, 3D] bf16 ->
// q', k' into qk [M, 2D] and v into vt [B][H][hd][Ns].  Without ids, rows n < lead of a
// clip (CLS rows) keep q and k unrotated and row n >= lead is grid token n - lead.
hipError_t launch_qkv_prepare(const uint16_t* qkv, uint16_t* qk, uint16_t* vt, int Ns, int B,
                              int N, int n_head, int head_dim, const int32_t* ids,
                              const RopeSpec& r, const void* tab, float qscale, hipStream_t s,
                              int lead = 0);
// Flash attention on prepared inputs: q (rotated, scaled by log2(e)/sqrt(hd)) and k
// (rotated) rows of leading dimension ld (elements), v transposed [B][H][hd][Ns];
// out [B*N, H*hd] bf16.  slot > 0: block-causal mask with n_cls (< 64) leading CLS rows
// that see every key, the other rows in temporal slots of `slot` tokens that see the
// non-CLS keys of their own and earlier slots.
// Long clips whose (head, query block) pairs would fill the compute units poorly take
// their keys in pieces, merged by a second kernel (a choice made from N and n_head
// only); those need split_ws, attention_split_bytes(B, N, n_head, head_dim) bytes
// (16-byte aligned, contents on entry do not matter).  Calls that overlap on one split_ws
// race.
hipError_t launch_attention_fwd(const uint16_t* q, const uint16_t* k, int ld, const uint16_t* vt,
                                int Ns, uint16_t* out, int B, int N, int n_head, int head_dim,
                                hipStream_t s, int n_cls = 0, int slot = 0,
                                void* split_ws = nullptr);
// Bytes of split_ws for B unmasked clips of N tokens (0: the keys are taken whole).
size_t attention_split_bytes(int B, int N, int n_head, int head_dim);
// Row stride (keys) of the transposed V layout for N tokens.
inline int vt_stride(int N) { return (N + 15) / 16 * 16; }
// Scale folded into q: log2(e) / sqrt(head_dim).
inline float attn_qscale(int head_dim) {
  return static_cast<float>(1.4426950408889634 / __builtin_sqrt(static_cast<double>(head_dim)));
}
// ids: grid ids of clip b at ids + b * ids_stride (NULL: row n is token n - n_cls, the
// n_cls leading CLS rows unrotated); slot > 0 adds the block-causal mask as above.
hipError_t launch_attention_f32(const float* qkv, float* out, int B, int N, int n_head,
                                int head_dim, const int32_t* ids, int ids_stride,
                                const RopeSpec& r, hipStream_t s, int n_cls = 0, int slot = 0);
// uint8 [B,T,H,W,3] -> normalised patch rows (bf16 or fp32): all B*N tokens ([B*N, 1536],
// ids NULL), or the K tokens ids[b*K + k] of each clip ([B*K, 1536], ids clamped to [0, N)).
hipError_t launch_patchify(const uint8_t* clip, int B, int T, int H, int W, void* A, int bf16,
                           hipStream_t s, const int32_t* ids = nullptr, int K = 0);
// uint8 images [B,H,W,3] -> normalised 1x16x16x3 patch rows [B*N, 768] (2.1 image path).
hipError_t launch_patchify_image(const uint8_t* img, int B, int H, int W, void* A, int bf16,
                                 hipStream_t s);
// dst[i, :] = src[clamp(ids[i]), :] (fp32 -> bf16 or fp32), i < n.
hipError_t launch_gather_rows(const float* src, int n_src, int D, const int32_t* ids, int n,
                              void* dst, int bf16, hipStream_t s);
// dst[i, :] = vec[:] for i < n (fp32).
hipError_t launch_fill_rows(float* dst, const float* vec, int n, int D, hipStream_t s);
// Single learned query over the N tokens of each clip (attentive-pool cross-attention):
// q fp32 [D] (projected), k and v fp32 rows of leading dimension ld (ld >= D, a multiple of 4),
// y[b] = q0 + concat_h softmax(q_h k_h^T / sqrt(hd)) v_h, fp32 [B, D].  N <= kXattnMaxTokens.
constexpr int kXattnMaxTokens = 16384;
hipError_t launch_xattn_query(const float* q, const float* k, const float* v, int ld,
                              const float* q0, float* y, int B, int N, int n_head, int head_dim,
                              hipStream_t s);
// Mean over the tokens of each clip: x fp32 [B, N, D] -> out fp32 [B, D].
hipError_t launch_mean_pool(const float* x, int B, int N, int D, float* out, hipStream_t s);
// dst[i] = a[i] + b[i] (fp32), i < n.
hipError_t launch_add_vec(float* dst, const float* a, const float* b, int n, hipStream_t s);

}  // namespace jepa
