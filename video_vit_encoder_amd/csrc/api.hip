// C ABI of libjepa: handles, argument checks, weight upload and the kernel sequence of
// the encoder and predictor forwards.  Declarations and conventions: include/jepa.h.
//
// Encoder forward ([Notes §3] "2.1 encoder forward"; block form [Notes §2]):
//   x = patchify(normalise(clip)) Wpe^T + bpe (+ mod_embed_video)
//   per block: x += attn(LN1(x)) Wout^T + bout ; x += GELU(LN2(x) Wup^T + bup) Wdown^T + bdown
//   out = LN_final(x)
// The residual stream x is fp32 and lives in the caller's output buffer; LayerNorm
// outputs, q|k|v, the attention output and the FFN hidden activations are in the
// compute dtype (bf16 on the MFMA path).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/jepa.h"
#include "kernels.h"

using namespace jepa;

namespace {

constexpr int kVersion = 100;  // 0.1.0

// ------------------------------------------------------------------ helpers

// Bytes past the last transposed-V row that the attention kernel's last key tile reads
// (at most 63 keys of 2 bytes; rounded up).
constexpr size_t kVtSlackBytes = 4096;

uint16_t host_f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) {  // inf / nan: keep, quiet the nan
    uint16_t h = static_cast<uint16_t>(u >> 16);
    if (u & 0x007FFFFFu) h |= 0x40;
    return h;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

float host_bf16_to_f32(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
};

int dev_alloc(DevBuf& b, size_t bytes) {
  if (b.p) return JEPA_OK;
  if (bytes == 0) bytes = 16;
  if (hipMalloc(&b.p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    b.p = nullptr;
    return JEPA_ERR_OOM;
  }
  b.bytes = bytes;
  return JEPA_OK;
}

void dev_free(DevBuf& b) {
  if (b.p) (void)hipFree(b.p);
  b.p = nullptr;
  b.bytes = 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? JEPA_OK : JEPA_ERR_HIP; }

#define JEPA_TRY(expr)                 \
  do {                                 \
    const int _st = (expr);            \
    if (_st != JEPA_OK) return _st;    \
  } while (0)

#define JEPA_HIP(expr)                               \
  do {                                               \
    if ((expr) != hipSuccess) {                      \
      (void)hipGetLastError();                       \
      return JEPA_ERR_HIP;                           \
    }                                                \
  } while (0)

// ------------------------------------------------------------------ kernel timing

// Event pairs around the launches of the forwards (jepa_timing_begin / _end).
struct Timing {
  bool on = false;
  int cap = 0;
  std::vector<hipEvent_t> ev[JEPA_KC_COUNT];  // per class: start, end of launch i at 2i, 2i+1
  int n[JEPA_KC_COUNT] = {};
};
Timing g_timing;

// Records the start event of one launch on construction and its end on destruction.
struct KTimer {
  int kc = -1;
  hipStream_t s;
  KTimer(int kind, hipStream_t st) : s(st) {
    if (g_timing.on && g_timing.n[kind] < g_timing.cap) {
      kc = kind;
      (void)hipEventRecord(g_timing.ev[kind][2 * g_timing.n[kind]], s);
    }
  }
  ~KTimer() {
    if (kc >= 0) {
      (void)hipEventRecord(g_timing.ev[kc][2 * g_timing.n[kc] + 1], s);
      ++g_timing.n[kc];
    }
  }
};

// A launch of kernel class kc on stream st, timed when timing is on.
#define JEPA_LAUNCH(kc, st, expr) \
  do {                            \
    KTimer _kt((kc), (st));       \
    JEPA_HIP(expr);               \
  } while (0)

// One weight tensor: expected shape, kind and device copy.
struct Tensor {
  std::string name;
  std::vector<int64_t> shape;
  bool matrix = false;   // stored in the compute dtype; vectors stay fp32
  bool set = false;
  bool required = true;
  DevBuf dev;
  std::vector<float> host;  // kept for vectors that are combined on the host
  bool keep_host = false;

  int64_t numel() const {
    int64_t n = 1;
    for (int64_t s : shape) n *= s;
    return n;
  }
};

struct TensorSet {
  std::vector<Tensor> t;
  int compute = JEPA_BF16;

  int add(const std::string& name, std::vector<int64_t> shape, bool matrix, bool keep_host = false) {
    Tensor x;
    x.name = name;
    x.shape = std::move(shape);
    x.matrix = matrix;
    x.keep_host = keep_host;
    t.push_back(std::move(x));
    return static_cast<int>(t.size()) - 1;
  }

  ~TensorSet() {
    for (Tensor& x : t) dev_free(x.dev);
  }

  int find(const char* name) const {
    for (size_t i = 0; i < t.size(); ++i)
      if (t[i].name == name) return static_cast<int>(i);
    return -1;
  }

  bool all_set() const {
    for (const Tensor& x : t)
      if (x.required && !x.set) return false;
    return true;
  }

  // Upload `host` (numel values of src_dtype) into tensor i.
  int upload(int i, const void* host, int src_dtype) {
    Tensor& x = t[i];
    const int64_t n = x.numel();
    std::vector<float> f(static_cast<size_t>(n));
    if (src_dtype == JEPA_F32) {
      std::memcpy(f.data(), host, static_cast<size_t>(n) * 4);
    } else {
      const uint16_t* h = static_cast<const uint16_t*>(host);
      for (int64_t k = 0; k < n; ++k) f[k] = host_bf16_to_f32(h[k]);
    }
    const bool as_bf16 = x.matrix && compute == JEPA_BF16;
    const size_t bytes = static_cast<size_t>(n) * (as_bf16 ? 2 : 4);
    JEPA_TRY(dev_alloc(x.dev, bytes));
    if (as_bf16) {
      std::vector<uint16_t> h(static_cast<size_t>(n));
      if (src_dtype == JEPA_BF16)
        std::memcpy(h.data(), host, static_cast<size_t>(n) * 2);
      else
        for (int64_t k = 0; k < n; ++k) h[k] = host_f32_to_bf16(f[k]);
      JEPA_HIP(hipMemcpy(x.dev.p, h.data(), bytes, hipMemcpyHostToDevice));
    } else {
      JEPA_HIP(hipMemcpy(x.dev.p, f.data(), bytes, hipMemcpyHostToDevice));
    }
    if (x.keep_host) x.host = std::move(f);
    x.set = true;
    return JEPA_OK;
  }

  int set_tensor(const char* name, const void* host, int src_dtype, const int64_t* shape,
                 int ndim) {
    if (!name || !host || !shape) return JEPA_ERR_ARG;
    if (src_dtype != JEPA_F32 && src_dtype != JEPA_BF16) return JEPA_ERR_ARG;
    const int i = find(name);
    if (i < 0) return JEPA_ERR_NAME;
    const Tensor& x = t[i];
    if (ndim != static_cast<int>(x.shape.size())) return JEPA_ERR_NAME;
    for (int k = 0; k < ndim; ++k)
      if (shape[k] != x.shape[k]) return JEPA_ERR_NAME;
    return upload(i, host, src_dtype);
  }

  const void* dev(int i) const { return t[i].dev.p; }
  const float* devf(int i) const { return static_cast<const float*>(t[i].dev.p); }
};

// Per-block tensor indices.
struct BlockIdx {
  int ln1w, ln1b, qkvw, qkvb, outw, outb, ln2w, ln2b, upw, upb, downw, downb;
};

BlockIdx add_block(TensorSet& ts, const std::string& p, int64_t d, int64_t f) {
  BlockIdx b;
  b.ln1w = ts.add(p + ".ln1.weight", {d}, false);
  b.ln1b = ts.add(p + ".ln1.bias", {d}, false);
  b.qkvw = ts.add(p + ".attn_qkv.weight", {3 * d, d}, true);
  b.qkvb = ts.add(p + ".attn_qkv.bias", {3 * d}, false);
  b.outw = ts.add(p + ".attn_out.weight", {d, d}, true);
  b.outb = ts.add(p + ".attn_out.bias", {d}, false);
  b.ln2w = ts.add(p + ".ln2.weight", {d}, false);
  b.ln2b = ts.add(p + ".ln2.bias", {d}, false);
  b.upw = ts.add(p + ".ffn_up.weight", {f, d}, true);
  b.upb = ts.add(p + ".ffn_up.bias", {f}, false);
  b.downw = ts.add(p + ".ffn_down.weight", {d, f}, true);
  b.downb = ts.add(p + ".ffn_down.bias", {d}, false);
  return b;
}

// Shape limits of the kernels, for a model width / FFN width / head dim.
int check_widths(int compute, int D, int F, int n_head, int head_dim) {
  if (compute != JEPA_F32 && compute != JEPA_BF16) return JEPA_ERR_ARG;
  if (D <= 0 || F <= 0 || n_head <= 0) return JEPA_ERR_ARG;
  if (head_dim * n_head != D) return JEPA_ERR_ARG;
  if (head_dim != 64 && head_dim != 32) return JEPA_ERR_ARG;
  if (!layernorm_width_ok(D)) return JEPA_ERR_ARG;  // LayerNorm kernel instantiations
  if (compute == JEPA_BF16 && (D % 128 != 0 || F % 128 != 0)) return JEPA_ERR_ARG;  // GEMM tiles
  if (compute == JEPA_F32 && (F % 4 != 0)) return JEPA_ERR_ARG;
  return JEPA_OK;
}

int check_grid(int gt, int gh, int gw, int ref_grid) {
  if (gt < 1 || gh < 1 || gw < 1) return JEPA_ERR_SHAPE;
  if (gt > kMaxGridSide || gh > kMaxGridSide || gw > kMaxGridSide) return JEPA_ERR_SHAPE;
  if (ref_grid < 0 || ref_grid == 1) return JEPA_ERR_ARG;
  // [Notes §4.3]: the interpolation divides by (side - 1)
  if (ref_grid > 1 && (gh < 2 || gw < 2)) return JEPA_ERR_SHAPE;
  return JEPA_OK;
}

// Workspace of the block sequence for `rows` token rows.
struct Workspace {
  DevBuf h, qkv, o, g, a, vt, tab, split;
  int rows = 0;
  size_t vt_rows = 0;  // capacity of vt in (clip, key) rows of D values
  ~Workspace() {
    dev_free(h);
    dev_free(qkv);
    dev_free(o);
    dev_free(g);
    dev_free(a);
    dev_free(vt);
    dev_free(tab);
    dev_free(split);
  }
  int alloc(int max_rows, int D, int F, int a_cols, int compute, int n_head) {
    rows = max_rows;
    const size_t es = compute == JEPA_BF16 ? 2 : 4;
    const size_t m = static_cast<size_t>(max_rows);
    JEPA_TRY(dev_alloc(h, m * D * es));
    JEPA_TRY(dev_alloc(qkv, m * 3 * D * es));
    JEPA_TRY(dev_alloc(o, m * D * es));
    JEPA_TRY(dev_alloc(g, m * F * es));
    if (a_cols > 0) JEPA_TRY(dev_alloc(a, m * a_cols * es));
    if (compute == JEPA_BF16) {
      // v transposed per (clip, head) with rows padded to 16 keys, plus the bytes the
      // attention kernel's last key tile reads past the final row
      vt_rows = 2 * m + 1024;
      JEPA_TRY(dev_alloc(vt, vt_rows * D * 2 + kVtSlackBytes));
      if (hipMemset(vt.p, 0, vt.bytes) != hipSuccess) return JEPA_ERR_HIP;
      JEPA_TRY(dev_alloc(tab, static_cast<size_t>(kRopeTabEntries) * 8));
      // key pieces of long clips: the most any B clips of N tokens with B N <= max_rows
      // need
      size_t most = 0;
      for (int n = 1; n <= max_rows; ++n)
        most = std::max(most, attention_split_bytes(max_rows / n, n, n_head, D / n_head));
      if (most > 0) JEPA_TRY(dev_alloc(split, most));
    }
    return JEPA_OK;
  }
  // The bf16 attention path fits B clips of N tokens.
  bool vt_fits(int B, int N) const { return static_cast<size_t>(B) * vt_stride(N) <= vt_rows; }
};

// GEMM in the compute dtype.  out_f32 selects fp32 output for the STORE/GELU epilogues.
hipError_t linear(int compute, const void* A, const void* W, const float* bias, void* C, int M,
                  int N, int K, int epi, int out_f32, hipStream_t s) {
  if (compute == JEPA_BF16)
    return launch_gemm_bf16(static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(W), bias,
                            C, M, N, K, epi, out_f32, s);
  return launch_gemm_f32(static_cast<const float*>(A), static_cast<const float*>(W), bias,
                         static_cast<float*>(C), M, N, K, epi, s);
}

// The pre-norm blocks over x (fp32 [B*N, D], in place).  On the bf16 path the QKV
// projection's epilogue applies the 3-D RoPE to q and k (q also takes log2(e)/sqrt(hd))
// and writes v transposed; the attention kernel then reads all three by DMA.  Token n of
// clip b sits at grid id ids[b * ids_stride + n] (ids NULL: n).
int run_blocks(const TensorSet& ts, const std::vector<BlockIdx>& blocks, int n_run, Workspace& ws,
               float* x, int B, int N, int D, int F, int n_head, float eps, const int32_t* ids,
               int ids_stride, const RopeSpec& rs, hipStream_t s) {
  const int compute = ts.compute;
  const int bf = compute == JEPA_BF16 ? 1 : 0;
  const int M = B * N;
  const int hd = D / n_head;
  const int Ns = vt_stride(N);
  if (bf && n_run > 0) {
    if (!ws.vt_fits(B, N)) return JEPA_ERR_SHAPE;
    if (attention_split_bytes(B, N, n_head, hd) > ws.split.bytes) return JEPA_ERR_SHAPE;
    JEPA_LAUNCH(JEPA_KC_OTHER, s, launch_rope_table(ws.tab.p, rs, hd, s));
  }
  for (int l = 0; l < n_run; ++l) {
    const BlockIdx& b = blocks[l];
    JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
                launch_layernorm(x, ts.devf(b.ln1w), ts.devf(b.ln1b), M, D, eps, ws.h.p, bf, s));
    if (bf) {
      uint16_t* qkv = static_cast<uint16_t*>(ws.qkv.p);
      uint16_t* vt = static_cast<uint16_t*>(ws.vt.p);
      JEPA_LAUNCH(JEPA_KC_GEMM_QKV, s,
                  launch_gemm_bf16_qkv(static_cast<const uint16_t*>(ws.h.p),
                                       static_cast<const uint16_t*>(ts.dev(b.qkvw)), ts.devf(b.qkvb),
                                       qkv, vt, Ns, M, D, D, hd, ids, ids_stride, N, rs, ws.tab.p,
                                       attn_qscale(hd), s));
      JEPA_LAUNCH(JEPA_KC_ATTENTION, s,
                  launch_attention_fwd(qkv, qkv + D, 3 * D, vt, Ns, static_cast<uint16_t*>(ws.o.p), B,
                                       N, n_head, hd, s, 0, 0, ws.split.p));
    } else {
      JEPA_LAUNCH(JEPA_KC_GEMM_QKV, s,
                  linear(compute, ws.h.p, ts.dev(b.qkvw), ts.devf(b.qkvb), ws.qkv.p, M, 3 * D, D,
                         JEPA_EPI_STORE, 1, s));
      JEPA_LAUNCH(JEPA_KC_ATTENTION, s,
                  launch_attention_f32(static_cast<const float*>(ws.qkv.p),
                                       static_cast<float*>(ws.o.p), B, N, n_head, hd, ids,
                                       ids_stride, rs, s));
    }
    JEPA_LAUNCH(JEPA_KC_GEMM_OUT, s,
                linear(compute, ws.o.p, ts.dev(b.outw), ts.devf(b.outb), x, M, D, D,
                       JEPA_EPI_RESIDUAL, 1, s));
    JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
                launch_layernorm(x, ts.devf(b.ln2w), ts.devf(b.ln2b), M, D, eps, ws.h.p, bf, s));
    JEPA_LAUNCH(JEPA_KC_GEMM_UP, s,
                linear(compute, ws.h.p, ts.dev(b.upw), ts.devf(b.upb), ws.g.p, M, F, D,
                       JEPA_EPI_GELU, !bf, s));
    JEPA_LAUNCH(JEPA_KC_GEMM_DOWN, s,
                linear(compute, ws.g.p, ts.dev(b.downw), ts.devf(b.downb), x, M, D, F,
                       JEPA_EPI_RESIDUAL, 1, s));
  }
  return JEPA_OK;
}

}  // namespace

// ==================================================================== encoder

struct jepa_encoder {
  jepa_encoder_config cfg;
  TensorSet ts;
  std::vector<BlockIdx> blocks;
  int pe_w = -1, pe_b = -1, mod = -1, norm_w = -1, norm_b = -1;
  int img_w = -1, img_b = -1, img_mod = -1;   // 2.1 image path (has_image_embed)
  DevBuf pe_bias_eff;   // bpe + mod_embed_video (when has_mod_embed), fp32 [D]
  DevBuf img_bias_eff;  // bpe_img + mod_embed_img (when has_mod_embed), fp32 [D]
  bool pe_bias_dirty = true;
  Workspace ws;
};

extern "C" {

int jepa_version(void) { return kVersion; }

const char* jepa_status_str(int status) {
  switch (status) {
    case JEPA_OK: return "ok";
    case JEPA_ERR_ARG: return "invalid argument";
    case JEPA_ERR_SHAPE: return "unsupported shape";
    case JEPA_ERR_STATE: return "handle not ready (a required tensor was never set)";
    case JEPA_ERR_NAME: return "unknown tensor name or shape mismatch";
    case JEPA_ERR_OOM: return "device allocation failed";
    case JEPA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int jepa_encoder_create(const jepa_encoder_config* cfg, jepa_encoder** out) {
  if (!cfg || !out) return JEPA_ERR_ARG;
  *out = nullptr;
  const jepa_encoder_config& c = *cfg;
  if (c.n_head <= 0 || c.embed_dim <= 0) return JEPA_ERR_ARG;
  const int hd = c.embed_dim / c.n_head;
  JEPA_TRY(check_widths(c.compute, c.embed_dim, c.ffn_dim, c.n_head, hd));
  if (c.n_layer < 0 || c.patch != 16 || c.tubelet != 2 || c.in_chans != 3) return JEPA_ERR_ARG;
  if ((c.has_image_embed | c.has_mod_embed | c.final_norm) & ~1) return JEPA_ERR_ARG;
  if (c.rope_layout != JEPA_ROPE_TILED && c.rope_layout != JEPA_ROPE_INTERLEAVED) return JEPA_ERR_ARG;
  if (c.rope_ref_grid < 0 || c.rope_ref_grid == 1) return JEPA_ERR_ARG;
  if (c.max_rows <= 0) return JEPA_ERR_ARG;
  if (!(c.ln_eps > 0.f) || !(c.rope_theta > 1.f)) return JEPA_ERR_ARG;

  jepa_encoder* e = new (std::nothrow) jepa_encoder();
  if (!e) return JEPA_ERR_OOM;
  e->cfg = c;
  e->ts.compute = c.compute;
  const int64_t D = c.embed_dim, F = c.ffn_dim;
  const int64_t feat = static_cast<int64_t>(c.in_chans) * c.tubelet * c.patch * c.patch;
  e->pe_w = e->ts.add("enc.patch_embed.weight", {D, feat}, true);
  e->pe_b = e->ts.add("enc.patch_embed.bias", {D}, false, true);
  if (c.has_mod_embed) e->mod = e->ts.add("enc.mod_embed_video", {D}, false, true);
  for (int i = 0; i < c.n_layer; ++i)
    e->blocks.push_back(add_block(e->ts, "enc.blk." + std::to_string(i), D, F));
  if (c.final_norm) {
    e->norm_w = e->ts.add("enc.norm.weight", {D}, false);
    e->norm_b = e->ts.add("enc.norm.bias", {D}, false);
  }
  if (c.has_image_embed) {
    e->img_w = e->ts.add("enc.patch_embed_img.weight", {D, feat / c.tubelet}, true);
    e->img_b = e->ts.add("enc.patch_embed_img.bias", {D}, false, true);
    if (c.has_mod_embed) e->img_mod = e->ts.add("enc.mod_embed_img", {D}, false, true);
  }
  int st = e->ws.alloc(c.max_rows, c.embed_dim, c.ffn_dim, static_cast<int>(feat), c.compute, c.n_head);
  if (st == JEPA_OK) st = dev_alloc(e->pe_bias_eff, static_cast<size_t>(D) * 4);
  if (st == JEPA_OK && c.has_image_embed) st = dev_alloc(e->img_bias_eff, static_cast<size_t>(D) * 4);
  if (st != JEPA_OK) {
    delete e;
    return st;
  }
  *out = e;
  return JEPA_OK;
}

void jepa_encoder_free(jepa_encoder* enc) {
  if (!enc) return;
  dev_free(enc->pe_bias_eff);
  dev_free(enc->img_bias_eff);
  delete enc;
}

int jepa_encoder_set_tensor(jepa_encoder* enc, const char* name, const void* host,
                            int src_dtype, const int64_t* shape, int ndim) {
  if (!enc) return JEPA_ERR_ARG;
  const int st = enc->ts.set_tensor(name, host, src_dtype, shape, ndim);
  if (st == JEPA_OK) enc->pe_bias_dirty = true;
  return st;
}

// Folds the modality vector into a patch-embedding bias on the host (fp32 sum of the two
// fp32 vectors, the same value the GPU would form).
static int fold_bias(const TensorSet& ts, int bias, int mod, DevBuf& dst) {
  const Tensor& b = ts.t[bias];
  std::vector<float> v(b.host);
  if (mod >= 0) {
    const Tensor& m = ts.t[mod];
    for (size_t i = 0; i < v.size(); ++i) v[i] = v[i] + m.host[i];
  }
  JEPA_HIP(hipMemcpy(dst.p, v.data(), v.size() * 4, hipMemcpyHostToDevice));
  return JEPA_OK;
}

static int refresh_pe_bias(jepa_encoder* e) {
  if (!e->pe_bias_dirty) return JEPA_OK;
  JEPA_TRY(fold_bias(e->ts, e->pe_b, e->mod, e->pe_bias_eff));
  if (e->img_b >= 0) JEPA_TRY(fold_bias(e->ts, e->img_b, e->img_mod, e->img_bias_eff));
  e->pe_bias_dirty = false;
  return JEPA_OK;
}

int jepa_encode(jepa_encoder* enc, const uint8_t* clip_dev, int B, int T, int H, int W,
                float* out_dev, void* stream) {
  if (!enc || !clip_dev || !out_dev) return JEPA_ERR_ARG;
  const jepa_encoder_config& c = enc->cfg;
  if (B < 1 || T < 2 || T % 2 || H < 16 || W < 16 || H % 16 || W % 16) return JEPA_ERR_SHAPE;
  const int gt = T / 2, gh = H / 16, gw = W / 16;
  JEPA_TRY(check_grid(gt, gh, gw, c.rope_ref_grid));
  const long long N = static_cast<long long>(gt) * gh * gw;
  if (static_cast<long long>(B) * N > c.max_rows) return JEPA_ERR_SHAPE;
  if (!enc->ts.all_set()) return JEPA_ERR_STATE;
  JEPA_TRY(refresh_pe_bias(enc));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = static_cast<int>(B * N);
  const int D = c.embed_dim, bf = c.compute == JEPA_BF16 ? 1 : 0;
  const int feat = c.in_chans * c.tubelet * c.patch * c.patch;
  JEPA_LAUNCH(JEPA_KC_PATCHIFY, s, launch_patchify(clip_dev, B, T, H, W, enc->ws.a.p, bf, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              linear(c.compute, enc->ws.a.p, enc->ts.dev(enc->pe_w),
                     static_cast<const float*>(enc->pe_bias_eff.p), out_dev, M, D, feat,
                     JEPA_EPI_STORE, 1, s));
  const RopeSpec rs{gt, gh, gw, c.rope_layout, c.rope_theta, c.rope_ref_grid};
  JEPA_TRY(run_blocks(enc->ts, enc->blocks, c.n_layer, enc->ws, out_dev, B, static_cast<int>(N), D,
                      c.ffn_dim, c.n_head, c.ln_eps, nullptr, 0, rs, s));
  if (c.final_norm)
    JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
                launch_layernorm(out_dev, enc->ts.devf(enc->norm_w), enc->ts.devf(enc->norm_b), M,
                                 D, c.ln_eps, out_dev, 0, s));
  return JEPA_OK;
}

int jepa_encode_tokens(jepa_encoder* enc, const float* x_dev, int B, int N,
                       const int32_t* ids_dev, int gt, int gh, int gw, float* out_dev,
                       void* stream) {
  if (!enc || !x_dev || !out_dev) return JEPA_ERR_ARG;
  const jepa_encoder_config& c = enc->cfg;
  if (B < 1 || N < 1) return JEPA_ERR_SHAPE;
  JEPA_TRY(check_grid(gt, gh, gw, c.rope_ref_grid));
  if (!ids_dev && static_cast<long long>(N) > static_cast<long long>(gt) * gh * gw)
    return JEPA_ERR_SHAPE;
  if (static_cast<long long>(B) * N > c.max_rows) return JEPA_ERR_SHAPE;
  if (!enc->ts.all_set()) return JEPA_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = B * N, D = c.embed_dim;
  if (out_dev != x_dev)
    JEPA_LAUNCH(JEPA_KC_OTHER, s,
                hipMemcpyAsync(out_dev, x_dev, static_cast<size_t>(M) * D * 4,
                               hipMemcpyDeviceToDevice, s));
  const RopeSpec rs{gt, gh, gw, c.rope_layout, c.rope_theta, c.rope_ref_grid};
  JEPA_TRY(run_blocks(enc->ts, enc->blocks, c.n_layer, enc->ws, out_dev, B, N, D, c.ffn_dim,
                      c.n_head, c.ln_eps, ids_dev, 0, rs, s));
  if (c.final_norm)
    JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
                launch_layernorm(out_dev, enc->ts.devf(enc->norm_w), enc->ts.devf(enc->norm_b), M,
                                 D, c.ln_eps, out_dev, 0, s));
  return JEPA_OK;
}

int jepa_encode_image(jepa_encoder* enc, const uint8_t* img_dev, int B, int H, int W,
                      float* out_dev, void* stream) {
  if (!enc || !img_dev || !out_dev || !enc->cfg.has_image_embed) return JEPA_ERR_ARG;
  const jepa_encoder_config& c = enc->cfg;
  if (B < 1 || H < 16 || W < 16 || H % 16 || W % 16) return JEPA_ERR_SHAPE;
  const int gh = H / 16, gw = W / 16;
  JEPA_TRY(check_grid(1, gh, gw, c.rope_ref_grid));
  const long long N = static_cast<long long>(gh) * gw;
  if (static_cast<long long>(B) * N > c.max_rows) return JEPA_ERR_SHAPE;
  if (!enc->ts.all_set()) return JEPA_ERR_STATE;
  JEPA_TRY(refresh_pe_bias(enc));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = static_cast<int>(B * N);
  const int D = c.embed_dim, bf = c.compute == JEPA_BF16 ? 1 : 0;
  const int feat = c.in_chans * c.patch * c.patch;
  // [Notes §3] "2.1 encoder forward", image line: tubelet-1 patches, the image embedding
  // and modality vector, then the blocks on the one-slot grid.
  JEPA_LAUNCH(JEPA_KC_PATCHIFY, s, launch_patchify_image(img_dev, B, H, W, enc->ws.a.p, bf, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              linear(c.compute, enc->ws.a.p, enc->ts.dev(enc->img_w),
                     static_cast<const float*>(enc->img_bias_eff.p), out_dev, M, D, feat,
                     JEPA_EPI_STORE, 1, s));
  const RopeSpec rs{1, gh, gw, c.rope_layout, c.rope_theta, c.rope_ref_grid};
  JEPA_TRY(run_blocks(enc->ts, enc->blocks, c.n_layer, enc->ws, out_dev, B, static_cast<int>(N), D,
                      c.ffn_dim, c.n_head, c.ln_eps, nullptr, 0, rs, s));
  if (c.final_norm)
    JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
                launch_layernorm(out_dev, enc->ts.devf(enc->norm_w), enc->ts.devf(enc->norm_b), M,
                                 D, c.ln_eps, out_dev, 0, s));
  return JEPA_OK;
}

int jepa_encode_masked(jepa_encoder* enc, const uint8_t* clip_dev, int B, int T, int H, int W,
                       const int32_t* ids_dev, int K, float* out_dev, void* stream) {
  if (!enc || !clip_dev || !ids_dev || !out_dev) return JEPA_ERR_ARG;
  const jepa_encoder_config& c = enc->cfg;
  if (B < 1 || T < 2 || T % 2 || H < 16 || W < 16 || H % 16 || W % 16) return JEPA_ERR_SHAPE;
  const int gt = T / 2, gh = H / 16, gw = W / 16;
  JEPA_TRY(check_grid(gt, gh, gw, c.rope_ref_grid));
  const long long N = static_cast<long long>(gt) * gh * gw;
  if (K < 1 || K > N) return JEPA_ERR_SHAPE;
  if (static_cast<long long>(B) * K > c.max_rows) return JEPA_ERR_SHAPE;
  if (!enc->ts.all_set()) return JEPA_ERR_STATE;
  JEPA_TRY(refresh_pe_bias(enc));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = B * K;
  const int D = c.embed_dim, bf = c.compute == JEPA_BF16 ? 1 : 0;
  const int feat = c.in_chans * c.tubelet * c.patch * c.patch;
  // [HFport "Usage"]: the tokens outside the context are dropped before the blocks.  The
  // patch embedding acts on each row alone, so only the K context tubelets of each clip
  // are patchified and embedded.
  JEPA_LAUNCH(JEPA_KC_PATCHIFY, s,
              launch_patchify(clip_dev, B, T, H, W, enc->ws.a.p, bf, s, ids_dev, K));
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              linear(c.compute, enc->ws.a.p, enc->ts.dev(enc->pe_w),
                     static_cast<const float*>(enc->pe_bias_eff.p), out_dev, M, D, feat,
                     JEPA_EPI_STORE, 1, s));
  const RopeSpec rs{gt, gh, gw, c.rope_layout, c.rope_theta, c.rope_ref_grid};
  JEPA_TRY(run_blocks(enc->ts, enc->blocks, c.n_layer, enc->ws, out_dev, B, K, D, c.ffn_dim,
                      c.n_head, c.ln_eps, ids_dev, K, rs, s));
  if (c.final_norm)
    JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
                launch_layernorm(out_dev, enc->ts.devf(enc->norm_w), enc->ts.devf(enc->norm_b), M,
                                 D, c.ln_eps, out_dev, 0, s));
  return JEPA_OK;
}

}  // extern "C"

// ==================================================================== predictor

struct jepa_predictor {
  jepa_predictor_config cfg;
  TensorSet ts;
  std::vector<BlockIdx> blocks;
  int emb_w = -1, emb_b = -1, mask = -1, norm_w = -1, norm_b = -1, proj_w = -1, proj_b = -1;
  int mod_v = -1, mod_i = -1, pctx_w = -1, pctx_b = -1;   // V-JEPA 2.1 options
  Workspace ws;
  DevBuf x;          // fp32 [max_rows, E] residual stream
  DevBuf ids;        // int32 [max_rows] concat(ids_ctx, ids_tgt)
  DevBuf emb_bias;   // fp32 [2, E]: bemb + mod_embed_video, bemb + mod_embed_img
  DevBuf mask_row;   // fp32 [E]: the mask token plus the modality vector
  bool bias_dirty = true;
};

extern "C" {

int jepa_predictor_create(const jepa_predictor_config* cfg, jepa_predictor** out) {
  if (!cfg || !out) return JEPA_ERR_ARG;
  *out = nullptr;
  const jepa_predictor_config& c = *cfg;
  if (c.n_head <= 0 || c.embed_dim <= 0) return JEPA_ERR_ARG;
  const int hd = c.embed_dim / c.n_head;
  JEPA_TRY(check_widths(c.compute, c.embed_dim, c.ffn_dim, c.n_head, hd));
  if (c.enc_dim <= 0 || c.out_dim <= 0 || c.n_layer < 0 || c.n_mask_tokens < 1) return JEPA_ERR_ARG;
  if (c.compute == JEPA_BF16 && (c.enc_dim % 64 != 0 || c.out_dim % 128 != 0)) return JEPA_ERR_ARG;
  if (c.compute == JEPA_F32 && (c.out_dim % 4 != 0)) return JEPA_ERR_ARG;
  if (c.rope_layout != JEPA_ROPE_TILED && c.rope_layout != JEPA_ROPE_INTERLEAVED) return JEPA_ERR_ARG;
  if (c.max_rows <= 0) return JEPA_ERR_ARG;
  if (!(c.ln_eps > 0.f) || !(c.rope_theta > 1.f)) return JEPA_ERR_ARG;
  if ((c.has_mod_embed | c.has_proj_context) & ~1) return JEPA_ERR_ARG;

  jepa_predictor* p = new (std::nothrow) jepa_predictor();
  if (!p) return JEPA_ERR_OOM;
  p->cfg = c;
  p->ts.compute = c.compute;
  const int64_t E = c.embed_dim, F = c.ffn_dim;
  p->emb_w = p->ts.add("pred.embed.weight", {E, c.enc_dim}, true);
  p->emb_b = p->ts.add("pred.embed.bias", {E}, false, true);
  p->mask = p->ts.add("pred.mask_tokens", {c.n_mask_tokens, E}, false);
  for (int i = 0; i < c.n_layer; ++i)
    p->blocks.push_back(add_block(p->ts, "pred.blk." + std::to_string(i), E, F));
  p->norm_w = p->ts.add("pred.norm.weight", {E}, false);
  p->norm_b = p->ts.add("pred.norm.bias", {E}, false);
  p->proj_w = p->ts.add("pred.proj.weight", {c.out_dim, E}, true);
  p->proj_b = p->ts.add("pred.proj.bias", {c.out_dim}, false);
  if (c.has_mod_embed) {
    p->mod_v = p->ts.add("pred.mod_embed_video", {E}, false, true);
    p->mod_i = p->ts.add("pred.mod_embed_img", {E}, false, true);
  }
  if (c.has_proj_context) {
    p->pctx_w = p->ts.add("pred.proj_context.weight", {c.out_dim, E}, true);
    p->pctx_b = p->ts.add("pred.proj_context.bias", {c.out_dim}, false);
  }
  int st = p->ws.alloc(c.max_rows, c.embed_dim, c.ffn_dim, c.enc_dim, c.compute, c.n_head);
  if (st == JEPA_OK) st = dev_alloc(p->x, static_cast<size_t>(c.max_rows) * E * 4);
  if (st == JEPA_OK) st = dev_alloc(p->ids, static_cast<size_t>(c.max_rows) * 4);
  if (st == JEPA_OK) st = dev_alloc(p->emb_bias, static_cast<size_t>(2) * E * 4);
  if (st == JEPA_OK) st = dev_alloc(p->mask_row, static_cast<size_t>(E) * 4);
  if (st != JEPA_OK) {
    dev_free(p->x);
    dev_free(p->ids);
    dev_free(p->emb_bias);
    dev_free(p->mask_row);
    delete p;
    return st;
  }
  *out = p;
  return JEPA_OK;
}

void jepa_predictor_free(jepa_predictor* pred) {
  if (!pred) return;
  dev_free(pred->x);
  dev_free(pred->ids);
  dev_free(pred->emb_bias);
  dev_free(pred->mask_row);
  delete pred;
}

int jepa_predictor_set_tensor(jepa_predictor* pred, const char* name, const void* host,
                              int src_dtype, const int64_t* shape, int ndim) {
  if (!pred) return JEPA_ERR_ARG;
  const int st = pred->ts.set_tensor(name, host, src_dtype, shape, ndim);
  if (st == JEPA_OK) pred->bias_dirty = true;
  return st;
}

int jepa_predict(jepa_predictor* pred, const float* z_dev, int n_enc,
                 const int32_t* ids_ctx_dev, int n_ctx, const int32_t* ids_tgt_dev, int n_tgt,
                 int mask_index, int gt, int gh, int gw, float* out_dev, void* stream) {
  return jepa_predict_mod(pred, z_dev, n_enc, ids_ctx_dev, n_ctx, ids_tgt_dev, n_tgt, mask_index,
                          JEPA_MODALITY_VIDEO, gt, gh, gw, out_dev, nullptr, stream);
}

int jepa_predict_mod(jepa_predictor* pred, const float* z_dev, int n_enc,
                     const int32_t* ids_ctx_dev, int n_ctx, const int32_t* ids_tgt_dev, int n_tgt,
                     int mask_index, int modality, int gt, int gh, int gw, float* out_dev,
                     float* ctx_out_dev, void* stream) {
  if (!pred || !z_dev || !ids_ctx_dev || !ids_tgt_dev || !out_dev) return JEPA_ERR_ARG;
  if (modality != JEPA_MODALITY_VIDEO && modality != JEPA_MODALITY_IMAGE &&
      modality != JEPA_MODALITY_AUTO)
    return JEPA_ERR_ARG;
  const jepa_predictor_config& c = pred->cfg;
  if (ctx_out_dev && !c.has_proj_context) return JEPA_ERR_ARG;
  if (n_ctx < 1 || n_tgt < 1 || n_enc < 1) return JEPA_ERR_SHAPE;
  if (static_cast<long long>(n_ctx) + n_tgt > c.max_rows) return JEPA_ERR_SHAPE;
  JEPA_TRY(check_grid(gt, gh, gw, 0));
  if (static_cast<long long>(gt) * gh * gw != n_enc) return JEPA_ERR_SHAPE;
  if (!pred->ts.all_set()) return JEPA_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = c.embed_dim, bf = c.compute == JEPA_BF16 ? 1 : 0;
  const int M = n_ctx + n_tgt;
  float* x = static_cast<float*>(pred->x.p);
  int32_t* ids = static_cast<int32_t*>(pred->ids.p);
  // V-JEPA 2.1: the modality vector goes onto every row.  On the context rows it is folded
  // into the embedding bias (host fp32 sums, refreshed after set_tensor), on the mask rows
  // it is added to the mask token before the fill.
  const bool mod = c.has_mod_embed != 0;
  const bool img = mod && (modality == JEPA_MODALITY_IMAGE || (modality == JEPA_MODALITY_AUTO && gt == 1));
  if (mod && pred->bias_dirty) {
    DevBuf v{pred->emb_bias.p, static_cast<size_t>(E) * 4};
    DevBuf i{static_cast<float*>(pred->emb_bias.p) + E, static_cast<size_t>(E) * 4};
    JEPA_TRY(fold_bias(pred->ts, pred->emb_b, pred->mod_v, v));
    JEPA_TRY(fold_bias(pred->ts, pred->emb_b, pred->mod_i, i));
    pred->bias_dirty = false;
  }
  const float* emb_bias = mod ? static_cast<const float*>(pred->emb_bias.p) + (img ? E : 0)
                              : pred->ts.devf(pred->emb_b);
  // [Notes §3] "2.1 predictor forward": embed the context rows, mask tokens at the
  // targets, concatenate; positions from the concatenated ids ([Notes §4.4]).
  JEPA_LAUNCH(JEPA_KC_OTHER, s,
              launch_gather_rows(z_dev, n_enc, c.enc_dim, ids_ctx_dev, n_ctx, pred->ws.a.p, bf, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              linear(c.compute, pred->ws.a.p, pred->ts.dev(pred->emb_w), emb_bias,
                     x, n_ctx, E, c.enc_dim, JEPA_EPI_STORE, 1, s));
  int mi = mask_index % c.n_mask_tokens;
  if (mi < 0) mi += c.n_mask_tokens;
  const float* mask_row = pred->ts.devf(pred->mask) + static_cast<size_t>(mi) * E;
  if (mod) {
    JEPA_LAUNCH(JEPA_KC_OTHER, s,
                launch_add_vec(static_cast<float*>(pred->mask_row.p), mask_row,
                               pred->ts.devf(img ? pred->mod_i : pred->mod_v), E, s));
    mask_row = static_cast<const float*>(pred->mask_row.p);
  }
  JEPA_LAUNCH(JEPA_KC_OTHER, s,
              launch_fill_rows(x + static_cast<size_t>(n_ctx) * E, mask_row, n_tgt, E, s));
  JEPA_LAUNCH(JEPA_KC_OTHER, s,
              hipMemcpyAsync(ids, ids_ctx_dev, static_cast<size_t>(n_ctx) * 4,
                             hipMemcpyDeviceToDevice, s));
  JEPA_LAUNCH(JEPA_KC_OTHER, s,
              hipMemcpyAsync(ids + n_ctx, ids_tgt_dev, static_cast<size_t>(n_tgt) * 4,
                             hipMemcpyDeviceToDevice, s));
  const RopeSpec rs{gt, gh, gw, c.rope_layout, c.rope_theta, 0};
  JEPA_TRY(run_blocks(pred->ts, pred->blocks, c.n_layer, pred->ws, x, 1, M, E, c.ffn_dim,
                      c.n_head, c.ln_eps, ids, 0, rs, s));
  // final norm and output projection: of the target rows only, or of all rows when the
  // context rows also go through pred.proj_context
  const size_t es = bf ? 2 : 4;
  const int first = ctx_out_dev ? 0 : n_ctx;
  JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
              launch_layernorm(x + static_cast<size_t>(first) * E, pred->ts.devf(pred->norm_w),
                               pred->ts.devf(pred->norm_b), M - first, E, c.ln_eps, pred->ws.h.p, bf, s));
  const unsigned char* ht = static_cast<const unsigned char*>(pred->ws.h.p) +
                            static_cast<size_t>(n_ctx - first) * E * es;
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              linear(c.compute, ht, pred->ts.dev(pred->proj_w), pred->ts.devf(pred->proj_b), out_dev,
                     n_tgt, c.out_dim, E, JEPA_EPI_STORE, 1, s));
  if (ctx_out_dev)
    JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
                linear(c.compute, pred->ws.h.p, pred->ts.dev(pred->pctx_w), pred->ts.devf(pred->pctx_b),
                       ctx_out_dev, n_ctx, c.out_dim, E, JEPA_EPI_STORE, 1, s));
  return JEPA_OK;
}

// ==================================================================== pooled outputs

struct jepa_head {
  jepa_head_config cfg;
  TensorSet ts;
  std::vector<BlockIdx> blocks;
  int query = -1, lnkv_w = -1, lnkv_b = -1, q_w = -1, q_b = -1, k_w = -1, k_b = -1, v_w = -1,
      v_b = -1, ln2_w = -1, ln2_b = -1, up_w = -1, up_b = -1, down_w = -1, down_b = -1,
      cls_w = -1, cls_b = -1;
  Workspace ws;
  DevBuf x;    // fp32 [max_rows, D] token rows through the pool blocks
  DevBuf kv;   // fp32 [2, max_rows, D]: k, then v of the cross-attention
  DevBuf q;    // fp32 [D] projected query
  DevBuf y;    // fp32 [max_rows, D] pooled rows (one per clip)
};

int jepa_head_create(const jepa_head_config* cfg, jepa_head** out) {
  if (!cfg || !out) return JEPA_ERR_ARG;
  *out = nullptr;
  const jepa_head_config& c = *cfg;
  if (c.n_head <= 0 || c.embed_dim <= 0 || c.n_layer < 0 || c.n_classes < 1) return JEPA_ERR_ARG;
  const int hd = c.embed_dim / c.n_head;
  JEPA_TRY(check_widths(c.compute, c.embed_dim, c.ffn_dim, c.n_head, hd));
  if (c.max_rows <= 0 || !(c.ln_eps > 0.f)) return JEPA_ERR_ARG;
  jepa_head* h = new (std::nothrow) jepa_head();
  if (!h) return JEPA_ERR_OOM;
  h->cfg = c;
  h->ts.compute = c.compute;
  const int64_t D = c.embed_dim, F = c.ffn_dim;
  h->query = h->ts.add("head.query", {1, D}, false);
  for (int i = 0; i < c.n_layer; ++i)
    h->blocks.push_back(add_block(h->ts, "head.blk." + std::to_string(i), D, F));
  h->lnkv_w = h->ts.add("head.xattn.ln_kv.weight", {D}, false);
  h->lnkv_b = h->ts.add("head.xattn.ln_kv.bias", {D}, false);
  // q sees one row and the classifier has any width: both stay fp32 for the fp32 GEMM
  h->q_w = h->ts.add("head.xattn.q.weight", {D, D}, false);
  h->q_b = h->ts.add("head.xattn.q.bias", {D}, false);
  h->k_w = h->ts.add("head.xattn.k.weight", {D, D}, true);
  h->k_b = h->ts.add("head.xattn.k.bias", {D}, false);
  h->v_w = h->ts.add("head.xattn.v.weight", {D, D}, true);
  h->v_b = h->ts.add("head.xattn.v.bias", {D}, false);
  h->ln2_w = h->ts.add("head.xattn.ln2.weight", {D}, false);
  h->ln2_b = h->ts.add("head.xattn.ln2.bias", {D}, false);
  h->up_w = h->ts.add("head.xattn.ffn_up.weight", {F, D}, true);
  h->up_b = h->ts.add("head.xattn.ffn_up.bias", {F}, false);
  h->down_w = h->ts.add("head.xattn.ffn_down.weight", {D, F}, true);
  h->down_b = h->ts.add("head.xattn.ffn_down.bias", {D}, false);
  h->cls_w = h->ts.add("head.cls.weight", {c.n_classes, D}, false);
  h->cls_b = h->ts.add("head.cls.bias", {c.n_classes}, false);
  const size_t m = static_cast<size_t>(c.max_rows);
  int st = h->ws.alloc(c.max_rows, c.embed_dim, c.ffn_dim, 0, c.compute, c.n_head);
  if (st == JEPA_OK) st = dev_alloc(h->x, m * D * 4);
  if (st == JEPA_OK) st = dev_alloc(h->kv, m * 2 * D * 4);
  if (st == JEPA_OK) st = dev_alloc(h->q, static_cast<size_t>(D) * 4);
  if (st == JEPA_OK) st = dev_alloc(h->y, m * D * 4);
  if (st != JEPA_OK) {
    jepa_head_free(h);
    return st;
  }
  *out = h;
  return JEPA_OK;
}

void jepa_head_free(jepa_head* head) {
  if (!head) return;
  dev_free(head->x);
  dev_free(head->kv);
  dev_free(head->q);
  dev_free(head->y);
  delete head;
}

int jepa_head_set_tensor(jepa_head* head, const char* name, const void* host, int src_dtype,
                         const int64_t* shape, int ndim) {
  if (!head) return JEPA_ERR_ARG;
  return head->ts.set_tensor(name, host, src_dtype, shape, ndim);
}

int jepa_head_forward(jepa_head* head, const float* x_dev, int B, int N, float* logits_dev,
                      void* stream) {
  if (!head || !x_dev || !logits_dev) return JEPA_ERR_ARG;
  const jepa_head_config& c = head->cfg;
  if (B < 1 || N < 1 || N > kXattnMaxTokens) return JEPA_ERR_SHAPE;
  if (static_cast<long long>(B) * N > c.max_rows) return JEPA_ERR_SHAPE;
  if (!head->ts.all_set()) return JEPA_ERR_STATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = c.embed_dim, M = B * N, hd = D / c.n_head, bf = c.compute == JEPA_BF16 ? 1 : 0;
  float* x = static_cast<float*>(head->x.p);
  float* kv = static_cast<float*>(head->kv.p);
  float* q = static_cast<float*>(head->q.p);
  float* y = static_cast<float*>(head->y.p);
  // [Notes §2] "Attentive-pool head": the pool blocks run without RoPE.  On the grid 1 x 1 x 1
  // every token sits at position 0, whose table entries are (cos, sin) = (1, 0) exactly.
  JEPA_LAUNCH(JEPA_KC_OTHER, s,
              hipMemcpyAsync(x, x_dev, static_cast<size_t>(M) * D * 4, hipMemcpyDeviceToDevice, s));
  const RopeSpec rs{1, 1, 1, JEPA_ROPE_TILED, 10000.f, 0};
  JEPA_TRY(run_blocks(head->ts, head->blocks, c.n_layer, head->ws, x, B, N, D, c.ffn_dim, c.n_head,
                      c.ln_eps, nullptr, 0, rs, s));
  // cross-attention: k, v (fp32) from the normed tokens, q from the raw query
  JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
              launch_layernorm(x, head->ts.devf(head->lnkv_w), head->ts.devf(head->lnkv_b), M, D,
                               c.ln_eps, head->ws.h.p, bf, s));
  float* kk = kv;
  float* vv = kv + static_cast<size_t>(c.max_rows) * D;
  JEPA_LAUNCH(JEPA_KC_GEMM_QKV, s,
              linear(c.compute, head->ws.h.p, head->ts.dev(head->k_w), head->ts.devf(head->k_b), kk, M,
                     D, D, JEPA_EPI_STORE, 1, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_QKV, s,
              linear(c.compute, head->ws.h.p, head->ts.dev(head->v_w), head->ts.devf(head->v_b), vv, M,
                     D, D, JEPA_EPI_STORE, 1, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              launch_gemv_f32(head->ts.devf(head->query), head->ts.devf(head->q_w),
                              head->ts.devf(head->q_b), q, 1, D, D, s));
  JEPA_LAUNCH(JEPA_KC_ATTENTION, s,
              launch_xattn_query(q, kk, vv, D, head->ts.devf(head->query), y, B, N, c.n_head, hd, s));
  // y += ffn_down(gelu(ffn_up(ln2(y)))), then the classifier (no final norm)
  JEPA_LAUNCH(JEPA_KC_LAYERNORM, s,
              launch_layernorm(y, head->ts.devf(head->ln2_w), head->ts.devf(head->ln2_b), B, D,
                               c.ln_eps, head->ws.h.p, bf, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_UP, s,
              linear(c.compute, head->ws.h.p, head->ts.dev(head->up_w), head->ts.devf(head->up_b),
                     head->ws.g.p, B, c.ffn_dim, D, JEPA_EPI_GELU, !bf, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_DOWN, s,
              linear(c.compute, head->ws.g.p, head->ts.dev(head->down_w), head->ts.devf(head->down_b),
                     y, B, D, c.ffn_dim, JEPA_EPI_RESIDUAL, 1, s));
  JEPA_LAUNCH(JEPA_KC_GEMM_EMBED, s,
              launch_gemv_f32(y, head->ts.devf(head->cls_w), head->ts.devf(head->cls_b), logits_dev, B,
                              c.n_classes, D, s));
  return JEPA_OK;
}

int jepa_pool_mean(const float* x_dev, int B, int N, int D, float* out_dev, void* stream) {
  if (!x_dev || !out_dev) return JEPA_ERR_ARG;
  if (B < 0 || N < 1 || D < 1) return JEPA_ERR_SHAPE;
  if (B == 0) return JEPA_OK;
  return hip_status(launch_mean_pool(x_dev, B, N, D, out_dev, static_cast<hipStream_t>(stream)));
}

// ==================================================================== stand-alone ops

int jepa_rope3d(const void* x_dev, void* y_dev, int dtype, int B, int N, int n_head,
                int head_dim, int64_t row_stride, const int32_t* ids_dev, int gt, int gh,
                int gw, int layout, float theta, int ref_grid, void* stream) {
  if (!x_dev || !y_dev) return JEPA_ERR_ARG;
  if (dtype != JEPA_F32 && dtype != JEPA_BF16) return JEPA_ERR_ARG;
  if (layout != JEPA_ROPE_TILED && layout != JEPA_ROPE_INTERLEAVED) return JEPA_ERR_ARG;
  if (!(theta > 1.f) || ref_grid < 0 || ref_grid == 1) return JEPA_ERR_ARG;
  if (B < 0 || N < 0 || n_head < 1) return JEPA_ERR_SHAPE;
  if (head_dim < 6 || head_dim > 96 || head_dim % 2) return JEPA_ERR_SHAPE;
  if (row_stride < static_cast<int64_t>(n_head) * head_dim || row_stride % 2) return JEPA_ERR_SHAPE;
  if (gt < 1 || gh < 1 || gw < 1) return JEPA_ERR_SHAPE;
  if (ref_grid > 1 && (gh < 2 || gw < 2)) return JEPA_ERR_SHAPE;
  if (!ids_dev && static_cast<long long>(N) > static_cast<long long>(gt) * gh * gw) return JEPA_ERR_SHAPE;
  if (B == 0 || N == 0) return JEPA_OK;
  const RopeSpec rs{gt, gh, gw, layout, theta, ref_grid};
  return hip_status(launch_rope3d(x_dev, y_dev, dtype == JEPA_BF16, B, N, n_head, head_dim,
                                  row_stride, ids_dev, rs, static_cast<hipStream_t>(stream)));
}

int jepa_layernorm(const float* x_dev, const float* weight_dev, const float* bias_dev, int M,
                   int D, float eps, void* out_dev, int out_dtype, void* stream) {
  if (!x_dev || !weight_dev || !bias_dev || !out_dev) return JEPA_ERR_ARG;
  if (out_dtype != JEPA_F32 && out_dtype != JEPA_BF16) return JEPA_ERR_ARG;
  if (!(eps > 0.f)) return JEPA_ERR_ARG;
  if (M < 0 || !layernorm_width_ok(D)) return JEPA_ERR_SHAPE;
  if (M == 0) return JEPA_OK;
  return hip_status(launch_layernorm(x_dev, weight_dev, bias_dev, M, D, eps, out_dev,
                                     out_dtype == JEPA_BF16, static_cast<hipStream_t>(stream)));
}

int jepa_linear(const void* A_dev, const void* W_dev, const float* bias_dev, void* C_dev, int M,
                int N, int K, int dtype, int epilogue, int out_dtype, void* stream) {
  if (!A_dev || !W_dev || !C_dev) return JEPA_ERR_ARG;
  if (dtype != JEPA_F32 && dtype != JEPA_BF16) return JEPA_ERR_ARG;
  if (out_dtype != JEPA_F32 && out_dtype != JEPA_BF16) return JEPA_ERR_ARG;
  if (epilogue != JEPA_EPI_STORE && epilogue != JEPA_EPI_GELU && epilogue != JEPA_EPI_RESIDUAL)
    return JEPA_ERR_ARG;
  if (epilogue == JEPA_EPI_RESIDUAL && out_dtype != JEPA_F32) return JEPA_ERR_ARG;
  if (dtype == JEPA_F32 && out_dtype != JEPA_F32) return JEPA_ERR_ARG;
  if (M < 0 || N <= 0 || K <= 0) return JEPA_ERR_SHAPE;
  if (dtype == JEPA_BF16 && (N % 128 || K % 64)) return JEPA_ERR_SHAPE;
  if (dtype == JEPA_F32 && (N % 4 || K % 4)) return JEPA_ERR_SHAPE;
  if (M == 0) return JEPA_OK;
  return hip_status(linear(dtype, A_dev, W_dev, bias_dev, C_dev, M, N, K, epilogue,
                           out_dtype == JEPA_F32, static_cast<hipStream_t>(stream)));
}

// Workspace of the bf16 stand-alone attention: RoPE table | q', k' [M, 2D] | V^T rows |
// key-piece buffer (long clips only).
static size_t attn_ws_parts(int B, int N, int n_head, int head_dim, size_t* off_qk,
                            size_t* off_vt, size_t* off_split) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int D = n_head * head_dim;
  const size_t tab = up(static_cast<size_t>(kRopeTabEntries) * 8);
  const size_t qk = up(static_cast<size_t>(B) * N * 2 * D * 2);
  const size_t vt = up(static_cast<size_t>(B) * D * vt_stride(N) * 2 + kVtSlackBytes);
  *off_qk = tab;
  *off_vt = tab + qk;
  *off_split = tab + qk + vt;
  return tab + qk + vt + attention_split_bytes(B, N, n_head, head_dim);
}

size_t jepa_attention_workspace_size(int dtype, int B, int N, int n_head, int head_dim) {
  if (dtype != JEPA_BF16 || B <= 0 || N <= 0 || n_head <= 0 || head_dim <= 0) return 0;
  size_t a, b, c;
  return attn_ws_parts(B, N, n_head, head_dim, &a, &b, &c);
}

// Shared by jepa_attention and jepa_attention_block_causal: ids (NULL: row n is grid
// token n - n_cls, the n_cls leading rows unrotated) and the mask (slot 0: none).
static int attention_common(const void* qkv_dev, void* out_dev, int dtype, int B, int N, int n_head,
                            int head_dim, const int32_t* ids_dev, const RopeSpec& rs, int n_cls,
                            int slot, void* work_dev, size_t work_bytes, hipStream_t s) {
  if (dtype == JEPA_F32) {
    JEPA_LAUNCH(JEPA_KC_ATTENTION, s,
                launch_attention_f32(static_cast<const float*>(qkv_dev), static_cast<float*>(out_dev),
                                     B, N, n_head, head_dim, ids_dev, 0, rs, s, n_cls, slot));
    return JEPA_OK;
  }
  const int D = n_head * head_dim;
  if (D % 32) return JEPA_ERR_SHAPE;
  size_t off_qk, off_vt, off_split;
  const size_t need = attn_ws_parts(B, N, n_head, head_dim, &off_qk, &off_vt, &off_split);
  if (!work_dev || work_bytes < need) return JEPA_ERR_ARG;
  // the kernels move 16-byte vectors
  if ((reinterpret_cast<uintptr_t>(qkv_dev) | reinterpret_cast<uintptr_t>(out_dev) |
       reinterpret_cast<uintptr_t>(work_dev)) % 16)
    return JEPA_ERR_ARG;
  unsigned char* w = static_cast<unsigned char*>(work_dev);
  uint16_t* qk = reinterpret_cast<uint16_t*>(w + off_qk);
  uint16_t* vt = reinterpret_cast<uint16_t*>(w + off_vt);
  const int Ns = vt_stride(N);
  JEPA_LAUNCH(JEPA_KC_OTHER, s, launch_rope_table(w, rs, head_dim, s));
  JEPA_LAUNCH(JEPA_KC_OTHER, s,
              launch_qkv_prepare(static_cast<const uint16_t*>(qkv_dev), qk, vt, Ns, B, N, n_head,
                                 head_dim, ids_dev, rs, w, attn_qscale(head_dim), s, n_cls));
  void* split = slot > 0 ? nullptr : w + off_split;
  JEPA_LAUNCH(JEPA_KC_ATTENTION, s,
              launch_attention_fwd(qk, qk + D, 2 * D, vt, Ns, static_cast<uint16_t*>(out_dev), B, N,
                                   n_head, head_dim, s, n_cls, slot, split));
  return JEPA_OK;
}

static int attention_args(const void* qkv_dev, void* out_dev, int dtype, int n_head, int head_dim,
                          int layout, float theta) {
  if (!qkv_dev || !out_dev) return JEPA_ERR_ARG;
  if (dtype != JEPA_F32 && dtype != JEPA_BF16) return JEPA_ERR_ARG;
  if (layout != JEPA_ROPE_TILED && layout != JEPA_ROPE_INTERLEAVED) return JEPA_ERR_ARG;
  if (!(theta > 1.f)) return JEPA_ERR_ARG;
  if (head_dim != 64 && head_dim != 32) return JEPA_ERR_SHAPE;
  if (n_head < 1) return JEPA_ERR_SHAPE;
  return JEPA_OK;
}

int jepa_attention(const void* qkv_dev, void* out_dev, int dtype, int B, int N, int n_head,
                   int head_dim, const int32_t* ids_dev, int gt, int gh, int gw, int layout,
                   float theta, int ref_grid, void* work_dev, size_t work_bytes, void* stream) {
  JEPA_TRY(attention_args(qkv_dev, out_dev, dtype, n_head, head_dim, layout, theta));
  if (B < 0 || N < 0) return JEPA_ERR_SHAPE;
  JEPA_TRY(check_grid(gt, gh, gw, ref_grid));
  if (!ids_dev && static_cast<long long>(N) > static_cast<long long>(gt) * gh * gw) return JEPA_ERR_SHAPE;
  if (B == 0 || N == 0) return JEPA_OK;
  const RopeSpec rs{gt, gh, gw, layout, theta, ref_grid};
  return attention_common(qkv_dev, out_dev, dtype, B, N, n_head, head_dim, ids_dev, rs, 0, 0,
                          work_dev, work_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// Scratch of jepa_attention_noalloc: one array per GPU, alive until the process ends.  In
// host code `attn_scratch` names a host-side stand-in, not device memory: kernels and
// copies get the address hipGetSymbolAddress returns for the current device instead.
static __device__ __align__(256) unsigned char attn_scratch[JEPA_ATTN_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's scratch array, looked up once per device.
int scratch_for_current_device(void** ptr) {
  int dev = 0;
  JEPA_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return JEPA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    JEPA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(attn_scratch)));
    if (!p) return JEPA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return JEPA_OK;
}
}  // namespace

extern "C" {

int jepa_attention_noalloc(const void* qkv_dev, void* out_dev, int dtype, int B, int N,
                           int n_head, int head_dim, const int32_t* ids_dev, int gt, int gh,
                           int gw, int layout, float theta, int ref_grid, void* stream) {
  JEPA_TRY(attention_args(qkv_dev, out_dev, dtype, n_head, head_dim, layout, theta));
  if (B < 0 || N < 0) return JEPA_ERR_SHAPE;
  JEPA_TRY(check_grid(gt, gh, gw, ref_grid));
  if (!ids_dev && static_cast<long long>(N) > static_cast<long long>(gt) * gh * gw) return JEPA_ERR_SHAPE;
  if (B == 0 || N == 0) return JEPA_OK;
  void* work = nullptr;
  size_t work_bytes = 0;
  if (dtype == JEPA_BF16) {
    size_t a, b, c;
    // a coarse bound first (6 bytes per q|k|v element), so that the exact size below
    // cannot overflow
    const double need = static_cast<double>(B) * N * n_head * head_dim * 6.0;
    if (need > static_cast<double>(JEPA_ATTN_SCRATCH_BYTES)) return JEPA_ERR_SHAPE;
    if (attn_ws_parts(B, N, n_head, head_dim, &a, &b, &c) > JEPA_ATTN_SCRATCH_BYTES) return JEPA_ERR_SHAPE;
    JEPA_TRY(scratch_for_current_device(&work));
    work_bytes = JEPA_ATTN_SCRATCH_BYTES;
  }
  const RopeSpec rs{gt, gh, gw, layout, theta, ref_grid};
  return attention_common(qkv_dev, out_dev, dtype, B, N, n_head, head_dim, ids_dev, rs, 0, 0,
                          work, work_bytes, static_cast<hipStream_t>(stream));
}

int jepa_attention_block_causal(const void* qkv_dev, void* out_dev, int dtype, int B, int n_cls,
                                int n_head, int head_dim, int gt, int gh, int gw, int layout,
                                float theta, int ref_grid, void* work_dev, size_t work_bytes,
                                void* stream) {
  JEPA_TRY(attention_args(qkv_dev, out_dev, dtype, n_head, head_dim, layout, theta));
  if (B < 0 || n_cls < 0 || n_cls >= 64) return JEPA_ERR_SHAPE;
  JEPA_TRY(check_grid(gt, gh, gw, ref_grid));
  if (B == 0) return JEPA_OK;
  const int N = n_cls + gt * gh * gw;
  const RopeSpec rs{gt, gh, gw, layout, theta, ref_grid};
  return attention_common(qkv_dev, out_dev, dtype, B, N, n_head, head_dim, nullptr, rs, n_cls,
                          gh * gw, work_dev, work_bytes, static_cast<hipStream_t>(stream));
}

int jepa_timing_begin(int cap) {
  if (cap < 1 || g_timing.on) return JEPA_ERR_ARG;
  for (int k = 0; k < JEPA_KC_COUNT; ++k) {
    g_timing.n[k] = 0;
    g_timing.ev[k].assign(2 * static_cast<size_t>(cap), nullptr);
    // timing-only events: no system-scope fence (cache write-back and invalidate) on
    // record, which would add its own cost to every bracketed launch
    for (hipEvent_t& e : g_timing.ev[k]) {
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipGetLastError();
        for (int j = 0; j <= k; ++j)
          for (hipEvent_t& f : g_timing.ev[j])
            if (f) (void)hipEventDestroy(f);
        for (int j = 0; j < JEPA_KC_COUNT; ++j) g_timing.ev[j].clear();
        return JEPA_ERR_HIP;
      }
    }
  }
  g_timing.cap = cap;
  g_timing.on = true;
  return JEPA_OK;
}

int jepa_timing_end(double* ms, int* launches) {
  if (!g_timing.on) return JEPA_ERR_STATE;
  g_timing.on = false;
  int st = JEPA_OK;
  for (int k = 0; k < JEPA_KC_COUNT; ++k) {
    double sum = 0.0;
    for (int i = 0; i < g_timing.n[k]; ++i) {
      float t = 0.f;
      if (hipEventSynchronize(g_timing.ev[k][2 * i + 1]) != hipSuccess ||
          hipEventElapsedTime(&t, g_timing.ev[k][2 * i], g_timing.ev[k][2 * i + 1]) != hipSuccess) {
        (void)hipGetLastError();
        st = JEPA_ERR_HIP;
        continue;
      }
      sum += t;
    }
    if (ms) ms[k] = sum;
    if (launches) launches[k] = g_timing.n[k];
    for (hipEvent_t& e : g_timing.ev[k]) (void)hipEventDestroy(e);
    g_timing.ev[k].clear();
    g_timing.n[k] = 0;
  }
  return st;
}

}  // extern "C"
