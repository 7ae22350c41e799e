/*
 * jepa.h -- C ABI of libjepa, a gfx950 (MI355X) implementation of the V-JEPA 2 / 2.1
 * video ViT encoder forward and of the V-JEPA 2 masked predictor.
 *
 * Sources, cited by page and section:
 *   [Notes]  "V-JEPA 2 / 2.1 tensor maps and RoPE derivation"
 *            (aselimc.github.io/jepa.cpp/vjepa-notes/)
 *   [Parity] "Parity -- image ViT encoders ... and video encoders (V-JEPA 2 / V-JEPA 2.1,
 *            LeVJEPA)" (aselimc.github.io/jepa.cpp/parity/)
 *   [HFport] "V-JEPA 2.1 ViT-B/16 384 -- HuggingFace port"
 *            (aimarketly.com/model/apiantonio/vjepa2.1-vit-base-384)
 *   [Card]   jepa.cpp V-JEPA 2 ViT-L/16 GGUF model card
 *            (graysoft.dev/models/jep/jepacpp-vjepa2-vitl-fpc64-256-gguf.html)
 *
 * Conventions shared by every entry point
 *   - Pointers named *_dev are device memory (HIP), allocated and owned by the caller;
 *     the library never frees caller memory.  Pointers named *_host are host memory,
 *     read during the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute entry points only
 *     enqueue work on it and return without synchronising; outputs are valid once the
 *     stream reaches that point.
 *   - Every call returns a jepa_status.  On an argument, shape or state error nothing is
 *     enqueued and no output is touched.  JEPA_ERR_HIP reports a HIP runtime error
 *     (allocation or launch); the state of the outputs is then unspecified.
 *   - Row-major everywhere.  bf16 data is passed as raw 16-bit patterns (uint16).
 *   - Token ids index a T-major grid (gt, gh, gw): id = t*gh*gw + h*gw + w ([Notes §4]).
 *     An ids pointer may be NULL, meaning ids 0..N-1.  Device ids outside [0, gt*gh*gw)
 *     are clamped to that range by the kernels (memory-safe; the result for such a
 *     token is unspecified).
 *   - A handle may be used by one stream at a time.
 */
#ifndef JEPA_H
#define JEPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ enums */

enum jepa_status {
  JEPA_OK = 0,
  JEPA_ERR_ARG = -1,    /* null pointer, bad enum, unsupported configuration value */
  JEPA_ERR_SHAPE = -2,  /* sizes that the method or this library does not accept */
  JEPA_ERR_STATE = -3,  /* handle not ready (a required tensor was never set) */
  JEPA_ERR_NAME = -4,   /* unknown tensor name, or a shape that does not match it */
  JEPA_ERR_OOM = -5,    /* device allocation failed */
  JEPA_ERR_HIP = -6     /* HIP runtime error (launch, copy) */
};

/* RoPE frequency layouts ([Notes §4.1] tiled = V-JEPA 2, [Notes §4.2] interleaved =
 * V-JEPA 2.1). */
enum jepa_rope_layout { JEPA_ROPE_TILED = 0, JEPA_ROPE_INTERLEAVED = 1 };

/* Modality vector of the V-JEPA 2.1 predictor ([Notes §3] "2.1 predictor forward"):
 * pred.mod_embed_video or pred.mod_embed_img; AUTO takes the image one when the grid has
 * a single temporal slot (gt = 1). */
enum jepa_modality { JEPA_MODALITY_VIDEO = 0, JEPA_MODALITY_IMAGE = 1, JEPA_MODALITY_AUTO = 2 };

/* Element types.  JEPA_F32 also selects the fp32 compute path (plain fp32 FMA
 * kernels); JEPA_BF16 selects bf16 MFMA operands with fp32 accumulation. */
enum jepa_dtype { JEPA_F32 = 0, JEPA_BF16 = 1 };

/* Epilogues of jepa_linear. */
enum jepa_epilogue {
  JEPA_EPI_STORE = 0,    /* C = A W^T + bias                  (C in out_dtype)        */
  JEPA_EPI_GELU = 1,     /* C = GELU_erf(A W^T + bias)         (C in out_dtype)        */
  JEPA_EPI_RESIDUAL = 2  /* C += A W^T + bias, C fp32 in place (out_dtype must be F32) */
};

/* Library version: major*10000 + minor*100 + patch. */
int jepa_version(void);

/* Human-readable text of a jepa_status (static storage). */
const char* jepa_status_str(int status);

/* ------------------------------------------------------------------ encoder */

/* Hyper-parameters of one encoder ([Notes §1] table).  ViT-L: 1024/24/16/4096,
 * 2.1 ViT-B: 768/12/12/3072; patch 16, tubelet 2, 3 channels, ln_eps 1e-6,
 * rope_theta 10000.  head_dim = embed_dim / n_head must be 64 or 32. */
typedef struct jepa_encoder_config {
  int32_t embed_dim;      /* D, a multiple of 128 on the bf16 path, of 64 on fp32,
                             and a LayerNorm width (see jepa_layernorm), else
                             JEPA_ERR_ARG at creation                            */
  int32_t n_layer;        /* >= 0 (0: patch embedding (+ final norm) only)        */
  int32_t n_head;
  int32_t ffn_dim;        /* F, a multiple of 128 on the bf16 path                */
  int32_t patch;          /* must be 16                                          */
  int32_t tubelet;        /* must be 2                                           */
  int32_t in_chans;       /* must be 3                                           */
  int32_t rope_layout;    /* jepa_rope_layout                                    */
  int32_t rope_ref_grid;  /* 0: integer positions; R > 1: interpolate the spatial
                             positions onto [0, R-1] ([Notes §4.3], R = 16)      */
  int32_t has_mod_embed;  /* 1: add enc.mod_embed_video after the patch embedding
                             ([Notes §3] "2.1 encoder forward")                   */
  int32_t final_norm;     /* 1: apply enc.norm at the end ([Notes §2], §3)        */
  int32_t compute;        /* jepa_dtype                                          */
  int32_t max_rows;       /* largest B*N a call may use (sizes the workspace)    */
  float ln_eps;           /* 1e-6                                                */
  float rope_theta;       /* 10000                                               */
  int32_t has_image_embed; /* 1: the V-JEPA 2.1 image path (jepa_encode_image) with
                              enc.patch_embed_img (+ enc.mod_embed_img when
                              has_mod_embed) ([Notes §2] key map, [Notes §3])    */
} jepa_encoder_config;

typedef struct jepa_encoder jepa_encoder;

/* Validate the configuration and allocate the handle: device weights (bf16 matrices,
 * fp32 vectors) and a workspace for max_rows token rows.  Must be called with the
 * target device current.  Errors: JEPA_ERR_ARG (null, bad value), JEPA_ERR_OOM. */
int jepa_encoder_create(const jepa_encoder_config* cfg, jepa_encoder** out);

/* Release the handle and everything it allocated.  NULL is ignored.  The caller must
 * make sure no enqueued work still uses it. */
void jepa_encoder_free(jepa_encoder* enc);

/* Upload one tensor by its GGUF name ([Notes §2] and [Notes §3] key maps):
 *   enc.patch_embed.weight [D, 1536] (feature order C, T, H, W), enc.patch_embed.bias [D],
 *   enc.mod_embed_video [D] (only when has_mod_embed),
 *   enc.blk.{i}.ln1.weight/bias [D], enc.blk.{i}.attn_qkv.weight [3D, D] (rows q; k; v),
 *   enc.blk.{i}.attn_qkv.bias [3D], enc.blk.{i}.attn_out.weight [D, D] / .bias [D],
 *   enc.blk.{i}.ln2.weight/bias [D], enc.blk.{i}.ffn_up.weight [F, D] / .bias [F],
 *   enc.blk.{i}.ffn_down.weight [D, F] / .bias [D], enc.norm.weight/bias [D];
 *   with has_image_embed: enc.patch_embed_img.weight [D, 768] / .bias [D] and, when
 *   has_mod_embed, enc.mod_embed_img [D].
 * `host` holds numel(shape) values of src_dtype (JEPA_F32 floats or JEPA_BF16 bit
 * patterns), row-major.  Matrices are stored on the device in the compute dtype
 * (fp32 -> bf16 by round-to-nearest-even); vectors stay fp32.  Synchronous.
 * Errors: JEPA_ERR_ARG, JEPA_ERR_NAME (unknown name or shape mismatch), JEPA_ERR_HIP. */
int jepa_encoder_set_tensor(jepa_encoder* enc, const char* name, const void* host,
                            int src_dtype, const int64_t* shape, int ndim);

/* Encode B uint8 clips ([Notes §3] "2.1 encoder forward"; [Notes §5] preprocessing):
 *   clip_dev: uint8 [B, T, H, W, 3] (frames, channels last, RGB);
 *   out_dev:  fp32 [B, N, D], N = (T/2)*(H/16)*(W/16), tokens T-major ([Notes §4]).
 * Pixels are normalised with the ImageNet mean/std in the fused form
 * (px - 255*mean)/(255*std) ([Parity "Preprocessing parity"]), patchified into
 * 2x16x16x3 tubelets and embedded; then the blocks and the final norm.
 * Shape errors (JEPA_ERR_SHAPE): T odd or < 2, H or W not a multiple of 16, B < 1,
 * B*N > max_rows, interpolation with a grid side of 1 ([Notes §4.3]); on the bf16 path
 * also B*ceil(N/16)*16 > 2*max_rows + 1024 (only reachable with fewer than 16 tokens per
 * clip).  JEPA_ERR_STATE if a required tensor was never set. */
int jepa_encode(jepa_encoder* enc, const uint8_t* clip_dev, int B, int T, int H, int W,
                float* out_dev, void* stream);

/* Run the blocks (and the final norm when configured) on token activations:
 *   x_dev: fp32 [B, N, D] (not modified); ids_dev: int32 [N] grid ids shared by all B
 *   rows of the batch (NULL = 0..N-1) on the grid (gt, gh, gw); out_dev: fp32 [B, N, D]
 *   (may alias x_dev).  Positions come from the ids ([Notes §4], [Notes §4.4]). */
int jepa_encode_tokens(jepa_encoder* enc, const float* x_dev, int B, int N,
                       const int32_t* ids_dev, int gt, int gh, int gw, float* out_dev,
                       void* stream);

/* Masked-encoder forward, the pre-training path ([HFport "Usage"]: masks passed to the
 * encoder; [HFport "Validation"], masked-encoder row): the tokens outside each clip's
 * context are dropped before the first block, so attention sees only the context and
 * RoPE takes each kept token's own grid position.  This differs from taking rows of
 * jepa_encode's output.
 *   clip_dev: uint8 [B, T, H, W, 3] as for jepa_encode (same preprocessing);
 *   ids_dev:  int32 [B, K] device array, the context tokens of clip b are
 *             ids_dev[b*K .. b*K + K) as T-major grid ids in [0, N), N = (T/2)(H/16)(W/16);
 *             any order, one clip's list may differ from another's; values outside
 *             [0, N) are clamped;
 *   out_dev:  fp32 [B, K, D], row k of clip b for token ids_dev[b*K + k].
 * Only the K context tubelets of each clip are patchified and embedded (the embedding
 * acts on each row alone), then the blocks and the final norm run on B clips of K tokens.
 * Needs B*K <= max_rows (not B*N).  Asynchronous on `stream`; the caller keeps ids_dev
 * alive until the work is done.
 * Errors: JEPA_ERR_ARG (null pointer); JEPA_ERR_SHAPE (T, H, W, interpolation as for
 * jepa_encode; K < 1 or K > N; B*K > max_rows; on the bf16 path also
 * B*ceil(K/16)*16 > 2*max_rows + 1024); JEPA_ERR_STATE (a tensor never set). */
int jepa_encode_masked(jepa_encoder* enc, const uint8_t* clip_dev, int B, int T, int H, int W,
                       const int32_t* ids_dev, int K, float* out_dev, void* stream);

/* V-JEPA 2.1 native image path ([Notes §3] "2.1 encoder forward", image line; [Notes §2]
 * patch_embed_img with tubelet 1): each image is one frame, patchified into 1x16x16x3
 * patches (features in C, T, H, W order with T = 1, 768 of them) and embedded with
 * enc.patch_embed_img [D, 768] / .bias (+ enc.mod_embed_img when has_mod_embed), then the
 * blocks and the final norm on the grid (1, H/16, W/16).
 *   img_dev: uint8 [B, H, W, 3]; out_dev: fp32 [B, N, D], N = (H/16)(W/16), row-major.
 * Needs has_image_embed.  Errors: JEPA_ERR_ARG (null pointer, no image path);
 * JEPA_ERR_SHAPE (H or W not a multiple of 16, a grid side above 64, interpolation with a
 * side of 1, B*N > max_rows); JEPA_ERR_STATE (a tensor never set). */
int jepa_encode_image(jepa_encoder* enc, const uint8_t* img_dev, int B, int H, int W,
                      float* out_dev, void* stream);

/* ------------------------------------------------------------------ predictor */

/* V-JEPA 2 masked predictor ([Notes §1]: 384 / 12 / 12 / 1536, 10 mask tokens, output
 * 1024, tiled RoPE, no interpolation).  head_dim = embed_dim / n_head must be 64 or 32. */
typedef struct jepa_predictor_config {
  int32_t enc_dim;        /* encoder width (input rows)   */
  int32_t embed_dim;      /* predictor width              */
  int32_t n_layer;
  int32_t n_head;
  int32_t ffn_dim;
  int32_t n_mask_tokens;
  int32_t out_dim;
  int32_t rope_layout;
  int32_t compute;        /* jepa_dtype */
  int32_t max_rows;       /* largest n_ctx + n_tgt */
  float ln_eps;
  float rope_theta;
  int32_t has_mod_embed;  /* 1: V-JEPA 2.1 modality vectors pred.mod_embed_video/_img [E]
                             added to every row ([Notes §3] "2.1 predictor forward") */
  int32_t has_proj_context; /* 1: pred.proj_context [Dout, E] projects the context rows */
} jepa_predictor_config;

typedef struct jepa_predictor jepa_predictor;

int jepa_predictor_create(const jepa_predictor_config* cfg, jepa_predictor** out);
void jepa_predictor_free(jepa_predictor* pred);

/* Names ([Notes §2]): pred.embed.weight [E, Denc] / .bias [E], pred.mask_tokens [n, E],
 * pred.blk.{i}.* as the encoder blocks at width E, pred.norm.weight/bias [E],
 * pred.proj.weight [Dout, E] / .bias [Dout]; with has_mod_embed pred.mod_embed_video and
 * pred.mod_embed_img [E]; with has_proj_context pred.proj_context.weight [Dout, E] /
 * .bias [Dout].  Same rules as jepa_encoder_set_tensor. */
int jepa_predictor_set_tensor(jepa_predictor* pred, const char* name, const void* host,
                              int src_dtype, const int64_t* shape, int ndim);

/* Predict the target tokens ([Notes §3] "2.1 predictor forward" order of operations,
 * [Notes §4.4] ids):
 *   z_dev: fp32 [n_enc, Denc] encoder token map of one clip;
 *   ids_ctx_dev: int32 [n_ctx] rows of z that form the context (also their grid ids);
 *   ids_tgt_dev: int32 [n_tgt] grid ids of the targets;
 *   every target row starts as mask_tokens[mask_index mod n_mask_tokens];
 *   positions are decoded from concat(ids_ctx, ids_tgt) on (gt, gh, gw);
 *   out_dev: fp32 [n_tgt, Dout] = projection of the normed target rows.
 * Errors: JEPA_ERR_SHAPE if n_ctx < 1, n_tgt < 1, n_ctx + n_tgt > max_rows or
 * gt*gh*gw != n_enc. */
int jepa_predict(jepa_predictor* pred, const float* z_dev, int n_enc,
                 const int32_t* ids_ctx_dev, int n_ctx, const int32_t* ids_tgt_dev, int n_tgt,
                 int mask_index, int gt, int gh, int gw, float* out_dev, void* stream);

/* jepa_predict with the V-JEPA 2.1 options ([Notes §3] "2.1 predictor forward"):
 *   modality: jepa_modality, which of pred.mod_embed_video / _img is added to every row
 *             after the concatenation (ignored without has_mod_embed; jepa_predict
 *             uses the video one);
 *   ctx_out_dev: NULL, or fp32 [n_ctx, Dout] = pred.proj_context of the normed context
 *             rows (needs has_proj_context).
 * Errors as jepa_predict, plus JEPA_ERR_ARG for a bad modality or ctx_out_dev without
 * has_proj_context. */
int jepa_predict_mod(jepa_predictor* pred, const float* z_dev, int n_enc,
                     const int32_t* ids_ctx_dev, int n_ctx, const int32_t* ids_tgt_dev, int n_tgt,
                     int mask_index, int modality, int gt, int gh, int gw, float* out_dev,
                     float* ctx_out_dev, void* stream);

/* ------------------------------------------------------------------ pooled outputs */

/* Mean over the tokens of each clip ([Card] "Run it", --pool mean):
 *   x_dev fp32 [B, N, D] -> out_dev fp32 [B, D], accumulated in fp64 in a fixed order.
 * Errors: JEPA_ERR_ARG (null pointer), JEPA_ERR_SHAPE (B < 0, N < 1, D < 1). */
int jepa_pool_mean(const float* x_dev, int B, int N, int D, float* out_dev, void* stream);

/* Attentive-pool classifier head ([Notes §2] "Attentive-pool head — exact forward"; the
 * V-JEPA 2 SSv2 classifier: D 1024, 3 pool blocks, 16 heads, FFN 4096, 174 classes). */
typedef struct jepa_head_config {
  int32_t embed_dim;      /* D, as the encoder; head_dim = D / n_head must be 64 or 32 */
  int32_t n_layer;        /* pool blocks (self-attention without RoPE), >= 0          */
  int32_t n_head;
  int32_t ffn_dim;
  int32_t n_classes;      /* >= 1, any width                                          */
  int32_t compute;        /* jepa_dtype of the blocks and the k / v / MLP projections */
  int32_t max_rows;       /* largest B*N a call may use                               */
  float ln_eps;           /* 1e-6                                                     */
} jepa_head_config;

typedef struct jepa_head jepa_head;

int jepa_head_create(const jepa_head_config* cfg, jepa_head** out);
void jepa_head_free(jepa_head* head);

/* Names ([Notes §2] key map): head.query [1, D]; head.blk.{i}.* as the encoder blocks;
 * head.xattn.ln_kv.weight/bias [D]; head.xattn.{q,k,v}.weight [D, D] / .bias [D];
 * head.xattn.ln2.weight/bias [D]; head.xattn.ffn_up.weight [F, D] / .bias [F];
 * head.xattn.ffn_down.weight [D, F] / .bias [D]; head.cls.weight [C, D] / .bias [C].
 * The query projection and the classifier stay fp32 (they see one row per clip); the
 * other matrices follow the compute dtype.  Same rules as jepa_encoder_set_tensor. */
int jepa_head_set_tensor(jepa_head* head, const char* name, const void* host, int src_dtype,
                         const int64_t* shape, int ndim);

/* Logits of B token maps:
 *   x_dev: fp32 [B, N, D] encoder output after its final norm (not modified);
 *   logits_dev: fp32 [B, C].
 * The pool blocks run on each clip's N tokens without RoPE; the learned query (raw, not
 * normed) attends over the normed tokens with fp32 k and v, heads concatenated, no output
 * projection; the raw query is the residual; then the MLP with its residual and the
 * classifier, no final norm.
 * Errors: JEPA_ERR_ARG (null pointer); JEPA_ERR_SHAPE (B < 1, N < 1, N > 16384,
 * B*N > max_rows); JEPA_ERR_STATE (a tensor never set). */
int jepa_head_forward(jepa_head* head, const float* x_dev, int B, int N, float* logits_dev,
                      void* stream);

/* ------------------------------------------------------------------ stand-alone ops */

/* 3-D RoPE ([Notes §4]; tiled [Notes §4.1], interleaved [Notes §4.2], interpolation
 * [Notes §4.3]) on head vectors, out of place or in place (y_dev may equal x_dev):
 *   element (b, n, e, j) of x/y is at [(b*N + n)*row_stride + e*head_dim + j],
 *   dtype JEPA_F32 or JEPA_BF16, row_stride >= n_head*head_dim (in elements);
 *   d = 2*((head_dim/3)/2) dims per axis: [0,d) follow t, [d,2d) h, [2d,3d) w, the
 *   rest pass through; omega_k = theta^(-k/(d/2)); angles are formed in fp64 and
 *   their cos/sin rounded to fp32.
 *   ref_grid 0: integer positions; R > 1: h' = h(R-1)/(gh-1), w' = w(R-1)/(gw-1).
 * head_dim must be even and >= 6. */
int jepa_rope3d(const void* x_dev, void* y_dev, int dtype, int B, int N, int n_head,
                int head_dim, int64_t row_stride, const int32_t* ids_dev, int gt, int gh,
                int gw, int layout, float theta, int ref_grid, void* stream);

/* LayerNorm over rows ([Notes §1] eps; centred variance as the CPU backend of
 * [Parity "Parity on a GPU"]): x_dev fp32 [M, D]; weight/bias fp32 [D] (device);
 * out_dev [M, D] in out_dtype (may alias x_dev when out_dtype is F32).
 * D = 64 * v with v in {1..6, 8, 10, 12, 16, 20, 22, 24, 32, 40, 48, 64}, else
 * JEPA_ERR_SHAPE. */
int jepa_layernorm(const float* x_dev, const float* weight_dev, const float* bias_dev,
                   int M, int D, float eps, void* out_dev, int out_dtype, void* stream);

/* Linear layer C = epilogue(A W^T + bias) ([Notes §2]: weights stored [out, in]):
 *   A_dev [M, K] and W_dev [N, K] in dtype; bias_dev fp32 [N] or NULL; C_dev [M, N].
 *   dtype JEPA_BF16: bf16 MFMA, fp32 accumulation; N a multiple of 128, K of 64.
 *   dtype JEPA_F32: fp32 FMA; N and K multiples of 4. */
int jepa_linear(const void* A_dev, const void* W_dev, const float* bias_dev, void* C_dev,
                int M, int N, int K, int dtype, int epilogue, int out_dtype, void* stream);

/* Multi-head softmax attention with the 3-D RoPE on q and k ([Notes §4]: RoPE on q and
 * k, not v, before the 1/sqrt(head_dim) scaling; softmax over every key, no mask):
 *   qkv_dev [B*N, 3*n_head*head_dim] in dtype: per row q | k | v, head e at columns
 *   e*head_dim of each third ([Notes §2]: fused rows [q; k; v]), not yet rotated;
 *   out_dev [B*N, n_head*head_dim] in dtype, heads concatenated;
 *   ids/grid/layout/theta/ref_grid as jepa_rope3d.  head_dim must be 64 or 32.
 * JEPA_BF16 (bf16 MFMA, fp32 softmax): q and k are first rotated (q also scaled by
 * log2(e)/sqrt(head_dim)) and v transposed into work_dev, a device buffer of at least
 * jepa_attention_workspace_size(...) bytes owned by the caller (contents on entry do not
 * matter; overwritten); then the flash-attention kernel runs on it.  The encoder forward
 * uses the same kernel with the rotation done by the QKV projection's epilogue.  Clips of
 * 4096 tokens or more whose (head, 512-query block) pairs would leave many of the GPU's
 * 256 compute units idle take each block's keys in 2-8 pieces, whose fp32 partial states
 * a second kernel merges in piece order (the workspace then also holds them); the choice
 * depends on N and n_head only, so a clip's output does not depend on B.
 * JEPA_F32 (plain fp32 FMA, RoPE applied as q and k are loaded): work_dev is unused and
 * may be NULL.
 * Errors: JEPA_ERR_ARG also when the bf16 workspace is NULL or smaller than needed, or
 * when a bf16 call's qkv_dev, out_dev or work_dev is not 16-byte aligned. */
int jepa_attention(const void* qkv_dev, void* out_dev, int dtype, int B, int N, int n_head,
                   int head_dim, const int32_t* ids_dev, int gt, int gh, int gw, int layout,
                   float theta, int ref_grid, void* work_dev, size_t work_bytes, void* stream);

/* Bytes of device workspace jepa_attention needs for these sizes (0 for JEPA_F32 or
 * non-positive sizes). */
size_t jepa_attention_workspace_size(int dtype, int B, int N, int n_head, int head_dim);

/* Block-causal attention with leading CLS rows ([Parity] "LeVJEPA ViT-L/16 -- CLS,
 * block-causal attention, tubelet 1": the CLS row first, then the patch tokens T-major;
 * the CLS carries no position, its RoPE row is the identity; the mask is bidirectional
 * inside a temporal slot, causal across slots, CLS row open, CLS column closed).
 *   Each clip has N = n_cls + gt*gh*gw rows: rows [0, n_cls) are CLS rows, row
 *   n_cls + n is grid token n (id n, as jepa_rope3d with ids NULL); a temporal slot is
 *   one grid slice of gh*gw tokens.
 *   CLS rows: q and k unrotated; the query sees every key of the clip.
 *   Patch row of slot t: the query sees the patch keys of slots 0..t and no CLS key.
 *   qkv_dev [B*N, 3*n_head*head_dim], out_dev [B*N, n_head*head_dim], dtype, layout,
 *   theta, ref_grid and the workspace (jepa_attention_workspace_size(dtype, B, N, ...))
 *   as jepa_attention.  0 <= n_cls < 64.
 * With n_cls = 0 and gt = 1 every row sees every key and the result equals
 * jepa_attention on the same rows (bit for bit when jepa_attention takes the keys in one
 * piece, as it always does below 4096 rows; up to rounding otherwise).
 * Errors: as jepa_attention; JEPA_ERR_SHAPE for n_cls outside [0, 64). */
int jepa_attention_block_causal(const void* qkv_dev, void* out_dev, int dtype, int B, int n_cls,
                                int n_head, int head_dim, int gt, int gh, int gw, int layout,
                                float theta, int ref_grid, void* work_dev, size_t work_bytes,
                                void* stream);

/* Bytes of the per-GPU scratch array jepa_attention_noalloc works in (64 MiB). */
#define JEPA_ATTN_SCRATCH_BYTES ((size_t)64 << 20)

/* jepa_attention for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * layouts, results and errors as jepa_attention minus the workspace: the bf16 path works
 * in a file-scope device array of JEPA_ATTN_SCRATCH_BYTES that each GPU holds until the
 * process ends, and the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  The caller still owns qkv_dev and out_dev.
 *   Limit: jepa_attention_workspace_size(dtype, B, N, n_head, head_dim) must not exceed
 *   JEPA_ATTN_SCRATCH_BYTES (e.g. B*N*n_head*head_dim up to about 11 M elements when the
 *   keys are taken whole; long clips whose keys go in pieces need more per element),
 *   else JEPA_ERR_SHAPE and nothing is enqueued.
 *   Every call on one GPU shares that GPU's array and leaves its contents behind (no
 *   state is read back: every byte a call reads was written earlier in the same call, or
 *   is masked); two calls that overlap on one GPU (different streams, or host threads
 *   without ordering) race on it.  The first call on a device looks up the array's
 *   address there (hipGetSymbolAddress), with that device current.
 * Errors: as jepa_attention; JEPA_ERR_HIP if the array's address cannot be found. */
int jepa_attention_noalloc(const void* qkv_dev, void* out_dev, int dtype, int B, int N,
                           int n_head, int head_dim, const int32_t* ids_dev, int gt, int gh,
                           int gw, int layout, float theta, int ref_grid, void* stream);

/* ------------------------------------------------------------------ kernel timing */

/* Kernel classes of the forwards, for jepa_timing_end. */
enum jepa_kernel_class {
  JEPA_KC_PATCHIFY = 0,   /* u8 clip -> normalised tubelet rows                     */
  JEPA_KC_GEMM_EMBED = 1, /* patch / predictor embedding and predictor output GEMMs  */
  JEPA_KC_LAYERNORM = 2,  /* LN1, LN2 and the final norm                            */
  JEPA_KC_GEMM_QKV = 3,   /* fused QKV projection                                   */
  JEPA_KC_ATTENTION = 4,  /* flash attention (fp32 path: RoPE on the Q/K load)       */
  JEPA_KC_GEMM_OUT = 5,   /* attention output projection + residual                 */
  JEPA_KC_GEMM_UP = 6,    /* FFN up-projection + GELU                               */
  JEPA_KC_GEMM_DOWN = 7,  /* FFN down-projection + residual                         */
  JEPA_KC_OTHER = 8,      /* row gathers, fills and device copies                   */
  JEPA_KC_COUNT = 9
};

/* Per-launch timing of the forwards, for measurement harnesses.  After
 * jepa_timing_begin(cap), every forward (jepa_encode*, jepa_predict*, jepa_head_forward)
 * and the stand-alone jepa_attention / jepa_attention_block_causal record a HIP event
 * pair on their own stream around each kernel launch, for at most
 * `cap` launches per class (later launches are not recorded).  Process-wide state, not
 * thread-safe; the events add a small gap between launches, so time throughput with
 * timing off.  Errors: JEPA_ERR_ARG (cap < 1, or timing already on), JEPA_ERR_HIP. */
int jepa_timing_begin(int cap);

/* Wait for every recorded event, write per class the summed launch duration in ms
 * (ms[JEPA_KC_COUNT]) and the number of recorded launches (launches[JEPA_KC_COUNT]),
 * release the events and turn timing off.  Either pointer may be NULL.
 * Errors: JEPA_ERR_STATE (timing is off), JEPA_ERR_HIP. */
int jepa_timing_end(double* ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* JEPA_H */
