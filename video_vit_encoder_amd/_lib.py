"""ctypes binding of libjepa (include/jepa.h): argument marshalling only.

Every function here has the name of the C entry point it calls and takes torch tensors
for device buffers (their data pointers are passed through) and numpy arrays for host
buffers.  Work is enqueued on ``torch.cuda.current_stream()``.  A non-zero status raises
``JepaError``.  If libjepa.so is missing the import of a function fails loudly: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libjepa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "jepa.h")

JEPA_OK, JEPA_ERR_ARG, JEPA_ERR_SHAPE, JEPA_ERR_STATE = 0, -1, -2, -3
JEPA_ERR_NAME, JEPA_ERR_OOM, JEPA_ERR_HIP = -4, -5, -6
JEPA_ROPE_TILED, JEPA_ROPE_INTERLEAVED = 0, 1
JEPA_F32, JEPA_BF16 = 0, 1
JEPA_EPI_STORE, JEPA_EPI_GELU, JEPA_EPI_RESIDUAL = 0, 1, 2
KERNEL_CLASSES = ("patchify", "gemm_embed", "layernorm", "gemm_qkv", "attention", "gemm_out",
                  "gemm_up", "gemm_down", "other")

LAYOUTS = {"tiled": JEPA_ROPE_TILED, "interleaved": JEPA_ROPE_INTERLEAVED}
DTYPES = {"f32": JEPA_F32, "bf16": JEPA_BF16}


class JepaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({_status_str(status)})")


class jepa_encoder_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "embed_dim", "n_layer", "n_head", "ffn_dim", "patch", "tubelet", "in_chans",
        "rope_layout", "rope_ref_grid", "has_mod_embed", "final_norm", "compute", "max_rows")] + [
        ("ln_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("has_image_embed", ctypes.c_int32)]


class jepa_predictor_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "enc_dim", "embed_dim", "n_layer", "n_head", "ffn_dim", "n_mask_tokens", "out_dim",
        "rope_layout", "compute", "max_rows")] + [
        ("ln_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("has_mod_embed", ctypes.c_int32), ("has_proj_context", ctypes.c_int32)]


class jepa_head_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "embed_dim", "n_layer", "n_head", "ffn_dim", "n_classes", "compute", "max_rows")] + [
        ("ln_eps", ctypes.c_float)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "jepa_version": ([], _I),
    "jepa_status_str": ([_I], ctypes.c_char_p),
    "jepa_encoder_create": ([ctypes.POINTER(jepa_encoder_config), ctypes.POINTER(_P)], _I),
    "jepa_encoder_free": ([_P], None),
    "jepa_encoder_set_tensor": ([_P, ctypes.c_char_p, _P, _I, ctypes.POINTER(_I64), _I], _I),
    "jepa_encode": ([_P, _P, _I, _I, _I, _I, _P, _P], _I),
    "jepa_encode_tokens": ([_P, _P, _I, _I, _P, _I, _I, _I, _P, _P], _I),
    "jepa_encode_masked": ([_P, _P, _I, _I, _I, _I, _P, _I, _P, _P], _I),
    "jepa_encode_image": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "jepa_predictor_create": ([ctypes.POINTER(jepa_predictor_config), ctypes.POINTER(_P)], _I),
    "jepa_predictor_free": ([_P], None),
    "jepa_predictor_set_tensor": ([_P, ctypes.c_char_p, _P, _I, ctypes.POINTER(_I64), _I], _I),
    "jepa_predict": ([_P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P], _I),
    "jepa_predict_mod": ([_P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "jepa_pool_mean": ([_P, _I, _I, _I, _P, _P], _I),
    "jepa_head_create": ([ctypes.POINTER(jepa_head_config), ctypes.POINTER(_P)], _I),
    "jepa_head_free": ([_P], None),
    "jepa_head_set_tensor": ([_P, ctypes.c_char_p, _P, _I, ctypes.POINTER(_I64), _I], _I),
    "jepa_head_forward": ([_P, _P, _I, _I, _P, _P], _I),
    "jepa_rope3d": ([_P, _P, _I, _I, _I, _I, _I, _I64, _P, _I, _I, _I, _I, _F, _I, _P], _I),
    "jepa_layernorm": ([_P, _P, _P, _I, _I, _F, _P, _I, _P], _I),
    "jepa_linear": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P], _I),
    "jepa_attention_noalloc": ([_P, _P, _I, _I, _I, _I, _I, _P, _I, _I, _I, _I, _F, _I, _P], _I),
    "jepa_attention": ([_P, _P, _I, _I, _I, _I, _I, _P, _I, _I, _I, _I, _F, _I, _P, ctypes.c_size_t,
                        _P], _I),
    "jepa_attention_workspace_size": ([_I, _I, _I, _I, _I], ctypes.c_size_t),
    "jepa_attention_block_causal": ([_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P,
                                     ctypes.c_size_t, _P], _I),
    "jepa_timing_begin": ([_I], _I),
    "jepa_timing_end": ([ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I)], _I),
}

_lib = None
_ENC_CFG = {}
_PRED_CFG = {}


def _torch():
    import torch
    return torch


def _enc_dim(handle: int) -> int:
    return _ENC_CFG[handle].embed_dim


def load() -> ctypes.CDLL:
    """Load libjepa.so from the package directory (raises if it was never built).

    torch is imported first: its HIP runtime (same soname as the system one) is then
    already in the process, so libjepa binds to it and shares torch's device memory and
    streams.  Loading libjepa first would bring a second, separate HIP runtime."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m video_vit_encoder_amd.build`")
        import torch  # noqa: F401  (see above)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/jepa.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jepa_[a-z0-9_]+)\s*\(", src)))


def _status_str(st: int) -> str:
    try:
        return load().jepa_status_str(st).decode()
    except Exception:  # pragma: no cover - only reached while reporting an error
        return "?"


def _check(fn: str, st: int) -> None:
    if st != JEPA_OK:
        raise JepaError(fn, st)


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _host_tensor(arr: np.ndarray):
    """(pointer, dtype code, shape array, keepalive) for a host tensor upload."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.float32:
        code = JEPA_F32
    elif a.dtype == np.uint16:
        code = JEPA_BF16
    else:
        a = np.ascontiguousarray(a, dtype=np.float32)
        code = JEPA_F32
    shape = (_I64 * a.ndim)(*a.shape)
    return a.ctypes.data_as(_P), code, shape, a


# ------------------------------------------------------------------ entry points


def jepa_version() -> int:
    return load().jepa_version()


def jepa_status_str(status: int) -> str:
    return load().jepa_status_str(status).decode()


def jepa_encoder_create(cfg: jepa_encoder_config) -> int:
    h = _P()
    _check("jepa_encoder_create", load().jepa_encoder_create(ctypes.byref(cfg), ctypes.byref(h)))
    _ENC_CFG[h.value] = cfg
    return h.value


def jepa_encoder_free(handle: int) -> None:
    load().jepa_encoder_free(handle)
    _ENC_CFG.pop(handle, None)


def jepa_encoder_set_tensor(handle: int, name: str, arr: np.ndarray) -> None:
    p, code, shape, keep = _host_tensor(arr)
    _check("jepa_encoder_set_tensor",
           load().jepa_encoder_set_tensor(handle, name.encode(), p, code, shape, keep.ndim))


def jepa_encode(handle: int, clip, out, stream=None) -> None:
    """clip: uint8 device tensor [B, T, H, W, 3]; out: fp32 device tensor [B, N, D]."""
    B, T, H, W, C = clip.shape
    _need(C == 3 and clip.dtype == _torch().uint8, "clip must be uint8 [B, T, H, W, 3]")
    N = (T // 2) * (H // 16) * (W // 16)
    _need(out.dtype == _torch().float32 and out.numel() == B * N * _enc_dim(handle),
          "out must be fp32 [B, N, D]")
    _check("jepa_encode", load().jepa_encode(handle, _ptr(clip), B, T, H, W, _ptr(out),
                                             _stream(stream)))


def jepa_encode_tokens(handle: int, x, ids, grid: Sequence[int], out, stream=None) -> None:
    """x: fp32 [B, N, D]; ids: int32 [N] device tensor or None; out: fp32 [B, N, D]."""
    B, N, D = x.shape
    _need(D == _enc_dim(handle) and x.dtype == _torch().float32, "x must be fp32 [B, N, D]")
    _need(out.shape == x.shape and out.dtype == x.dtype, "out must match x")
    _need(ids is None or (ids.numel() == N and ids.dtype == _torch().int32), "ids must be int32 [N]")
    gt, gh, gw = grid
    _check("jepa_encode_tokens",
           load().jepa_encode_tokens(handle, _ptr(x), B, N, _ptr(ids), gt, gh, gw, _ptr(out),
                                     _stream(stream)))


def jepa_encode_masked(handle: int, clip, ids, out, stream=None) -> None:
    """clip: uint8 device tensor [B, T, H, W, 3]; ids: int32 device tensor [B, K] (context
    grid ids of each clip); out: fp32 device tensor [B, K, D]."""
    B, T, H, W, C = clip.shape
    _need(C == 3 and clip.dtype == _torch().uint8, "clip must be uint8 [B, T, H, W, 3]")
    _need(ids is not None and ids.dtype == _torch().int32 and ids.dim() == 2 and ids.shape[0] == B
          and ids.is_contiguous(), "ids must be contiguous int32 [B, K]")
    K = ids.shape[1]
    _need(out.dtype == _torch().float32 and out.numel() == B * K * _enc_dim(handle),
          "out must be fp32 [B, K, D]")
    _check("jepa_encode_masked", load().jepa_encode_masked(handle, _ptr(clip), B, T, H, W, _ptr(ids), K,
                                                           _ptr(out), _stream(stream)))


def jepa_encode_image(handle: int, img, out, stream=None) -> None:
    """img: uint8 device tensor [B, H, W, 3]; out: fp32 device tensor [B, N, D]."""
    B, H, W, C = img.shape
    _need(C == 3 and img.dtype == _torch().uint8, "img must be uint8 [B, H, W, 3]")
    N = (H // 16) * (W // 16)
    _need(out.dtype == _torch().float32 and out.numel() == B * N * _enc_dim(handle),
          "out must be fp32 [B, N, D]")
    _check("jepa_encode_image", load().jepa_encode_image(handle, _ptr(img), B, H, W, _ptr(out),
                                                         _stream(stream)))


def jepa_predictor_create(cfg: jepa_predictor_config) -> int:
    h = _P()
    _check("jepa_predictor_create",
           load().jepa_predictor_create(ctypes.byref(cfg), ctypes.byref(h)))
    _PRED_CFG[h.value] = cfg
    return h.value


def jepa_predictor_free(handle: int) -> None:
    load().jepa_predictor_free(handle)
    _PRED_CFG.pop(handle, None)


def jepa_predictor_set_tensor(handle: int, name: str, arr: np.ndarray) -> None:
    p, code, shape, keep = _host_tensor(arr)
    _check("jepa_predictor_set_tensor",
           load().jepa_predictor_set_tensor(handle, name.encode(), p, code, shape, keep.ndim))


def jepa_predict(handle: int, z, ids_ctx, ids_tgt, mask_index: int, grid: Sequence[int], out,
                 stream=None) -> None:
    """z: fp32 [n_enc, Denc]; ids_ctx/ids_tgt: int32 device tensors; out: fp32 [n_tgt, Dout]."""
    c = _PRED_CFG[handle]
    _need(z.dim() == 2 and z.shape[1] == c.enc_dim and z.dtype == _torch().float32,
          "z must be fp32 [n_enc, enc_dim]")
    for t in (ids_ctx, ids_tgt):
        _need(t.dtype == _torch().int32, "ids must be int32")
    _need(out.dtype == _torch().float32 and out.numel() == ids_tgt.numel() * c.out_dim,
          "out must be fp32 [n_tgt, out_dim]")
    gt, gh, gw = grid
    _check("jepa_predict",
           load().jepa_predict(handle, _ptr(z), z.shape[0], _ptr(ids_ctx), ids_ctx.numel(),
                               _ptr(ids_tgt), ids_tgt.numel(), mask_index, gt, gh, gw, _ptr(out),
                               _stream(stream)))


def jepa_pool_mean(x, out, stream=None) -> None:
    """x: fp32 device tensor [B, N, D]; out: fp32 device tensor [B, D]."""
    B, N, D = x.shape
    _need(x.dtype == _torch().float32 and out.dtype == x.dtype and out.numel() == B * D,
          "x must be fp32 [B, N, D] and out fp32 [B, D]")
    _check("jepa_pool_mean", load().jepa_pool_mean(_ptr(x), B, N, D, _ptr(out), _stream(stream)))


_HEAD_CFG = {}


def jepa_head_create(cfg: jepa_head_config) -> int:
    h = _P()
    _check("jepa_head_create", load().jepa_head_create(ctypes.byref(cfg), ctypes.byref(h)))
    _HEAD_CFG[h.value] = cfg
    return h.value


def jepa_head_free(handle: int) -> None:
    load().jepa_head_free(handle)
    _HEAD_CFG.pop(handle, None)


def jepa_head_set_tensor(handle: int, name: str, arr: np.ndarray) -> None:
    p, code, shape, keep = _host_tensor(arr)
    _check("jepa_head_set_tensor",
           load().jepa_head_set_tensor(handle, name.encode(), p, code, shape, keep.ndim))


def jepa_head_forward(handle: int, x, logits, stream=None) -> None:
    """x: fp32 device tensor [B, N, D]; logits: fp32 device tensor [B, n_classes]."""
    c = _HEAD_CFG[handle]
    B, N, D = x.shape
    _need(D == c.embed_dim and x.dtype == _torch().float32, "x must be fp32 [B, N, D]")
    _need(logits.dtype == _torch().float32 and logits.numel() == B * c.n_classes,
          "logits must be fp32 [B, n_classes]")
    _check("jepa_head_forward", load().jepa_head_forward(handle, _ptr(x), B, N, _ptr(logits),
                                                         _stream(stream)))


MODALITIES = {"video": 0, "image": 1, "auto": 2}


def jepa_predict_mod(handle: int, z, ids_ctx, ids_tgt, mask_index: int, modality: str,
                     grid: Sequence[int], out, ctx_out=None, stream=None) -> None:
    """jepa_predict with the 2.1 modality vector ('video', 'image' or 'auto') and, when
    ctx_out (fp32 [n_ctx, Dout]) is given, the context projection."""
    c = _PRED_CFG[handle]
    _need(z.dim() == 2 and z.shape[1] == c.enc_dim and z.dtype == _torch().float32,
          "z must be fp32 [n_enc, enc_dim]")
    for t in (ids_ctx, ids_tgt):
        _need(t.dtype == _torch().int32, "ids must be int32")
    _need(out.dtype == _torch().float32 and out.numel() == ids_tgt.numel() * c.out_dim,
          "out must be fp32 [n_tgt, out_dim]")
    _need(ctx_out is None or (ctx_out.dtype == _torch().float32 and
                              ctx_out.numel() == ids_ctx.numel() * c.out_dim),
          "ctx_out must be fp32 [n_ctx, out_dim]")
    _need(modality in MODALITIES, "modality must be 'video', 'image' or 'auto'")
    gt, gh, gw = grid
    _check("jepa_predict_mod",
           load().jepa_predict_mod(handle, _ptr(z), z.shape[0], _ptr(ids_ctx), ids_ctx.numel(),
                                   _ptr(ids_tgt), ids_tgt.numel(), mask_index, MODALITIES[modality],
                                   gt, gh, gw, _ptr(out), _ptr(ctx_out), _stream(stream)))


def jepa_rope3d(x, y, B: int, N: int, n_head: int, head_dim: int, row_stride: int, ids,
                grid: Sequence[int], layout: str, theta: float = 10000.0, ref_grid: int = 0,
                stream=None) -> None:
    """x, y: fp32 or bf16 (torch.bfloat16) device tensors; y may be x."""
    import torch
    dt = JEPA_BF16 if x.dtype == torch.bfloat16 else JEPA_F32
    _need(x.dtype in (torch.float32, torch.bfloat16) and y.dtype == x.dtype, "x, y: fp32 or bf16")
    if B * N > 0:
        need = (B * N - 1) * row_stride + n_head * head_dim
        _need(x.numel() >= need and y.numel() >= need, "x/y smaller than B*N rows of row_stride")
    _need(ids is None or (ids.numel() >= N and ids.dtype == torch.int32), "ids must be int32 [N]")
    gt, gh, gw = grid
    _check("jepa_rope3d",
           load().jepa_rope3d(_ptr(x), _ptr(y), dt, B, N, n_head, head_dim, row_stride, _ptr(ids),
                              gt, gh, gw, LAYOUTS[layout], theta, ref_grid, _stream(stream)))


def jepa_layernorm(x, weight, bias, eps: float, out, stream=None) -> None:
    import torch
    M, D = x.shape
    _need(x.dtype == torch.float32 and weight.numel() == D and bias.numel() == D
          and weight.dtype == torch.float32 and bias.dtype == torch.float32, "fp32 x, weight, bias")
    _need(out.numel() == M * D and out.dtype in (torch.float32, torch.bfloat16), "out [M, D]")
    od = JEPA_BF16 if out.dtype == torch.bfloat16 else JEPA_F32
    _check("jepa_layernorm",
           load().jepa_layernorm(_ptr(x), _ptr(weight), _ptr(bias), M, D, eps, _ptr(out), od,
                                 _stream(stream)))


def jepa_linear(A, W, bias, C, epilogue: int = JEPA_EPI_STORE, stream=None) -> None:
    """C = epilogue(A W^T + bias); A [M, K], W [N, K] (same dtype), C [M, N]."""
    import torch
    M, K = A.shape
    N = W.shape[0]
    _need(W.dim() == 2 and W.shape[1] == K and W.dtype == A.dtype, "W must be [N, K] like A")
    _need(C.dim() == 2 and tuple(C.shape) == (M, N), "C must be [M, N]")
    _need(bias is None or (bias.numel() == N and bias.dtype == torch.float32), "bias fp32 [N]")
    dt = JEPA_BF16 if A.dtype == torch.bfloat16 else JEPA_F32
    od = JEPA_BF16 if C.dtype == torch.bfloat16 else JEPA_F32
    _check("jepa_linear",
           load().jepa_linear(_ptr(A), _ptr(W), _ptr(bias), _ptr(C), M, N, K, dt, epilogue, od,
                              _stream(stream)))


def jepa_attention_workspace_size(dtype: int, B: int, N: int, n_head: int, head_dim: int) -> int:
    return load().jepa_attention_workspace_size(dtype, B, N, n_head, head_dim)


def jepa_attention(qkv, out, B: int, N: int, n_head: int, head_dim: int, ids,
                   grid: Sequence[int], layout: str, theta: float = 10000.0, ref_grid: int = 0,
                   stream=None, work=None) -> None:
    """qkv [B*N, 3D] and out [B*N, D] device tensors of one dtype.  The bf16 path needs a
    device workspace: ``work`` (a uint8 tensor) or one allocated here."""
    import torch
    dt = JEPA_BF16 if qkv.dtype == torch.bfloat16 else JEPA_F32
    D = n_head * head_dim
    _need(qkv.numel() == B * N * 3 * D and out.numel() == B * N * D and out.dtype == qkv.dtype,
          "qkv [B*N, 3D] and out [B*N, D] of one dtype")
    _need(ids is None or (ids.numel() >= N and ids.dtype == torch.int32), "ids must be int32 [N]")
    nbytes = jepa_attention_workspace_size(dt, B, N, n_head, head_dim)
    if work is None and nbytes > 0:
        work = torch.empty(nbytes, dtype=torch.uint8, device=qkv.device)
    wbytes = 0 if work is None else work.numel() * work.element_size()
    gt, gh, gw = grid
    _check("jepa_attention",
           load().jepa_attention(_ptr(qkv), _ptr(out), dt, B, N, n_head, head_dim, _ptr(ids),
                                 gt, gh, gw, LAYOUTS[layout], theta, ref_grid, _ptr(work), wbytes,
                                 _stream(stream)))


def jepa_attention_noalloc(qkv, out, B: int, N: int, n_head: int, head_dim: int, ids,
                           grid: Sequence[int], layout: str, theta: float = 10000.0,
                           ref_grid: int = 0, stream=None) -> None:
    """jepa_attention without a workspace: the library's per-GPU scratch array is used
    and nothing is allocated."""
    import torch
    dt = JEPA_BF16 if qkv.dtype == torch.bfloat16 else JEPA_F32
    D = n_head * head_dim
    _need(qkv.numel() == B * N * 3 * D and out.numel() == B * N * D and out.dtype == qkv.dtype,
          "qkv [B*N, 3D] and out [B*N, D] of one dtype")
    _need(ids is None or (ids.numel() >= N and ids.dtype == torch.int32), "ids must be int32 [N]")
    gt, gh, gw = grid
    _check("jepa_attention_noalloc",
           load().jepa_attention_noalloc(_ptr(qkv), _ptr(out), dt, B, N, n_head, head_dim, _ptr(ids),
                                         gt, gh, gw, LAYOUTS[layout], theta, ref_grid,
                                         _stream(stream)))


def jepa_attention_block_causal(qkv, out, B: int, n_cls: int, n_head: int, head_dim: int,
                                grid: Sequence[int], layout: str, theta: float = 10000.0,
                                ref_grid: int = 0, stream=None, work=None) -> None:
    """Block-causal attention with n_cls leading CLS rows: qkv [B*N, 3D] and out [B*N, D]
    device tensors of one dtype, N = n_cls + gt*gh*gw."""
    import torch
    dt = JEPA_BF16 if qkv.dtype == torch.bfloat16 else JEPA_F32
    gt, gh, gw = grid
    N = n_cls + gt * gh * gw
    D = n_head * head_dim
    _need(qkv.numel() == B * N * 3 * D and out.numel() == B * N * D and out.dtype == qkv.dtype,
          "qkv [B*N, 3D] and out [B*N, D] of one dtype, N = n_cls + gt*gh*gw")
    nbytes = jepa_attention_workspace_size(dt, B, N, n_head, head_dim)
    if work is None and nbytes > 0:
        work = torch.empty(nbytes, dtype=torch.uint8, device=qkv.device)
    wbytes = 0 if work is None else work.numel() * work.element_size()
    _check("jepa_attention_block_causal",
           load().jepa_attention_block_causal(_ptr(qkv), _ptr(out), dt, B, n_cls, n_head, head_dim,
                                              gt, gh, gw, LAYOUTS[layout], theta, ref_grid,
                                              _ptr(work), wbytes, _stream(stream)))


def jepa_timing_begin(cap: int) -> None:
    """Record a HIP event pair around each launch of the forwards (at most cap per class)."""
    _check("jepa_timing_begin", load().jepa_timing_begin(cap))


def jepa_timing_end() -> dict:
    """{class name: (summed launch ms, launches)} of the launches recorded since begin."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (_I * n)()
    _check("jepa_timing_end", load().jepa_timing_end(ms, cnt))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_CLASSES)}
