"""The C-ABI library loads and exports every function include/jepa.h declares; argument
checks that return before any device work behave as documented.  CPU only: no call here
reaches the GPU (each returns from its host-side validation first)."""
import ctypes
import os
import subprocess

import pytest

import video_vit_encoder_amd as J
from video_vit_encoder_amd import _lib


def test_library_exports_every_header_function():
    lib = J.load()
    names = J.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_version_and_status_strings():
    assert J.jepa_version() == 100
    for st in range(0, -7, -1):
        assert J.jepa_status_str(st) != "unknown status"
    assert J.jepa_status_str(42) == "unknown status"


def _enc_cfg(**kw):
    c = dict(embed_dim=1024, n_layer=24, n_head=16, ffn_dim=4096, patch=16, tubelet=2,
             in_chans=3, rope_layout=0, rope_ref_grid=0, has_mod_embed=0, final_norm=1,
             compute=1, max_rows=8192, ln_eps=1e-6, rope_theta=10000.0)
    c.update(kw)
    return _lib.jepa_encoder_config(**c)


@pytest.mark.parametrize("bad", [
    dict(n_head=0), dict(embed_dim=1000), dict(n_head=8),          # head dim 128
    dict(n_head=32, embed_dim=1024, ffn_dim=4000),                 # F not a multiple of 128
    dict(patch=14), dict(tubelet=1), dict(in_chans=1), dict(rope_layout=2),
    dict(rope_ref_grid=1), dict(rope_ref_grid=-3), dict(max_rows=0), dict(compute=5),
    dict(ln_eps=0.0), dict(rope_theta=1.0), dict(n_layer=-1),
    # width 896 (14 x 64) fits the GEMM tiles but has no LayerNorm instantiation
    dict(embed_dim=896, n_head=14),
])
def test_encoder_create_rejects_bad_config(bad):
    lib = J.load()
    h = ctypes.c_void_p()
    cfg = _enc_cfg(**bad)
    assert lib.jepa_encoder_create(ctypes.byref(cfg), ctypes.byref(h)) == _lib.JEPA_ERR_ARG
    assert h.value is None


def test_predictor_and_head_create_reject_unnormable_width():
    lib = J.load()
    h = ctypes.c_void_p()
    pc = _lib.jepa_predictor_config(enc_dim=1024, embed_dim=896, n_layer=2, n_head=14, ffn_dim=1536,
                                    n_mask_tokens=10, out_dim=1024, rope_layout=0, compute=1,
                                    max_rows=64, ln_eps=1e-6, rope_theta=10000.0)
    assert lib.jepa_predictor_create(ctypes.byref(pc), ctypes.byref(h)) == _lib.JEPA_ERR_ARG
    hc = _lib.jepa_head_config(embed_dim=896, n_layer=1, n_head=14, ffn_dim=1536, n_classes=10,
                               compute=1, max_rows=64, ln_eps=1e-6)
    assert lib.jepa_head_create(ctypes.byref(hc), ctypes.byref(h)) == _lib.JEPA_ERR_ARG
    assert h.value is None


def test_null_arguments_are_rejected():
    lib = J.load()
    assert lib.jepa_encoder_create(None, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_encode(None, None, 1, 2, 16, 16, None, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_encode_tokens(None, None, 1, 1, None, 1, 1, 1, None, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_predict(None, None, 1, None, 1, None, 1, 0, 1, 1, 1, None, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_encoder_set_tensor(None, b"x", None, 0, None, 0) == _lib.JEPA_ERR_ARG
    assert lib.jepa_predictor_set_tensor(None, b"x", None, 0, None, 0) == _lib.JEPA_ERR_ARG
    lib.jepa_encoder_free(None)
    lib.jepa_predictor_free(None)


def test_standalone_ops_validate_before_launch():
    lib = J.load()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation
    # rope3d: odd head dim, stride below the row, bad layout, grid side 1 with interpolation
    assert lib.jepa_rope3d(fake, fake, 0, 1, 4, 1, 63, 63, None, 1, 2, 2, 0, 1e4, 0, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_rope3d(fake, fake, 0, 1, 4, 2, 64, 64, None, 1, 2, 2, 0, 1e4, 0, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_rope3d(fake, fake, 0, 1, 4, 1, 64, 64, None, 1, 2, 2, 7, 1e4, 0, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_rope3d(fake, fake, 0, 1, 4, 1, 64, 64, None, 4, 1, 1, 0, 1e4, 16, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_rope3d(fake, fake, 0, 1, 5, 1, 64, 64, None, 1, 2, 2, 0, 1e4, 0, None) == _lib.JEPA_ERR_SHAPE
    # empty inputs are no-ops that touch nothing
    assert lib.jepa_rope3d(fake, fake, 0, 0, 4, 1, 64, 64, None, 1, 2, 2, 0, 1e4, 0, None) == _lib.JEPA_OK
    assert lib.jepa_layernorm(fake, fake, fake, 0, 1024, 1e-6, fake, 0, None) == _lib.JEPA_OK
    assert lib.jepa_linear(fake, fake, None, fake, 0, 128, 64, 1, 0, 1, None) == _lib.JEPA_OK
    # layernorm: width not a multiple of 64 / above 4096 / not instantiated
    assert lib.jepa_layernorm(fake, fake, fake, 4, 100, 1e-6, fake, 0, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_layernorm(fake, fake, fake, 4, 8192, 1e-6, fake, 0, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_layernorm(fake, fake, fake, 4, 64 * 7, 1e-6, fake, 0, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_layernorm(fake, fake, fake, 4, 896, 1e-6, fake, 0, None) == _lib.JEPA_ERR_SHAPE
    # the ViT-g width (1408 = 22 x 64) is instantiated
    assert lib.jepa_layernorm(fake, fake, fake, 0, 1408, 1e-6, fake, 0, None) == _lib.JEPA_OK
    # linear: bf16 tiles need N % 128 and K % 64; residual needs fp32 output
    assert lib.jepa_linear(fake, fake, None, fake, 4, 100, 64, 1, 0, 1, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_linear(fake, fake, None, fake, 4, 128, 60, 1, 0, 1, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_linear(fake, fake, None, fake, 4, 128, 64, 1, 2, 1, None) == _lib.JEPA_ERR_ARG
    # attention: head dim 48, grid side above the table limit
    assert lib.jepa_attention(fake, fake, 1, 1, 8, 1, 48, None, 1, 2, 4, 0, 1e4, 0, None, 0, None) == _lib.JEPA_ERR_SHAPE
    assert lib.jepa_attention(fake, fake, 1, 1, 65, 1, 64, None, 65, 1, 1, 0, 1e4, 0, None, 0, None) == _lib.JEPA_ERR_SHAPE
    # bf16 needs a workspace of jepa_attention_workspace_size bytes
    need = lib.jepa_attention_workspace_size(1, 1, 8, 1, 64)
    assert need > 8 * 3 * 64 * 2
    assert lib.jepa_attention(fake, fake, 1, 1, 8, 1, 64, None, 1, 2, 4, 0, 1e4, 0, None, 0, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_attention(fake, fake, 1, 1, 8, 1, 64, None, 1, 2, 4, 0, 1e4, 0, fake, need - 1, None) == _lib.JEPA_ERR_ARG
    # bf16 buffers must be 16-byte aligned (checked before anything is launched)
    odd = ctypes.c_void_p(fake.value + 8)
    assert lib.jepa_attention(fake, odd, 1, 1, 8, 1, 64, None, 1, 2, 4, 0, 1e4, 0, fake, need, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_attention(odd, fake, 1, 1, 8, 1, 64, None, 1, 2, 4, 0, 1e4, 0, fake, need, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_attention(fake, fake, 1, 1, 8, 1, 64, None, 1, 2, 4, 0, 1e4, 0, odd, need, None) == _lib.JEPA_ERR_ARG
    assert lib.jepa_attention_workspace_size(0, 1, 8, 1, 64) == 0
    assert lib.jepa_attention_workspace_size(1, 0, 8, 1, 64) == 0



def _attn_ws_without_pieces(B, N, H, hd):
    # RoPE table (3 axes x 64 coordinates x 16 frequencies of (cos, sin)) | q', k' bf16
    # [B N, 2 D] | V^T bf16 [B][H][hd][N up to 16] + 4 KB read past the last row, each part
    # rounded up to 256 bytes
    up = lambda v: (v + 255) // 256 * 256
    D = H * hd
    return up(3 * 64 * 16 * 8) + up(B * N * 2 * D * 2) + up(B * D * ((N + 15) // 16 * 16) * 2 + 4096)


@pytest.mark.parametrize("B,N,H,hd,blocks,pieces", [
    # (clip, head) pairs of 512-query blocks against 256 compute units
    (4, 2048, 16, 64, 4, 1),     # ViT-L at 16 frames: below 4096 tokens, keys whole
    (1, 18432, 12, 64, 36, 1),   # 2.1 ViT-B at 18,432: 432 pairs, pieces would not save a tenth
    (1, 8192, 16, 64, 16, 1),    # ViT-L at 64 frames: 256 pairs, one full round
    (1, 8192, 12, 32, 16, 4),    # V-JEPA 2 predictor: 192 pairs -> 768 workgroups, 3 rounds
    (1, 4608, 12, 32, 9, 2),     # 2.1 predictor: 108 pairs -> 216 workgroups
    (3, 4608, 12, 32, 9, 2),     # the same clips in a batch: the same pieces
    (1, 4096, 16, 64, 8, 2),     # ViT-L at 32 frames, one clip: 128 pairs -> 256
    (1, 4225, 2, 32, 9, 8),      # few heads: 18 pairs, the most pieces
    (1, 4095, 2, 32, 8, 1),      # below 4096 tokens
])
def test_attention_key_pieces_follow_clip_length_and_heads(B, N, H, hd, blocks, pieces):
    """The flash kernel's key pieces, read off the workspace size on the host: the records
    take (hd/2 + 2) fp32 values per lane, 64 lanes, 2 query groups and 8 waves per (clip,
    head, query block, piece), and the piece count depends on N and the head count only."""
    got = _lib.load().jepa_attention_workspace_size(1, B, N, H, hd)
    rec = 0 if pieces == 1 else B * H * blocks * pieces * 8 * 2 * (hd // 2 + 2) * 64 * 4
    assert got == _attn_ws_without_pieces(B, N, H, hd) + rec

def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libjepa.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()


def test_one_hip_runtime_in_the_process():
    # libjepa must bind to the HIP runtime torch loaded, not bring a second one
    import subprocess, sys
    code = ("import video_vit_encoder_amd as J; J.load();"
            "m = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l};"
            "print(len(m))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_timing_state_errors():
    lib = J.load()
    # neither call reaches the GPU: begin rejects cap < 1 before creating events, end
    # rejects a timing session that was never begun
    assert lib.jepa_timing_begin(0) == _lib.JEPA_ERR_ARG
    assert lib.jepa_timing_end(None, None) == _lib.JEPA_ERR_STATE
