"""CPU-side checks of the C ABI: the library loads, exports exactly what the
header declares, plans its workspace correctly, and rejects every bad
argument before touching the GPU.  No kernel is launched here: every call
either fails validation or (valid arguments, no device) reports ERR_HIP,
and the latter only runs on a machine without a GPU."""
import ctypes
import os
import re

import pytest

import video_diffusion_transformer_adaln_amd as h3k
from video_diffusion_transformer_adaln_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3k.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3k_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = h3k.lib()
    declared = _declared()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTED) == declared


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(B.DitConfig) == 72
    assert ctypes.sizeof(B.DitBlockWeights) == 14 * 8
    assert ctypes.sizeof(B.DitStats) == 48
    assert ctypes.sizeof(B.DitPlanInfo) == 9 * 8 * 2 + 9 * 4 * 2 + 8 * 5 + 8 + 32
    assert ctypes.sizeof(B.DeviceInfo) == 4 * 4 + 8 + 64


def test_device_info_rejects_null_and_missing_devices():
    lib = h3k.lib()
    assert lib.h3k_get_device_info(0, None) == B.H3K_ERR_NULL
    d = B.DeviceInfo()
    assert lib.h3k_get_device_info(-1, ctypes.byref(d)) == B.H3K_ERR_HIP
    assert lib.h3k_get_device_info(1 << 20, ctypes.byref(d)) == B.H3K_ERR_HIP
    assert d.compute_units == 0 and d.arch == b""   # untouched on error


def cfg_c2(**kw):
    base = dict(n_tokens=22680, hidden=5120, n_heads=40, head_dim=128, mlp_hidden=13824, cond_dim=5120,
                act_dtype=B.H3K_BF16)
    base.update(kw)
    return B.make_config(**base)


def _live(info, t, s):
    return info.first_step[t] <= s <= info.last_step[t]


@pytest.mark.parametrize("alias", [True, False])
@pytest.mark.parametrize("shape", [
    dict(n_tokens=22680, hidden=5120, n_heads=40, head_dim=128, mlp_hidden=13824, cond_dim=5120, act_dtype=1),
    dict(n_tokens=6144, hidden=3072, n_heads=24, head_dim=128, mlp_hidden=12288, cond_dim=3072, act_dtype=1),
    dict(n_tokens=512, hidden=256, n_heads=4, head_dim=64, mlp_hidden=1024, cond_dim=256, act_dtype=0),
    dict(n_tokens=1, hidden=128, n_heads=2, head_dim=64, mlp_hidden=64, cond_dim=8, act_dtype=1),
    dict(n_tokens=333, hidden=320, n_heads=5, head_dim=64, mlp_hidden=2048, cond_dim=64, act_dtype=1),
    dict(n_tokens=22680, hidden=5120, n_heads=40, head_dim=128, mlp_hidden=13824, cond_dim=5120, act_dtype=1,
         weight_dtype=2, int8_fc2_rows=True),
    dict(n_tokens=37, hidden=256, n_heads=2, head_dim=128, mlp_hidden=384, cond_dim=64, act_dtype=1,
         weight_dtype=2, int8_fc2_rows=True),
])
def test_plan_no_live_overlap(shape, alias):
    cfg = B.make_config(alias=alias, **shape)
    info = h3k.h3k_dit_plan(cfg)
    n = len(B.TENSOR_NAMES)
    for t in range(n):
        assert info.offset[t] % 256 == 0
        assert info.offset[t] + info.bytes[t] <= info.workspace_bytes
    for s in range(9):
        live = [t for t in range(n) if _live(info, t, s)]
        for i in live:
            for j in live:
                if i < j:
                    a0, a1 = info.offset[i], info.offset[i] + info.bytes[i]
                    b0, b1 = info.offset[j], info.offset[j] + info.bytes[j]
                    assert a1 <= b0 or b1 <= a0, (B.TENSOR_NAMES[i], B.TENSOR_NAMES[j], s)
    if alias:
        assert info.workspace_bytes < info.unaliased_bytes
        assert info.workspace_bytes >= info.peak_live_bytes
    else:
        assert info.workspace_bytes == info.unaliased_bytes
    assert h3k.h3k_dit_workspace_size(cfg, 3) == info.workspace_bytes


def test_plan_c2_sizes_and_layout():
    """The 864x480x56-frame block: tensor sizes and the aliasing it yields."""
    N, D, F = 22680, 5120, 13824
    on = h3k.h3k_dit_plan(cfg_c2(alias=True))
    off = h3k.h3k_dit_plan(cfg_c2(alias=False))
    act = N * D * 2
    assert on.bytes[1] == act and on.bytes[3] == act and on.bytes[4] == act and on.bytes[5] == act
    assert on.bytes[6] == N * F * 2
    assert on.bytes[2] == N * 2 * D * 2 + D * N * 2          # [Q | K] + V^T (22680 is a multiple of 8)
    assert on.vt_pitch == N
    # first fit: o and h2 reuse h's region; x1 sits at the start of the dead qkv; u follows x1
    assert on.offset[3] == on.offset[1] and on.offset[5] == on.offset[1]
    assert on.offset[4] == on.offset[2]
    assert on.offset[6] == on.offset[4] + act
    assert on.workspace_bytes == on.offset[6] + N * F * 2
    assert off.workspace_bytes - on.workspace_bytes > 1_000_000_000      # > 1 GB saved
    assert on.peak_live_bytes == on.workspace_bytes


def test_token_reduction_adds_the_merged_stream_to_the_workspace():
    plain = h3k.h3k_dit_workspace_size(cfg_c2())
    red = h3k.h3k_dit_workspace_size(cfg_c2(token_reduction=(12, 38)))
    merged = ((22680 // 2) * 5120 * 2 + 255) // 256 * 256
    info = h3k.h3k_dit_plan(cfg_c2(token_reduction=(12, 38)))
    # 22680 tokens: no GEMM tail is split (no scratch); the reduced blocks' 11340 tokens leave
    # 126 MLP-up tiles in the last wave, split two ways: 126 * 2 partial tiles of 256 KiB
    assert h3k.h3k_dit_plan(cfg_c2()).part_bytes == 0
    assert info.part_bytes == 126 * 2 * 256 * 256 * 4
    assert red - plain == merged + info.part_bytes
    tensors_end = max(info.offset[t] + info.bytes[t] for t in range(9))
    assert tensors_end <= info.part_offset
    assert info.part_offset + info.part_bytes == info.workspace_bytes - merged


def test_int8_weight_staging_buffer():
    """INT8 weights with BF16 activations: a staging buffer of the largest bf16 projection
    weight (QKV, 3D x D) after the k-split scratch; nothing for bf16 or fp32 weights."""
    D, F = 5120, 13824
    info = h3k.h3k_dit_plan(cfg_c2(weight_dtype=B.H3K_INT8))
    assert info.wstage_bytes == 3 * D * D * 2
    assert info.wstage_offset == info.part_offset + info.part_bytes
    assert info.wstage_offset + info.wstage_bytes == info.workspace_bytes
    wide = h3k.h3k_dit_plan(B.make_config(512, 1024, 8, 128, 8192, 1024, B.H3K_BF16, B.H3K_INT8))
    assert wide.wstage_bytes == 1024 * 8192 * 2                 # D x F > 3D x D
    assert h3k.h3k_dit_plan(cfg_c2()).wstage_bytes == 0
    assert h3k.h3k_dit_plan(B.make_config(512, 256, 4, 64, 1024, 256, B.H3K_F32)).wstage_bytes == 0


def _rule_part_bytes(N, D, H, d, F, int8_fc2=False, reduction=False):
    """The split-tail scratch from the rules restated in tests/gpu_util.py at
    256 CUs: the largest need of the out / up / down GEMMs and the attention,
    over N tokens and (with token reduction) N/2."""
    import gpu_util as G

    def need(n):
        tm = (n + 255) // 256
        best = 0
        for i, (nn, k) in enumerate(((D, D), (F, D), (D, F))):
            if i == 2 and int8_fc2:
                continue
            tiles = tm * ((nn + 255) // 256)
            S = G.tail_split_ways(tiles, k // 64, 256, 256)
            if S:
                best = max(best, (tiles % 256) * S * 256 * 256 * 4)
        if d == 128:
            tiles = (n + 31) // 32
            unit = lambda nw: nw * 32 * 130 * 4
            b8 = (n + 255) // 256 * H
            s8 = G.attn_split_ways(b8, tiles, 256, 1 << 40)
            four = (n + 255) // 256 * H < 1024 and n <= 8192
            if s8:
                best = max(best, (b8 % 256) * s8 * unit(8))
            elif four:
                b4 = (n + 127) // 128 * H
                s4 = G.attn_split_ways(b4, tiles, 512, 1 << 40)
                if s4:
                    best = max(best, (b4 % 512) * s4 * unit(4))
        return best

    b = need(N)
    if reduction:
        b = max(b, need(N // 2))
    return (b + 255) // 256 * 256


@pytest.mark.parametrize("N", [1, 300, 2000, 4096, 6000, 6144, 8192, 11340, 12000, 22680])
@pytest.mark.parametrize("H,F", [(2, 1024), (8, 4096), (24, 12288), (40, 13824)])
def test_split_scratch_matches_the_launch_rules(N, H, F):
    """The plan's split-tail scratch is what the GEMM and attention launchers
    would use on 256 CUs, for bf16 and int8 weights, with and without token
    reduction (tests/gpu_util.py restates both rules)."""
    d = 128
    D = H * d
    for w8, fc2 in ((False, False), (True, False), (True, True)):
        for red in ((False,) if N % 2 else (False, True)):
            cfg = B.make_config(N, D, H, d, F, D, B.H3K_BF16, B.H3K_INT8 if w8 else B.H3K_BF16,
                                int8_fc2_rows=fc2, token_reduction=(0, 1) if red else None)
            want = _rule_part_bytes(N, D, H, d, F, int8_fc2=fc2, reduction=red)
            assert h3k.h3k_dit_plan(cfg).part_bytes == want, (N, H, F, w8, fc2, red)


def test_tail_split_scratch_sizes():
    """The k-split scratch the plan reserves: the largest of the out / up / down GEMMs' last-wave
    tiles times their split ways, on 256 compute units (one 256x256 tile per CU and wave)."""
    # 6144 x 3072 (F = 12288): out and down have 24 x 12 = 288 tiles, 32 in the last wave, split
    # 8 ways (256 partial tiles); up has 24 x 48 = 1152, 128 in the last wave, whose 2-way split
    # would shed only 1536 of its k = 3072 per workgroup: not split
    c1 = B.make_config(6144, 3072, 24, 128, 12288, 3072, B.H3K_BF16)
    assert h3k.h3k_dit_plan(c1).part_bytes == 256 * 256 * 256 * 4
    # the same up GEMM with k = 4096 sheds 2048: 128 tiles split 2 ways, out and down 32 x 8
    wide = B.make_config(6144, 4096, 32, 128, 12288, 64, B.H3K_BF16)   # out/down: 24 x 16 = 384, tail 128
    assert h3k.h3k_dit_plan(wide).part_bytes == 128 * 2 * 256 * 256 * 4
    # fp32 and int8-weight configs never split
    assert h3k.h3k_dit_plan(B.make_config(512, 256, 4, 64, 1024, 256, B.H3K_F32)).part_bytes == 0
    assert h3k.h3k_dit_plan(cfg_c2(weight_dtype=B.H3K_INT8)).part_bytes == 0
    # a one-tile GEMM with 64 k-tiles splits 8 ways; with 4 k-tiles it does not split
    small = B.make_config(200, 256, 2, 128, 4096, 64, B.H3K_BF16)   # down: 1 tile, k = 4096
    assert h3k.h3k_dit_plan(small).part_bytes == 1 * 8 * 256 * 256 * 4
    tiny = B.make_config(200, 256, 2, 128, 256, 64, B.H3K_BF16)     # every k = 256: 4 k-tiles
    assert h3k.h3k_dit_plan(tiny).part_bytes == 0


def test_env_switch_disables_aliasing(monkeypatch):
    monkeypatch.setenv("H3K_DISABLE_ACTIVATION_ALIAS", "1")
    info = h3k.h3k_dit_plan(cfg_c2(alias=True))
    assert info.alias_activations == 0
    assert info.workspace_bytes == info.unaliased_bytes
    monkeypatch.delenv("H3K_DISABLE_ACTIVATION_ALIAS")
    assert h3k.h3k_dit_plan(cfg_c2(alias=True)).alias_activations == 1


def test_config_rejects_int8_fc2_beyond_int32_range():
    """The row-quantised FC2 sums mlp_hidden int8 products in int32: F <= 2^17."""
    ok = B.make_config(8, 128, 2, 64, 1 << 17, 128, B.H3K_BF16, B.H3K_INT8, int8_fc2_rows=True)
    assert h3k.h3k_dit_workspace_size(ok) > 0
    bad = B.make_config(8, 128, 2, 64, (1 << 17) + 128, 128, B.H3K_BF16, B.H3K_INT8, int8_fc2_rows=True)
    out = ctypes.c_uint64()
    assert h3k.lib().h3k_dit_workspace_size(ctypes.byref(bad), 1, ctypes.byref(out)) == B.H3K_ERR_UNSUPPORTED
    assert "2^17" in h3k.last_error()


# ---------------------------------------------------------------- validation
FAKE = 0x7f0000000000          # never dereferenced: every call below fails before a launch


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


# The calls below pass never-mapped device addresses and rely on validation
# rejecting them before any launch; they run only where no GPU is visible, so
# a validation regression can never send a kernel to those addresses.
fake_pointers = pytest.mark.skipif(not _no_gpu(), reason="fake device pointers: run only without a GPU")


def _weights(**over):
    base = {f: FAKE + (i + 1) * (1 << 32) for i, f in enumerate(B.WEIGHT_FIELDS) if not f.startswith("s_")}
    base.update(over)
    return B.DitBlockWeights(*[base.get(f) for f in B.WEIGHT_FIELDS])


def _block(cfg, weights=None, x=FAKE + (100 << 32), c=FAKE + (101 << 32), out=FAKE + (102 << 32),
           ws=FAKE + (110 << 32), ws_bytes=None):
    lib = h3k.lib()
    if ws_bytes is None:
        ws_bytes = h3k.h3k_dit_workspace_size(cfg) if lib.h3k_dit_workspace_size(
            ctypes.byref(cfg), 1, ctypes.byref(ctypes.c_uint64())) == 0 else 1 << 40
    w = weights if weights is not None else _weights()
    return lib.h3k_dit_block_forward(ctypes.byref(cfg), ctypes.byref(w), x, c, out, ws, ws_bytes, None, None)


@fake_pointers
def test_reject_null_config_and_pointers():
    lib = h3k.lib()
    assert lib.h3k_dit_block_forward(None, None, 0, 0, 0, 0, 0, None, None) == B.H3K_ERR_NULL
    assert _block(cfg_c2(), x=None) == B.H3K_ERR_NULL
    assert _block(cfg_c2(), weights=_weights(w_qkv=None)) == B.H3K_ERR_NULL
    assert "w_qkv" in h3k.last_error()


@fake_pointers
def test_reject_bad_shapes_and_dtypes():
    assert _block(cfg_c2(hidden=5000)) == B.H3K_ERR_SHAPE                        # D != H*d
    assert _block(cfg_c2(n_tokens=0)) == B.H3K_ERR_SHAPE
    assert _block(cfg_c2(head_dim=96, n_heads=40, hidden=3840)) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(mlp_hidden=13800)) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(act_dtype=B.H3K_INT8)) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(act_dtype=7)) == B.H3K_ERR_DTYPE
    assert _block(cfg_c2(act_dtype=B.H3K_F32, weight_dtype=B.H3K_INT8)) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(ln_eps=0.0)) == B.H3K_ERR_SHAPE
    # the row-quantised FC2 needs int8 weights, bf16 activations, F a multiple of 128
    assert _block(cfg_c2(int8_fc2_rows=True)) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(weight_dtype=B.H3K_INT8, mlp_hidden=13824 - 64, int8_fc2_rows=True)) == B.H3K_ERR_UNSUPPORTED
    bad = cfg_c2(weight_dtype=B.H3K_INT8)
    bad.int8_fc2_rows = 2
    assert _block(bad) == B.H3K_ERR_SHAPE
    # group-wise int8 MLP: G in {32, 64, 128}, int8 weights with bf16 activations, D and F multiples of G,
    # and not together with the row-quantised FC2
    assert _block(cfg_c2(weight_dtype=B.H3K_INT8, int8_mlp_group=16)) == B.H3K_ERR_SHAPE
    assert _block(cfg_c2(int8_mlp_group=64)) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(weight_dtype=B.H3K_INT8, mlp_hidden=13824 - 64, int8_mlp_group=128)) == B.H3K_ERR_SHAPE
    assert _block(cfg_c2(weight_dtype=B.H3K_INT8, int8_mlp_group=64, int8_fc2_rows=True)) == B.H3K_ERR_UNSUPPORTED
    # 3D RoPE: the grid must hold the tokens; bf16 activations; the halving flag needs a grid
    assert _block(cfg_c2(rope=(14, 30, 53, False))) == B.H3K_ERR_SHAPE
    assert _block(cfg_c2(rope=(14, 0, 54, False))) == B.H3K_ERR_SHAPE
    f32 = dict(n_tokens=512, hidden=256, n_heads=4, head_dim=64, mlp_hidden=1024, cond_dim=256, act_dtype=B.H3K_F32)
    assert _block(B.make_config(**f32, rope=(2, 16, 16, False))) == B.H3K_ERR_UNSUPPORTED
    half_only = cfg_c2()
    half_only.rope_half_spatial = 1
    assert _block(half_only) == B.H3K_ERR_SHAPE
    # token reduction: an inverted range, an odd token count, together with RoPE, a range past the blocks
    assert _block(cfg_c2(token_reduction=(3, 2))) == B.H3K_ERR_SHAPE
    assert _block(cfg_c2(n_tokens=22679, token_reduction=(0, 1))) == B.H3K_ERR_SHAPE
    assert _block(cfg_c2(token_reduction=(0, 1), rope=(14, 30, 54, False))) == B.H3K_ERR_UNSUPPORTED
    assert _block(cfg_c2(token_reduction=(0, 2))) == B.H3K_ERR_SHAPE       # one block only
    assert "beyond" in h3k.last_error()


@fake_pointers
def test_reject_int8_without_scales():
    cfg = cfg_c2(weight_dtype=B.H3K_INT8)
    assert _block(cfg) == B.H3K_ERR_NULL
    assert "scale" in h3k.last_error()


@fake_pointers
def test_reject_misalignment_workspace_overlap():
    cfg = cfg_c2()
    assert _block(cfg, x=FAKE + (100 << 32) + 4) == B.H3K_ERR_ALIGN
    assert _block(cfg, ws=FAKE + (110 << 32) + 64) == B.H3K_ERR_ALIGN
    need = h3k.h3k_dit_workspace_size(cfg)
    assert _block(cfg, ws_bytes=need - 1) == B.H3K_ERR_WORKSPACE
    assert _block(cfg, out=FAKE + (100 << 32) + 4096) == B.H3K_ERR_OVERLAP          # out inside x
    assert _block(cfg, out=FAKE + (110 << 32) + 1024) == B.H3K_ERR_OVERLAP          # out inside workspace
    w = _weights(w_up=FAKE + (110 << 32) + 4096)                                    # weight inside workspace
    assert _block(cfg, weights=w) == B.H3K_ERR_OVERLAP


@fake_pointers
def test_reject_bad_kernel_level_arguments():
    lib = h3k.lib()
    # linear: k not a multiple of 64 for bf16
    assert lib.h3k_linear(1, 1, 10, 64, 100, FAKE, 100, FAKE + (1 << 32), 100, None, None, 0, None, 0, None,
                          FAKE + (2 << 32), 64, None, 0, 64, None) == B.H3K_ERR_SHAPE
    # gated residual without gate
    assert lib.h3k_linear(1, 1, 10, 64, 64, FAKE, 64, FAKE + (1 << 32), 64, None, None, 2, FAKE + (3 << 32), 64,
                          None, FAKE + (2 << 32), 64, None, 0, 64, None) == B.H3K_ERR_NULL
    # transposed part with GELU is not supported
    assert lib.h3k_linear(1, 1, 10, 64, 64, FAKE, 64, FAKE + (1 << 32), 64, None, None, 1, None, 0, None,
                          FAKE + (2 << 32), 64, FAKE + (4 << 32), 16, 32, None) == B.H3K_ERR_UNSUPPORTED
    # RoPE beyond 2^24 tokens (coordinates come from an exact fp32 quotient)
    assert lib.h3k_rope_3d(1 << 25, 128, 128, 1 << 13, 1 << 6, 1 << 6, 0, FAKE, 128, None) == B.H3K_ERR_UNSUPPORTED
    # attention: head_dim 32, pitch too small
    assert lib.h3k_attention(1, 100, 2, 32, FAKE, 64, FAKE, 64, FAKE, 104, FAKE, 64, 0, None) == B.H3K_ERR_UNSUPPORTED
    # prescaled q: bf16 only, flag 0 or 1
    assert lib.h3k_attention(0, 100, 2, 64, FAKE, 128, FAKE + (1 << 32), 128, FAKE + (2 << 32), 104,
                             FAKE + (3 << 32), 128, 1, None) == B.H3K_ERR_UNSUPPORTED
    assert lib.h3k_attention(1, 100, 2, 64, FAKE, 128, FAKE + (1 << 32), 128, FAKE + (2 << 32), 104,
                             FAKE + (3 << 32), 128, 2, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_attention(1, 100, 2, 64, FAKE, 128, FAKE + (1 << 32), 128, FAKE + (2 << 32), 96,
                             FAKE + (3 << 32), 128, 0, None) == B.H3K_ERR_SHAPE
    # quantiser: int8 source, overlapping q / w
    assert lib.h3k_quantize_weights_int8(FAKE, 2, 4, 64, FAKE + (1 << 32), FAKE + (2 << 32), None) == B.H3K_ERR_UNSUPPORTED
    assert lib.h3k_quantize_weights_int8(FAKE, 0, 4, 64, FAKE + 64, FAKE + (2 << 32), None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_ln_modulate(1, 4, 100, 1e-6, FAKE, 100, FAKE, FAKE, FAKE + (1 << 32), 100, None) == B.H3K_ERR_SHAPE
    # int8 x int8 linear: k not a multiple of 128, missing x_scale, misaligned xq, y overlapping wq
    X, XS, W, WS, Y = FAKE, FAKE + (1 << 32), FAKE + (2 << 32), FAKE + (3 << 32), FAKE + (4 << 32)
    assert lib.h3k_linear_int8(10, 64, 192, X, 192, XS, W, 192, WS, None, 0, None, 0, None, Y, 64, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_linear_int8(10, 64, 256, X, 256, None, W, 256, WS, None, 0, None, 0, None, Y, 64, None) == B.H3K_ERR_NULL
    assert lib.h3k_linear_int8(10, 64, 256, X + 8, 256, XS, W, 256, WS, None, 0, None, 0, None, Y, 64, None) == B.H3K_ERR_ALIGN
    assert lib.h3k_linear_int8(10, 64, 256, X, 256, XS, W, 256, WS, None, 0, None, 0, None, W + 256, 64, None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_linear_int8(10, 64, 256, X, 256, XS, W, 256, WS, None, 2, None, 0, None, Y, 64, None) == B.H3K_ERR_NULL
    assert lib.h3k_linear_int8(10, 64, 1 << 18, X, 1 << 18, XS, W, 1 << 18, WS, None, 0, None, 0, None, Y, 64,
                               None) == B.H3K_ERR_SHAPE
    assert lib.h3k_adaln_modulation(1, 10, 12, FAKE, None, FAKE, FAKE + (1 << 32), None) == B.H3K_ERR_SHAPE
    # group quantiser: group 16, cols not a multiple of the group, scales overlapping q
    Q, S = FAKE + (1 << 32), FAKE + (2 << 32)
    assert lib.h3k_quantize_weights_int8_groups(FAKE, 1, 4, 128, 16, Q, S, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_quantize_weights_int8_groups(FAKE, 1, 4, 96, 64, Q, S, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_quantize_weights_int8_groups(FAKE, 1, 4, 128, 64, Q, Q + 256, None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_quantize_weights_int8_groups(FAKE, 2, 4, 128, 64, Q, S, None) == B.H3K_ERR_UNSUPPORTED
    # group-wise int8 linear: k not a multiple of the group, no scales, y overlapping the scales, bad group
    assert lib.h3k_linear_int8_groups(10, 64, 192, 128, X, 192, W, 192, WS, None, 0, None, 0, None, Y, 64,
                                      None) == B.H3K_ERR_SHAPE
    assert lib.h3k_linear_int8_groups(10, 64, 256, 64, X, 256, W, 256, None, None, 0, None, 0, None, Y, 64,
                                      None) == B.H3K_ERR_NULL
    assert lib.h3k_linear_int8_groups(10, 64, 256, 64, X, 256, W, 256, WS, None, 0, None, 0, None, WS + 64, 64,
                                      None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_linear_int8_groups(10, 64, 256, 48, X, 256, W, 256, WS, None, 0, None, 0, None, Y, 64,
                                      None) == B.H3K_ERR_SHAPE
    # RoPE: head_dim not a multiple of 16, cols not a multiple of head_dim, grid / token mismatch, misaligned x
    assert lib.h3k_rope_3d(24, 96, 24, 2, 3, 4, 0, X, 96, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_rope_3d(24, 96, 64, 2, 3, 4, 0, X, 96, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_rope_3d(24, 128, 64, 2, 3, 5, 0, X, 128, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_rope_3d(24, 128, 64, 2, 3, 4, 2, X, 128, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_rope_3d(24, 128, 64, 2, 3, 4, 0, X + 8, 128, None) == B.H3K_ERR_ALIGN
    # token merge / unmerge: odd token count, xm overlapping x, out partially overlapping entry
    assert lib.h3k_token_merge(1, 7, 64, X, 64, Y, 64, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_token_merge(1, 8, 64, X, 64, X + 256, 64, None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_token_merge(1, 8, 60, X, 64, Y, 64, None) == B.H3K_ERR_SHAPE
    assert lib.h3k_token_unmerge(1, 8, 64, X, 64, Y, 64, X + 128, 64, None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_token_unmerge(1, 8, 64, X, 64, Y, 64, Y + 64, 64, None) == B.H3K_ERR_OVERLAP
    assert lib.h3k_token_unmerge(1, 8, 64, X, 64, Y, 64, X, 72, None) == B.H3K_ERR_SHAPE


@fake_pointers
def test_valid_arguments_without_device_report_hip_error():
    assert _block(cfg_c2()) == B.H3K_ERR_HIP
    assert "device" in h3k.last_error()
    # group-wise int8 MLP: scales are [F, D/G] and [D, F/G]; everything valid, so only the device is missing
    scales = {f: FAKE + (60 + i) * (1 << 32) for i, f in enumerate(("s_qkv", "s_out", "s_up", "s_down"))}
    assert _block(cfg_c2(weight_dtype=B.H3K_INT8, int8_mlp_group=128), weights=_weights(**scales)) == B.H3K_ERR_HIP
    lib = h3k.lib()
    assert lib.h3k_quantize_weights_int8_groups(FAKE, 1, 4, 128, 64, FAKE + (1 << 32), FAKE + (2 << 32),
                                                None) == B.H3K_ERR_HIP
    assert _block(cfg_c2(rope=(14, 30, 54, True))) == B.H3K_ERR_HIP
    assert _block(cfg_c2(token_reduction=(0, 1))) == B.H3K_ERR_HIP
    assert lib.h3k_token_merge(1, 8, 64, FAKE, 64, FAKE + (1 << 32), 64, None) == B.H3K_ERR_HIP
    assert lib.h3k_token_unmerge(1, 8, 64, FAKE, 64, FAKE + (1 << 32), 64, FAKE, 64, None) == B.H3K_ERR_HIP
    assert lib.h3k_rope_3d(24, 128, 64, 2, 3, 4, 1, FAKE, 128, None) == B.H3K_ERR_HIP
