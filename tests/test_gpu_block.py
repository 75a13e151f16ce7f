"""Block- and stack-level parity of the HIP path against the CPU oracle.

  * the small fp32 block, every element (fp32 vs fp32: 1e-4);
  * the 512x512x22-frame block (N=6144, D=3072), every element;
  * the 864x480x56-frame block (N=22680, D=5120) and its int8-weight
    variant, on sampled token rows (the oracle computes k and v for all
    tokens, the rest for those rows);
  * aliasing on vs off: byte-identical outputs, with the workspace filled
    with 0xFF (bf16/fp32 NaN) before each run so that a read of an unwritten
    or stale aliased byte would show;
  * the layer stack: a 50-block bf16 stack at reduced width against the
    oracle (the full-size 50-block step is in test_gpu_c3_step.py).
Tolerance for bf16 paths: relative L2 <= 2e-2 per output tensor.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import (config_for, dev, device_cus, expected_tail_splits, flush, has_gpu, sample_rows, to_np,
                      upload_block)
from helpers import record, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

TOL = 2e-2


@pytest.fixture(scope="module")
def R():
    from video_diffusion_transformer_adaln_amd import binding, runtime
    binding.lib()
    return runtime


def _run_block(R, shape, dw, xd, cd, alias=True, poison=True, stats=None, int8_fc2_rows=False, int8_mlp_group=0,
               rope=None):
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    cfg = config_for(shape, alias, int8_fc2_rows, int8_mlp_group, rope)
    ws = R.alloc_workspace(cfg)
    if poison:
        ws.fill_(0xFF)
    out = torch.empty_like(xd)
    B.h3k_dit_block_forward(cfg, B.make_weights(dw), xd, cd, out, ws, stats=stats)
    torch.cuda.synchronize()
    return out


def _want(shape, n_tokens, part_bytes, cus=None):
    """Kernels of a bf16 block of `shape` at n_tokens that split their last wave."""
    return expected_tail_splits(n_tokens, shape.hidden, shape.mlp_hidden, part_bytes,
                                device_cus() if cus is None else cus, shape.n_heads, shape.head_dim)


def _block_case(shape, bias_std=0.0):
    hx, hc = si.gen_activation(shape)
    hw = si.gen_block_weights(shape, 0, bias_std=bias_std)
    return hx, hc, hw


def test_block_c0_fp32_full(R):
    shape = si.C0
    flush(f"block {shape.name}")
    hx, hc, hw = _block_case(shape, bias_std=0.05)
    dw, ow = upload_block(shape, hw)
    from video_diffusion_transformer_adaln_amd import binding as B
    st = B.DitStats()
    out = _run_block(R, shape, dw, dev(hx), dev(hc), stats=st)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads)
    got = to_np(out)
    assert st.dispatches == 8 and st.tail_splits == 0
    assert record("block c0 fp32 (512x256)", rel_l2(got, ref), 1e-4) < 1e-4


@pytest.mark.parametrize("n", [1, 37, 300])
def test_block_ragged_bf16_full(R, n):
    shape = si.custom_shape(f"ragged{n}", 950 + n, n, 4, 128, 1024, "bf16")
    flush(f"block {shape.name}")
    hx, hc, hw = _block_case(shape, bias_std=0.05)
    dw, ow = upload_block(shape, hw)
    got = to_np(_run_block(R, shape, dw, dev(hx), dev(hc)))
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads)
    assert np.isfinite(got).all()
    assert record(f"block ragged N={n} bf16", rel_l2(got, ref), TOL) < TOL


def test_block_c1_full(R):
    """The 512x512x22-frame block, every element, with the split tails (on 256
    CUs the out-projection and MLP-down leave 32 tiles in their last wave and
    split them 8 ways along k; the attention then takes 576 eight-wave
    workgroups, 64 in the last round of 256, and splits those 4 ways along the
    keys) and
    without them (H3K_DISABLE_TAIL_SPLIT=1): both against the oracle, the split
    no further from it, and the two within the rounding of P (see below)."""
    _split_on_off(R, si.C1, "block c1 (6144x3072)", 3)


def test_block_ragged_tail_split(R):
    """The split tails with ragged edges: 6000 tokens (the last m-tile holds 112
    rows, the last 128-query workgroup 112 queries, the last key tile 16 keys)
    and D = 2944 (the last n-tile 128 columns); out and down leave 32 of 288
    tiles in the last wave and split them 8 ways, the attention 40 of its 552
    eight-wave workgroups 6 ways along the keys."""
    shape = si.custom_shape("ragged_split", 990, 6000, 23, 128, 11776, "bf16")
    _split_on_off(R, shape, "block ragged 6000x2944", 3)


@pytest.mark.parametrize("int8", [False, True])
def test_block_wide_tail_split_all_gemms(R, int8):
    """6144 tokens at D = 4096 (32 x 128 heads), F = 12288: the out-projection
    and MLP-down (384 tiles) and the MLP-up with its GELU epilogue (1152 tiles)
    each leave 128 tiles in their last wave on 256 CUs and split them 2 ways
    along k.  With int8 weights the same happens to the bf16 GEMMs on the
    staged (widened) weights, the channel scale in the split epilogue."""
    shape = si.custom_shape("wide_split" + ("_int8" if int8 else ""), 992 + int8, 6144, 32, 128, 12288, "bf16",
                            int8_weights=int8)
    _split_on_off(R, shape, f"block 6144x4096{' int8 weights' if int8 else ''}", 3)


def _split_on_off(R, shape, label, want_256):
    import os
    from video_diffusion_transformer_adaln_amd import binding as B
    flush(f"block {shape.name}")
    hx, hc, hw = _block_case(shape)
    dw, ow = upload_block(shape, hw)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads)
    cfg = config_for(shape)
    part = B.h3k_dit_plan(cfg).part_bytes
    outs = {}
    for split in (True, False):
        st = B.DitStats()
        if not split:
            os.environ["H3K_DISABLE_TAIL_SPLIT"] = "1"
        try:
            outs[split] = to_np(_run_block(R, shape, dw, dev(hx), dev(hc), stats=st))
        finally:
            os.environ.pop("H3K_DISABLE_TAIL_SPLIT", None)
        want = _want(shape, shape.n_tokens, part) if split else 0
        staged = 4 if shape.int8_weights else 0                # int8: the four weight-widening passes
        assert st.tail_splits == want and st.dispatches == 8 + staged + want
        err = rel_l2(outs[split], ref)
        flush(f"  split={split}: {st.tail_splits} kernels split, rel_l2 = {err:.3e}")
        record(f"{label}{'' if split else ', tail split off'}", err, TOL)
        assert err < TOL
    if device_cus() == 256:
        assert _want(shape, shape.n_tokens, part, 256) == want_256
    # The split moves the result no further from the oracle.  The two runs are
    # not bit-equal: the GEMM tails sum in another fp32 order, and each key
    # range of a split attention workgroup rounds its probabilities to bf16
    # against its own running reference, so the outputs carry independent bf16
    # roundings of P (about 3e-3 apart after a full block at 6144 tokens,
    # each 4.4e-3 from the oracle).
    errs = {k: rel_l2(v, ref) for k, v in outs.items()}
    assert errs[True] <= 1.05 * errs[False]
    assert rel_l2(outs[True], outs[False]) < 5e-3


@pytest.fixture(scope="module")
def c2_case():
    flush("generating the 864x480x56-frame block inputs")
    return _block_case(si.C2)


def test_block_c2_sampled_rows(R, c2_case):
    shape = si.C2
    flush(f"block {shape.name}")
    hx, hc, hw = c2_case
    dw, ow = upload_block(shape, hw)
    got = to_np(_run_block(R, shape, dw, dev(hx), dev(hc)))
    rows = sample_rows(shape.n_tokens)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads, rows=rows)
    assert np.isfinite(got).all()
    err = rel_l2(got[rows], ref)
    flush(f"  rel_l2 = {err:.3e}")
    record("block c2 (22680x5120) sampled rows", err, TOL)
    assert err < TOL


def test_alias_on_off_byte_identical_c2(R, c2_case):
    import torch
    shape = si.C2
    flush("alias on/off")
    hx, hc, hw = c2_case
    dw, _ = upload_block(shape, hw)
    xd, cd = dev(hx), dev(hc)
    on = _run_block(R, shape, dw, xd, cd, alias=True)
    off = _run_block(R, shape, dw, xd, cd, alias=False)
    again = _run_block(R, shape, dw, xd, cd, alias=True)
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))
    assert torch.equal(on.view(torch.int16), again.view(torch.int16))


def test_block_c4_int8_sampled_rows(R):
    shape = si.C4
    flush(f"block {shape.name}")
    hx, hc, hw = _block_case(shape)
    dw, ow = upload_block(shape, hw)
    # the GPU quantiser and the oracle's agree bit for bit
    for name in si.MATRIX_NAMES:
        q, s = ow[name]
        assert np.array_equal(dw[name].cpu().numpy(), q)
        assert np.array_equal(dw["s_" + name[2:]].cpu().numpy(), s)
    from video_diffusion_transformer_adaln_amd import binding as B
    st = B.DitStats()
    got_t = _run_block(R, shape, dw, dev(hx), dev(hc), stats=st)
    assert st.dispatches == 8 + 4 and st.tail_splits == 0   # four weight-widening passes; no tail split
    got = to_np(got_t)
    rows = sample_rows(shape.n_tokens)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads, rows=rows)
    err = rel_l2(got[rows], ref)
    flush(f"  rel_l2 = {err:.3e}")
    record("block c4 int8 weights (22680x5120) sampled rows", err, TOL)
    assert err < TOL
    # widening inside the GEMM instead of into the staging buffer: the same bits
    _assert_staging_identical(R, shape, dw, dev(hx), dev(hc), got_t)


def _assert_staging_identical(R, shape, dw, xd, cd, staged, **kw):
    """The int8 projections with their weights widened in the GEMM's ring
    (H3K_DISABLE_WEIGHT_STAGING=1) give the bytes of the staged path: the same
    bf16 operands (bf16(q), or bf16(q s) with group scales) in the same
    order, and the channel scale applied before the bias in both."""
    import os
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    os.environ["H3K_DISABLE_WEIGHT_STAGING"] = "1"
    try:
        st = B.DitStats()
        ring = _run_block(R, shape, dw, xd, cd, stats=st, **kw)
    finally:
        os.environ.pop("H3K_DISABLE_WEIGHT_STAGING", None)
    assert st.tail_splits == 0
    assert torch.equal(ring.view(torch.int16), staged.view(torch.int16))


@pytest.mark.parametrize("case", ["c4", "small"])
def test_block_int8_fc2_rows(R, case):
    """The row-quantised FC2 (u quantised per token row, int8 x int8 MLP-down):
    against the oracle's block with the same option, and byte-identical with
    aliasing on and off."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    shape = si.C4 if case == "c4" else si.custom_shape("int8fc2", 971, 333, 2, 128, 640, "bf16", int8_weights=True)
    flush(f"block {shape.name} int8_fc2_rows")
    hx, hc, hw = _block_case(shape, bias_std=0.05)
    dw, ow = upload_block(shape, hw)
    xd, cd = dev(hx), dev(hc)
    st = B.DitStats()
    got_t = _run_block(R, shape, dw, xd, cd, stats=st, int8_fc2_rows=True)
    assert st.dispatches == 9 + 3 and st.tail_splits == 0   # QKV, out and up widen their weights first
    _assert_staging_identical(R, shape, dw, xd, cd, got_t, int8_fc2_rows=True)
    got = to_np(got_t)
    rows = sample_rows(shape.n_tokens) if case == "c4" else np.arange(shape.n_tokens)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads, rows=rows, int8_fc2_rows=True)
    err = rel_l2(got[rows], ref)
    flush(f"  rel_l2 = {err:.3e}")
    record(f"block int8 FC2 rows ({case})", err, TOL)
    assert err < TOL
    if case == "small":
        off = _run_block(R, shape, dw, xd, cd, alias=False, int8_fc2_rows=True)
        assert torch.equal(off.view(torch.int16), got_t.view(torch.int16))


@pytest.mark.parametrize("case,group", [("c4", 128), ("small", 32), ("small", 64)])
def test_block_int8_mlp_groups(R, case, group):
    """The group-wise int8 MLP (w_up and w_down with one scale per group of
    input channels, dequantised to bf16 on the way to the matrix cores):
    against the oracle's block with the same grouped weights, and
    byte-identical with aliasing on and off."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    shape = si.C4 if case == "c4" else si.custom_shape("int8grp", 973, 333, 2, 128, 640, "bf16", int8_weights=True)
    flush(f"block {shape.name} int8_mlp_group={group}")
    hx, hc, hw = _block_case(shape, bias_std=0.05)
    dw, ow = upload_block(shape, hw, mlp_group=group)
    assert tuple(dw["s_up"].shape) == (shape.mlp_hidden, shape.hidden // group)
    xd, cd = dev(hx), dev(hc)
    st = B.DitStats()
    got_t = _run_block(R, shape, dw, xd, cd, stats=st, int8_mlp_group=group)
    assert st.dispatches == 8 + 4 and st.tail_splits == 0
    _assert_staging_identical(R, shape, dw, xd, cd, got_t, int8_mlp_group=group)
    got = to_np(got_t)
    rows = sample_rows(shape.n_tokens) if case == "c4" else np.arange(shape.n_tokens)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads, rows=rows)
    err = rel_l2(got[rows], ref)
    flush(f"  rel_l2 = {err:.3e}")
    record(f"block int8 MLP groups G={group} ({case})", err, TOL)
    assert err < TOL
    if case == "small":
        off = _run_block(R, shape, dw, xd, cd, alias=False, int8_mlp_group=group)
        assert torch.equal(off.view(torch.int16), got_t.view(torch.int16))


@pytest.mark.parametrize("case,grid,half", [("c2", (14, 30, 54), False), ("ragged", (3, 3, 37), False),
                                             ("ragged", (3, 3, 37), True), ("d64", (2, 8, 16), True),
                                             ("ragged_int8", (3, 3, 37), True)])
def test_block_rope(R, case, grid, half):
    """3D RoPE of q and k fused into the QKV projection's epilogue, against the
    oracle's block with the same grid; byte-identical with aliasing on and
    off.  c2: the 864x480x56-frame latent (14 frames, 30 rows, 54 columns).
    The QKV weights are scaled up so that the output depends on the
    positions: the block without RoPE must be far from the reference.
    ragged_int8: int8 projection weights, the QKV weights widened into the
    staging buffer before the rotary epilogue (the same bytes as widening in
    the GEMM)."""
    import torch
    if case == "c2":
        shape = si.C2
    elif case == "ragged":
        shape = si.custom_shape("rope", 974, 333, 2, 128, 640, "bf16")
    elif case == "ragged_int8":
        shape = si.custom_shape("rope8", 977, 333, 2, 128, 640, "bf16", int8_weights=True)
    else:
        shape = si.custom_shape("rope64", 975, 256, 4, 64, 512, "bf16")
    flush(f"block {shape.name} rope grid={grid} half={half}")
    hx, hc, hw = _block_case(shape, bias_std=0.05)
    # QKV weights scaled so that q and k have std ~1.4 (logits of std ~2) at every width, as the
    # N(0, 0.02^2) weights give at D = 5120: attention, and the block, then depend on the positions
    boost = max(1.0, 70.0 / np.sqrt(shape.hidden))
    hw["w_qkv"] = si._finish(np.ascontiguousarray(hw["w_qkv"].values * boost, dtype=np.float32),
                             "f32" if shape.int8_weights else shape.dtype)   # int8: fp32 before quantising
    dw, ow = upload_block(shape, hw)
    xd, cd = dev(hx), dev(hc)
    rope = (grid[0], grid[1], grid[2], half)
    got_t = _run_block(R, shape, dw, xd, cd, rope=rope)
    got = to_np(got_t)
    rows = sample_rows(shape.n_tokens) if case == "c2" else np.arange(shape.n_tokens)
    ref = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads, rows=rows, rope=rope)
    err = rel_l2(got[rows], ref)
    flush(f"  rel_l2 = {err:.3e}")
    record(f"block RoPE {case} grid={grid} half={half}", err, TOL)
    assert err < TOL
    if case == "ragged_int8":
        _assert_staging_identical(R, shape, dw, xd, cd, got_t, rope=rope)
    plain = oracle.block_forward(hx.values, hc.values, ow, shape.n_heads, rows=rows)
    flush(f"  rel_l2 to the block without RoPE = {rel_l2(got[rows], plain):.3e}")
    assert rel_l2(got[rows], plain) > 5 * err          # the positions are in the output
    if case != "c2":
        off = _run_block(R, shape, dw, xd, cd, alias=False, rope=rope)
        assert torch.equal(off.view(torch.int16), got_t.view(torch.int16))


def test_stack50_reduced_width_vs_oracle(R):
    """50 blocks (bf16 residual stream between blocks) at N=512, D=512."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    shape = si.custom_shape("stack50", 960, 512, 4, 128, 2048, "bf16", n_blocks=50)
    flush("stack of 50 reduced-width blocks")
    hx, hc = si.gen_activation(shape)
    blocks_h = [si.gen_block_weights(shape, l) for l in range(50)]
    up = [upload_block(shape, hw) for hw in blocks_h]
    stack = R.DitStack(config_for(shape), [u[0] for u in up])
    stack.workspace.fill_(0xFF)
    xd, cd = dev(hx), dev(hc)
    out = torch.empty_like(xd)
    st = B.DitStats()
    stack.forward(xd, cd, out, stats=st)
    torch.cuda.synchronize()
    part = B.h3k_dit_plan(config_for(shape)).part_bytes
    assert st.tail_splits == 50 * _want(shape, shape.n_tokens, part)
    assert st.dispatches == 8 * 50 + st.tail_splits
    ref = oracle.stack_forward(hx.values, hc.values, [u[1] for u in up], shape.n_heads)
    err = rel_l2(to_np(out), ref)
    flush(f"  rel_l2 after 50 blocks = {err:.3e}")
    record("stack 50 blocks reduced width (512x512)", err, TOL)
    assert err < TOL
    # L = 1 is the block call
    one = torch.empty_like(xd)
    stack.forward(xd, cd, one, n_layers=1)
    single = _run_block(R, shape, up[0][0], xd, cd)
    assert torch.equal(one.view(torch.int16), single.view(torch.int16))


@pytest.mark.parametrize("n_blocks,rng_", [(6, (2, 5)), (4, (0, 4)), (3, (0, 1)), (5, (4, 5))])
def test_stack_token_reduction(R, n_blocks, rng_):
    """Token reduction over a layer range against the oracle's stack with the
    same range: merge before the first reduced block, the range on N/2
    tokens, restore after it.  Aliasing on and off give the same bytes, and
    the stack makes two dispatches more than without the range."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    shape = si.custom_shape("tokred", 976, 334, 2, 128, 640, "bf16", n_blocks=n_blocks)
    flush(f"stack of {n_blocks} with token reduction {rng_}")
    hx, hc = si.gen_activation(shape)
    blocks_h = [si.gen_block_weights(shape, l, bias_std=0.05) for l in range(n_blocks)]
    up = [upload_block(shape, hw) for hw in blocks_h]
    xd, cd = dev(hx), dev(hc)
    outs = []
    for alias in (True, False):
        cfg = config_for(shape, alias)
        cfg.token_reduction_first, cfg.token_reduction_last = rng_
        stack = R.DitStack(cfg, [u[0] for u in up])
        stack.workspace.fill_(0xFF)
        out = torch.full_like(xd, float("nan"))
        st = B.DitStats()
        stack.forward(xd, cd, out, stats=st)
        torch.cuda.synchronize()
        part = B.h3k_dit_plan(cfg).part_bytes
        n_red = rng_[1] - rng_[0]
        want = ((n_blocks - n_red) * _want(shape, shape.n_tokens, part)
                + n_red * _want(shape, shape.n_tokens // 2, part))
        assert st.tail_splits == want
        assert st.dispatches == 8 * n_blocks + 2 + st.tail_splits
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got = to_np(outs[0])
    ref = oracle.stack_forward(hx.values, hc.values, [u[1] for u in up], shape.n_heads, token_reduction=rng_)
    err = rel_l2(got, ref)
    plain = oracle.stack_forward(hx.values, hc.values, [u[1] for u in up], shape.n_heads)
    flush(f"  rel_l2 = {err:.3e}; to the stack without reduction {rel_l2(got, plain):.3e}")
    record(f"stack {n_blocks} token reduction {rng_}", err, TOL)
    assert err < TOL
    assert rel_l2(got, plain) > 3 * err                   # the reduction is visible in the output


def test_stack_token_reduction_split_attention(R):
    """Token reduction where the attention splits its last round along the keys
    in the full blocks (8192 tokens: 64 eight-wave workgroups on 256 CUs) and
    in the reduced ones (4096 tokens: 32 workgroups), both using the one
    scratch region of the full plan: against the oracle's stack with the same
    range, and byte-identical with aliasing on and off."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    shape = si.custom_shape("tokred_split", 978, 8192, 2, 128, 1024, "bf16", n_blocks=4)
    rng_ = (1, 3)
    flush(f"stack of 4 at 8192 tokens with token reduction {rng_}")
    hx, hc = si.gen_activation(shape)
    blocks_h = [si.gen_block_weights(shape, l, bias_std=0.05) for l in range(4)]
    up = [upload_block(shape, hw) for hw in blocks_h]
    xd, cd = dev(hx), dev(hc)
    outs = []
    for alias in (True, False):
        cfg = config_for(shape, alias)
        cfg.token_reduction_first, cfg.token_reduction_last = rng_
        stack = R.DitStack(cfg, [u[0] for u in up])
        stack.workspace.fill_(0xFF)
        out = torch.full_like(xd, float("nan"))
        st = B.DitStats()
        stack.forward(xd, cd, out, stats=st)
        torch.cuda.synchronize()
        part = B.h3k_dit_plan(cfg).part_bytes
        want = 2 * _want(shape, shape.n_tokens, part) + 2 * _want(shape, shape.n_tokens // 2, part)
        assert st.tail_splits == want and st.dispatches == 8 * 4 + 2 + want
        if device_cus() == 256:
            assert want == 4                                   # the attention of every block
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    got = to_np(outs[0])
    ref = oracle.stack_forward(hx.values, hc.values, [u[1] for u in up], shape.n_heads, token_reduction=rng_)
    err = rel_l2(got, ref)
    flush(f"  rel_l2 = {err:.3e}")
    record("stack 4 at 8192 tokens, token reduction (1, 3), split attention", err, TOL)
    assert err < TOL


def test_stack50_reduced_width_token_reduction(R):
    """50 reduced-width blocks with the middle half (blocks 12..37) on merged tokens."""
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    shape = si.custom_shape("stack50", 960, 512, 4, 128, 2048, "bf16", n_blocks=50)
    flush("stack of 50 reduced-width blocks, token reduction 12..37")
    hx, hc = si.gen_activation(shape)
    blocks_h = [si.gen_block_weights(shape, l) for l in range(50)]
    up = [upload_block(shape, hw) for hw in blocks_h]
    cfg = config_for(shape)
    cfg.token_reduction_first, cfg.token_reduction_last = 12, 38
    stack = R.DitStack(cfg, [u[0] for u in up])
    stack.workspace.fill_(0xFF)
    xd, cd = dev(hx), dev(hc)
    out = torch.empty_like(xd)
    st = B.DitStats()
    stack.forward(xd, cd, out, stats=st)
    torch.cuda.synchronize()
    part = B.h3k_dit_plan(cfg).part_bytes
    want = (24 * _want(shape, shape.n_tokens, part)
            + 26 * _want(shape, shape.n_tokens // 2, part))
    assert st.tail_splits == want
    assert st.dispatches == 8 * 50 + 2 + st.tail_splits
    ref = oracle.stack_forward(hx.values, hc.values, [u[1] for u in up], shape.n_heads, token_reduction=(12, 38))
    err = rel_l2(to_np(out), ref)
    flush(f"  rel_l2 after 50 blocks = {err:.3e}")
    record("stack 50 blocks reduced width, token reduction 12..37", err, TOL)
    assert err < TOL
