"""Kernel-level parity of the HIP path against the CPU oracle's stages.

Each kernel is called through the C ABI on seeded inputs and compared with
the oracle function of the same stage: element-wise at small, ragged sizes
(several tiles plus a tail), and on sampled rows at the full 864x480x56-frame
shapes in the launch configuration the block uses.

Tolerances (relative L2 per output tensor): the bf16 kernels read
bf16-exact inputs, accumulate in fp32 and round once at the store, which
alone gives an rms relative error of about 2^-9/sqrt(3) ~ 1.1e-3; attention
adds one bf16 rounding of the probabilities.  The bound used is 1e-2 (the
block-level bound is 2e-2).  fp32 kernels differ from the oracle only in
summation order: 1e-5.  The int8 quantiser must be bit-exact.
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import dev, flush, has_gpu, sample_rows, to_np
from helpers import record, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

BF16_TOL = 1e-2
F32_TOL = 1e-5


@pytest.fixture(scope="module")
def B():
    from video_diffusion_transformer_adaln_amd import binding
    binding.lib()
    return binding


def _f32(shape, std, cid, tensor="x", block=0):
    return si.normal_f32(shape, std, 42, cid, block, tensor)


def _ht(a, dtype):
    return si._finish(np.ascontiguousarray(a, dtype=np.float32), dtype)


# ------------------------------------------------------------------ device query

def test_device_info_matches_runtime(B):
    import torch
    d = B.h3k_get_device_info(0)
    p = torch.cuda.get_device_properties(0)
    flush(f"device info {d}")
    assert d["compute_units"] == p.multi_processor_count
    assert d["arch"].split(":")[0] == p.gcnArchName.split(":")[0]
    assert d["wavefront_size"] == 64
    assert d["hbm_bytes"] == p.total_memory
    assert 1_000_000 <= d["peak_clock_khz"] <= 4_000_000
    assert d["lds_bytes_per_cu"] >= 160 * 1024   # the GEMM's operand ring uses all of it


# ------------------------------------------------------------------ AdaLN GEMV

@pytest.mark.parametrize("rows,cols,dtype", [(6 * 5120, 5120, "bf16"), (6 * 256, 256, "f32"), (72, 24, "bf16"), (30, 40, "bf16"), (42, 16, "f32"),
                                             (6 * 3072, 3072, "bf16")])
def test_adaln_gemv(B, rows, cols, dtype):
    import torch
    flush(f"adaln gemv rows={rows} cols={cols} {dtype}")
    w = _ht(_f32((rows, cols), 0.02, 800, "w_ada"), dtype)
    b = _ht(_f32((rows,), 0.1, 800, "b_ada"), dtype)
    c = _ht(_f32((cols,), 1.0, 800, "c"), dtype)
    mod = torch.empty(rows, dtype=torch.float32, device="cuda")
    code = B.H3K_F32 if dtype == "f32" else B.H3K_BF16
    B.h3k_adaln_modulation(code, rows, cols, dev(w), dev(b), dev(c), mod)
    torch.cuda.synchronize()
    ref = np.concatenate(list(oracle.adaln_modulation(w.values, b.values, c.values).values()))
    assert rel_l2(to_np(mod), ref) < 1e-5


# ------------------------------------------------------------------ LayerNorm + modulation

@pytest.mark.parametrize("n,D,dtype,full", [(22680, 5120, "bf16", False), (512, 256, "f32", True),
                                             (37, 320, "bf16", True), (1, 64, "bf16", True),
                                             (6144, 3072, "bf16", False), (100, 8192, "bf16", True),
                                             (3, 8192, "f32", True)])
def test_ln_modulate(B, n, D, dtype, full):
    import torch
    flush(f"ln_modulate n={n} D={D} {dtype}")
    x = _ht(_f32((n, D), 1.0, 801) * 3 + 0.5, dtype)
    shift = _f32((D,), 0.5, 801, "b_ada")
    scale = _f32((D,), 0.5, 801, "b_qkv")
    xd = dev(x)
    out = torch.empty_like(xd)
    code = B.H3K_F32 if dtype == "f32" else B.H3K_BF16
    B.h3k_ln_modulate(code, n, D, 1e-6, xd, D, torch.from_numpy(shift).cuda(), torch.from_numpy(scale).cuda(),
                      out, D)
    torch.cuda.synchronize()
    rows = np.arange(n) if full else sample_rows(n)
    ref = oracle.modulate(oracle.layer_norm(x.values[rows]), shift, scale)
    got = to_np(out)[rows]
    assert rel_l2(got, ref) < (F32_TOL if dtype == "f32" else BF16_TOL / 2)


# ------------------------------------------------------------------ GEMMs

def _linear_ref(x, w, b, epi, residual=None, gate=None):
    z = oracle.linear(x, w, b)
    if epi == 1:
        return oracle.gelu_tanh(z)
    if epi == 2:
        return residual + gate * z
    return z


GEMM_CASES = [
    # m, n, k, epilogue, dtype, int8, split, full
    (300, 320, 128, 0, "bf16", False, None, True),
    (300, 320, 128, 1, "bf16", False, None, True),
    (300, 320, 128, 2, "bf16", False, None, True),
    (1, 64, 64, 0, "bf16", False, None, True),
    (513, 768, 256, 0, "bf16", False, 512, True),     # Q|K row-major, V transposed (straddling tile)
    (300, 1536, 256, 0, "bf16", False, 1024, True),   # split on a tile boundary
    (257, 328, 192, 2, "bf16", False, None, True),    # 3 k-tiles, ragged n
    (129, 264, 320, 1, "bf16", False, None, True),    # 5 k-tiles: the operand ring wraps
    (700, 520, 704, 0, "bf16", False, 264, True),     # 11 k-tiles, straddling transposed split
    (4200, 4096, 128, 2, "bf16", False, None, True),  # 272 tiles: a second, partial round of workgroups
    (4200, 4352, 192, 0, "bf16", False, 2824, True),  # 289 tiles, straddling split, a second round
    (300, 320, 128, 0, "bf16", True, None, True),
    (300, 576, 192, 2, "bf16", True, None, True),
    (97, 1024, 256, 0, "bf16", True, 512, True),
    (1, 64, 64, 0, "bf16", True, None, True),         # int8 weights, one k-tile
    (257, 328, 320, 2, "bf16", True, None, True),     # int8 weights, 5 k-tiles (the ring wraps), ragged m and n
    (700, 520, 704, 0, "bf16", True, 264, True),      # int8 weights, 11 k-tiles, straddling transposed split
    (512, 768, 256, 0, "f32", False, 512, True),
    (512, 1024, 256, 1, "f32", False, None, True),
    (512, 256, 1024, 2, "f32", False, None, True),
    (22680, 15360, 5120, 0, "bf16", False, 10240, False),   # QKV projection
    (22680, 5120, 5120, 2, "bf16", False, None, False),     # out projection
    (22680, 13824, 5120, 1, "bf16", False, None, False),    # MLP up
    (22680, 5120, 13824, 2, "bf16", False, None, False),    # MLP down
    (22680, 13824, 5120, 1, "bf16", True, None, False),     # MLP up, int8 weights
    (22680, 15360, 5120, 0, "bf16", True, 10240, False),    # QKV, int8 weights
    (2835, 15360, 5120, 0, "bf16", False, 10240, False),    # QKV on one GPU's 1/8 share of the tokens
    (2835, 5120, 13824, 2, "bf16", False, None, False),     # MLP down on the same share
]


@pytest.mark.parametrize("m,n,k,epi,dtype,int8,split,full", GEMM_CASES)
def test_linear(B, m, n, k, epi, dtype, int8, split, full):
    import torch
    flush(f"linear m={m} n={n} k={k} epi={epi} {dtype} int8={int8} split={split}")
    cid = 810 + epi
    x = _ht(_f32((m, k), 1.0, cid), dtype)
    w32 = _f32((n, k), 0.02, cid, "w_up")
    bias = _ht(_f32((n,), 0.05, cid, "b_up"), dtype)
    split = n if split is None else split
    code = B.H3K_F32 if dtype == "f32" else B.H3K_BF16
    if int8:
        q_ref, s_ref = oracle.quantize_int8(w32)
        from video_diffusion_transformer_adaln_amd import runtime as R
        q, s = R.quantize_int8(torch.from_numpy(w32).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q_ref) and np.array_equal(s.cpu().numpy(), s_ref)
        wd, wcode, w_ref = q, B.H3K_INT8, oracle.dequantize_int8(q_ref, s_ref)
        sd = s
    else:
        wt = _ht(w32, dtype)
        wd, wcode, w_ref, sd = dev(wt), code, wt.values, None
    res = gate = None
    resd = gated = None
    if epi == 2:
        res = _ht(_f32((m, split), 1.0, cid, "x", 1), dtype)
        gate = _f32((split,), 0.5, cid, "b_down")
        resd, gated = dev(res), torch.from_numpy(gate).cuda()
    xd = dev(x)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    y = torch.full((m, split), float("nan"), dtype=tdt, device="cuda")
    ldyt = ((m + 7) // 8) * 8
    yt = torch.full((n - split, ldyt), float("nan"), dtype=tdt, device="cuda") if split < n else None
    B.h3k_linear(code, wcode, m, n, k, xd, k, wd, k, sd, dev(bias), epi, resd, split, gated, y, split,
                 yt, ldyt if yt is not None else 0, split)
    torch.cuda.synchronize()
    rows = np.arange(m) if full else sample_rows(m)
    if epi == 2:
        ref = _linear_ref(x.values[rows], w_ref, bias.values, 2, res.values[rows], gate)
    else:
        ref = _linear_ref(x.values[rows], w_ref, bias.values, epi)
    got = to_np(y)[rows]
    tol = F32_TOL if dtype == "f32" else BF16_TOL / 2
    assert np.isfinite(got).all()
    case = f"linear {m}x{n}x{k} epi={epi} {dtype}{' int8' if int8 else ''}"
    if not full:
        record(case, rel_l2(got, ref[:, :split] if split < n else ref), tol)
    assert rel_l2(got, ref[:, :split] if split < n else ref) < tol
    if split < n:
        got_t = to_np(yt)[:, :m].T[rows]
        assert np.isfinite(got_t).all()
        if not full:
            record(case + " (transposed part)", rel_l2(got_t, ref[:, split:]), tol)
        assert rel_l2(got_t, ref[:, split:]) < tol
        assert np.isnan(to_np(yt)[:, m:]).all()                # padding columns untouched


NO_BIAS_CASES = [
    # m, n, k, epilogue, weights, split
    (300, 320, 128, 0, "bf16", None),
    (513, 768, 256, 0, "bf16", 512),     # transposed part, straddling tile
    (300, 1536, 256, 0, "bf16", 1024),   # transposed part on a tile boundary
    (257, 328, 192, 2, "bf16", None),
    (300, 576, 192, 2, "int8", None),
    (97, 1024, 256, 0, "int8", 512),
    (129, 264, 256, 1, "int8x8", None),
    (257, 328, 384, 2, "int8x8", None),
]


@pytest.mark.parametrize("m,n,k,epi,weights,split", NO_BIAS_CASES)
def test_linear_without_bias(B, m, n, k, epi, weights, split):
    """A null bias (the epilogue adds -0, which leaves every value as it is)
    on the bf16, int8-weight and int8 x int8 paths, row-major and transposed
    parts, against the oracle's linear without a bias."""
    import torch
    from video_diffusion_transformer_adaln_amd import runtime as R
    flush(f"linear without bias m={m} n={n} k={k} epi={epi} {weights} split={split}")
    cid = 870 + epi
    x32 = _f32((m, k), 1.0, cid)
    w32 = _f32((n, k), 0.02, cid, "w_up")
    split = n if split is None else split
    res = gate = resd = gated = None
    if epi == 2:
        res = _ht(_f32((m, split), 1.0, cid, "x", 1), "bf16")
        gate = _f32((split,), 0.5, cid, "b_down")
        resd, gated = dev(res), torch.from_numpy(gate).cuda()
    y = torch.full((m, split), float("nan"), dtype=torch.bfloat16, device="cuda")
    ldyt = ((m + 7) // 8) * 8
    yt = torch.full((n - split, ldyt), float("nan"), dtype=torch.bfloat16, device="cuda") if split < n else None
    if weights == "int8x8":
        xq, xs = R.quantize_int8(torch.from_numpy(x32).cuda())
        wq, ws = R.quantize_int8(torch.from_numpy(w32).cuda())
        B.h3k_linear_int8(m, n, k, xq, k, xs, wq, k, ws, None, epi, resd, split, gated, y, split)
        torch.cuda.synchronize()
        qx, sx = oracle.quantize_int8(x32)
        qw, sw = oracle.quantize_int8(w32)
        z = oracle.linear_w8a8(qx, sx, qw, sw, None)
    else:
        x = _ht(x32, "bf16")
        if weights == "int8":
            wd, sd = R.quantize_int8(torch.from_numpy(w32).cuda())
            qw, sw = oracle.quantize_int8(w32)
            w_ref, wcode = oracle.dequantize_int8(qw, sw), B.H3K_INT8
        else:
            wt = _ht(w32, "bf16")
            wd, sd, w_ref, wcode = dev(wt), None, wt.values, B.H3K_BF16
        B.h3k_linear(B.H3K_BF16, wcode, m, n, k, dev(x), k, wd, k, sd, None, epi, resd, split, gated, y, split,
                     yt, ldyt if yt is not None else 0, split)
        torch.cuda.synchronize()
        z = oracle.linear(x.values, w_ref, None)
    if epi == 1:
        ref = oracle.gelu_tanh(z)
    elif epi == 2:
        ref = res.values + gate * z[:, :split]
    else:
        ref = z
    got = to_np(y)
    assert np.isfinite(got).all()
    assert rel_l2(got, ref[:, :split]) < BF16_TOL / 2
    if split < n:
        got_t = to_np(yt)[:, :m].T
        assert rel_l2(got_t, z[:, split:]) < BF16_TOL / 2
        assert np.isnan(to_np(yt)[:, m:]).all()


# ------------------------------------------------------------------ int8 x int8 linear

LINEAR_INT8_CASES = [
    # m, n, k, epilogue, full
    (300, 320, 256, 0, True),
    (300, 320, 256, 1, True),
    (300, 320, 256, 2, True),
    (1, 64, 128, 0, True),
    (257, 328, 384, 2, True),      # 3 k-tiles, ragged n
    (129, 264, 640, 1, True),      # 5 k-tiles: the operand ring wraps
    (22680, 5120, 13824, 2, False),   # the MLP-down projection of the 864x480x56-frame block
]


@pytest.mark.parametrize("m,n,k,epi,full", LINEAR_INT8_CASES)
def test_linear_int8(B, m, n, k, epi, full):
    """Both operands quantised on the GPU (checked bit for bit against the
    oracle's quantiser), then the int8 x int8 product against the oracle's
    linear_w8a8 with the same epilogue."""
    import torch
    from video_diffusion_transformer_adaln_amd import runtime as R
    flush(f"linear int8 m={m} n={n} k={k} epi={epi}")
    cid = 840 + epi
    x32 = _f32((m, k), 1.0, cid)
    w32 = _f32((n, k), 0.02, cid, "w_up")
    bias = _ht(_f32((n,), 0.05, cid, "b_up"), "bf16")
    xq, xs = R.quantize_int8(torch.from_numpy(x32).cuda())
    wq, ws = R.quantize_int8(torch.from_numpy(w32).cuda())
    torch.cuda.synchronize()
    rows = np.arange(m) if full else sample_rows(m)
    qx_ref, sx_ref = oracle.quantize_int8(x32[rows])
    qw_ref, sw_ref = oracle.quantize_int8(w32)
    assert np.array_equal(xq.cpu().numpy()[rows], qx_ref) and np.array_equal(xs.cpu().numpy()[rows], sx_ref)
    assert np.array_equal(wq.cpu().numpy(), qw_ref) and np.array_equal(ws.cpu().numpy(), sw_ref)
    res = gate = resd = gated = None
    if epi == 2:
        res = _ht(_f32((m, n), 1.0, cid, "x", 1), "bf16")
        gate = _f32((n,), 0.5, cid, "b_down")
        resd, gated = dev(res), torch.from_numpy(gate).cuda()
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.h3k_linear_int8(m, n, k, xq, k, xs, wq, k, ws, dev(bias), epi, resd, n, gated, y, n)
    torch.cuda.synchronize()
    z = oracle.linear_w8a8(qx_ref, sx_ref, qw_ref, sw_ref, bias.values)
    if epi == 1:
        ref = oracle.gelu_tanh(z)
    elif epi == 2:
        ref = res.values[rows] + gate * z
    else:
        ref = z
    got = to_np(y)[rows]
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) < BF16_TOL / 2


LINEAR_GROUP_CASES = [
    # m, n, k, group, epilogue, full
    (300, 320, 256, 64, 0, True),
    (300, 320, 256, 32, 1, True),
    (257, 328, 384, 128, 2, True),     # 6 k-tiles, ragged m and n
    (1, 64, 128, 128, 0, True),
    (129, 264, 640, 64, 1, True),
    (22680, 13824, 5120, 128, 1, False),   # the MLP-up projection of the 864x480x56-frame block
    (22680, 5120, 13824, 128, 2, False),   # and its MLP-down
]


@pytest.mark.parametrize("m,n,k,group,epi,full", LINEAR_GROUP_CASES)
def test_linear_int8_groups(B, m, n, k, group, epi, full):
    """Weights quantised on the GPU in groups (checked bit for bit against the
    oracle's group quantiser), bf16 activations, against the oracle's product
    with the dequantised weights and the same epilogue."""
    import torch
    from video_diffusion_transformer_adaln_amd import runtime as R
    flush(f"linear int8 groups m={m} n={n} k={k} group={group} epi={epi}")
    cid = 850 + epi
    x = _ht(_f32((m, k), 1.0, cid), "bf16")
    w32 = _f32((n, k), 0.02, cid, "w_up")
    w32[3, :group] = 0.0                               # a zero group
    bias = _ht(_f32((n,), 0.05, cid, "b_up"), "bf16")
    wq, ws = R.quantize_int8_groups(torch.from_numpy(w32).cuda(), group)
    torch.cuda.synchronize()
    qw_ref, sw_ref = oracle.quantize_int8_groups(w32, group)
    assert np.array_equal(wq.cpu().numpy(), qw_ref) and np.array_equal(ws.cpu().numpy(), sw_ref)
    res = gate = resd = gated = None
    if epi == 2:
        res = _ht(_f32((m, n), 1.0, cid, "x", 1), "bf16")
        gate = _f32((n,), 0.5, cid, "b_down")
        resd, gated = dev(res), torch.from_numpy(gate).cuda()
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.h3k_linear_int8_groups(m, n, k, group, dev(x), k, wq, k, ws, dev(bias), epi, resd, n, gated, y, n)
    torch.cuda.synchronize()
    rows = np.arange(m) if full else sample_rows(m)
    z = oracle.linear(x.values[rows], oracle.dequantize_int8(qw_ref, sw_ref), bias.values)
    if epi == 1:
        ref = oracle.gelu_tanh(z)
    elif epi == 2:
        ref = res.values[rows] + gate * z
    else:
        ref = z
    got = to_np(y)[rows]
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) < BF16_TOL / 2


# ------------------------------------------------------------------ token reduction

@pytest.mark.parametrize("n,D,dtype", [(22680, 5120, "bf16"), (334, 256, "bf16"), (2, 8, "f32"), (1000, 64, "f32")])
def test_token_merge_unmerge(B, n, D, dtype):
    """merge: bit-exact (the fp32 mean of two bf16 or fp32 values, rounded
    once); unmerge of the unchanged merge: the entry back bit for bit, also
    in place; unmerge after a change: the oracle's restore."""
    import torch
    flush(f"token merge/unmerge n={n} D={D} {dtype}")
    code = B.H3K_F32 if dtype == "f32" else B.H3K_BF16
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    e = _ht(_f32((n, D), 1.0, 870, "x"), dtype)
    ed = dev(e)
    xm = torch.full((n // 2, D), float("nan"), dtype=tdt, device="cuda")
    B.h3k_token_merge(code, n, D, ed, D, xm, D)
    torch.cuda.synchronize()
    ref_m = si._finish(oracle.token_merge(e.values), dtype).values       # exact fp32 mean, rounded like the store
    assert np.array_equal(to_np(xm), ref_m)
    out = torch.full_like(ed, float("nan"))
    B.h3k_token_unmerge(code, n, D, ed, D, xm, D, out, D)
    torch.cuda.synchronize()
    assert torch.equal(out, ed)
    delta = _ht(_f32((n // 2, D), 0.3, 871, "c"), dtype)
    xm2 = (xm.float() + dev(delta).float()).to(tdt)
    inplace = ed.clone()
    B.h3k_token_unmerge(code, n, D, inplace, D, xm2, D, inplace, D)
    torch.cuda.synchronize()
    ref = oracle.token_unmerge(e.values, to_np(xm2))
    assert rel_l2(to_np(inplace), ref) < (F32_TOL if dtype == "f32" else BF16_TOL / 2)


# ------------------------------------------------------------------ 3D RoPE

@pytest.mark.parametrize("grid,heads,hd,half", [((2, 3, 4), 2, 128, False), ((3, 3, 37), 4, 64, True),
                                                ((1, 1, 1), 2, 64, False), ((14, 30, 54), 2, 128, False),
                                                ((14, 30, 54), 2, 128, True), ((5, 7, 9), 3, 128, True),
                                                ((64, 127, 129), 1, 16, False)])
def test_rope_3d(B, grid, heads, hd, half):
    """In-place rotation of a [tokens, heads * d] bf16 matrix (with a wider
    row pitch) against the oracle's float64 rope_3d of the same bf16 values."""
    import torch
    n = grid[0] * grid[1] * grid[2]
    cols = heads * hd
    flush(f"rope n={n} grid={grid} heads={heads} d={hd} half={half}")
    x = _ht(_f32((n, cols), 1.0, 860, "x"), "bf16")
    ld = cols + 8
    xd = torch.full((n, ld), 7.0, dtype=torch.bfloat16, device="cuda")
    xd[:, :cols] = dev(x)
    B.h3k_rope_3d(n, cols, hd, grid[0], grid[1], grid[2], half, xd, ld)
    torch.cuda.synchronize()
    got = to_np(xd)
    assert (got[:, cols:] == 7.0).all()                 # the pitch padding is untouched
    ref = oracle.rope_3d(x.values, heads, grid, half)
    assert rel_l2(got[:, :cols], ref) < 4e-3           # one bf16 rounding of the result
    # every token at its own grid position: a wrong coordinate turns a pair by
    # a wrong angle, far beyond one bf16 rounding (|values| < 8 here)
    assert np.max(np.abs(got[:, :cols].astype(np.float64) - ref)) < 0.05
    assert np.array_equal(got[0, :cols], x.values[0])   # token (0, 0, 0) is not rotated


# ------------------------------------------------------------------ attention

ATTN_CASES = [
    # n, heads, head_dim, dtype, full
    (1, 2, 128, "bf16", True),
    (37, 2, 128, "bf16", True),
    (300, 3, 64, "bf16", True),
    (1000, 2, 128, "bf16", True),
    (513, 4, 64, "f32", True),
    (512, 4, 64, "f32", True),
    (100, 2, 128, "f32", True),
    (6144, 24, 128, "bf16", False),
    (22680, 40, 128, "bf16", False),
    (9000, 40, 64, "bf16", False),
    (22680, 5, 128, "bf16", False),    # one GPU's 5 of 40 heads over all tokens
]


def _prescaled_q(q32, hd):
    """q in the kernel's prescaled form, bf16(q * log2(e) / sqrt(d)) (one rounding, as the
    block's QKV epilogue writes it), and the fp32 q the oracle's softmax(q k^T / sqrt(d))
    then sees: the stored value times sqrt(d) / log2(e), i.e. times sqrt(d) ln 2."""
    c = np.float32(1.4426950408889634 / np.sqrt(hd))
    qp = _ht((q32 * c).astype(np.float32), "bf16")
    q_oracle = (qp.values.astype(np.float64) * np.sqrt(hd) * np.log(2.0)).astype(np.float32)
    return qp, q_oracle


# prescaled q is a bf16 layout: fp32 cases run with unscaled q only
ATTN_RUNS = [(*c, pre) for c in ATTN_CASES for pre in (False, True) if not (pre and c[3] != "bf16")]


@pytest.mark.parametrize("n,heads,hd,dtype,full,pre", ATTN_RUNS)
def test_attention(B, n, heads, hd, dtype, full, pre):
    import torch
    flush(f"attention n={n} heads={heads} d={hd} {dtype} prescaled={pre}")
    D = heads * hd
    # q and k entries ~ N(0, 3^2), so q.k / sqrt(d) has std 3^2 = 9: softmax rows as peaked as the
    # block's (its logits have std about 10); test_attention_moving_reference moves the reference
    # after the first tile
    q32 = _f32((n, D), 1.0, 820, "x") * 3.0
    q = _ht(q32, dtype)
    q_in, q_ref = (q, q.values) if not pre else _prescaled_q(q32, hd)
    k = _ht(_f32((n, D), 1.0, 820, "c") * 3.0, dtype)
    v = _ht(_f32((n, D), 1.0, 820, "w_qkv"), dtype)
    ldvt = ((n + 7) // 8) * 8
    vt = np.zeros((D, ldvt), dtype=np.float32)
    vt[:, :n] = v.values.T
    code = B.H3K_F32 if dtype == "f32" else B.H3K_BF16
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    vtd = torch.from_numpy(vt).to(tdt).cuda()
    if ldvt > n:
        vtd[:, n:] = float("nan")        # padding must never reach the output
    o = torch.full((n, D), float("nan"), dtype=tdt, device="cuda")
    B.h3k_attention(code, n, heads, hd, dev(q_in), D, dev(k), D, vtd, ldvt, o, D, q_prescaled=pre)
    torch.cuda.synchronize()
    rows = np.arange(n) if full else sample_rows(n)
    ref = oracle.attention(q_ref[rows], k.values, v.values, heads)
    got = to_np(o)[rows]
    assert np.isfinite(got).all()
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    if not full:
        record(f"attention N={n} {heads}x{hd} {dtype}{' prescaled q' if pre else ''} (logit std 9)",
               rel_l2(got, ref), tol)
    assert rel_l2(got, ref) < tol


@pytest.mark.parametrize("pre", [False, True])
@pytest.mark.parametrize("n,hd,kind", [(700, 128, "ramp"), (2000, 128, "ramp"), (700, 64, "ramp"), (333, 128, "huge"),
                                        (100, 64, "huge")])
def test_attention_moving_reference(B, n, hd, kind, pre):
    """The kernel's softmax reference moves only when a tile's probabilities
    would exceed a bound; these inputs make it move after the first tile.
    ramp: key rows scaled by 1 + 60 j / n, so later keys score ever higher
    (the logits' std grows from about 0.5 to about 30 in log2 units: for
    nearly every query a later tile's probabilities pass the kernel's bound
    of 2^48 against the first tile's reference, once, checked on the CPU);
    huge: queries scaled by 300 (logits of std ~100 in log2 units), where
    exponentials taken without moving the reference would overflow."""
    import torch
    flush(f"attention moving reference n={n} d={hd} {kind} prescaled={pre}")
    heads = 2
    D = heads * hd
    q = _f32((n, D), 1.0, 821, "x") * 0.6
    k = _f32((n, D), 1.0, 821, "c") * 0.6
    if kind == "ramp":
        k = k * (1.0 + 60.0 * np.arange(n, dtype=np.float32)[:, None] / n)
    else:
        q = q * 300.0
    q_in, q_ref = (_ht(q, "bf16"), None) if not pre else _prescaled_q(q, hd)
    if not pre:
        q_ref = q_in.values
    k = _ht(k, "bf16")
    v = _ht(_f32((n, D), 1.0, 821, "w_qkv"), "bf16")
    ldvt = ((n + 7) // 8) * 8
    vt = np.zeros((D, ldvt), dtype=np.float32)
    vt[:, :n] = v.values.T
    vtd = torch.from_numpy(vt).to(torch.bfloat16).cuda()
    o = torch.full((n, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.h3k_attention(B.H3K_BF16, n, heads, hd, dev(q_in), D, dev(k), D, vtd, ldvt, o, D, q_prescaled=pre)
    torch.cuda.synchronize()
    ref = oracle.attention(q_ref, k.values, v.values, heads)
    got = to_np(o)
    assert np.isfinite(got).all()
    assert rel_l2(got, ref) < BF16_TOL


# ------------------------------------------------------------------ int8 quantiser

@pytest.mark.parametrize("rows,cols,group,dtype", [(13824, 5120, 128, "f32"), (5120, 13824, 128, "bf16"),
                                                   (300, 256, 32, "f32"), (257, 1024, 64, "bf16"),
                                                   (7, 64, 64, "bf16"), (3, 96, 32, "f32"), (64, 640, 128, "f32")])
def test_quantize_int8_groups_bit_exact(B, rows, cols, group, dtype):
    import torch
    flush(f"quantize groups rows={rows} cols={cols} group={group} {dtype}")
    w = _f32((rows, cols), 0.02, 831, "w_up")
    w[min(1, rows - 1)] = 0.0                      # a zero row
    w[rows - 1, group:2 * group] = 0.0             # a zero group inside a row
    w[0, 3] = 0.5                                  # one large value: only its group's scale moves
    ht = _ht(w, dtype)
    from video_diffusion_transformer_adaln_amd import runtime as R
    q, s = R.quantize_int8_groups(dev(ht), group)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_int8_groups(ht.values, group)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("rows,cols,dtype", [(15360, 5120, "f32"), (5120, 13824, "f32"), (300, 77, "f32"),
                                             (257, 1000, "bf16"), (3, 1, "f32"), (5120, 13824, "bf16"),
                                             (301, 8, "bf16"), (7, 20, "bf16"),
                                             (22680, 13824, "bf16"),   # the rows of u (row-quantised FC2)
                                             (64, 4104, "bf16"),       # one wave per row, a part-filled chunk column
                                             (33, 24576, "bf16"),      # a workgroup per row, 12 chunks per lane
                                             (5, 34816, "f32")])       # longer rows: the two-pass kernel
def test_quantize_int8_bit_exact(B, rows, cols, dtype):
    import torch
    flush(f"quantize rows={rows} cols={cols} {dtype}")
    w = _f32((rows, cols), 0.02, 830, "w_up")
    w[min(1, rows - 1)] = 0.0                      # a zero row
    ht = _ht(w, dtype)
    from video_diffusion_transformer_adaln_amd import runtime as R
    q, s = R.quantize_int8(dev(ht))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_int8(ht.values)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("cols,dtype", [(4096, "bf16"), (13824, "bf16"), (5120, "f32")])
def test_quantize_int8_exact_ties(B, cols, dtype):
    """Rows of k + 1/2 values with scale 2^e, so that w / s lands exactly on
    rounding ties: the reciprocal fast path must hand these to the correctly
    rounded division and round them half to even, bit-exact with the oracle."""
    import torch
    flush(f"quantize ties cols={cols} {dtype}")
    rng = np.random.default_rng(cols)
    rows = 64
    k = rng.integers(-127, 127, size=(rows, cols)).astype(np.float32) + np.float32(0.5)
    k[:, 0] = 127.0                                 # max |w| / 127 = 2^e exactly
    w = (k * np.exp2(rng.integers(-12, 4, size=(rows, 1)))).astype(np.float32)
    ht = _ht(w, dtype)
    assert np.array_equal(ht.values, w)             # exactly representable in bf16 as well
    from video_diffusion_transformer_adaln_amd import runtime as R
    q, s = R.quantize_int8(dev(ht))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_int8(ht.values)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert (np.abs(q_ref[:, 1:]) % 2 == 0).all()    # every tie went to the even neighbour


@pytest.mark.parametrize("group", [32, 128])
def test_quantize_int8_groups_exact_ties(B, group):
    """The group-wise quantiser on rows of k + 1/2 values whose every group
    has max |w| = 127 * 2^e: all other entries are exact rounding ties."""
    import torch
    flush(f"group quantize ties G={group}")
    rng = np.random.default_rng(group)
    rows, cols = 48, 2048
    k = rng.integers(-127, 127, size=(rows, cols)).astype(np.float32) + np.float32(0.5)
    k[:, ::group] = -127.0
    w = (k * np.exp2(rng.integers(-12, 4, size=(rows, 1)))).astype(np.float32)
    ht = _ht(w, "f32")
    from video_diffusion_transformer_adaln_amd import runtime as R
    q, s = R.quantize_int8_groups(dev(ht), group)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_int8_groups(ht.values, group)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
