"""Pins of the CPU oracle against things other than itself.

Each test fixes one part of the oracle with an independent route: a torch
CPU library routine, a pure-Python brute force, a closed form, a golden
fixture derived by hand, or an invariant of the mathematics.  A plausible
mistake (a dropped term, a swapped modulation chunk, a transposed weight, a
wrong softmax axis, a bad rounding rule) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import brute_force as bf
import oracle
import seeded_inputs as si
from helpers import host_values, rel_l2, tiny_problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- LayerNorm

def test_layernorm_closed_form_fixture():
    g = _golden("layernorm_closed_form.json")
    x = np.array([g["x"]], dtype=np.float32)
    got = oracle.layer_norm(x, g["eps"])[0]
    np.testing.assert_allclose(got, g["ln"], rtol=2e-7, atol=2e-7)


def test_layernorm_matches_torch_library():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((37, 256)) * 3 + 1.5).astype(np.float32)
    ref = F.layer_norm(torch.from_numpy(x).double(), (256,), eps=1e-6).numpy()
    assert rel_l2(oracle.layer_norm(x), ref) < 1e-6


def test_zero_modulation_is_plain_layernorm():
    shape, x, c, w = tiny_problem(n_tokens=6, n_heads=2, head_dim=8)
    w["w_ada"][:] = 0
    w["b_ada"][:] = 0
    inter = {}
    oracle.block_forward(x, c, w, shape.n_heads, intermediates=inter)
    ref = F.layer_norm(torch.from_numpy(x).double(), (shape.hidden,), eps=1e-6).numpy()
    assert rel_l2(inter["h"], ref) < 1e-6
    assert rel_l2(inter["h2"], F.layer_norm(torch.from_numpy(inter["x1"]).double(), (shape.hidden,),
                                          eps=1e-6).numpy()) < 1e-6


@pytest.mark.parametrize("chunk", range(6))
def test_modulation_chunk_order(chunk):
    """Only one chunk of b_ada is non-zero; its effect must show where it belongs."""
    shape, x, c, w = tiny_problem(n_tokens=6, n_heads=2, head_dim=8)
    D = shape.hidden
    w["w_ada"][:] = 0
    w["b_ada"][:] = 0
    w["b_ada"][chunk * D:(chunk + 1) * D] = 0.5
    inter = {}
    y = oracle.block_forward(x, c, w, shape.n_heads, intermediates=inter)
    ln_x = F.layer_norm(torch.from_numpy(x).double(), (D,), eps=1e-6).numpy()
    if chunk == 0:      # shift_a: h = LN(x) + 0.5
        np.testing.assert_allclose(inter["h"], ln_x + 0.5, rtol=1e-5, atol=1e-5)
    elif chunk == 1:    # scale_a: h = 1.5 LN(x)
        np.testing.assert_allclose(inter["h"], 1.5 * ln_x, rtol=1e-5, atol=1e-5)
    else:
        np.testing.assert_allclose(inter["h"], ln_x, rtol=1e-5, atol=1e-5)
    if chunk == 2:      # gate_a opens the attention branch
        assert np.abs(inter["x1"] - x).max() > 1e-3
    else:               # gate_a = 0: attention branch contributes nothing
        assert np.array_equal(inter["x1"], x)
    ln_x1 = F.layer_norm(torch.from_numpy(inter["x1"]).double(), (D,), eps=1e-6).numpy()
    if chunk == 3:
        np.testing.assert_allclose(inter["h2"], ln_x1 + 0.5, rtol=1e-5, atol=1e-5)
    elif chunk == 4:
        np.testing.assert_allclose(inter["h2"], 1.5 * ln_x1, rtol=1e-5, atol=1e-5)
    else:
        np.testing.assert_allclose(inter["h2"], ln_x1, rtol=1e-5, atol=1e-5)
    if chunk == 5:
        assert np.abs(y - inter["x1"]).max() > 1e-3
    else:
        assert np.array_equal(y, inter["x1"])


def test_gate_zero_is_identity_bitwise():
    shape, x, c, w = tiny_problem(n_tokens=9, n_heads=2, head_dim=8, mlp=40)
    D = shape.hidden
    for g in (2, 5):     # gate_a and gate_m rows of the AdaLN map
        w["w_ada"][g * D:(g + 1) * D] = 0
        w["b_ada"][g * D:(g + 1) * D] = 0
    y = oracle.block_forward(x, c, w, shape.n_heads)
    assert np.array_equal(y, x)


# ---------------------------------------------------------------- GELU, linear

def test_gelu_matches_torch_and_limits():
    z = np.linspace(-12, 12, 20001).astype(np.float32)
    ref = F.gelu(torch.from_numpy(z).double(), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z), ref, rtol=2e-6, atol=2e-7)
    assert oracle.gelu_tanh(np.zeros(1, np.float32))[0] == 0.0
    big = np.array([30.0, -30.0], np.float32)
    np.testing.assert_allclose(oracle.gelu_tanh(big), [30.0, 0.0], atol=1e-6)
    # closed form at 1: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    assert abs(oracle.gelu_tanh(np.ones(1, np.float32))[0] -
               0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))) < 1e-6


def test_linear_matches_torch_and_brute_force():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 12)).astype(np.float32)
    w = rng.standard_normal((5, 12)).astype(np.float32)      # [out, in], non-square
    b = rng.standard_normal(5).astype(np.float32)
    got = oracle.linear(x, w, b)
    ref_t = F.linear(torch.from_numpy(x).double(), torch.from_numpy(w).double(), torch.from_numpy(b).double())
    assert rel_l2(got, ref_t.numpy()) < 1e-6
    assert rel_l2(got, bf.dense(x.tolist(), w.tolist(), b.tolist())) < 1e-6


# ---------------------------------------------------------------- attention

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(11)
    s = (rng.standard_normal((64, 300)) * 10).astype(np.float32)
    p = oracle.softmax_rows(s)
    assert np.abs(p.sum(axis=-1) - 1).max() < 1e-6
    assert (p >= 0).all()


@pytest.mark.parametrize("n,heads,d", [(1, 2, 4), (7, 2, 4), (13, 3, 8)])
def test_attention_matches_naive_brute_force(n, heads, d):
    rng = np.random.default_rng(n * 31 + d)
    D = heads * d
    q, k, v = (rng.standard_normal((n, D)).astype(np.float32) * 2 for _ in range(3))
    got = oracle.attention(q, k, v, heads, chunk=4)
    ref = bf.attention_naive(q.tolist(), k.tolist(), v.tolist(), heads)
    assert rel_l2(got, ref) < 2e-6


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(19)
    n, heads, d = 300, 3, 16
    q, k, v = (rng.standard_normal((n, heads * d)).astype(np.float32) for _ in range(3))
    got = oracle.attention(q, k, v, heads, chunk=128)
    t = lambda a: torch.from_numpy(a).double().view(n, heads, d).transpose(0, 1)
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v)).transpose(0, 1).reshape(n, heads * d)
    assert rel_l2(got, ref.numpy()) < 1e-6


def test_attention_special_cases():
    rng = np.random.default_rng(23)
    v = rng.standard_normal((1, 8)).astype(np.float32)
    q = rng.standard_normal((1, 8)).astype(np.float32)
    # one token: softmax over one key is exactly 1, so o = v
    assert np.array_equal(oracle.attention(q, q, v, 2), v)
    # identical keys and values: o is that value row, whatever the queries
    kk = np.repeat(rng.standard_normal((1, 8)).astype(np.float32), 6, axis=0)
    vv = np.repeat(v, 6, axis=0)
    qq = rng.standard_normal((6, 8)).astype(np.float32)
    np.testing.assert_allclose(oracle.attention(qq, kk, vv, 2), vv, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- whole block

@pytest.mark.parametrize("n,heads,d,mlp", [(1, 2, 4, 12), (5, 2, 4, 12), (6, 3, 4, 20)])
def test_block_matches_brute_force(n, heads, d, mlp):
    shape, x, c, w = tiny_problem(n_tokens=n, n_heads=heads, head_dim=d, mlp=mlp)
    got = oracle.block_forward(x, c, w, heads)
    ref = bf.block(x.tolist(), c.tolist(), {k: v.tolist() for k, v in w.items()}, heads)
    assert rel_l2(got, ref) < 1e-5


def test_block_matches_torch_composition_c0():
    """The c0 block through torch CPU library routines (fp64)."""
    shape = si.C0
    x, c = si.gen_activation(shape)
    w = host_values(si.gen_block_weights(shape, 0, bias_std=0.05))
    got = oracle.block_forward(x.values, c.values, w, shape.n_heads)
    T = lambda a: torch.from_numpy(np.asarray(a)).double()
    D, H, d, N = shape.hidden, shape.n_heads, shape.head_dim, shape.n_tokens
    mod = F.linear(T(c.values)[None], T(w["w_ada"]), T(w["b_ada"]))[0]
    sa, ca, ga, sm, cm, gm = mod.split(D)
    xx = T(x.values)
    h = F.layer_norm(xx, (D,), eps=1e-6) * (1 + ca) + sa
    qkv = F.linear(h, T(w["w_qkv"]), T(w["b_qkv"]))
    q, k, v = (t.view(N, H, d).transpose(0, 1) for t in qkv.split(D, dim=1))
    o = F.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(N, D)
    x1 = xx + ga * F.linear(o, T(w["w_out"]), T(w["b_out"]))
    h2 = F.layer_norm(x1, (D,), eps=1e-6) * (1 + cm) + sm
    u = F.gelu(F.linear(h2, T(w["w_up"]), T(w["b_up"])), approximate="tanh")
    y = x1 + gm * F.linear(u, T(w["w_down"]), T(w["b_down"]))
    assert rel_l2(got, y.numpy()) < 1e-5


def test_block_matches_torch_fp64_c1_sampled_rows():
    """The fp32 oracle at the 6144-token width (D = 3072, 24 x 128 heads,
    F = 12288) against the same block in fp64 through torch CPU routines, on
    the first 8, the last 8 and 16 seeded token rows (k and v over every
    token).  fp32 dot products over up to K = 12288 terms carry a relative
    error of at most about sqrt(K) 2^-24 ~ 7e-6 each; the bound is the c0
    pin's 1e-5 (measured: about 1e-6)."""
    shape = si.C1
    x, c = si.gen_activation(shape)
    w = host_values(si.gen_block_weights(shape, 0, bias_std=0.05))
    n = shape.n_tokens
    rng = np.random.default_rng(5)
    rows = np.array(sorted(set(range(8)) | set(range(n - 8, n)) | set(rng.choice(n, 16, replace=False).tolist())))
    got = oracle.block_forward(x.values, c.values, w, shape.n_heads, rows=rows)
    T = lambda a: torch.from_numpy(np.asarray(a)).double()
    D, H, d = shape.hidden, shape.n_heads, shape.head_dim
    with torch.no_grad():
        mod = F.linear(T(c.values)[None], T(w["w_ada"]), T(w["b_ada"]))[0]
        sa, ca, ga, sm, cm, gm = mod.split(D)
        xx = T(x.values)
        h = F.layer_norm(xx, (D,), eps=1e-6) * (1 + ca) + sa
        wq, wk, wv = T(w["w_qkv"]).split(D)
        bq, bk, bv = T(w["b_qkv"]).split(D)
        q = F.linear(h[rows], wq, bq).view(len(rows), H, d).transpose(0, 1)
        k = F.linear(h, wk, bk).view(n, H, d).transpose(0, 1)
        v = F.linear(h, wv, bv).view(n, H, d).transpose(0, 1)
        p = torch.softmax(q @ k.transpose(1, 2) / math.sqrt(d), dim=-1)
        o = (p @ v).transpose(0, 1).reshape(len(rows), D)
        x1 = xx[rows] + ga * F.linear(o, T(w["w_out"]), T(w["b_out"]))
        h2 = F.layer_norm(x1, (D,), eps=1e-6) * (1 + cm) + sm
        u = F.gelu(F.linear(h2, T(w["w_up"]), T(w["b_up"])), approximate="tanh")
        y = x1 + gm * F.linear(u, T(w["w_down"]), T(w["b_down"]))
    err = rel_l2(got, y.numpy())
    print(f"c1 block, fp32 oracle against fp64 torch, sampled rows: rel-L2 {err:.2e}")
    assert err < 1e-5, err


def test_block_rows_subset_equals_full():
    shape, x, c, w = tiny_problem(n_tokens=40, n_heads=2, head_dim=8, mlp=24)
    full = oracle.block_forward(x, c, w, shape.n_heads)
    rows = [0, 3, 17, 39]
    np.testing.assert_allclose(oracle.block_forward(x, c, w, shape.n_heads, rows=rows), full[rows],
                               rtol=1e-6, atol=1e-6)


def test_block_permutation_equivariance():
    """No positional terms: permuting tokens permutes the output rows."""
    shape, x, c, w = tiny_problem(n_tokens=48, n_heads=4, head_dim=8, mlp=64)
    perm = np.random.default_rng(1).permutation(shape.n_tokens)
    a = oracle.block_forward(x[perm], c, w, shape.n_heads)
    b = oracle.block_forward(x, c, w, shape.n_heads)[perm]
    assert rel_l2(a, b) < 1e-5


# ---------------------------------------------------------------- stack

def test_stack_one_layer_is_block_and_prefix():
    shape, x, c, _ = tiny_problem(n_tokens=16, n_heads=2, head_dim=8, mlp=32)
    blocks = []
    for l in range(4):
        w = host_values(si.gen_block_weights(shape, l, 7, bias_std=0.1))
        blocks.append(w)
    one = oracle.stack_forward(x, c, blocks[:1], shape.n_heads)
    assert np.array_equal(one, oracle.block_forward(x, c, blocks[0], shape.n_heads))
    two = oracle.stack_forward(x, c, blocks, shape.n_heads, n_layers=2)
    manual = oracle.block_forward(oracle.block_forward(x, c, blocks[0], shape.n_heads), c, blocks[1],
                                  shape.n_heads)
    assert np.array_equal(two, manual)
    three = oracle.stack_forward(x, c, blocks, shape.n_heads, n_layers=3)
    assert np.array_equal(three, oracle.stack_forward(x, c, blocks[:3], shape.n_heads))


# ---------------------------------------------------------------- 3D RoPE

def _grid_positions(grid, half=False):
    T, H, W = grid
    return [(t, h * (0.5 if half else 1.0), w * (0.5 if half else 1.0))
            for t in range(T) for h in range(H) for w in range(W)]


@pytest.mark.parametrize("d,grid,half", [(16, (2, 3, 4), False), (32, (3, 2, 2), True), (64, (1, 4, 5), False)])
def test_rope_matches_brute_force(d, grid, half):
    n = grid[0] * grid[1] * grid[2]
    heads = 2
    rng = np.random.default_rng(61)
    x = rng.standard_normal((n, heads * d)).astype(np.float32)
    got = oracle.rope_3d(x, heads, grid, half)
    ref = bf.rope_rows(x.astype(np.float64).tolist(), heads, _grid_positions(grid, half), oracle.rope_axis_dims(d))
    assert np.allclose(got, np.array(ref), rtol=1e-6, atol=1e-6)


def test_rope_axis_split_and_positions():
    assert oracle.rope_axis_dims(128) == (32, 48, 48)
    assert oracle.rope_axis_dims(64) == (16, 24, 24)
    with pytest.raises(ValueError):
        oracle.rope_axis_dims(8)
    pos = oracle.rope_positions(2 * 3 * 5, (2, 3, 5))
    assert pos[0].tolist() == [0, 0, 0] and pos[1].tolist() == [0, 0, 1] and pos[5].tolist() == [0, 1, 0]
    assert pos[15].tolist() == [1, 0, 0] and pos[29].tolist() == [1, 2, 4]
    assert oracle.rope_positions(30, (2, 3, 5), True)[29].tolist() == [1, 1.0, 2.0]
    with pytest.raises(ValueError):
        oracle.rope_positions(31, (2, 3, 5))


def test_rope_identity_at_origin_and_pair_norms():
    rng = np.random.default_rng(67)
    grid = (2, 3, 4)
    x = rng.standard_normal((24, 128)).astype(np.float32)
    y = oracle.rope_3d(x, 1, grid)
    assert np.array_equal(y[0], x[0])                         # token (0, 0, 0): every angle is 0
    nx = np.hypot(x[:, 0::2].astype(np.float64), x[:, 1::2])
    ny = np.hypot(y[:, 0::2].astype(np.float64), y[:, 1::2])
    assert np.allclose(nx, ny, rtol=1e-6)


def test_rope_scores_depend_on_relative_position_only():
    """<R(p) q, R(p') k> is a function of p - p' for every axis: shifting both
    tokens by the same offset leaves every head's score unchanged."""
    rng = np.random.default_rng(71)
    grid = (3, 4, 5)
    n = 60
    d, heads = 64, 2
    qv = rng.standard_normal(heads * d)
    kv = rng.standard_normal(heads * d)
    X = np.tile(qv, (n, 1)).astype(np.float32)
    K = np.tile(kv, (n, 1)).astype(np.float32)
    rq, rk = oracle.rope_3d(X, heads, grid), oracle.rope_3d(K, heads, grid)
    tok = lambda t, h, w: (t * 4 + h) * 5 + w
    for h_ in range(heads):
        sl = slice(h_ * d, (h_ + 1) * d)
        s1 = float(rq[tok(0, 1, 1), sl].astype(np.float64) @ rk[tok(1, 0, 3), sl])
        s2 = float(rq[tok(1, 3, 2), sl].astype(np.float64) @ rk[tok(2, 2, 4), sl])
        assert abs(s1 - s2) < 1e-4 * max(1.0, abs(s1))
        s3 = float(rq[tok(0, 1, 1), sl].astype(np.float64) @ rk[tok(1, 0, 4), sl])   # a different offset
        assert abs(s1 - s3) > 1e-3


def test_rope_axes_act_on_their_own_slices():
    """Tokens in the same frame get the same time slice; tokens in the same
    row the same height slice; tokens in the same column the same width slice."""
    rng = np.random.default_rng(73)
    grid = (2, 3, 4)
    v = rng.standard_normal(64).astype(np.float32)
    y = oracle.rope_3d(np.tile(v, (24, 1)), 1, grid)
    dt, dh, dw = oracle.rope_axis_dims(64)
    tok = lambda t, h, w: (t * 3 + h) * 4 + w
    assert np.array_equal(y[tok(1, 0, 0), :dt], y[tok(1, 2, 3), :dt])
    assert np.array_equal(y[tok(0, 2, 1), dt:dt + dh], y[tok(1, 2, 3), dt:dt + dh])
    assert np.array_equal(y[tok(0, 0, 3), dt + dh:], y[tok(1, 2, 3), dt + dh:])
    assert not np.array_equal(y[tok(0, 0, 0), :dt], y[tok(1, 0, 0), :dt])


def test_block_with_rope_matches_brute_force():
    shape, x, c, w = tiny_problem(n_tokens=6, n_heads=2, head_dim=16, mlp=12)
    grid = (1, 2, 3)
    got = oracle.block_forward(x, c, w, shape.n_heads, rope=(1, 2, 3, False))
    ref = bf.block(x.tolist(), c.tolist(), {k: (v.tolist() if v is not None else None) for k, v in w.items()},
                   shape.n_heads, rope=(_grid_positions(grid), oracle.rope_axis_dims(16)))
    assert rel_l2(got, ref) < 1e-5
    plain = oracle.block_forward(x, c, w, shape.n_heads)
    assert rel_l2(got, plain) > 1e-3                    # the positions do change the block
    rows = [1, 4]
    part = oracle.block_forward(x, c, w, shape.n_heads, rows=rows, rope=(1, 2, 3, False))
    assert np.allclose(part, got[rows], rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------- token reduction

def test_token_merge_pairs_and_identity_restore():
    rng = np.random.default_rng(79)
    x = rng.standard_normal((10, 6)).astype(np.float32)
    m = oracle.token_merge(x)
    ref = bf.token_merge_rows(x.astype(np.float64).tolist())
    assert np.allclose(m, np.array(ref), rtol=1e-6, atol=1e-7)
    dup = np.repeat(x[:5], 2, axis=0)                      # equal pairs merge to themselves
    assert np.array_equal(oracle.token_merge(dup), x[:5])
    assert np.array_equal(oracle.token_unmerge(x, m), x)   # reduced layers that change nothing
    d = rng.standard_normal((5, 6)).astype(np.float32)     # a change of the merged stream reaches both tokens
    assert np.allclose(oracle.token_unmerge(x, m + d), x + np.repeat(d, 2, axis=0), rtol=1e-6, atol=1e-6)
    with pytest.raises(ValueError):
        oracle.token_merge(x[:9])


def test_reduced_stack_matches_brute_force_and_empty_range():
    shape, x, c, w = tiny_problem(n_tokens=8, n_heads=2, head_dim=4, mlp=12)
    blocks = [w, {k: (v * 0.9 if v is not None else None) for k, v in w.items()},
              {k: (v * 1.1 if v is not None else None) for k, v in w.items()}, w]
    got = oracle.stack_forward(x, c, blocks, shape.n_heads, token_reduction=(1, 3))
    lists = [{k: (v.tolist() if v is not None else None) for k, v in b.items()} for b in blocks]
    ref = bf.reduced_stack(x.tolist(), c.tolist(), lists, shape.n_heads, 1, 3)
    assert rel_l2(got, ref) < 1e-5
    plain = oracle.stack_forward(x, c, blocks, shape.n_heads)
    assert np.array_equal(oracle.stack_forward(x, c, blocks, shape.n_heads, token_reduction=(2, 2)), plain)
    assert rel_l2(got, plain) > 1e-3                       # the reduction does change the result
    # reducing from the first block to the last is merge, the stack on N/2 tokens, restore
    whole = oracle.stack_forward(x, c, blocks, shape.n_heads, token_reduction=(0, 4))
    mid = oracle.stack_forward(oracle.token_merge(x), c, blocks, shape.n_heads)
    assert np.allclose(whole, oracle.token_unmerge(x, mid), rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- int8 quantiser

def test_quantize_golden_ties():
    g = _golden("quantize_int8_ties.json")
    q, s = oracle.quantize_int8(np.array(g["w"], dtype=np.float32))
    assert q.tolist() == g["q"]
    assert s.tolist() == g["s"]


def test_quantize_matches_pure_python_fp32():
    rng = np.random.default_rng(29)
    w = (rng.standard_normal((9, 50)) * 0.02).astype(np.float32)
    w[3] = 0.0                      # zero row
    w[4] = 0.0
    w[4, 7] = -1e-3                 # single non-zero
    w[5, :10] = 0.5 * w[5].max()    # repeated values
    q, s = oracle.quantize_int8(w)
    for o in range(w.shape[0]):
        qr, sr = bf.quantize_row_int8(w[o].tolist())
        assert q[o].tolist() == qr
        assert float(s[o]) == sr


def test_quantize_bounds_and_error():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    q, s = oracle.quantize_int8(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(q.astype(np.int32)).max() <= 127
    assert (np.abs(q.astype(np.int32)).max(axis=1) == 127).all()
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    # |w - q s| <= s (1/2 + 127 * 2^-24): half a step plus the fp32 rounding of w/s
    assert (err <= s.astype(np.float64)[:, None] * (0.5 + 127 * 2.0 ** -24)).all()
    # the oracle's per-channel dequantisation lands within the same step of w
    # (plus the fp32 rounding of q s); a dropped, transposed or wrong-row scale
    # fails this on the non-square matrix
    deq = oracle.dequantize_int8(q, s)
    assert deq.dtype == np.float32 and deq.shape == w.shape
    err_d = np.abs(w.astype(np.float64) - deq.astype(np.float64))
    assert (err_d <= s.astype(np.float64)[:, None] * (0.5 + 2 * 127 * 2.0 ** -24)).all()


def test_int8_block_uses_dequantised_weights():
    shape, x, c, w = tiny_problem(n_tokens=5, n_heads=2, head_dim=4, mlp=12)
    wq = dict(w)
    deq = dict(w)
    for name in si.MATRIX_NAMES:
        qs = oracle.quantize_int8(w[name])
        wq[name] = qs
        deq[name] = oracle.dequantize_int8(*qs)
    got = oracle.block_forward(x, c, wq, shape.n_heads)
    ref = bf.block(x.tolist(), c.tolist(), {k: v.tolist() for k, v in deq.items()}, shape.n_heads)
    assert rel_l2(got, ref) < 1e-5


def test_quantize_groups_golden():
    g = _golden("quantize_int8_groups.json")
    q, s = oracle.quantize_int8_groups(np.array(g["w"], dtype=np.float32), g["group"])
    assert q.tolist() == g["q"]
    assert s.tolist() == g["s"]


@pytest.mark.parametrize("group", [4, 32, 64])
def test_quantize_groups_matches_pure_python_fp32(group):
    rng = np.random.default_rng(43)
    w = (rng.standard_normal((7, 128)) * 0.02).astype(np.float32)
    w[2] = 0.0                            # a zero row: every group zero
    w[3, :group] = 0.0                    # one zero group inside a row
    w[4, 5] = 1.0                         # one large value: its group's scale only
    q, s = oracle.quantize_int8_groups(w, group)
    assert s.shape == (7, 128 // group)
    for o in range(w.shape[0]):
        qr, sr = bf.quantize_groups_int8(w[o].tolist(), group)
        assert q[o].tolist() == qr
        assert s[o].tolist() == sr


def test_quantize_groups_whole_row_is_per_channel():
    rng = np.random.default_rng(47)
    w = (rng.standard_normal((9, 96)) * 0.02).astype(np.float32)
    qg, sg = oracle.quantize_int8_groups(w, 96)
    q, s = oracle.quantize_int8(w)
    assert np.array_equal(qg, q)
    assert np.array_equal(sg[:, 0], s)


def test_quantize_groups_bounds_error_and_dequantise():
    rng = np.random.default_rng(53)
    w = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    q, s = oracle.quantize_int8_groups(w, 64)
    qi = q.astype(np.int32).reshape(32, 4, 64)
    assert np.abs(qi).max() <= 127
    assert (np.abs(qi).max(axis=2) == 127).all()        # every group reaches the full range
    deq = oracle.dequantize_int8(q, s)                   # 2-D scales select the group rule
    for o in range(0, 32, 7):
        for k in range(0, 256, 13):
            assert deq[o, k] == np.float32(np.float32(q[o, k]) * s[o, k // 64])
    err = np.abs(w.astype(np.float64) - deq.astype(np.float64))
    bound = np.repeat(s.astype(np.float64), 64, axis=1) * (0.5 + 127 * 2.0 ** -24)
    assert (err <= bound).all()
    # group scales never exceed the row scale, so the group rule is at least as fine
    _, s_row = oracle.quantize_int8(w)
    assert (s <= s_row[:, None]).all()


def test_int8_group_mlp_block_uses_dequantised_weights():
    shape, x, c, w = tiny_problem(n_tokens=5, n_heads=2, head_dim=4, mlp=16)
    wq = dict(w)
    deq = dict(w)
    for name in si.MATRIX_NAMES:
        qs = oracle.quantize_int8_groups(w[name], 4) if name in ("w_up", "w_down") else oracle.quantize_int8(w[name])
        wq[name] = qs
        deq[name] = oracle.dequantize_int8(*qs)
    got = oracle.block_forward(x, c, wq, shape.n_heads)
    ref = bf.block(x.tolist(), c.tolist(), {k: v.tolist() for k, v in deq.items()}, shape.n_heads)
    assert rel_l2(got, ref) < 1e-5


def test_w8a8_linear_is_the_exact_integer_sum():
    rng = np.random.default_rng(37)
    qx = rng.integers(-127, 128, size=(5, 96)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(7, 96)).astype(np.int8)
    ones_x, ones_w = np.ones(5, np.float32), np.ones(7, np.float32)
    got = oracle.linear_w8a8(qx, ones_x, qw, ones_w, None)
    for n in range(5):
        for o in range(7):
            exact = sum(int(a) * int(w) for a, w in zip(qx[n], qw[o]))   # |sum| < 2^24: exact in fp32
            assert float(got[n, o]) == float(exact)


def test_w8a8_linear_matches_the_dequantised_product():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    w = (rng.standard_normal((9, 128)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(9) * 0.05).astype(np.float32)
    qx, sx = oracle.quantize_int8(x)
    qw, sw = oracle.quantize_int8(w)
    got = oracle.linear_w8a8(qx, sx, qw, sw, b)
    ref = (qx.astype(np.float64) * sx.astype(np.float64)[:, None]) @ \
          (qw.astype(np.float64) * sw.astype(np.float64)[:, None]).T + b.astype(np.float64)
    assert rel_l2(got, ref) < 1e-6


def test_int8_fc2_block_stage_matches_brute_force():
    """The row-quantised FC2 stage of the oracle block against the pure-Python
    quantiser and integer sums, fed the same u (so every rounding decision
    is taken on identical values); the residual and gate around it as in
    the float block."""
    shape, x, c, w = tiny_problem(n_tokens=6, n_heads=2, head_dim=4, mlp=40)
    wq = dict(w)
    for name in si.MATRIX_NAMES:
        wq[name] = oracle.quantize_int8(w[name])
    inter = {}
    got = oracle.block_forward(x, c, wq, shape.n_heads, intermediates=inter, int8_fc2_rows=True)
    q_down, s_down = wq["w_down"]
    b_down = w.get("b_down")
    down = bf.fc2_int8_rows(inter["u"].tolist(), q_down.astype(int).tolist(), s_down.tolist(),
                            None if b_down is None else b_down.tolist())
    gate_m = inter["mod"]["gate_m"].astype(np.float64)
    ref = inter["x1"].astype(np.float64) + gate_m * np.array(down)
    assert rel_l2(got, ref) < 1e-6
    # and the int8 FC2 stays close to the dequantised-weight block (one quantisation of u)
    plain = oracle.block_forward(x, c, wq, shape.n_heads)
    assert rel_l2(got, plain) < 2e-2


# ---------------------------------------------------------------- generator sanity

def test_bf16_rounding_of_generator():
    a = np.array([1.0, 1.00390625, 1.005859375, -2.0 ** -130, 3.4e38], dtype=np.float32)
    bits = si.bf16_bits(a)
    back = si.bf16_to_f32(bits)
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    assert np.array_equal(back, ref)
    rng = np.random.default_rng(2)
    r = rng.standard_normal(100000).astype(np.float32)
    assert np.array_equal(si.bf16_to_f32(si.bf16_bits(r)),
                          torch.from_numpy(r).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_distributed():
    shape = si.C0
    w1 = si.gen_block_weights(shape, 0)
    w2 = si.gen_block_weights(shape, 0)
    w3 = si.gen_block_weights(shape, 1)
    assert np.array_equal(w1["w_qkv"].values, w2["w_qkv"].values)
    assert not np.array_equal(w1["w_qkv"].values, w3["w_qkv"].values)
    assert abs(float(w1["w_up"].values.std()) - 0.02) < 1e-3
    assert not w1["b_qkv"].values.any()
