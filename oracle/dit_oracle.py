"""CPU oracle for the AdaLN-modulated DiT block forward (plain numpy, fp32).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  It shares no code with the GPU library and never imports it; the
only module both sides use is ``seeded_inputs`` (random draws, no method
arithmetic).

Sources.  Two pages describe the block this oracle computes:
  [H3-review]  "Redis 之父下场手写推理引擎：antirez 用约 24000 行原生代码驯服视频生成模型"
               (text-matrix.pages.dev, review of antirez's h3-metal engine).
  [H3-memory]  "37GiB模型如何装进统一内存 h3.c 零拷贝权重与激活内存别名技巧详解"
               (m.nxbn.cn, zero-copy weights and activation aliasing in h3.c).
[H3-memory], technique 2 (activation aliasing), fixes the order inside a block
(QKV projection, then attention, then the MLP) and that a denoising step runs
50 such blocks; technique 3 says AdaLN is precomputed before the block's
heavy work.  [H3-review], knob list, gives the layer counts 50 / 45 / 40 and,
in its speed/quality section, the int8 weight variants (int8 MLP, then int8
QKV projection).  The pages print no formula for the block, so each function
below states the reading it implements; every reading is listed again in the
repository's design notes.

Everything is float32, as a plain fp32 reference.  Matmuls use numpy's BLAS
as a library step; nothing else is blocked, fused or reordered.

Pins (tests/test_oracle_pins.py): textbook LayerNorm via torch on the CPU,
pure-Python brute force of the whole block and of attention on tiny inputs,
torch's scaled-dot-product attention and tanh-GELU, closed-form values,
permutation equivariance, gate = 0 identity, softmax rows summing to one,
the layer-prefix property of the stack, a pure-Python fp32 quantiser (per
channel and per group), and pure-Python integer sums for the int8 x int8
projection.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

LN_EPS = 1e-6
# Order of the six length-D chunks of the AdaLN modulation vector:
# shift, scale, gate for the attention branch, then the same for the MLP.
MOD_CHUNKS = ("shift_a", "scale_a", "gate_a", "shift_m", "scale_m", "gate_m")

f32 = np.float32


def adaln_modulation(w_ada: np.ndarray, b_ada: Optional[np.ndarray], c: np.ndarray) -> Dict[str, np.ndarray]:
    """mod = W_ada c + b_ada, split into six chunks of length D.

    Reading: no SiLU on c before the linear map (a caller wanting one passes
    SiLU(c)); [H3-memory] technique 3 only says the modulation is computed
    once, ahead of the block's heavy stages.
    """
    mod = w_ada.astype(f32) @ c.astype(f32)
    if b_ada is not None:
        mod = mod + b_ada.astype(f32)
    D = mod.shape[0] // 6
    return {name: mod[i * D:(i + 1) * D] for i, name in enumerate(MOD_CHUNKS)}


def layer_norm(z: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """Row-wise LayerNorm without affine parameters; biased variance."""
    z = z.astype(f32)
    mu = z.mean(axis=-1, keepdims=True)
    var = np.square(z - mu).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + f32(eps))


def modulate(zn: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """AdaLN modulation zn * (1 + scale) + shift, broadcast over tokens.

    The (1 + scale) form makes zero modulation reduce to plain LayerNorm.
    """
    return zn * (f32(1.0) + scale) + shift


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """y = x W^T + b with W in [out, in] layout."""
    y = x.astype(f32) @ w.astype(f32).T
    if b is not None:
        y = y + b.astype(f32)
    return y


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, the row maximum subtracted first."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int, chunk: int = 512) -> np.ndarray:
    """Full (non-causal) multi-head self-attention without positional terms.

    q: [Nq, D] query rows, k and v: [N, D] all tokens.  Head j uses columns
    j*d .. (j+1)*d-1.  Per head o = softmax(q k^T / sqrt(d)) v.  Query rows are
    taken ``chunk`` at a time only to bound memory; every row's softmax is
    computed over all N keys at once, so the chunking changes nothing.
    [H3-memory] technique 2: attention runs over the whole token sequence
    between the QKV projection and the MLP.
    """
    nq, D = q.shape
    d = D // n_heads
    scale = f32(1.0 / math.sqrt(d))
    o = np.empty((nq, D), dtype=f32)
    for j in range(n_heads):
        cols = slice(j * d, (j + 1) * d)
        kh = k[:, cols]
        vh = v[:, cols]
        for r0 in range(0, nq, chunk):
            r = slice(r0, min(nq, r0 + chunk))
            s = (q[r, cols] @ kh.T) * scale
            o[r, cols] = softmax_rows(s) @ vh
    return o


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    z = z.astype(f32)
    c = f32(math.sqrt(2.0 / math.pi))
    return f32(0.5) * z * (f32(1.0) + np.tanh(c * (z + f32(0.044715) * z * z * z)))


ROPE_BASE = 10000.0


def rope_axis_dims(head_dim: int):
    """Head dimensions given to the (time, height, width) axes: d/4, 3d/8, 3d/8
    (each even, so d must be a multiple of 16)."""
    if head_dim % 16:
        raise ValueError("RoPE needs head_dim a multiple of 16")
    dt = head_dim // 4
    dh = (head_dim - dt) // 2
    return dt, dh, head_dim - dt - dh


def rope_positions(n_tokens: int, grid, half_spatial: bool = False) -> np.ndarray:
    """[n_tokens, 3] (t, h, w) coordinates of tokens laid out frame by frame,
    then row by row, then column by column over the latent grid (T, H, W);
    the spatial two are halved under the native-256 rule."""
    T, H, W = grid
    if T * H * W != n_tokens:
        raise ValueError("grid does not match the token count")
    n = np.arange(n_tokens)
    pos = np.stack([n // (H * W), (n // W) % H, n % W], axis=1).astype(np.float64)
    if half_spatial:
        pos[:, 1:] *= 0.5
    return pos


def rope_3d(x: np.ndarray, n_heads: int, grid, half_spatial: bool = False) -> np.ndarray:
    """3D rotary position embedding of q or k ([n_tokens, n_heads * d]).

    [H3-review], its note on native-256 RoPE: rotary position embedding
    injects each token's position, and on 256 square canvases the spatial
    RoPE coordinates are halved.  The page gives no more; the readings here
    (listed again in the design notes) are the plainest ones for a video
    latent: each head's d dimensions are split into a time, a height and a
    width slice (rope_axis_dims), and within the slice of axis a the pair
    (2i, 2i+1) is rotated by the angle pos_a * base^(-2i / d_a), base 10000:
        (x, y) -> (x cos phi - y sin phi, x sin phi + y cos phi).
    Angles and rotation in float64, result rounded to fp32.
    """
    N, D = x.shape
    d = D // n_heads
    pos = rope_positions(N, grid, half_spatial)
    x = x.astype(np.float64).reshape(N, n_heads, d)
    out = np.empty_like(x)
    c0 = 0
    for a, da in enumerate(rope_axis_dims(d)):
        i = np.arange(da // 2, dtype=np.float64)
        theta = ROPE_BASE ** (-2.0 * i / da)
        phi = pos[:, a:a + 1] * theta[None, :]                 # [N, da/2]
        cs, sn = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
        xe, xo = x[:, :, c0:c0 + da:2], x[:, :, c0 + 1:c0 + da:2]
        out[:, :, c0:c0 + da:2] = xe * cs - xo * sn
        out[:, :, c0 + 1:c0 + da:2] = xe * sn + xo * cs
        c0 += da
    return out.reshape(N, D).astype(f32)


def quantize_int8(w: np.ndarray):
    """Per-output-channel symmetric int8: s[o] = max_k |w[o,k]| / 127,
    q = clip(rint(w / s), -127, 127) with ties to even.

    One fp32 division for s and one per element for w / s.  A row of zeros
    gets s = 0 and q = 0.  [H3-review] speed/quality section: the engine's
    int8 path quantises the MLP and then the QKV projection weights.
    """
    w = np.ascontiguousarray(w, dtype=f32)
    s = (np.abs(w).max(axis=1) / f32(127.0)).astype(f32)
    safe = np.where(s == 0, f32(1.0), s).astype(f32)
    q = np.rint(w / safe[:, None])
    q = np.clip(q, -127, 127)
    q[s == 0] = 0
    return q.astype(np.int8), s


def dequantize_int8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q * s in fp32; s is [rows] (per-channel) or [rows, cols / G] (groups of G)."""
    if s.ndim == 2:
        return dequantize_int8_groups(q, s)
    return q.astype(f32) * s.astype(f32)[:, None]


def quantize_int8_groups(w: np.ndarray, group: int):
    """Group-wise symmetric int8: each output channel's input axis is cut into
    consecutive blocks of ``group`` weights, and every block gets its own
    scale, s[o, g] = max |w[o, gG:(g+1)G]| / 127, with
    q = clip(rint(w / s), -127, 127), ties to even, one fp32 division per
    element.  A block of zeros gets s = 0 and q = 0.

    [H3-review] speed/quality section: the engine's default MLP path on the
    M5 is int8 with group quantisation.  The page gives no group size; the
    library takes G in {32, 64, 128}.  With G = cols this is quantize_int8.
    """
    w = np.ascontiguousarray(w, dtype=f32)
    rows, cols = w.shape
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    wg = w.reshape(rows, cols // group, group)
    s = (np.abs(wg).max(axis=2) / f32(127.0)).astype(f32)
    safe = np.where(s == 0, f32(1.0), s).astype(f32)
    q = np.rint(wg / safe[:, :, None])
    q = np.clip(q, -127, 127)
    q[s == 0] = 0
    return q.reshape(rows, cols).astype(np.int8), s


def dequantize_int8_groups(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """w[o, k] = q[o, k] * s[o, k // G] in fp32, G = cols / s.shape[1]."""
    rows, cols = q.shape
    ng = s.shape[1]
    wg = q.astype(f32).reshape(rows, ng, cols // ng) * s.astype(f32)[:, :, None]
    return wg.reshape(rows, cols)


def linear_w8a8(qx: np.ndarray, sx: np.ndarray, qw: np.ndarray, sw: np.ndarray,
                b: Optional[np.ndarray]) -> np.ndarray:
    """Both operands int8: y[n, o] = sx[n] sw[o] sum_k qx[n, k] qw[o, k] + b[o].

    The k-sum of int8 products is an exact integer (computed in float64,
    which holds every integer below 2^53); it is rounded once to fp32, then
    multiplied by the activation row scale and the weight channel scale,
    and the bias is added, in fp32.  [H3-review] speed/quality section: the
    row-quantised FC2 variant gives the MLP's second projection one
    activation scale per token row.
    """
    acc = qx.astype(np.float64) @ qw.astype(np.float64).T
    y = acc.astype(f32) * sx.astype(f32)[:, None] * sw.astype(f32)[None, :]
    if b is not None:
        y = y + b.astype(f32)
    return y.astype(f32)


def _weight(wts: Dict[str, np.ndarray], name: str) -> np.ndarray:
    """fp32 view of a projection matrix, dequantising int8 (q, s) pairs."""
    w = wts[name]
    if isinstance(w, tuple):
        return dequantize_int8(*w)
    return w.astype(f32)


def block_forward(x: np.ndarray, c: np.ndarray, wts: Dict[str, np.ndarray], n_heads: int,
                  rows: Optional[Sequence[int]] = None, eps: float = LN_EPS,
                  intermediates: Optional[dict] = None, int8_fc2_rows: bool = False,
                  rope: Optional[tuple] = None) -> np.ndarray:
    """One AdaLN DiT block.

        mod = W_ada c + b_ada -> shift_a, scale_a, gate_a, shift_m, scale_m, gate_m
        h   = LN(x) (1 + scale_a) + shift_a
        q, k, v = h W_q^T + b_q, h W_k^T + b_k, h W_v^T + b_v   (W_qkv rows [Q | K | V])
        o   = attention(q, k, v)
        x1  = x + gate_a * (o W_o^T + b_o)
        h2  = LN(x1) (1 + scale_m) + shift_m
        u   = GELU_tanh(h2 W_1^T + b_1)
        y   = x1 + gate_m * (u W_2^T + b_2)

    Block order from [H3-memory] technique 2.  ``rows`` restricts the output
    to some token rows: keys and values still come from every token, the
    per-token stages run only on those rows (each output row depends on its
    own row and on k, v of all rows).  Projection weights may be given as
    (q_int8, scale) pairs, which are dequantised in fp32: scale [rows] per
    output channel, or [rows, cols / G] for groups of G input channels
    (quantize_int8_groups; the group-wise int8 MLP).

    ``int8_fc2_rows`` selects the row-quantised FC2 of [H3-review]'s
    speed/quality section: u is quantised per token row with the same
    symmetric rule as the weights (quantize_int8), and the MLP-down
    projection is the int8 x int8 product of linear_w8a8 with the int8
    w_down (which must then be a (q_int8, scale) pair).

    ``rope`` = (T, H, W, half_spatial) rotates q and k after their bias by
    rope_3d over the latent grid (T, H, W) (the native-256 note of
    [H3-review]); None leaves attention without positional terms.
    """
    x = x.astype(f32)
    D = x.shape[1]
    m = adaln_modulation(wts["w_ada"], wts.get("b_ada"), c)
    sel = slice(None) if rows is None else np.asarray(rows)

    h = modulate(layer_norm(x, eps), m["shift_a"], m["scale_a"])
    w_qkv = _weight(wts, "w_qkv")
    b_qkv = wts.get("b_qkv")
    bq = bk = bv = None
    if b_qkv is not None:
        bq, bk, bv = b_qkv[:D], b_qkv[D:2 * D], b_qkv[2 * D:]
    q = linear(h, w_qkv[:D], bq) if rope is not None else linear(h[sel], w_qkv[:D], bq)
    k = linear(h, w_qkv[D:2 * D], bk)
    v = linear(h, w_qkv[2 * D:], bv)
    if rope is not None:
        grid, half = tuple(rope[:3]), bool(rope[3])
        q = rope_3d(q, n_heads, grid, half)[sel]
        k = rope_3d(k, n_heads, grid, half)
    o = attention(q, k, v, n_heads)
    x1 = x[sel] + m["gate_a"] * linear(o, _weight(wts, "w_out"), wts.get("b_out"))
    h2 = modulate(layer_norm(x1, eps), m["shift_m"], m["scale_m"])
    u = gelu_tanh(linear(h2, _weight(wts, "w_up"), wts.get("b_up")))
    if int8_fc2_rows:
        q_down, s_down = wts["w_down"]
        q_u, s_u = quantize_int8(u)
        down = linear_w8a8(q_u, s_u, q_down, s_down, wts.get("b_down"))
    else:
        down = linear(u, _weight(wts, "w_down"), wts.get("b_down"))
    y = x1 + m["gate_m"] * down
    if intermediates is not None:
        intermediates.update(mod=m, h=h, q=q, k=k, v=v, o=o, x1=x1, h2=h2, u=u)
    return y.astype(f32)


def token_merge(x: np.ndarray) -> np.ndarray:
    """Tokens (2m, 2m+1) -> their mean, in fp32: [N, D] -> [N/2, D].

    [H3-review] knob list: token reduction pairs the video tokens two by two
    along rows to shorten the sequence in the middle layers.  With tokens
    laid out row by row and an even row length, tokens 2m and 2m+1 are such
    row neighbours.  The mean is the reading for the merge (the page gives
    no formula).
    """
    x = x.astype(f32)
    if x.shape[0] % 2:
        raise ValueError("token reduction needs an even token count")
    return ((x[0::2] + x[1::2]) * f32(0.5)).astype(f32)


def token_unmerge(entry: np.ndarray, merged_out: np.ndarray) -> np.ndarray:
    """Back to N tokens: each token gets its own state from before the merge
    plus the change the reduced layers made to its pair's mean,
        y[2m + j] = entry[2m + j] + (merged_out[m] - token_merge(entry)[m]),
    so reduced layers that change nothing give back ``entry`` exactly (the
    reading for the restore; the page gives no formula)."""
    delta = merged_out.astype(f32) - token_merge(entry)
    return (entry.astype(f32) + np.repeat(delta, 2, axis=0)).astype(f32)


def stack_forward(x: np.ndarray, c: np.ndarray, blocks: Sequence[Dict[str, np.ndarray]], n_heads: int,
                  n_layers: Optional[int] = None, eps: float = LN_EPS, int8_fc2_rows: bool = False,
                  rope: Optional[tuple] = None, token_reduction: Optional[tuple] = None) -> np.ndarray:
    """x_{l+1} = block_l(x_l, c) for the first ``n_layers`` blocks, one shared c.

    [H3-review] knob list: the layer count runs the first 50, 45 or 40 blocks.
    No final norm or unpatchify (they are outside the block).
    ``token_reduction`` = (first, last) runs blocks first .. last-1 on the
    merged tokens (token_merge before block first, token_unmerge after block
    last-1); None runs every block on all tokens.
    """
    L = len(blocks) if n_layers is None else n_layers
    first, last = token_reduction if token_reduction is not None else (0, 0)
    entry = None
    for l in range(L):
        if first < last and l == first:
            entry = x
            x = token_merge(x)
        x = block_forward(x, c, blocks[l], n_heads, eps=eps, int8_fc2_rows=int8_fc2_rows, rope=rope)
        if first < last and l == last - 1:
            x = token_unmerge(entry, x)
    return x
