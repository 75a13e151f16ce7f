"""Pure-Python brute force of the AdaLN DiT block for tiny inputs.

Written independently of ``oracle/`` (plain loops over Python floats, i.e.
fp64, with ``math``), to pin the oracle's composition: a dropped term, a
wrong chunk, sign or index, or a transposed operand in the oracle makes the
two disagree.  Use only for a few tokens and a hidden size of a few dozen.
"""
import math
import struct


def _mat(a):
    return [[float(v) for v in row] for row in a]


def _vec(a):
    return [float(v) for v in a]


def matvec(w, x):
    return [sum(w[o][k] * x[k] for k in range(len(x))) for o in range(len(w))]


def dense(rows, w, b):
    """Every row r: out[r][o] = sum_k rows[r][k] * w[o][k] + b[o]."""
    out = []
    for r in rows:
        out.append([sum(r[k] * w[o][k] for k in range(len(r))) + (b[o] if b else 0.0)
                    for o in range(len(w))])
    return out


def layernorm_row(z, eps):
    n = len(z)
    mean = sum(z) / n
    var = sum((v - mean) ** 2 for v in z) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(v - mean) * inv for v in z]


def gelu_tanh_scalar(z):
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def attention_naive(q, k, v, n_heads):
    """Materialises every score S[i][j] for every head; fp64 exp."""
    n_q, D = len(q), len(q[0])
    n_k = len(k)
    d = D // n_heads
    out = [[0.0] * D for _ in range(n_q)]
    for h in range(n_heads):
        c0 = h * d
        for i in range(n_q):
            s = [sum(q[i][c0 + t] * k[j][c0 + t] for t in range(d)) / math.sqrt(d) for j in range(n_k)]
            mx = max(s)
            e = [math.exp(v_ - mx) for v_ in s]
            tot = sum(e)
            for t in range(d):
                out[i][c0 + t] = sum(e[j] * v[j][c0 + t] for j in range(n_k)) / tot
    return out


def rope_rows(rows, n_heads, positions, split):
    """Rotary embedding on nested lists: for every token, head and axis a, the
    pair (2i, 2i+1) of the axis's slice (widths ``split`` = (d_t, d_h, d_w), in
    that order inside the head) turns by positions[token][a] * 10000^(-2i/d_a)."""
    out = []
    for row, pos in zip(rows, positions):
        d = len(row) // n_heads
        new = list(row)
        for hd in range(n_heads):
            c0 = hd * d
            for a, da in enumerate(split):
                for i in range(da // 2):
                    phi = pos[a] * 10000.0 ** (-2.0 * i / da)
                    x, y = row[c0 + 2 * i], row[c0 + 2 * i + 1]
                    new[c0 + 2 * i] = x * math.cos(phi) - y * math.sin(phi)
                    new[c0 + 2 * i + 1] = x * math.sin(phi) + y * math.cos(phi)
                c0 += da
        out.append(new)
    return out


def block(x, c, w, n_heads, eps=1e-6, rope=None):
    """x: N x D nested lists, c: C list, w: dict of nested lists (biases may be None).
    rope = (positions, split) rotates q and k by rope_rows."""
    x = _mat(x)
    c = _vec(c)
    D = len(x[0])
    W = {k_: (_mat(v_) if v_ is not None and hasattr(v_[0], "__len__") else (_vec(v_) if v_ is not None else None))
         for k_, v_ in w.items()}
    mod = matvec(W["w_ada"], c)
    if W.get("b_ada") is not None:
        mod = [m + b for m, b in zip(mod, W["b_ada"])]
    shift_a, scale_a, gate_a = mod[0:D], mod[D:2 * D], mod[2 * D:3 * D]
    shift_m, scale_m, gate_m = mod[3 * D:4 * D], mod[4 * D:5 * D], mod[5 * D:6 * D]

    h = []
    for row in x:
        n = layernorm_row(row, eps)
        h.append([n[i] * (1.0 + scale_a[i]) + shift_a[i] for i in range(D)])
    qkv = dense(h, W["w_qkv"], W.get("b_qkv"))
    q = [r[0:D] for r in qkv]
    k = [r[D:2 * D] for r in qkv]
    v = [r[2 * D:3 * D] for r in qkv]
    if rope is not None:
        q = rope_rows(q, n_heads, *rope)
        k = rope_rows(k, n_heads, *rope)
    o = attention_naive(q, k, v, n_heads)
    proj = dense(o, W["w_out"], W.get("b_out"))
    x1 = [[x[t][i] + gate_a[i] * proj[t][i] for i in range(D)] for t in range(len(x))]
    h2 = []
    for row in x1:
        n = layernorm_row(row, eps)
        h2.append([n[i] * (1.0 + scale_m[i]) + shift_m[i] for i in range(D)])
    u = [[gelu_tanh_scalar(z) for z in r] for r in dense(h2, W["w_up"], W.get("b_up"))]
    down = dense(u, W["w_down"], W.get("b_down"))
    return [[x1[t][i] + gate_m[i] * down[t][i] for i in range(D)] for t in range(len(x))]


def fp32(v):
    """Round a Python float to the nearest fp32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def quantize_row_int8(row):
    """Symmetric int8 of one row, with fp32 arithmetic emulated exactly.

    The division of two fp32 values is done in fp64 and rounded once to fp32;
    for division that double rounding cannot change the result (53 >= 2*24+2).
    ``round`` in Python 3 rounds half to even.
    """
    row = [fp32(v) for v in row]
    mx = max(abs(v) for v in row)
    s = fp32(mx / 127.0)
    if s == 0.0:
        return [0] * len(row), 0.0
    q = []
    for v in row:
        t = fp32(v / s)
        qi = int(round(t))
        q.append(max(-127, min(127, qi)))
    return q, s


def quantize_groups_int8(row, group):
    """Group-wise symmetric int8 of one row: each block of ``group`` consecutive
    values is quantised by quantize_row_int8 on its own; returns the row's q
    and its list of group scales."""
    q, s = [], []
    for g in range(0, len(row), group):
        qg, sg = quantize_row_int8(row[g:g + group])
        q.extend(qg)
        s.append(sg)
    return q, s


def fc2_int8_rows(u, q_w, s_w, b):
    """int8 x int8 MLP-down on nested lists: each row of u quantised by
    quantize_row_int8, then y[t][o] = s_u[t] s_w[o] sum_k q_u[t][k] q_w[o][k] + b[o]
    with the integer sum exact and the scaling in Python floats."""
    out = []
    for row in u:
        qu, su = quantize_row_int8(row)
        r = []
        for o in range(len(q_w)):
            acc = sum(a * w for a, w in zip(qu, q_w[o]))      # exact integer
            r.append(su * s_w[o] * acc + (b[o] if b is not None else 0.0))
        out.append(r)
    return out


def token_merge_rows(x):
    """Pairs of consecutive rows -> their mean (nested lists)."""
    return [[0.5 * (a + b) for a, b in zip(x[2 * m], x[2 * m + 1])] for m in range(len(x) // 2)]


def reduced_stack(x, c, blocks, n_heads, first, last, eps=1e-6):
    """Blocks first .. last-1 on the merged rows; on exit each row gets its own
    entry state plus its pair's change."""
    entry = None
    for l, w in enumerate(blocks):
        if l == first:
            entry = x
            x = token_merge_rows(x)
        x = block(x, c, w, n_heads, eps)
        if l == last - 1:
            merged_in = token_merge_rows(entry)
            x = [[e + (x[r // 2][i] - merged_in[r // 2][i]) for i, e in enumerate(entry[r])]
                 for r in range(len(entry))]
    return x
