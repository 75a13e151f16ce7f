"""Helpers for GPU tests: upload seeded inputs, run the library, sample rows.

Inputs come from ``seeded_inputs`` on the host, so the oracle and the GPU see
the same values; nothing here computes any part of the block.
"""
import sys

import numpy as np

import seeded_inputs as si

ROWS_PER_SAMPLE = 48


def flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def dev(ht):
    from video_diffusion_transformer_adaln_amd import runtime as R
    return R.upload(ht.storage, ht.dtype)


def act_code(shape):
    from video_diffusion_transformer_adaln_amd import binding as B
    return B.H3K_F32 if shape.dtype == "f32" else B.H3K_BF16


def config_for(shape, alias=True, int8_fc2_rows=False, int8_mlp_group=0, rope=None):
    from video_diffusion_transformer_adaln_amd import binding as B
    act = act_code(shape)
    return B.make_config(shape.n_tokens, shape.hidden, shape.n_heads, shape.head_dim, shape.mlp_hidden,
                         shape.cond_dim, act, B.H3K_INT8 if shape.int8_weights else act, alias,
                         int8_fc2_rows=int8_fc2_rows, int8_mlp_group=int8_mlp_group, rope=rope)


def sample_rows(n, count=ROWS_PER_SAMPLE, seed=5):
    """Deterministic rows: the first few, the ragged tail and a random middle."""
    rng = np.random.default_rng(seed)
    head = list(range(min(n, 8)))
    tail = list(range(max(0, n - 8), n))
    mid = rng.choice(n, size=min(n, max(0, count - 16)), replace=False).tolist() if n > 16 else []
    return np.array(sorted(set(head + tail + mid)), dtype=np.int64)


def to_np(t):
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def upload_block(shape, hw, mlp_group=0):
    """Device tensors of one block; int8 matrices are quantised on the GPU.

    Returns (device dict, oracle weight dict).  For int8 the oracle gets its
    own quantisation of the same fp32 matrices; tests assert bit-equality of
    the two quantisations separately.  mlp_group > 0 quantises w_up and
    w_down in groups of that many input channels."""
    import oracle
    from video_diffusion_transformer_adaln_amd import runtime as R
    d = {}
    ow = {}
    for name, ht in hw.items():
        if shape.int8_weights and name in si.MATRIX_NAMES:
            w32 = R.upload(ht.storage, "f32")
            grouped = mlp_group > 0 and name in ("w_up", "w_down")
            q, s = R.quantize_int8_groups(w32, mlp_group) if grouped else R.quantize_int8(w32)
            del w32
            d[name] = q
            d["s_" + name[2:]] = s
            ow[name] = oracle.quantize_int8_groups(ht.values, mlp_group) if grouped else oracle.quantize_int8(ht.values)
        else:
            d[name] = dev(ht)
            ow[name] = ht.values
    return d, ow


def tail_split_ways(tiles, kt, cus, cap_tiles):
    """The block's k-split rule for a bf16 GEMM of `tiles` 256x256 tiles and `kt`
    k-tiles of 64 on `cus` compute units, restated for the tests: the last
    tiles % cus tiles split S ways when they would leave at least half the
    CUs idle, S <= 8, >= 4 k-tiles per split, tail * S <= min(cus, cap), and
    only if each split sheds at least 2048 of k, (1 - 1/S) 64 kt >= 2048."""
    if tiles < 1 or cus < 1:
        return 0
    tail = tiles % cus
    if tail == 0 or 2 * tail > cus:
        return 0
    s = min(8, kt // 4, min(cap_tiles, cus) // tail)
    return s if s >= 2 and (s - 1) * kt >= 32 * s else 0


def attn_split_ways(blocks, tiles, slots, cap_units):
    """The block's key-split rule for the bf16 attention (head_dim 128), restated
    for the tests: `blocks` workgroups, `slots` resident at once, `tiles` key
    tiles of 32; the last round splits S ways when it would leave at least half
    the slots idle, S <= 8, >= 8 tiles per range, tail * S <= min(slots, cap),
    and only if each range sheds at least 2048 keys, (1 - 1/S) 32 tiles >= 2048."""
    if blocks < 1 or slots < 1:
        return 0
    tail = blocks % slots
    if tail == 0 or 2 * tail > slots:
        return 0
    s = min(8, tiles // 8, min(cap_units, slots) // tail)
    return s if s >= 2 and (s - 1) * tiles >= 64 * s else 0


def expected_tail_splits(n_tokens, hidden, mlp, part_bytes, cus, n_heads=None, head_dim=128):
    """How many of a bf16 block's kernels split their last wave: the out / up /
    down GEMMs and (head_dim 128) the attention."""
    tm = (n_tokens + 255) // 256
    cap = part_bytes // (256 * 256 * 4)
    n = sum(tail_split_ways(tm * ((nn + 255) // 256), k // 64, cus, cap) > 0
            for nn, k in ((hidden, hidden), (mlp, hidden), (hidden, mlp)))
    if head_dim == 128:
        # 8-wave workgroups when their last round can split, else the 4-wave
        # shape (short sequences, few workgroups) with its own split, if any
        heads = hidden // head_dim if n_heads is None else n_heads
        tiles = (n_tokens + 31) // 32
        unit = lambda nw: nw * 32 * 130 * 4
        s8 = attn_split_ways((n_tokens + 255) // 256 * heads, tiles, cus, part_bytes // unit(8))
        four = (n_tokens + 255) // 256 * heads < 1024 and n_tokens <= 8192
        s4 = attn_split_ways((n_tokens + 127) // 128 * heads, tiles, 2 * cus, part_bytes // unit(4)) if four else 0
        n += (s8 > 0 or s4 > 0) and part_bytes > 0
    return n


def device_cus():
    from video_diffusion_transformer_adaln_amd import binding as B
    return B.h3k_get_device_info(0)["compute_units"]
