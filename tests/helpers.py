"""Shared test helpers (no method arithmetic, no GPU calls)."""
import numpy as np

import seeded_inputs as si


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def host_values(wts):
    """name -> fp32 values of a generated weight dict."""
    return {k: v.values for k, v in wts.items()}


def tiny_problem(n_tokens=5, n_heads=2, head_dim=4, mlp=12, weight_std=0.3, bias_std=0.2,
                 seed=7, config_id=900, dtype="f32", cond_dim=None):
    """A tiny block whose modulation and biases are large enough to matter."""
    shape = si.custom_shape("tiny", config_id, n_tokens, n_heads, head_dim, mlp, dtype, cond_dim=cond_dim)
    x, c = si.gen_activation(shape, seed)
    w = si.gen_block_weights(shape, 0, seed, bias_std=bias_std)
    vals = host_values(w)
    for k in list(vals):
        if k.startswith("w_"):
            vals[k] = (vals[k] * np.float32(weight_std / si.WEIGHT_STD)).astype(np.float32)
    return shape, x.values, c.values, vals


# (case, rel-L2, bound) of every parity comparison that calls ``record``; the
# terminal summary (conftest.py) prints them, so a quiet run still shows how
# far each result is from the oracle.
PARITY = []


def record(case: str, err: float, bound: float) -> float:
    PARITY.append((case, float(err), float(bound)))
    return err
