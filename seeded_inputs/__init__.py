"""Seeded synthetic inputs for the AdaLN DiT block.

This module is shared by the CPU oracle (``oracle/``) and by the GPU side
(tests, ``bench.py``).  It holds none of the block's arithmetic: it only
draws Gaussian tensors of the workload shapes and rounds them to the storage
type the workload uses (bf16 round-to-nearest-even, done with integer ops).
Quantisation to int8 is part of the method and is NOT done here; each side
quantises the fp32 weights itself.

Shapes follow the video-latent geometries the pages describe: a 512x512,
22-frame render and the default 864x480, 56-frame render (h3-metal review,
intro and "fox" profiling example), reduced 16x spatially and 4x temporally
to 6x32x32 = 6144 and 14x54x30 = 22680 latent tokens.

Recipe: x, c ~ N(0, 1); every weight matrix ~ N(0, 0.02^2); biases zero
unless ``bias_std`` asks otherwise.  One numpy PCG64 stream per tensor,
seeded by SeedSequence([seed, config_id, block, tensor_id]).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BASE_SEED = 42
WEIGHT_STD = 0.02

# tensor ids inside a block's seed sequence
TENSOR_IDS = {
    "x": 0, "c": 1,
    "w_ada": 2, "b_ada": 3,
    "w_qkv": 4, "b_qkv": 5,
    "w_out": 6, "b_out": 7,
    "w_up": 8, "b_up": 9,
    "w_down": 10, "b_down": 11,
}
MATRIX_NAMES = ("w_qkv", "w_out", "w_up", "w_down")


@dataclasses.dataclass(frozen=True)
class DitShape:
    """Sizes of one DiT block: N tokens, D hidden, H heads x d, F MLP width, C cond."""
    name: str
    config_id: int
    n_tokens: int
    hidden: int
    n_heads: int
    head_dim: int
    mlp_hidden: int
    cond_dim: int
    dtype: str            # "f32" or "bf16": storage type of x, c, weights, biases
    int8_weights: bool = False
    n_blocks: int = 1

    def __post_init__(self):
        assert self.hidden == self.n_heads * self.head_dim

    def weight_shapes(self) -> Dict[str, tuple]:
        D, F, C = self.hidden, self.mlp_hidden, self.cond_dim
        return {
            "w_ada": (6 * D, C), "b_ada": (6 * D,),
            "w_qkv": (3 * D, D), "b_qkv": (3 * D,),
            "w_out": (D, D), "b_out": (D,),
            "w_up": (F, D), "b_up": (F,),
            "w_down": (D, F), "b_down": (D,),
        }

    def replace(self, **kw) -> "DitShape":
        return dataclasses.replace(self, **kw)


# The five workloads: a small fp32 block, the 512x512x22-frame block, the
# 864x480x56-frame block, the 50-block denoising step at that shape and the
# same block with int8 weights.
C0 = DitShape("c0_block_n512_d256_f32", 0, 512, 256, 4, 64, 1024, 256, "f32")
C1 = DitShape("c1_block_n6144_d3072_bf16", 1, 6144, 3072, 24, 128, 12288, 3072, "bf16")
C2 = DitShape("c2_block_n22680_d5120_bf16", 2, 22680, 5120, 40, 128, 13824, 5120, "bf16")
C3 = C2.replace(name="c3_step50_n22680_d5120_bf16", config_id=3, n_blocks=50)
C4 = C2.replace(name="c4_block_n22680_d5120_int8w", config_id=4, int8_weights=True)
CONFIGS = {s.config_id: s for s in (C0, C1, C2, C3, C4)}


def _rng(seed: int, config_id: int, block: int, tensor: str) -> np.random.Generator:
    ss = np.random.SeedSequence([seed, config_id, block, TENSOR_IDS[tensor]])
    return np.random.Generator(np.random.PCG64(ss))


def normal_f32(shape, std: float, seed: int, config_id: int, block: int, tensor: str) -> np.ndarray:
    """fp32 N(0, std^2) draw from the tensor's own stream."""
    out = np.empty(shape, dtype=np.float32)
    _rng(seed, config_id, block, tensor).standard_normal(out=out, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16-bit patterns.

    Storage conversion only.  NaN is not expected in generated data.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class HostTensor:
    """A generated tensor: fp32 values (exactly representable in ``dtype``)
    plus the raw storage (fp32 array, or uint16 bf16 patterns)."""
    values: np.ndarray
    storage: np.ndarray
    dtype: str


def _finish(a: np.ndarray, dtype: str) -> HostTensor:
    if dtype == "bf16":
        bits = bf16_bits(a)
        return HostTensor(bf16_to_f32(bits), bits, "bf16")
    if dtype == "f32":
        return HostTensor(a, a, "f32")
    raise ValueError(dtype)


def gen_activation(shape: DitShape, seed: int = BASE_SEED):
    """x [N, D] and c [C], both N(0, 1) in the workload's storage dtype."""
    x = normal_f32((shape.n_tokens, shape.hidden), 1.0, seed, shape.config_id, 0, "x")
    c = normal_f32((shape.cond_dim,), 1.0, seed, shape.config_id, 0, "c")
    return _finish(x, shape.dtype), _finish(c, shape.dtype)


def gen_block_weights(shape: DitShape, block: int = 0, seed: int = BASE_SEED,
                      bias_std: float = 0.0, only: Optional[tuple] = None) -> Dict[str, HostTensor]:
    """All weights of one block.

    Matrices ~ N(0, 0.02^2), biases zero (or N(0, bias_std^2) when asked).
    With ``int8_weights`` the four projection matrices are returned in fp32
    (their quantisation is the method's job); the AdaLN matrix and all biases
    use the activation dtype.
    """
    out = {}
    for name, shp in shape.weight_shapes().items():
        if only is not None and name not in only:
            continue
        is_bias = name.startswith("b_")
        if is_bias:
            if bias_std == 0.0:
                a = np.zeros(shp, dtype=np.float32)
            else:
                a = normal_f32(shp, bias_std, seed, shape.config_id, block, name)
        else:
            a = normal_f32(shp, WEIGHT_STD, seed, shape.config_id, block, name)
        if shape.int8_weights and name in MATRIX_NAMES:
            out[name] = HostTensor(a, a, "f32")
        else:
            out[name] = _finish(a, shape.dtype)
    return out


def block_weight_bf16_bits(shape: DitShape, block: int, name: str, seed: int = BASE_SEED) -> np.ndarray:
    """The bf16 storage of one weight matrix of a block (``gen_block_weights(shape,
    block, seed)[name].storage`` without the fp32 copy), for uploading many
    blocks quickly.  Only for bf16 workloads."""
    if shape.dtype != "bf16" or name not in shape.weight_shapes() or name.startswith("b_"):
        raise ValueError(f"{name} of {shape.name}: bf16 weight matrices only")
    return bf16_bits(normal_f32(shape.weight_shapes()[name], WEIGHT_STD, seed, shape.config_id, block, name))


def custom_shape(name: str, config_id: int, n_tokens: int, n_heads: int, head_dim: int,
                 mlp_hidden: int, dtype: str, int8_weights: bool = False, n_blocks: int = 1,
                 cond_dim: Optional[int] = None) -> DitShape:
    """A test shape outside the five workloads (ragged sizes, tiny cases)."""
    hidden = n_heads * head_dim
    return DitShape(name, config_id, n_tokens, hidden, n_heads, head_dim, mlp_hidden,
                    hidden if cond_dim is None else cond_dim, dtype, int8_weights, n_blocks)


def torch_device_normal(shape, std: float, seed: int, tag: int, device, dtype):
    """Throughput-run inputs drawn on the device with torch's seeded generator.

    Same distribution and storage rounding as the numpy streams, different
    numbers; used only where no oracle value is compared (timing runs and
    GPU-side properties such as aliasing on/off or the layer-prefix check).
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tag)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)
