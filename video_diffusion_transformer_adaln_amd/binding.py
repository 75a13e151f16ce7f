"""ctypes binding of libh3k.so (argument marshalling only).

Every function named ``h3k_*`` here calls the C entry point of the same name
in ``include/h3k.h``; tensors are passed as device pointers (``data_ptr()``)
and the stream defaults to torch's current HIP stream.  All computation runs
in the library's HIP kernels: there is no fallback path, and loading fails
with an error if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libh3k.so")

H3K_OK, H3K_ERR_NULL, H3K_ERR_SHAPE, H3K_ERR_DTYPE, H3K_ERR_ALIGN = 0, 1, 2, 3, 4
H3K_ERR_WORKSPACE, H3K_ERR_OVERLAP, H3K_ERR_UNSUPPORTED, H3K_ERR_HIP = 5, 6, 7, 8
STATUS_NAMES = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_ALIGN", 5: "ERR_WORKSPACE",
                6: "ERR_OVERLAP", 7: "ERR_UNSUPPORTED", 8: "ERR_HIP"}
H3K_F32, H3K_BF16, H3K_INT8 = 0, 1, 2
H3K_EPI_BIAS, H3K_EPI_GELU, H3K_EPI_GATED_RESIDUAL = 0, 1, 2
KERNEL_KINDS = ("adaln", "ln_mod", "qkv", "attention", "out_proj", "mlp_up", "mlp_down", "act_quant",
                "token_merge", "token_unmerge")
TENSOR_NAMES = ("mod", "h", "qkv", "o", "x1", "h2", "u", "uq", "us")

c_int32, c_int64, c_uint64, c_float, c_void_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                                  ctypes.c_float, ctypes.c_void_p)


class DitConfig(ctypes.Structure):
    _fields_ = [("n_tokens", c_int32), ("hidden", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
                ("mlp_hidden", c_int32), ("cond_dim", c_int32), ("ln_eps", c_float), ("act_dtype", c_int32),
                ("weight_dtype", c_int32), ("alias_activations", c_int32), ("int8_fc2_rows", c_int32),
                ("int8_mlp_group", c_int32), ("rope_frames", c_int32), ("rope_height", c_int32),
                ("rope_width", c_int32), ("rope_half_spatial", c_int32), ("token_reduction_first", c_int32),
                ("token_reduction_last", c_int32)]


class DitBlockWeights(ctypes.Structure):
    _fields_ = [("w_ada", c_void_p), ("b_ada", c_void_p),
                ("w_qkv", c_void_p), ("b_qkv", c_void_p), ("s_qkv", c_void_p),
                ("w_out", c_void_p), ("b_out", c_void_p), ("s_out", c_void_p),
                ("w_up", c_void_p), ("b_up", c_void_p), ("s_up", c_void_p),
                ("w_down", c_void_p), ("b_down", c_void_p), ("s_down", c_void_p)]


class DitStats(ctypes.Structure):
    _fields_ = [("workspace_bytes", c_uint64), ("peak_live_bytes", c_uint64), ("unaliased_bytes", c_uint64),
                ("dispatches", c_int32), ("alias_activations", c_int32), ("tail_splits", c_int32),
                ("_reserved", c_int32), ("profiler", c_void_p)]


class DitPlanInfo(ctypes.Structure):
    _fields_ = [("offset", c_uint64 * 9), ("bytes", c_uint64 * 9), ("first_step", c_int32 * 9),
                ("last_step", c_int32 * 9), ("qkv_vt_offset", c_uint64), ("vt_pitch", c_int64),
                ("workspace_bytes", c_uint64), ("peak_live_bytes", c_uint64), ("unaliased_bytes", c_uint64),
                ("alias_activations", c_int32), ("_reserved", c_int32), ("part_offset", c_uint64),
                ("part_bytes", c_uint64), ("wstage_offset", c_uint64), ("wstage_bytes", c_uint64)]


class DeviceInfo(ctypes.Structure):
    _fields_ = [("compute_units", c_int32), ("peak_clock_khz", c_int32), ("lds_bytes_per_cu", c_int32),
                ("wavefront_size", c_int32), ("hbm_bytes", c_uint64), ("arch", ctypes.c_char * 64)]


class H3KError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"h3k {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_LIB = None

# (name, restype, argtypes) of every exported entry point
_SIGNATURES = [
    ("h3k_last_error", ctypes.c_char_p, []),
    ("h3k_dit_workspace_size", c_int32, [ctypes.POINTER(DitConfig), c_int32, ctypes.POINTER(c_uint64)]),
    ("h3k_dit_plan", c_int32, [ctypes.POINTER(DitConfig), ctypes.POINTER(DitPlanInfo)]),
    ("h3k_dit_block_forward", c_int32, [ctypes.POINTER(DitConfig), ctypes.POINTER(DitBlockWeights), c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_uint64, c_void_p,
                                        ctypes.POINTER(DitStats)]),
    ("h3k_dit_stack_forward", c_int32, [ctypes.POINTER(DitConfig), ctypes.POINTER(DitBlockWeights), c_int32,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_uint64, c_void_p,
                                        ctypes.POINTER(DitStats)]),
    ("h3k_dit_block_forward_noalloc", c_int32, [ctypes.POINTER(DitConfig), ctypes.POINTER(DitBlockWeights),
                                                c_void_p, c_void_p, c_void_p, c_void_p, ctypes.POINTER(DitStats)]),
    ("h3k_quantize_weights_int8", c_int32, [c_void_p, c_int32, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
    ("h3k_quantize_weights_int8_groups", c_int32, [c_void_p, c_int32, c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                                   c_void_p]),
    ("h3k_adaln_modulation", c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p]),
    ("h3k_ln_modulate", c_int32, [c_int32, c_int32, c_int32, c_float, c_void_p, c_int64, c_void_p, c_void_p,
                                  c_void_p, c_int64, c_void_p]),
    ("h3k_linear", c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                             c_void_p, c_void_p, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                             c_void_p, c_int64, c_int64, c_void_p]),
    ("h3k_linear_int8", c_int32, [c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                  c_void_p, c_void_p, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                  c_void_p]),
    ("h3k_linear_int8_groups", c_int32, [c_int64, c_int64, c_int64, c_int32, c_void_p, c_int64, c_void_p, c_int64,
                                         c_void_p, c_void_p, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                         c_void_p]),
    ("h3k_rope_3d", c_int32, [c_int64, c_int64, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int64,
                              c_void_p]),
    ("h3k_token_merge", c_int32, [c_int32, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p]),
    ("h3k_token_unmerge", c_int32, [c_int32, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                    c_int64, c_void_p]),
    ("h3k_attention", c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_int64, c_void_p, c_int64,
                                c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p]),
    ("h3k_profiler_create", c_int32, [c_int32, ctypes.POINTER(c_void_p)]),
    ("h3k_profiler_destroy", c_int32, [c_void_p]),
    ("h3k_profiler_reset", c_int32, [c_void_p]),
    ("h3k_profiler_read", c_int32, [c_void_p, c_int32, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(c_int32)]),
    ("h3k_get_device_info", c_int32, [c_int32, ctypes.POINTER(DeviceInfo)]),
]
EXPORTED = tuple(n for n, _, _ in _SIGNATURES)


def lib() -> ctypes.CDLL:
    """Load libh3k.so (built by ``python -m video_diffusion_transformer_adaln_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m video_diffusion_transformer_adaln_amd.build` (needs ROCm hipcc)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def last_error() -> str:
    return lib().h3k_last_error().decode()


def check(status: int) -> None:
    if status != H3K_OK:
        raise H3KError(status, last_error())


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor, an int address, or None for NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(n_tokens: int, hidden: int, n_heads: int, head_dim: int, mlp_hidden: int, cond_dim: int,
                act_dtype: int, weight_dtype: Optional[int] = None, alias: bool = True,
                ln_eps: float = 1e-6, int8_fc2_rows: bool = False, int8_mlp_group: int = 0,
                rope: Optional[tuple] = None, token_reduction: Optional[tuple] = None) -> DitConfig:
    """rope = (frames, height, width, half_spatial) turns on the 3D RoPE of q and k;
    token_reduction = (first, last) runs layers first .. last-1 of a stack on merged tokens."""
    rt, rh, rw, rhalf = (0, 0, 0, 0) if rope is None else (rope[0], rope[1], rope[2], 1 if rope[3] else 0)
    tf, tl = (0, 0) if token_reduction is None else token_reduction
    return DitConfig(n_tokens, hidden, n_heads, head_dim, mlp_hidden, cond_dim, ln_eps, act_dtype,
                     act_dtype if weight_dtype is None else weight_dtype, 1 if alias else 0,
                     1 if int8_fc2_rows else 0, int8_mlp_group, rt, rh, rw, rhalf, tf, tl)


WEIGHT_FIELDS = ("w_ada", "b_ada", "w_qkv", "b_qkv", "s_qkv", "w_out", "b_out", "s_out",
                 "w_up", "b_up", "s_up", "w_down", "b_down", "s_down")


def make_weights(tensors: dict) -> DitBlockWeights:
    """Struct of device pointers from a dict of tensors (missing keys are NULL)."""
    return DitBlockWeights(*[_ptr(tensors.get(f)) for f in WEIGHT_FIELDS])


# ---------------------------------------------------------------- entry points

def h3k_dit_workspace_size(cfg: DitConfig, n_blocks: int = 1) -> int:
    out = c_uint64()
    check(lib().h3k_dit_workspace_size(ctypes.byref(cfg), n_blocks, ctypes.byref(out)))
    return out.value


def h3k_dit_plan(cfg: DitConfig) -> DitPlanInfo:
    info = DitPlanInfo()
    check(lib().h3k_dit_plan(ctypes.byref(cfg), ctypes.byref(info)))
    return info


def h3k_dit_block_forward(cfg: DitConfig, weights: DitBlockWeights, x, c, out, workspace, workspace_bytes=None,
                          stream=None, stats: Optional[DitStats] = None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    check(lib().h3k_dit_block_forward(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(c), _ptr(out),
                                      _ptr(workspace), nbytes, _stream(stream),
                                      ctypes.byref(stats) if stats is not None else None))


def h3k_dit_stack_forward(cfg: DitConfig, blocks: Sequence[DitBlockWeights], x, c, out, workspace,
                          workspace_bytes=None, stream=None, stats: Optional[DitStats] = None,
                          n_blocks: Optional[int] = None) -> None:
    arr = (DitBlockWeights * len(blocks))(*blocks)
    nb = len(blocks) if n_blocks is None else n_blocks
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    check(lib().h3k_dit_stack_forward(ctypes.byref(cfg), arr, nb, _ptr(x), _ptr(c), _ptr(out), _ptr(workspace),
                                      nbytes, _stream(stream), ctypes.byref(stats) if stats is not None else None))


NOALLOC_SCRATCH_BYTES = 128 << 20


def h3k_dit_block_forward_noalloc(cfg: DitConfig, weights: DitBlockWeights, x, c, out, stream=None,
                                  stats: Optional[DitStats] = None) -> None:
    check(lib().h3k_dit_block_forward_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(x), _ptr(c), _ptr(out),
                                              _stream(stream), ctypes.byref(stats) if stats is not None else None))


def h3k_quantize_weights_int8(w, w_dtype: int, rows: int, cols: int, q, scales, stream=None) -> None:
    check(lib().h3k_quantize_weights_int8(_ptr(w), w_dtype, rows, cols, _ptr(q), _ptr(scales), _stream(stream)))


def h3k_quantize_weights_int8_groups(w, w_dtype: int, rows: int, cols: int, group: int, q, scales,
                                     stream=None) -> None:
    check(lib().h3k_quantize_weights_int8_groups(_ptr(w), w_dtype, rows, cols, group, _ptr(q), _ptr(scales),
                                                 _stream(stream)))


def h3k_adaln_modulation(dtype: int, rows: int, cols: int, w, b, c, mod, stream=None) -> None:
    check(lib().h3k_adaln_modulation(dtype, rows, cols, _ptr(w), _ptr(b), _ptr(c), _ptr(mod), _stream(stream)))


def h3k_ln_modulate(dtype: int, n: int, D: int, eps: float, x, ldx: int, shift, scale, out, ldo: int,
                    stream=None) -> None:
    check(lib().h3k_ln_modulate(dtype, n, D, eps, _ptr(x), ldx, _ptr(shift), _ptr(scale), _ptr(out), ldo,
                                _stream(stream)))


def h3k_linear(act_dtype: int, weight_dtype: int, m: int, n: int, k: int, x, ldx: int, w, ldw: int, w_scale,
               bias, epilogue: int, residual, ldr: int, gate, y, ldy: int, yt=None, ldyt: int = 0,
               split_col: Optional[int] = None, stream=None) -> None:
    check(lib().h3k_linear(act_dtype, weight_dtype, m, n, k, _ptr(x), ldx, _ptr(w), ldw, _ptr(w_scale), _ptr(bias),
                           epilogue, _ptr(residual), ldr, _ptr(gate), _ptr(y), ldy, _ptr(yt), ldyt,
                           n if split_col is None else split_col, _stream(stream)))


def h3k_linear_int8(m: int, n: int, k: int, xq, ldx: int, x_scale, wq, ldw: int, w_scale, bias, epilogue: int,
                    residual, ldr: int, gate, y, ldy: int, stream=None) -> None:
    check(lib().h3k_linear_int8(m, n, k, _ptr(xq), ldx, _ptr(x_scale), _ptr(wq), ldw, _ptr(w_scale), _ptr(bias),
                                epilogue, _ptr(residual), ldr, _ptr(gate), _ptr(y), ldy, _stream(stream)))


def h3k_linear_int8_groups(m: int, n: int, k: int, group: int, x, ldx: int, wq, ldw: int, w_scale, bias,
                           epilogue: int, residual, ldr: int, gate, y, ldy: int, stream=None) -> None:
    check(lib().h3k_linear_int8_groups(m, n, k, group, _ptr(x), ldx, _ptr(wq), ldw, _ptr(w_scale), _ptr(bias),
                                       epilogue, _ptr(residual), ldr, _ptr(gate), _ptr(y), ldy, _stream(stream)))


def h3k_token_merge(dtype: int, n_tokens: int, D: int, x, ldx: int, xm, ldxm: int, stream=None) -> None:
    check(lib().h3k_token_merge(dtype, n_tokens, D, _ptr(x), ldx, _ptr(xm), ldxm, _stream(stream)))


def h3k_token_unmerge(dtype: int, n_tokens: int, D: int, entry, ld_entry: int, xm, ldxm: int, out, ldo: int,
                      stream=None) -> None:
    check(lib().h3k_token_unmerge(dtype, n_tokens, D, _ptr(entry), ld_entry, _ptr(xm), ldxm, _ptr(out), ldo,
                                  _stream(stream)))


def h3k_rope_3d(n_tokens: int, cols: int, head_dim: int, frames: int, height: int, width: int, half_spatial: bool,
                x, ldx: int, stream=None) -> None:
    check(lib().h3k_rope_3d(n_tokens, cols, head_dim, frames, height, width, 1 if half_spatial else 0, _ptr(x), ldx,
                            _stream(stream)))


def h3k_attention(dtype: int, n: int, n_heads: int, head_dim: int, q, ldq: int, k, ldk: int, vt, ldvt: int, o,
                  ldo: int, q_prescaled: bool = False, stream=None) -> None:
    check(lib().h3k_attention(dtype, n, n_heads, head_dim, _ptr(q), ldq, _ptr(k), ldk, _ptr(vt), ldvt, _ptr(o),
                              ldo, 1 if q_prescaled else 0, _stream(stream)))


def h3k_get_device_info(device: int = 0) -> dict:
    d = DeviceInfo()
    check(lib().h3k_get_device_info(device, ctypes.byref(d)))
    return {"compute_units": d.compute_units, "peak_clock_khz": d.peak_clock_khz,
            "lds_bytes_per_cu": d.lds_bytes_per_cu, "wavefront_size": d.wavefront_size,
            "hbm_bytes": d.hbm_bytes, "arch": d.arch.decode(errors="replace")}


class Profiler:
    """Per-kernel GPU-event timer (h3k_profiler_*)."""

    def __init__(self, capacity: int):
        h = c_void_p()
        check(lib().h3k_profiler_create(capacity, ctypes.byref(h)))
        self.handle = h

    def reset(self) -> None:
        check(lib().h3k_profiler_reset(self.handle))

    def read(self, kind: int):
        ms = ctypes.c_double()
        n = c_int32()
        check(lib().h3k_profiler_read(self.handle, kind, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def summary(self) -> dict:
        return {name: dict(zip(("total_ms", "launches"), self.read(i))) for i, name in enumerate(KERNEL_KINDS)}

    def close(self) -> None:
        if self.handle:
            check(lib().h3k_profiler_destroy(self.handle))
            self.handle = None

    def stats(self) -> DitStats:
        s = DitStats()
        s.profiler = self.handle
        return s

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
