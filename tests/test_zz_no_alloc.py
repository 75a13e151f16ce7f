"""The block forward without a caller workspace (h3k_dit_block_forward_noalloc),
for callers that cannot allocate device memory, against the block forward
with a workspace (h3k_dit_block_forward): the same kernels on the same plan,
so the outputs must be byte-identical.  Two bf16 calls in a row, the second
with a smaller input, then an fp32 block; the scratch array keeps the last
call's contents, which no kernel may read.  A config whose workspace exceeds
the static array is rejected before anything is enqueued."""
import pytest

import seeded_inputs as si
from gpu_util import config_for, dev, flush, has_gpu, upload_block

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _case(shape):
    hx, hc = si.gen_activation(shape)
    hw = si.gen_block_weights(shape, 0, bias_std=0.05)
    dw, _ = upload_block(shape, hw)
    return dev(hx), dev(hc), dw


def test_noalloc_matches_workspace_entry_point():
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    from video_diffusion_transformer_adaln_amd import runtime as R
    B.lib()
    shapes = [si.custom_shape("noalloc_a", 980, 1000, 4, 128, 2048, "bf16"),
              si.custom_shape("noalloc_b", 981, 300, 2, 128, 1024, "bf16"),
              si.C0]
    for shape in shapes:
        flush(f"no-alloc block {shape.name}")
        x, c, dw = _case(shape)
        cfg = config_for(shape)
        need = B.h3k_dit_workspace_size(cfg)
        assert need <= B.NOALLOC_SCRATCH_BYTES
        w = B.make_weights(dw)
        st = B.DitStats()
        got = torch.full_like(x, float("nan"))
        B.h3k_dit_block_forward_noalloc(cfg, w, x, c, got, stats=st)
        ws = R.alloc_workspace(cfg)
        ws.fill_(0xFF)
        ref = torch.full_like(x, float("nan"))
        B.h3k_dit_block_forward(cfg, w, x, c, ref, ws)
        torch.cuda.synchronize()
        assert st.dispatches == 8 + st.tail_splits and st.workspace_bytes == need
        assert torch.isfinite(got.float()).all()
        bits = torch.int32 if got.dtype == torch.float32 else torch.int16
        assert torch.equal(got.view(bits), ref.view(bits))


def test_noalloc_rejects_configs_beyond_the_scratch_array():
    import torch
    from video_diffusion_transformer_adaln_amd import binding as B
    B.lib()
    shape = si.C2                                   # about 1.1 GB of workspace
    cfg = config_for(shape)
    assert B.h3k_dit_workspace_size(cfg) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    out = torch.full((64,), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.H3KError) as e:
        B.h3k_dit_block_forward_noalloc(cfg, B.make_weights({}), x, x, out)
    assert e.value.status == B.H3K_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()           # nothing was enqueued
