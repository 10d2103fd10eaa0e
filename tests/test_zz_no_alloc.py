"""The allocation-free LM head entry point (dg_k_lm_argmax_noalloc) against
dg_k_lm_argmax: the same kernels with their partials in the library's static
scratch instead of the context's workspace, so the two agree bit for bit.
Two calls in a row, the second with a smaller batch, then the size limit."""
import dataclasses

import numpy as np
import pytest

from gpu_util import needs_gpu, say
from synth import C1, C3, gen, upload

pytestmark = [pytest.mark.gpu, needs_gpu]

# a small bf16 model whose LM head takes the fused path (H % 128 == 0, V % 16 == 0)
SMALL = dataclasses.replace(C1.model, dtype="bf16", hidden=256, vocab=4096)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    return _t


@pytest.fixture(scope="module")
def dg():
    import canvas_denoising_moe_amd as _dg
    _dg.lib()
    return _dg


def test_noalloc_lm_head_equals_the_workspace_path(torch, dg):
    m = SMALL
    N = m.canvas_len
    w = dataclasses.replace(C1, model=m, batch=4, name="small-bf16")
    with dg.Context(m, max_batch=4, max_prompt_len=w.prompt_len) as ctx:
        e = upload.to_device(gen.embed(w), "bf16")
        nf = upload.to_device(gen.norm_final(w), "bf16")
        ctx.set_embedding(e, nf)
        torch.cuda.synchronize()
        for call, batch in enumerate((4, 1)):
            M = batch * N
            say("no-alloc LM head, call", call, "batch", batch)
            h = upload.to_device(gen.activations(40 + call, 1, (M, m.hidden), std=1.0, dtype="bf16"), "bf16")
            p0 = torch.empty(M, dtype=torch.int32, device="cuda")
            c0 = torch.empty(M, dtype=torch.float32, device="cuda")
            p1 = torch.full((M,), -7, dtype=torch.int32, device="cuda")
            c1 = torch.full((M,), -7.0, dtype=torch.float32, device="cuda")
            ctx.k_lm_argmax(batch, h, p0, c0)
            ctx.k_lm_argmax_noalloc(batch, h, p1, c1)
            torch.cuda.synchronize()
            assert torch.equal(p0, p1), call
            assert torch.equal(c0, c1), call
            assert int(p1.min()) >= 0 and int(p1.max()) < m.vocab
            print(f"call {call} (batch {batch}): pred and conf equal to dg_k_lm_argmax bit for bit")


def test_noalloc_lm_head_rejects_batches_beyond_the_scratch(torch, dg):
    # at V = 262144 the scratch holds 1024 rows: 4 canvases of 256, not 5;
    # the size is checked before anything else, so no weights are needed
    m = C3.model
    with dg.Context(m, max_batch=5, max_prompt_len=0) as ctx:
        h = torch.zeros((5 * m.canvas_len, m.hidden), dtype=torch.bfloat16, device="cuda")
        pred = torch.zeros(5 * m.canvas_len, dtype=torch.int32, device="cuda")
        conf = torch.zeros(5 * m.canvas_len, dtype=torch.float32, device="cuda")
        with pytest.raises(dg.DGError) as ei:
            ctx.k_lm_argmax_noalloc(5, h, pred, conf)
        assert ei.value.status == dg.DG_EINVAL and "static scratch" in str(ei.value)
        # within the limit the call gets as far as the state check (no embedding)
        with pytest.raises(dg.DGError) as ei:
            ctx.k_lm_argmax_noalloc(4, h[: 4 * m.canvas_len], pred[: 4 * m.canvas_len], conf[: 4 * m.canvas_len])
        assert ei.value.status == dg.DG_ESTATE
