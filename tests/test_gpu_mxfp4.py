"""MXFP4 expert weights on the GPU against the oracle, through the C ABI: the
quantised codes and scales bit for bit, the dequantised values exactly, the
routed MoE and a one-layer forward at full size within the bf16 tolerance,
and a whole denoise block, decisions shadowed."""
import dataclasses

import numpy as np
import pytest

from gpu_util import DELTA_REL, TOL, host64, needs_gpu, rel_err, run_block_stepwise, say, shadow_compare
from oracle import model as om
from oracle import quant
from oracle.inputs import prompt_kv_fn, weights_for
from synth import C1, C2, configs, gen, upload

pytestmark = [pytest.mark.gpu, needs_gpu]

# bf16 with MXFP4 experts; F = 160 leaves a padded k-group in the down operand
TINY_Q = dataclasses.replace(
    C1, name="mxfp4-tiny",
    model=configs.ModelConfig(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                              n_experts=16, top_k=2, expert_ffn=160, vocab=1024, canvas_len=32,
                              window=1024, global_layer_mask=0b10, dtype="bf16", expert_format="mxfp4"),
    batch=1, prompt_len=64, n_steps=4, seed=51)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    return _t


@pytest.fixture(scope="module")
def dg():
    import canvas_denoising_moe_amd as _dg
    _dg.lib()
    return _dg


def _bf16_bits(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("w", [TINY_Q, dataclasses.replace(C2, model=dataclasses.replace(C2.model,
                                                                                           expert_format="mxfp4"))],
                         ids=["tiny", "C2"])
def test_quantised_experts_match_oracle(torch, dg, w):
    m = w.model
    H, F, E = m.hidden, m.expert_ffn, m.n_experts
    raw = gen.layer_weights(w, 0)
    with dg.Context(m, max_batch=1, max_prompt_len=w.prompt_len) as ctx:
        say(w.name, "load")
        upload.load_context(ctx, w, layers=[0])
        for expert in (0, E // 2 + 1, E):  # E: the shared expert
            for which, name in enumerate(("gate", "up", "down")):
                K, N = (F, H) if which == 2 else (H, F)
                vals = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
                codes = torch.empty((K, N), dtype=torch.uint8, device="cuda")
                scales = torch.empty((K // 32, N), dtype=torch.uint8, device="cuda")
                say(w.name, "expert", expert, name)
                ctx.get_expert_weight(0, expert, which, vals, codes, scales)
                torch.cuda.synchronize()
                key = ("sh_" + name) if expert == E else ("w_" + name)
                src = raw[key] if expert == E else raw[key][expert]
                w64 = om.bf16_bits_to_f64(src)
                c_ref, s_ref = quant.quantize_weight(w64)
                assert np.array_equal(codes.cpu().numpy(), c_ref), (expert, name)
                assert np.array_equal(scales.cpu().numpy(), s_ref), (expert, name)
                deq = om.bf16_bits_to_f64(_bf16_bits(vals))
                assert np.array_equal(deq, quant.dequantize_weight(c_ref, s_ref)), (expert, name)
        print(f"{w.name}: codes, scales and dequantised values identical to the oracle")


# "random": distinct random experts per token; "same2": four canvases whose
# every token picks experts 3 and 9 (in its own order), so each of the two
# takes all 128 rows over several work entries and the other 14 stay empty
@pytest.mark.parametrize("batch,pattern", [(1, "random"), (4, "same2")])
def test_moe_ffn_mxfp4(torch, dg, batch, pattern):
    w = TINY_Q
    m = w.model
    M = batch * m.canvas_len
    rng = np.random.default_rng(3 if pattern == "random" else 4)
    f_bits = gen.activations(7, 2, (M, m.hidden), std=1.0, dtype="bf16")
    if pattern == "random":
        idx = np.stack([rng.choice(m.n_experts, m.top_k, replace=False) for _ in range(M)]).astype(np.int32)
    else:
        idx = np.stack([rng.permutation(np.array([3, 9])) for _ in range(M)]).astype(np.int32)
    gates = rng.dirichlet(np.ones(m.top_k), size=M).astype(np.float32)
    with dg.Context(m, max_batch=batch, max_prompt_len=w.prompt_len) as ctx:
        upload.load_context(ctx, w, layers=[0, 1])
        out = torch.empty((M, m.hidden), dtype=torch.float32, device="cuda")
        say("mxfp4 moe", pattern, "batch", batch)
        ctx.k_moe_ffn(0, batch, upload.to_device(f_bits, "bf16"), torch.from_numpy(idx).cuda(),
                      torch.from_numpy(gates).cuda(), out)
        torch.cuda.synchronize()
        got = host64(out)
    lw = weights_for(w).layer(0)
    f = om.bf16_bits_to_f64(f_bits)
    ref = np.zeros_like(got)
    for t in range(M):
        for s in range(m.top_k):
            e = idx[t, s]
            ref[t] += gates[t, s] * om.expert_ffn(f[t:t + 1], lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e],
                                                  om.bf16_round)[0]
        ref[t] += om.expert_ffn(f[t:t + 1], lw["sh_gate"], lw["sh_up"], lw["sh_down"], om.bf16_round)[0]
    e = rel_err(got, ref)
    print(f"mxfp4 routed MoE ({pattern}, {M} rows): rel err {e:.3e}")
    assert e <= TOL["bf16"]


def test_one_layer_c2_mxfp4(torch, dg):
    # the full-size layer (128 experts, F = 704: a padded k-group in down)
    w = dataclasses.replace(C2, name="C2-mxfp4", model=dataclasses.replace(C2.model, expert_format="mxfp4"))
    m = w.model
    say("C2 mxfp4 forward_hidden")
    with dg.Context(m, max_batch=1, max_prompt_len=w.prompt_len) as ctx:
        upload.load_context(ctx, w)
        M = w.batch * m.canvas_len
        x_np = gen.x_in(w)
        x_in = torch.from_numpy(x_np).cuda()
        x_out = torch.empty_like(x_in)
        trace = torch.empty((m.n_layers, M, m.top_k), dtype=torch.int32, device="cuda")
        ctx.set_trace(trace)
        ctx.forward_hidden(x_in, x_out)
        torch.cuda.synchronize()
        tr = trace.cpu().numpy()
        got = host64(x_out)
    W = weights_for(w)
    sh = om.Shadow(route_idx=[tr[l] for l in range(m.n_layers)], delta_route=DELTA_REL["bf16"])
    ref = om.forward_hidden(x_np.astype(np.float64), W, m, prompt_kv_fn(w), [w.prompt_len], shadow=sh)
    e = rel_err(got - x_np, ref - x_np)
    print(f"C2 mxfp4 one layer: residual update rel err {e:.3e}; adopted {sh.adopted}")
    assert not sh.failures, sh.failures[:5]
    assert e <= TOL["bf16"]


def test_block_mxfp4_tiny(torch, dg):
    w = TINY_Q
    with dg.Context(w.model, max_batch=1, max_prompt_len=w.prompt_len) as ctx:
        upload.load_context(ctx, w)
        tok0, lk0, passes = run_block_stepwise(torch, ctx, w)
    report, worst = shadow_compare(w, tok0, lk0, passes, DELTA_REL["bf16"], TOL["bf16"])
    print(f"mxfp4 tiny block: adopted {report}, worst conf rel err {worst:.3e}")
    assert passes[-1]["locked"].all()


def test_c3_mxfp4_sampled_layers(torch, dg):
    # the benchmark's MXFP4 configuration (30-layer stack, 4096-position prompt
    # KV): layers 0 and 29, each from the GPU's own input to it, against the
    # oracle with the dequantised experts; routing shadowed
    from synth import C3
    w = dataclasses.replace(C3, name="C3-mxfp4", model=dataclasses.replace(C3.model, expert_format="mxfp4"))
    m = w.model
    M = w.batch * m.canvas_len
    tok0, _ = gen.canvas(w)
    x_np = om.bf16_bits_to_f64(gen.embed(w)[tok0.reshape(-1)])
    with dg.Context(m, max_batch=1, max_prompt_len=w.prompt_len) as ctx:
        say("C3 mxfp4 load")
        upload.load_context(ctx, w)
        x0 = torch.from_numpy(x_np.astype(np.float32)).cuda()
        x28 = torch.empty_like(x0)
        x29 = torch.empty_like(x0)
        x1 = torch.empty_like(x0)
        trace = torch.zeros((m.n_layers, M, m.top_k), dtype=torch.int32, device="cuda")
        ctx.set_trace(trace)
        say("C3 mxfp4 layers")
        ctx.forward_layers(0, 1, x0, x1)
        ctx.forward_layers(0, 29, x0, x28)
        ctx.forward_layers(29, 1, x28, x29)
        torch.cuda.synchronize()
        tr = trace.cpu().numpy()
        ctx.set_trace(None)
        got = {0: (x_np, host64(x1)), 29: (host64(x28), host64(x29))}
    W = weights_for(w)
    kvf = prompt_kv_fn(w)
    for l, (xin, xout) in got.items():
        route = [None] * m.n_layers
        route[l] = tr[l]
        sh = om.Shadow(route_idx=route, delta_route=DELTA_REL["bf16"])
        ref = om.forward_hidden(xin, W, m, kvf, [w.prompt_len], layers=[l], shadow=sh)
        e = rel_err(xout, ref)
        print(f"C3 mxfp4 layer {l}: rel err {e:.3e}, routing adopted {sh.adopted['route']}", flush=True)
        assert not sh.failures, sh.failures[:5]
        assert e <= TOL["bf16"], (l, e)
