"""Parity at the full sizes of the 30-layer bf16 workloads, in the launch
configuration the benchmark times: one context per workload sized for its
batch and prompt length, every kernel on the library's own stream.

Two comparisons of whole passes, both with the GPU's discrete decisions
(routing, argmax, lock set) adopted by the oracle only at near-ties:

* end to end: the oracle's own 30-layer stack from the embedded canvas
  against the GPU's; the residual stream after the last layer is held to the
  bf16 tolerance, while the decision deltas and the confidence carry the
  stack's own amplification of rounding noise (the oracle's response to a
  half-ulp input perturbation, tests/golden/sensitivity_c3.json);
* anchored: every layer of every pass starts the oracle from the GPU's own
  residual stream, so each layer is held to the bf16 tolerance with one-layer
  decision deltas, and the head runs from the GPU's final state; the tokens
  and locked mask after every pass must equal the GPU's.

Workloads: the 256-slot canvas over a 4096-position prompt (the whole 8-pass
block anchored, its first pass end to end); the 131072-position prompt and
the four pre-locked canvases over 32768-position prompts with gate logits
N(0, 2^2) (first pass both ways).  Also: the LM head on sampled rows of the
262144-entry vocabulary, the routed MoE on sampled tokens, global-layer
attention over 131072 + 256 keys on sampled queries, the lock schedules
against their closed forms, and each canvas of a batched pass equal to the
same canvas run alone."""
import json
import os

import numpy as np
import pytest

from gpu_util import (DELTA_REL, TOL, anchored_pass_compare, anchored_passes_compare, host64, needs_gpu,
                      oracle_head_step, rel_err, rms, run_block_stepwise, say)
from oracle import eb
from oracle import model as om
from oracle.inputs import prompt_kv_fn, weights_for
from synth import C3, C4, C5, gen, upload

pytestmark = [pytest.mark.gpu, needs_gpu]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    return _t


@pytest.fixture(scope="module")
def dg():
    import canvas_denoising_moe_amd as _dg
    _dg.lib()
    return _dg


def _context(dg, w, extra_positions=0):
    say("load", w.name)
    ctx = dg.Context(w.model, max_batch=w.batch, max_prompt_len=w.prompt_len + extra_positions)
    upload.load_context(ctx, w)
    return ctx


def _oracle_weights(w, cache_layers=False):
    """Oracle weights whose layer provider reports progress (a 30-layer pass
    takes a while on the host)."""
    W = weights_for(w, cache_layers=cache_layers)
    inner = W.layer_fn

    def layer_fn(l):
        print(f"[oracle] {w.name} layer {l}", flush=True)
        return inner(l)
    W.layer_fn = layer_fn
    return W


def _schedule(w):
    with open(os.path.join(GOLDEN, "lock_schedules.json")) as f:
        return json.load(f)[w.name.split("-")[0]]["counts"]


def _check_schedule(w, tok0, lk0, passes):
    counts = _schedule(w)
    prev_t, prev_l = tok0, lk0
    for t, p in enumerate(passes):
        new = (p["locked"].astype(int) - prev_l.astype(int)).sum(axis=1)
        assert [int(c) for c in new] == [counts[b][t] for b in range(w.batch)], (t, new)
        assert np.array_equal(p["tokens"][prev_l == 1], prev_t[prev_l == 1])  # locked never change
        un = p["locked"] == 0
        assert np.array_equal(p["tokens"][un], tok0[un])  # the rest keep their placeholder
        prev_t, prev_l = p["tokens"], p["locked"]
    assert passes[-1]["locked"].all()


# ----------------------------------------------- 256 canvas, 4096 prompt ---

@pytest.fixture(scope="module")
def c3ctx(torch, dg):
    # room for one block commit (the last test on this context)
    ctx = _context(dg, C3, extra_positions=C3.model.canvas_len)
    yield ctx
    ctx.close()
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def c3_oracle():
    # the oracle's float64 layers of the 30-layer workload, generated once for
    # every test of this module that runs the oracle's whole stack
    return _oracle_weights(C3, cache_layers=True)


def _stack_tolerance():
    """End-to-end tolerance of the 30-layer bf16 stack: four times the
    oracle's own response, after 30 layers, to a half-ulp perturbation of its
    input (tests/golden/sensitivity_c3.json, written by the oracle alone).
    Rounding differences enter at every layer of the GPU path, and the stack
    carries them forward like that perturbation; router and vocabulary logits
    (RMS near 1 here) move by the same relative amount, so the same figure is
    the decision delta (absolute on logits, times the RMS for confidence)."""
    with open(os.path.join(GOLDEN, "sensitivity_c3.json")) as f:
        return 4.0 * json.load(f)["rel_diff_max"]


@pytest.fixture(scope="module")
def c3_block(torch, c3ctx):
    # the whole 8-pass block on the GPU, pass by pass, with every decision recorded
    say("C3 block")
    tok0, lk0, passes = run_block_stepwise(torch, c3ctx, C3)
    _check_schedule(C3, tok0, lk0, passes)
    return tok0, lk0, passes


def _end_to_end_first_pass(torch, ctx, w, W, tok0, lk0, p0, route_scale=1.0):
    """The first pass end to end: the GPU's decoder stack on the embedded
    canvas against the oracle's own stack with the GPU's routing adopted at
    near-ties; the residual stream after the last layer within the bf16
    tolerance; then the oracle's head from its own final state, the GPU's
    argmax and lock set adopted at near-ties, and the tokens and locked mask
    equal to the GPU pass's.  ``route_scale``: the router logits' RMS in units
    of the 256-slot workload's."""
    m = w.model
    B, N, L = w.batch, m.canvas_len, m.n_layers
    x_np = om.bf16_bits_to_f64(gen.embed(w)[tok0.reshape(-1)])
    x0 = torch.from_numpy(x_np.astype(np.float32)).cuda()
    trace = torch.zeros((L, B * N, m.top_k), dtype=torch.int32, device="cuda")
    say(w.name, "decoder stack")
    ctx.set_trace(trace)
    x_out = torch.empty_like(x0)
    ctx.forward_hidden(x0, x_out)
    torch.cuda.synchronize()
    ctx.set_trace(None)
    tol = _stack_tolerance()
    tr = trace.cpu().numpy()
    # the routing the stack records equals the pass's own (same kernels, same inputs)
    assert np.array_equal(tr, p0["trace"])
    sh = om.Shadow(route_idx=[tr[l] for l in range(L)], delta_route=tol * route_scale)
    ref = om.forward_hidden(x_np, W, m, prompt_kv_fn(w), [w.prompt_len] * B, shadow=sh)
    assert not sh.failures, sh.failures[:5]
    e = rel_err(host64(x_out), ref)
    t_o, l_o, pred_o, conf_o, shh = oracle_head_step(ref, W, m, tok0, lk0, [w.n_steps] * B, p0, tol, tol)
    assert not shh.failures, shh.failures[:5]
    ce = rel_err(p0["conf"], conf_o)
    ce_el = float(np.max(np.abs(p0["conf"] - conf_o) / conf_o))
    print(f"{w.name} first pass end to end: residual after {L} layers rel err {e:.3e} (tolerance "
          f"{TOL['bf16']:.0e}); routing adopted {sh.adopted['route']} (max margin {sh.max_margin['route']:.3e}, "
          f"delta {tol * route_scale:.3e}); argmax adopted {shh.adopted['pred']}, lock sets {shh.adopted['lock']}; "
          f"conf rel err {ce:.3e} (largest per position {ce_el:.3e}, stack tolerance {tol:.3e})", flush=True)
    assert e <= TOL["bf16"]
    assert ce <= tol
    assert np.array_equal(p0["tokens"], t_o)
    assert np.array_equal(p0["locked"], l_o)


def test_c3_first_pass_end_to_end(torch, c3ctx, c3_oracle, c3_block):
    w = C3
    tok0, lk0, passes = c3_block
    _end_to_end_first_pass(torch, c3ctx, w, c3_oracle, tok0, lk0, passes[0])
    assert int(passes[0]["locked"].sum()) == 32


def _route_delta(w):
    """One-layer decision delta of the routing: the survey's cap of 2e-2 times
    the router logits' RMS (weight std x sqrt(H) for unit-RMS inputs: 0.9 in
    the N(0, 0.02) workloads, 2 under gate logits N(0, 2^2)).  Four times the
    one-layer router-logit error measured on the GPU (up to 3.3e-2 at RMS 2
    behind 32768-position prompts, where P's bf16 rounding meets tens of
    thousands of keys) exceeds that cap, so the cap applies."""
    return 2e-2 * w.router_std * float(np.sqrt(w.model.hidden))


def _anchored_block(torch, ctx, w, W, tok0, lk0, passes, t0, t1, route_delta):
    kvf = prompt_kv_fn(w)
    tokens, locked = (tok0, lk0) if t0 == 0 else (passes[t0 - 1]["tokens"], passes[t0 - 1]["locked"])
    out = anchored_passes_compare(torch, ctx, w, W, kvf, t0, t1, tokens, locked, passes, route_delta,
                                  DELTA_REL["bf16"], DELTA_REL["bf16"], w.name)
    torch.cuda.empty_cache()
    return out


# The anchored block runs as two tests of four passes each, so that no single
# test stays silent for minutes.
def test_c3_block_anchored_passes_0_to_3(torch, c3ctx, c3_oracle, c3_block):
    tok0, lk0, passes = c3_block
    _anchored_block(torch, c3ctx, C3, c3_oracle, tok0, lk0, passes, 0, 4, _route_delta(C3))


def test_c3_block_anchored_passes_4_to_7(torch, c3ctx, c3_oracle, c3_block):
    w = C3
    tok0, lk0, passes = c3_block
    _anchored_block(torch, c3ctx, w, c3_oracle, tok0, lk0, passes, 4, 8, _route_delta(w))
    # every pass ended with the oracle's tokens equal to the GPU's: the final
    # canvases agree in full after the near-tie decisions are adopted
    assert passes[-1]["locked"].all()
    with open(os.path.join(GOLDEN, "agreement_c3.json")) as f:
        floor = json.load(f)
    print(f"C3 block: final canvas agreement with the shadowed oracle 100% (256 of 256). Without "
          f"shadowing, the oracle agrees with itself on {floor['final_token_agreement']:.1%} of the final tokens "
          f"when its input moves by half a bf16 ulp (tests/golden/agreement_c3.json)")


def test_c3_passes_repeat_bit_for_bit(torch, c3ctx, c3_block):
    """Run twice, compare bits: the block's first two passes run again from
    the same canvas on the same context give the same routing at every
    layer, confidence, argmax, tokens and lock mask, bit for bit (no float
    atomics anywhere; every sum runs in a fixed order)."""
    w = C3
    tok0, lk0, passes = c3_block
    t0, l0, again = run_block_stepwise(torch, c3ctx, w, steps=2)
    assert np.array_equal(t0, tok0) and np.array_equal(l0, lk0)
    for t, p in enumerate(again):
        for key in ("trace", "conf", "pred", "tokens", "locked"):
            assert np.array_equal(p[key], passes[t][key]), (t, key)
    print(f"{w.name}: passes 0 and 1 run again from the same canvas equal the first run bit for bit "
          f"(routing of all {w.model.n_layers} layers, confidence, argmax, tokens, lock mask)")


def test_c3_lm_head_sampled_rows(torch, c3ctx):
    w = C3
    m = w.model
    M = w.batch * m.canvas_len
    say("C3 LM head")
    h_bits = gen.activations(21, 1, (M, m.hidden), std=1.0, dtype="bf16")
    h = upload.to_device(h_bits, "bf16")
    logits = torch.empty((M, m.vocab), dtype=torch.float32, device="cuda")
    c3ctx.k_lm_head(w.batch, h, logits)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 77, 128, 200, 255])
    E = om.bf16_bits_to_f64(gen.embed(w))
    ref = om.lm_logits(om.bf16_bits_to_f64(h_bits[rows]), E)
    got = host64(logits[torch.from_numpy(rows).cuda()])
    e = rel_err(got, ref)
    print(f"C3 LM head: sampled rows rel err {e:.3e}")
    assert e <= TOL["bf16"]
    # the argmax of each sampled row, where the oracle's top-2 gap clears the noise
    srt = np.sort(ref, axis=1)
    clear = (srt[:, -1] - srt[:, -2]) > 1e-2 * np.sqrt(np.mean(ref ** 2))
    assert np.array_equal(np.argmax(got, axis=1)[clear], np.argmax(ref, axis=1)[clear])


def test_c3_fused_argmax_equals_row_reduction(torch, c3ctx):
    # the pass's fused LM head + argmax against the row reduction of the
    # same kernel's logits over the whole 262144-entry vocabulary
    w = C3
    m = w.model
    M = w.batch * m.canvas_len
    say("C3 fused argmax")
    h = upload.to_device(gen.activations(26, 1, (M, m.hidden), std=1.0, dtype="bf16"), "bf16")
    logits = torch.empty((M, m.vocab), dtype=torch.float32, device="cuda")
    c3ctx.k_lm_head(w.batch, h, logits)
    pred = torch.empty(M, dtype=torch.int32, device="cuda")
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    c3ctx.k_lm_argmax(w.batch, h, pred, conf)
    pred2 = torch.empty_like(pred)
    conf2 = torch.empty_like(conf)
    dg_mod = __import__("canvas_denoising_moe_amd")
    dg_mod.k_argmax_conf(logits, pred2, conf2)
    torch.cuda.synchronize()
    assert torch.equal(pred, pred2)
    c, c2 = conf.cpu().numpy().astype(np.float64), conf2.cpu().numpy().astype(np.float64)
    e = float(np.max(np.abs(c - c2) / c2))
    print(f"C3 fused argmax: pred equal, conf rel diff {e:.3e}")
    assert e <= 1e-6


def test_c3_fused_sampler_on_its_own_logits(torch, c3ctx):
    # the fused LM head's sampler statistics over the 262144-entry vocabulary
    # against the oracle's on the same kernel's logits: greedy ids exactly,
    # entropies of every row, samples of sampled rows
    w = C3
    m = w.model
    M = w.batch * m.canvas_len
    say("C3 fused sampler")
    h = upload.to_device(gen.activations(27, 1, (M, m.hidden), std=1.0, dtype="bf16"), "bf16")
    logits = torch.empty((M, m.vocab), dtype=torch.float32, device="cuda")
    pred = torch.empty(M, dtype=torch.int32, device="cuda")
    ent = torch.empty(M, dtype=torch.float32, device="cuda")
    samp = torch.empty(M, dtype=torch.int32, device="cuda")
    t, t_max, seeds = 5, eb.T_MAX, [2024]
    c3ctx.k_lm_head(w.batch, h, logits)
    c3ctx.k_lm_sample(w.batch, h, t, t_max, seeds, 1, pred, ent, samp)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert np.array_equal(pred.cpu().numpy(), np.argmax(lg, axis=1))
    tau = eb.temperature(t, t_max)
    H = eb.entropy(lg.astype(np.float64), tau)
    herr = np.abs(ent.cpu().numpy().astype(np.float64) - H)
    print(f"C3 fused sampler: entropy max |err| {herr.max():.3e} (H {H.min():.3f}..{H.max():.3f})")
    assert np.all(herr <= 2e-5 * (1.0 + H))
    rows = np.array([0, 3, 64, 100, 129, 200, 254, 255])
    noise = eb.gumbel_noise(seeds[0], 1, t, rows, m.vocab)
    score = eb.sample_scores(lg[rows].astype(np.float64), tau, noise).astype(np.float64)
    got = samp.cpu().numpy()[rows]
    mine = np.argmax(score, axis=1)
    for j in np.nonzero(mine != got)[0]:
        assert score[j, mine[j]] - score[j, got[j]] <= 4e-6 * (1.0 + abs(score[j, mine[j]])), (rows[j],)
    print(f"C3 fused sampler: {int((mine == got).sum())}/{rows.size} sampled rows identical")


def test_c3_eb_pass_matches_oracle(torch, c3ctx, c3_oracle):
    # one entropy-bounded pass of the full stack against the oracle, decisions shadowed
    w = C3
    m = w.model
    B, N, L = w.batch, m.canvas_len, m.n_layers
    say("C3 EB pass")
    tok0, lk0 = gen.canvas(w)
    tokens = torch.from_numpy(tok0).cuda()
    locked = torch.from_numpy(lk0).cuda()
    prev = torch.zeros((B, N), dtype=torch.int32, device="cuda")
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    ent = torch.empty((B, N), dtype=torch.float32, device="cuda")
    samp = torch.empty((B, N), dtype=torch.int32, device="cuda")
    pred = torch.empty((B, N), dtype=torch.int32, device="cuda")
    trace = torch.empty((L, B * N, m.top_k), dtype=torch.int32, device="cuda")
    seeds = [99]
    c3ctx.set_trace(trace)
    c3ctx.eb_step(tokens, locked, 0, eb.T_MAX, seeds, 0, prev, status, ent, samp, pred)
    torch.cuda.synchronize()
    c3ctx.set_trace(None)
    tol = _stack_tolerance()
    tr = trace.cpu().numpy()
    W = c3_oracle
    kvf = prompt_kv_fn(w)
    sh = om.Shadow(route_idx=[tr[l] for l in range(L)], delta_route=tol)
    x = W.embed_rows(tok0.reshape(-1).astype(np.int64)).copy()
    x = om.forward_hidden(x, W, m, kvf, [w.prompt_len], shadow=sh)
    hh = om.bf16_round(om.rmsnorm(x, W.norm_final(), m.rms_eps))
    lg = om.lm_logits(hh, W.embed()).reshape(B, N, -1)
    assert not sh.failures, sh.failures[:5]
    H = eb.entropy(lg[0], eb.temperature(0))
    g_ent = ent.cpu().numpy()[0].astype(np.float64)
    herr = float(np.max(np.abs(g_ent - H) / H))
    rms = float(np.sqrt(np.mean(lg ** 2)))
    esh = eb.EBShadow(sample=samp.cpu().numpy(), pred=pred.cpu().numpy(), locked_after=locked.cpu().numpy(),
                      stopped=(status.cpu().numpy() & 4) != 0, dlogit=tol * max(1.0, rms))
    state = eb.EBState(B)
    t_o, l_o, info = eb.eb_update(lg, tok0, lk0, 0, state, seeds, 0, eb.T_MAX, shadow=esh)
    print(f"C3 EB pass: entropy rel err {herr:.3e}, routing adopted {sh.adopted['route']}, "
          f"decisions adopted {esh.adopted}, locked {[len(s) for s in info['selected']]}")
    assert not esh.failures, esh.failures[:5]
    assert herr <= tol
    assert np.array_equal(tokens.cpu().numpy(), t_o)
    assert np.array_equal(locked.cpu().numpy(), l_o)


def test_c3_moe_sampled_tokens(torch, c3ctx):
    w = C3
    m = w.model
    M = w.batch * m.canvas_len
    layer = 7
    say("C3 MoE layer", layer)
    f_bits = gen.activations(22, 1, (M, m.hidden), std=1.0, dtype="bf16")
    r = gen.router_logits(23, M, m.n_experts, std=1.0)
    idx, gates = om.route(r.astype(np.float64), m.top_k)
    f = upload.to_device(f_bits, "bf16")
    out = torch.empty((M, m.hidden), dtype=torch.float32, device="cuda")
    c3ctx.k_moe_ffn(layer, w.batch, f, torch.from_numpy(idx.astype(np.int32)).cuda(),
                    torch.from_numpy(gates.astype(np.float32)).cuda(), out)
    torch.cuda.synchronize()
    toks = np.array([0, 3, 64, 129, 250])
    lw = _oracle_weights(w).layer(layer)
    f64 = om.bf16_bits_to_f64(f_bits[toks])
    ref = np.zeros((toks.size, m.hidden))
    for i in range(toks.size):
        for s in range(m.top_k):
            e = int(idx[toks[i], s])
            ref[i] += gates[toks[i], s] * om.expert_ffn(f64[i:i + 1], lw["w_gate"][e], lw["w_up"][e],
                                                         lw["w_down"][e], om.bf16_round)[0]
        ref[i] += om.expert_ffn(f64[i:i + 1], lw["sh_gate"], lw["sh_up"], lw["sh_down"], om.bf16_round)[0]
    got = host64(out)[toks]
    e = rel_err(got, ref)
    print(f"C3 MoE: sampled tokens rel err {e:.3e}")
    assert e <= TOL["bf16"]


def test_c3_block_commit_sampled_layers(torch, c3ctx, c3_oracle):
    # block continuation at full size, last on this context (it grows the
    # caches): the copied part of each cache is bit-exact, the block's K/V
    # meet the one-layer tolerance on layer 0 and the stack's end-to-end
    # tolerance deeper in
    w = C3
    m = w.model
    N, L = m.canvas_len, m.n_layers
    tok0, _ = gen.canvas(w)
    layers = [0, 5, 11, 29]
    before = {}
    for l in layers:
        n = c3ctx.prompt_kv_len(0, l)
        k = torch.empty((n, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        c3ctx.get_prompt_kv(0, l, k, v)
        before[l] = (host64(k), host64(v))
    trace = torch.zeros((L, N, m.top_k), dtype=torch.int32, device="cuda")
    c3ctx.set_trace(trace)
    say("C3 block commit")
    c3ctx.commit_block(torch.from_numpy(tok0).cuda())
    torch.cuda.synchronize()
    c3ctx.set_trace(None)
    tr = trace.cpu().numpy()
    tol = _stack_tolerance()
    W = c3_oracle
    kvf = prompt_kv_fn(w)
    sh = om.Shadow(route_idx=[tr[l] for l in range(L - 1)] + [None], delta_route=tol)
    blk = om.commit_block(tok0, W, m, kvf, [w.prompt_len], shadow=sh)
    assert not sh.failures, sh.failures[:5]
    print(f"C3 commit: routing adopted {sh.adopted}, max margin {sh.max_margin}")
    for l in layers:
        vis = w.prompt_len + N if m.is_global(l) else min(w.prompt_len + N, m.window)
        n = c3ctx.prompt_kv_len(0, l)
        assert n == vis, (l, n, vis)
        k = torch.empty((n, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        c3ctx.get_prompt_kv(0, l, k, v)
        torch.cuda.synchronize()
        gk, gv = host64(k), host64(v)
        old = vis - N
        bk, bv = before[l]
        assert np.array_equal(gk[:old], bk[len(bk) - old:]) and np.array_equal(gv[:old], bv[len(bv) - old:]), l
        ek, ev = rel_err(gk[old:], blk[l][0][0]), rel_err(gv[old:], blk[l][1][0])
        lim = TOL["bf16"] if l == 0 else tol
        print(f"C3 commit layer {l}: len {vis}, block K rel err {ek:.3e}, V {ev:.3e} (tolerance {lim:.3e})")
        assert ek <= lim and ev <= lim, (l, ek, ev)


# ------------------------------------------ 256 canvas, 131072 prompt ----

def test_c4_long_prompt_attention_and_first_pass(torch, dg):
    w = C4
    m = w.model
    N = m.canvas_len
    ctx = _context(dg, w)
    try:
        layer = next(l for l in range(m.n_layers) if m.is_global(l))
        say("C4 attention layer", layer, "prompt", w.prompt_len)
        a_bits = gen.activations(24, 1, (N, m.hidden), std=1.0, dtype="bf16")
        a = upload.to_device(a_bits, "bf16")
        q = torch.empty((1, N, m.n_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((1, N, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        o = torch.empty((1, N, m.n_heads * m.head_dim), dtype=torch.bfloat16, device="cuda")
        ctx.k_qkv(layer, 1, a, q, k, v)
        ctx.k_canvas_attn(layer, 1, q, k, v, o)
        torch.cuda.synchronize()
        rows = np.array([0, 31, 128, 255])
        qh, kh, vh = host64(q), host64(k), host64(v)
        Kp, Vp = gen.prompt_kv(w, layer, 0)
        kv = [(om.bf16_bits_to_f64(Kp), om.bf16_bits_to_f64(Vp))]
        ref = om.canvas_attention(qh[:, rows], kh, vh, kv, om.bf16_round)
        e = rel_err(host64(o)[0, rows], ref)
        print(f"C4 global attention over {w.prompt_len} + {N} keys: sampled rows rel err {e:.3e}")
        assert e <= TOL["bf16"]
        del kv, Kp, Vp

        say("C4 block")
        tok0, lk0, passes = run_block_stepwise(torch, ctx, w)
        _check_schedule(w, tok0, lk0, passes)
        W = _oracle_weights(w, cache_layers=True)
        _end_to_end_first_pass(torch, ctx, w, W, tok0, lk0, passes[0])
        anchored_pass_compare(torch, ctx, w, W, prompt_kv_fn(w), 0, tok0, lk0, passes[0], _route_delta(w),
                              DELTA_REL["bf16"], DELTA_REL["bf16"], w.name)
    finally:
        ctx.close()
        torch.cuda.empty_cache()


# --------------------------- four canvases, pre-locked, 32768 prompts ----

def test_c5_batch_first_pass_and_independence(torch, dg):
    w = C5
    m = w.model
    N = m.canvas_len
    ctx = _context(dg, w)
    try:
        say("C5 block, batch", w.batch)
        tok0, lk0, passes = run_block_stepwise(torch, ctx, w)
        _check_schedule(w, tok0, lk0, passes)
        # the first pass against the oracle, with the workload's own router
        # (gate logits N(0, 2^2): twice the logit RMS of the other workloads,
        # so the routing deltas double with it)
        W = _oracle_weights(w, cache_layers=True)
        _end_to_end_first_pass(torch, ctx, w, W, tok0, lk0, passes[0], route_scale=2.0)
        anchored_pass_compare(torch, ctx, w, W, prompt_kv_fn(w), 0, tok0, lk0, passes[0],
                              _route_delta(w), DELTA_REL["bf16"], DELTA_REL["bf16"], w.name)
        del W
        # each canvas of the batched first pass equals that canvas run alone
        for b in range(w.batch):
            say("C5 canvas", b, "alone")
            ks, vs = upload.prompt_kv_to_device(w, b)
            ctx.load_prompt_kv(0, w.prompt_len, ks, vs)
            del ks, vs
            tokens = torch.from_numpy(tok0[b:b + 1].copy()).cuda()
            locked = torch.from_numpy(lk0[b:b + 1].copy()).cuda()
            conf = torch.empty((1, N), dtype=torch.float32, device="cuda")
            pred = torch.empty((1, N), dtype=torch.int32, device="cuda")
            ctx.denoise_step(tokens, locked, [w.n_steps], conf, pred)
            torch.cuda.synchronize()
            # every kernel computes a canvas's rows from that canvas alone, in
            # an order fixed by the canvas itself: the results are identical
            p0 = passes[0]
            assert np.array_equal(conf.cpu().numpy()[0], p0["conf"][b]), b
            assert np.array_equal(pred.cpu().numpy()[0], p0["pred"][b]), b
            assert np.array_equal(tokens.cpu().numpy()[0], p0["tokens"][b]), b
            assert np.array_equal(locked.cpu().numpy()[0], p0["locked"][b]), b
            print(f"C5 canvas {b}: the batched pass and the canvas alone agree bit for bit")
    finally:
        ctx.close()
        torch.cuda.empty_cache()
