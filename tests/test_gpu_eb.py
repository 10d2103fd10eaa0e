"""Entropy-bounded denoising on the GPU against the oracle, through the C ABI:
the counter-based Gumbel noise, the per-row sampler statistics (stored fp32
logits and the fused bf16 LM head), the lock step bit for bit on identical
inputs, and whole EB blocks on small models with the shadowed comparison of
the discrete decisions."""
import dataclasses

import numpy as np
import pytest

from gpu_util import DELTA_REL, needs_gpu, say
from oracle import eb
from oracle import model as om
from oracle.inputs import prompt_kv_fn, weights_for
from synth import C1, configs, gen, upload

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    return _t


@pytest.fixture(scope="module")
def dg():
    import canvas_denoising_moe_amd as _dg
    _dg.lib()
    return _dg


# noise: GPU log2-based against the oracle's float64 logs, both rounded to float32
def _noise_tol(g):
    return 2e-6 * (1.0 + np.abs(g))


@pytest.mark.parametrize("V,N,B,t,block", [(1000, 32, 2, 5, 3), (262144, 4, 1, 47, 0), (64, 16, 3, 0, 7)])
def test_noise_matches_oracle(torch, dg, V, N, B, t, block):
    seeds = [11 + 1000 * b for b in range(B)]
    out = torch.empty((B * N, V), dtype=torch.float32, device="cuda")
    say("noise", V, N, B, t, block)
    dg.k_eb_noise(B * N, V, N, t, seeds, block, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(B, N, V).astype(np.float64)
    for b in range(B):
        ref = eb.gumbel_noise(seeds[b], block, t, np.arange(N), V).astype(np.float64)
        err = np.abs(got[b] - ref)
        print(f"noise V={V} canvas {b}: max |err| {err.max():.3e}")
        assert np.all(err <= _noise_tol(ref)), (b, float(err.max()))


def _logits(kind, rows, V, rng):
    if kind == "normal":
        return rng.normal(0, 1, size=(rows, V)).astype(np.float32)
    if kind == "peaked":  # low entropies
        x = rng.normal(0, 1, size=(rows, V)).astype(np.float32)
        x[np.arange(rows), rng.integers(0, V, size=rows)] += rng.uniform(5, 40, size=rows).astype(np.float32)
        return x
    if kind == "ties":  # integer logits: equal maxima, argmax to the lower id
        return rng.integers(-3, 4, size=(rows, V)).astype(np.float32)
    raise ValueError(kind)


def _check_rows(logits, N, t, t_max, seeds, block, pred, ent, samp, tag):
    rows, V = logits.shape
    tau = eb.temperature(t, t_max)
    l64 = logits.astype(np.float64)
    assert np.array_equal(pred, np.argmax(logits, axis=1)), tag
    H = eb.entropy(l64, tau)
    herr = np.abs(ent - H)
    assert np.all(herr <= 2e-5 * (1.0 + H)), (tag, float(herr.max()))
    adopted = 0
    for b in range(rows // N):
        noise = eb.gumbel_noise(seeds[b], block, t, np.arange(N), V)
        score = eb.sample_scores(l64[b * N:(b + 1) * N], tau, noise).astype(np.float64)
        mine = np.argmax(score, axis=1)
        for i in np.nonzero(mine != samp[b * N:(b + 1) * N])[0]:
            g = samp[b * N + i]
            margin = score[i, mine[i]] - score[i, g]
            assert margin <= 4e-6 * (1.0 + abs(score[i, mine[i]])), (tag, b, i, margin)
            adopted += 1
    print(f"{tag}: entropy max |err| {herr.max():.3e}, samples within noise rounding {adopted}")


@pytest.mark.parametrize("kind,V,N,B,t,t_max", [
    ("normal", 1024, 32, 2, 0, 48), ("peaked", 1000, 32, 2, 47, 48), ("ties", 1024, 16, 1, 3, 8),
    ("normal", 262144, 16, 1, 10, 48), ("peaked", 4096, 64, 4, 0, 1)])
def test_eb_rows_match_oracle(torch, dg, kind, V, N, B, t, t_max):
    rng = np.random.default_rng(V + N + t)
    lg = _logits(kind, B * N, V, rng)
    seeds = [int(x) for x in rng.integers(0, 2 ** 32, size=B)]
    dlg = torch.from_numpy(lg).cuda()
    pred = torch.empty(B * N, dtype=torch.int32, device="cuda")
    ent = torch.empty(B * N, dtype=torch.float32, device="cuda")
    samp = torch.empty(B * N, dtype=torch.int32, device="cuda")
    say("eb rows", kind, V, N, B, t, t_max)
    dg.k_eb_rows(dlg, N, t, t_max, seeds, 9, pred, ent, samp)
    torch.cuda.synchronize()
    _check_rows(lg, N, t, t_max, seeds, 9, pred.cpu().numpy(), ent.cpu().numpy().astype(np.float64),
                samp.cpu().numpy(), f"rows {kind} V={V}")


# --------------------------------------------------------------------------
# the lock step, bit for bit on identical inputs
# --------------------------------------------------------------------------

def _select_case(rng, B, N, kind):
    """Entropies, samples, greedy tokens, tokens, locks and state of B canvases."""
    H = np.zeros((B, N), dtype=np.float32)
    for b in range(B):
        k = (kind + b) % 5
        if k == 0:    # vague
            H[b] = rng.uniform(0.2, 8.0, size=N)
        elif k == 1:  # mostly confident, a spread at the bound
            H[b] = rng.exponential(0.01, size=N)
        elif k == 2:  # ties on a coarse grid (lock order by position)
            H[b] = rng.integers(0, 8, size=N) / 256.0
        elif k == 3:  # f32(0.05) pairs: the float32 sum decides the bound
            H[b] = rng.uniform(0.3, 1.0, size=N)
            H[b, rng.choice(N, 4, replace=False)] = np.float32(0.05)
        else:         # low entropy everywhere: the stop rule
            H[b] = rng.uniform(0.0, 0.008, size=N)
    samp = rng.integers(0, 50000, size=(B, N)).astype(np.int32)
    pred = rng.integers(0, 50000, size=(B, N)).astype(np.int32)
    tokens = rng.integers(0, 50000, size=(B, N)).astype(np.int32)
    locked = (rng.random((B, N)) < rng.uniform(0, 0.6, size=(B, 1))).astype(np.uint8)
    prev = pred.copy()
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        r = rng.integers(0, 4)
        if r == 1:
            status[b] = 2  # stable: a previous pass with the same greedy tokens
        elif r == 2:
            status[b] = 2
            prev[b, rng.integers(0, N)] += 1  # one greedy token moved
        elif r == 3:
            status[b] = 3  # done
    return H, samp, pred, tokens, locked, prev, status


@pytest.mark.parametrize("B,N,t,t_max,kind", [(8, 256, 3, 48, 0), (16, 32, 0, 48, 1), (5, 1000, 10, 48, 2),
                                              (64, 256, 47, 48, 3), (3, 4096, 1, 48, 4), (10, 256, 0, 1, 0)])
def test_eb_select_bit_exact(torch, dg, B, N, t, t_max, kind):
    rng = np.random.default_rng(B * 7 + N + t + kind)
    H, samp, pred, tokens, locked, prev, status = _select_case(rng, B, N, kind)
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda()
         for k, v in dict(H=H, samp=samp, pred=pred, tokens=tokens, locked=locked, prev=prev,
                          status=status).items()}
    say("eb select", B, N, t, t_max, kind)
    dg.k_eb_select(d["H"], d["samp"], d["pred"], d["tokens"], d["locked"], d["prev"], d["status"], t, t_max)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in d.items()}
    stops = 0
    for b in range(B):
        if status[b] & 1:
            assert np.array_equal(g["tokens"][b], tokens[b]) and np.array_equal(g["locked"][b], locked[b])
            assert np.array_equal(g["prev"][b], prev[b]) and g["status"][b] == status[b]
            continue
        ref_prev = prev[b] if status[b] & 2 else None
        tk, lk, sel, stop, done = eb.eb_apply(H[b].astype(np.float64), samp[b], pred[b], tokens[b], locked[b], t,
                                               t_max, ref_prev)
        assert np.array_equal(g["tokens"][b], tk), b
        assert np.array_equal(g["locked"][b], lk), b
        assert np.array_equal(g["prev"][b], pred[b]), b
        assert g["status"][b] == 2 | (4 if stop else 0) | (1 if done else 0), (b, g["status"][b], stop, done)
        stops += stop
    print(f"eb select B={B} N={N}: {stops} canvases stopped")


# --------------------------------------------------------------------------
# the fused LM head in sampler mode
# --------------------------------------------------------------------------

LM_BF16 = dataclasses.replace(
    C1, name="eb-lm-bf16",
    model=configs.ModelConfig(n_layers=1, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                              n_experts=16, top_k=2, expert_ffn=128, vocab=4112, canvas_len=32,
                              window=64, global_layer_mask=0b1, dtype="bf16"),
    batch=2, prompt_len=32, n_steps=4, seed=41, final_norm_shift=30.0)


@pytest.mark.parametrize("t,t_max", [(0, 48), (30, 48), (0, 1)])
def test_fused_lm_head_sampler_mode(torch, dg, t, t_max):
    w = LM_BF16
    m = w.model
    B, N = w.batch, m.canvas_len
    with dg.Context(m, max_batch=B, max_prompt_len=w.prompt_len) as ctx:
        upload.load_context(ctx, w)
        rng = np.random.default_rng(t)
        h = torch.from_numpy(rng.normal(0, 3, size=(B * N, m.hidden)).astype(np.float32)).cuda().to(torch.bfloat16)
        logits = torch.empty((B * N, m.vocab), dtype=torch.float32, device="cuda")
        pred = torch.empty(B * N, dtype=torch.int32, device="cuda")
        ent = torch.empty(B * N, dtype=torch.float32, device="cuda")
        samp = torch.empty(B * N, dtype=torch.int32, device="cuda")
        seeds = [5, 6]
        say("lm sample", t, t_max)
        ctx.k_lm_head(B, h, logits)
        ctx.k_lm_sample(B, h, t, t_max, seeds, 2, pred, ent, samp)
        torch.cuda.synchronize()
        # the fused statistics against the oracle's on the same (GPU) logits
        _check_rows(logits.cpu().numpy(), N, t, t_max, seeds, 2, pred.cpu().numpy(),
                    ent.cpu().numpy().astype(np.float64), samp.cpu().numpy(), f"fused t={t}")


# --------------------------------------------------------------------------
# whole EB blocks on small models
# --------------------------------------------------------------------------

def _eb_block(torch, dg, w, t_max, seeds, block=0, delta_scale=1.0):
    """Pass by pass: the GPU's EB step against the oracle's, shadowed; then
    dg_generate_block_eb from the same start must give the same block.
    delta_scale widens the shadow deltas (routing and logits) for workloads
    with many more near-ties than the small ones."""
    m = w.model
    B, N, L = w.batch, m.canvas_len, m.n_layers
    tok0, lk0 = gen.canvas(w)
    W = weights_for(w)
    kvf = prompt_kv_fn(w)
    rnd = om._rounder(m)
    with dg.Context(m, max_batch=B, max_prompt_len=w.prompt_len) as ctx:
        upload.load_context(ctx, w)
        tokens = torch.from_numpy(tok0).cuda()
        locked = torch.from_numpy(lk0).cuda()
        prev = torch.zeros((B, N), dtype=torch.int32, device="cuda")
        status = torch.zeros(B, dtype=torch.int32, device="cuda")
        ent = torch.empty((B, N), dtype=torch.float32, device="cuda")
        samp = torch.empty((B, N), dtype=torch.int32, device="cuda")
        pred = torch.empty((B, N), dtype=torch.int32, device="cuda")
        trace = torch.empty((L, B * N, m.top_k), dtype=torch.int32, device="cuda")
        ctx.set_trace(trace)
        state = eb.EBState(B)
        t_o, l_o = tok0.copy(), lk0.copy()
        adopted = {"route": 0, "sample": 0, "pred": 0, "lock": 0, "stop": 0}
        passes = [0] * B
        t = 0
        while t < t_max and not state.done.all():
            say(w.name, "EB pass", t)
            ctx.eb_step(tokens, locked, t, t_max, seeds, block, prev, status, ent, samp, pred)
            torch.cuda.synchronize()
            tr = trace.cpu().numpy()
            st = status.cpu().numpy()
            # the oracle's logits of this pass, the GPU's routing adopted at near-ties
            sh = om.Shadow(route_idx=[tr[l] for l in range(L)], delta_route=DELTA_REL[m.dtype] * delta_scale)
            x = W.embed_rows(t_o.reshape(-1).astype(np.int64)).copy()
            x = om.forward_hidden(x, W, m, kvf, [w.prompt_len] * B, shadow=sh)
            h = rnd(om.rmsnorm(x, W.norm_final(), m.rms_eps))
            lg = om.lm_logits(h, W.embed()).reshape(B, N, -1)
            assert not sh.failures, sh.failures[:3]
            adopted["route"] += sh.adopted["route"]
            g_ent = ent.cpu().numpy().astype(np.float64)
            Hs = np.stack([eb.entropy(lg[b], eb.temperature(t, t_max)) for b in range(B)])
            herr = float(np.max(np.abs(g_ent - Hs) / (1.0 + Hs)))
            rms = float(np.sqrt(np.mean(lg ** 2)))
            esh = eb.EBShadow(sample=samp.cpu().numpy(), pred=pred.cpu().numpy(), locked_after=locked.cpu().numpy(),
                              stopped=(st & 4) != 0, dlogit=DELTA_REL[m.dtype] * delta_scale * max(1.0, rms))
            t_o, l_o, info = eb.eb_update(lg, t_o, l_o, t, state, seeds, block, t_max, shadow=esh)
            assert not esh.failures, esh.failures[:3]
            for k in ("sample", "pred", "lock", "stop"):
                adopted[k] += esh.adopted[k]
            assert np.array_equal(tokens.cpu().numpy(), t_o), t
            assert np.array_equal(locked.cpu().numpy(), l_o), t
            assert np.array_equal((st & 1) != 0, state.done), t
            for b in range(B):
                if state.done[b] and not passes[b]:
                    passes[b] = t + 1
            print(f"{w.name} pass {t}: locked {[len(s) for s in info['selected']]}, entropy err {herr:.2e}, "
                  f"stopped {info['stopped']}")
            t += 1
        ctx.set_trace(None)
        final = tokens.cpu().numpy()
        print(f"{w.name}: passes {passes}, adopted {adopted}")
        assert state.done.all() and l_o.all()
        # the whole block in one call: the same result and pass counts
        tokens2 = torch.from_numpy(tok0).cuda()
        locked2 = torch.from_numpy(lk0).cuda()
        say(w.name, "generate_block_eb")
        got_passes = ctx.generate_block_eb(tokens2, locked2, seeds, block, t_max)
        torch.cuda.synchronize()
        assert got_passes == passes
        assert np.array_equal(tokens2.cpu().numpy(), final)
        assert locked2.cpu().numpy().all()
        return passes


def test_eb_block_fp32_tiny(torch, dg):
    w = dataclasses.replace(C1, final_norm_shift=60.0)
    passes = _eb_block(torch, dg, w, 48, [7])
    assert 1 < passes[0] < 48  # several positions per pass


def test_eb_block_fp32_vague_runs_to_the_last_pass(torch, dg):
    # random-init logits are vague: one lock per pass, the last pass locks the rest
    passes = _eb_block(torch, dg, C1, 6, [3])
    assert passes == [6]


def test_eb_block_bf16_two_canvases_with_prelocks(torch, dg):
    w = dataclasses.replace(LM_BF16, name="eb-bf16-2", prelock=(0, 12), final_norm_shift=40.0)
    passes = _eb_block(torch, dg, w, 48, [21, 22], block=5)
    assert all(p >= 1 for p in passes)


def test_eb_block_max_capacity_batch(torch, dg):
    # 64 canvases of 64 slots (4096 rows, the most a context takes; 64 canvases
    # is also the sampler-mode LM head's bound), 128 experts top-8, pre-lock
    # counts 0..63, every canvas with its own seed
    m = configs.ModelConfig(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, n_experts=128, top_k=8,
                            expert_ffn=128, vocab=1024, canvas_len=64, window=64, global_layer_mask=0b10,
                            dtype="bf16")
    w = dataclasses.replace(C1, name="eb-max-capacity", model=m, batch=64, prompt_len=96, n_steps=4, seed=93,
                            prelock=tuple(range(64)), final_norm_shift=40.0)
    # 4096 positions hold far more near-ties than the small workloads: the
    # shadow deltas are 3% of the logits' RMS here (the bf16 tolerance, 2e-2
    # of the largest logit, is about 8% of the RMS of Gaussian logits)
    passes = _eb_block(torch, dg, w, 6, list(range(1000, 1064)), block=2, delta_scale=3.0)
    assert all(1 <= p <= 6 for p in passes)
