"""Block continuation on the GPU against the oracle: dg_commit_block runs the
decoder stack causally over a finished block and appends every layer's K/V
to the prompt caches; the grown caches, and a denoise pass at the moved
canvas positions, are compared with the oracle's commit and append.

The copied part of a cache must be bit-exact; the block's K/V (and the pass
after the commits) meet the storage format's tolerance, with the routing of
the commit pass compared in the shadowed mode."""
import dataclasses

import numpy as np
import pytest

from gpu_util import DELTA_REL, TOL, host64, needs_gpu, rel_err, say
from oracle import model as om
from oracle.inputs import prompt_kv_fn, weights_for
from synth import C1, configs, gen, upload

pytestmark = [pytest.mark.gpu, needs_gpu]

# bf16, a sliding-window layer (window 64 < the grown context) and a global one
COMMIT_BF16 = dataclasses.replace(
    C1, name="commit-bf16",
    model=configs.ModelConfig(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                              n_experts=16, top_k=2, expert_ffn=128, vocab=1024, canvas_len=32,
                              window=64, global_layer_mask=0b10, dtype="bf16"),
    batch=1, prompt_len=48, n_steps=4, seed=31)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    return _t


@pytest.fixture(scope="module")
def dg():
    import canvas_denoising_moe_amd as _dg
    _dg.lib()
    return _dg


def _gpu_cache(torch, ctx, m, l):
    n = ctx.prompt_kv_len(0, l)
    dt = torch.bfloat16 if m.dtype == "bf16" else torch.float32
    k = torch.empty((n, m.n_kv_heads, m.head_dim), dtype=dt, device="cuda")
    v = torch.empty_like(k)
    if n:
        ctx.get_prompt_kv(0, l, k, v)
    torch.cuda.synchronize()
    return host64(k), host64(v)


def _visible(m, l, total):
    return total if m.is_global(l) else min(total, m.window)


def _commit_and_compare(torch, ctx, w, W, cache, pos, tokens_np, tol, tag, n=None):
    """One GPU commit (of the first n tokens of each row; all N when n is
    None) against the oracle's; returns the oracle's new caches."""
    m = w.model
    L, N = m.n_layers, m.canvas_len
    n = N if n is None else n
    trace = torch.empty((L, N, m.top_k), dtype=torch.int32, device="cuda")
    ctx.set_trace(trace)
    say(tag, "commit at", pos, "of", n)
    if n == N:
        ctx.commit_block(torch.from_numpy(tokens_np.astype(np.int32)).cuda())
    else:
        ctx.commit_tokens(torch.from_numpy(tokens_np.astype(np.int32)).cuda(), n)
    torch.cuda.synchronize()
    ctx.set_trace(None)
    tr = trace.cpu().numpy()
    # the last layer's FFN is not run by the commit: its routing is not compared;
    # the oracle commits the n tokens alone, so only their routing is compared
    sh = om.Shadow(route_idx=[tr[l][:n] for l in range(L - 1)] + [None], delta_route=DELTA_REL[m.dtype])
    mn = dataclasses.replace(m, canvas_len=n)
    blk = om.commit_block(tokens_np[:, :n], W, mn, lambda l, b: cache[l], [pos], shadow=sh)
    assert not sh.failures, sh.failures[:5]
    new = []
    for l in range(L):
        vis = _visible(m, l, pos + n)
        K, V = om.append_kv(cache[l][0], cache[l][1], blk[l][0][0], blk[l][1][0], vis)
        gk, gv = _gpu_cache(torch, ctx, m, l)
        assert gk.shape == K.shape, (l, gk.shape, K.shape)
        old = vis - n  # positions copied from the previous cache
        if old > 0:
            assert np.array_equal(gk[:old], _gpu_prev[l][0][len(_gpu_prev[l][0]) - old:]), (tag, l)
            assert np.array_equal(gv[:old], _gpu_prev[l][1][len(_gpu_prev[l][1]) - old:]), (tag, l)
        ek, ev = rel_err(gk[old:], K[old:]), rel_err(gv[old:], V[old:])
        print(f"{tag} layer {l}: len {vis}, block K rel err {ek:.3e}, V {ev:.3e}")
        assert ek <= tol and ev <= tol, (tag, l, ek, ev)
        _gpu_prev[l] = (gk, gv)
        new.append((K, V))
    print(f"{tag}: routing adopted {sh.adopted}, max margin {sh.max_margin}")
    return new


_gpu_prev = {}


def _run_commits(torch, dg, w, n_commits, prefill_from_empty=False, counts=None):
    m = w.model
    L, N = m.n_layers, m.canvas_len
    p0 = 0 if prefill_from_empty else w.prompt_len
    counts = counts if counts is not None else [N] * n_commits
    ctx = dg.Context(m, max_batch=1, max_prompt_len=p0 + sum(counts))
    try:
        say("load", w.name, "prompt", p0)
        ww = dataclasses.replace(w, prompt_len=p0)
        upload.load_context(ctx, ww)
        W = weights_for(ww)
        kvf = prompt_kv_fn(ww)
        cache = [kvf(l, 0) for l in range(L)]
        _gpu_prev.clear()
        for l in range(L):
            _gpu_prev[l] = _gpu_cache(torch, ctx, m, l)
            assert np.array_equal(_gpu_prev[l][0], cache[l][0]) and np.array_equal(_gpu_prev[l][1], cache[l][1])
        rng = np.random.default_rng(w.seed + 1000)
        pos = p0
        for c, n in enumerate(counts):
            toks = rng.integers(0, m.vocab, size=(1, N))
            if n < N:
                toks[:, n:] = rng.integers(-5, 2 * m.vocab, size=(1, N - n))  # ignored, may be anything
            cache = _commit_and_compare(torch, ctx, ww, W, cache, pos, toks, TOL[m.dtype], f"{w.name} #{c}", n)
            pos += n
        return ctx, W, cache, pos
    except Exception:
        ctx.close()
        raise


def _pass_after(torch, ctx, w, W, cache, pos):
    """A denoise pass on the canvas at positions pos + i, GPU vs oracle."""
    m = w.model
    L, N = m.n_layers, m.canvas_len
    tok0, lk0 = gen.canvas(dataclasses.replace(w, batch=1))
    tokens = torch.from_numpy(tok0).cuda()
    locked = torch.from_numpy(lk0).cuda()
    conf = torch.empty((1, N), dtype=torch.float32, device="cuda")
    pred = torch.empty((1, N), dtype=torch.int32, device="cuda")
    trace = torch.empty((L, N, m.top_k), dtype=torch.int32, device="cuda")
    ctx.set_trace(trace)
    say(w.name, "pass after the commits at", pos)
    ctx.denoise_step(tokens, locked, [w.n_steps], conf, pred)
    torch.cuda.synchronize()
    ctx.set_trace(None)
    tr = trace.cpu().numpy()
    c_g = conf.cpu().numpy()
    sh = om.Shadow(route_idx=[tr[l] for l in range(L)], pred=pred.cpu().numpy(),
                   locked_after=locked.cpu().numpy())
    d = DELTA_REL[m.dtype]
    sh.delta_route = d
    sh.delta_logit = d
    sh.delta_conf = d * float(np.sqrt(np.mean(c_g.astype(np.float64) ** 2)))
    t_o, l_o, pred_o, conf_o, _ = om.denoise_pass(tok0, lk0, [w.n_steps], W, m, lambda l, b: cache[l], [pos],
                                                   shadow=sh)
    assert not sh.failures, sh.failures[:5]
    ce = rel_err(c_g, conf_o)
    ce_el = float(np.max(np.abs(c_g - conf_o) / conf_o))
    print(f"{w.name} pass after commits: conf rel err {ce:.3e} (largest per position {ce_el:.3e}), "
          f"adopted {sh.adopted}")
    assert ce <= TOL[m.dtype]
    assert np.array_equal(tokens.cpu().numpy(), t_o)
    assert np.array_equal(locked.cpu().numpy(), l_o)


def test_commit_bf16_window_and_global_then_pass(torch, dg):
    w = COMMIT_BF16
    ctx, W, cache, pos = _run_commits(torch, dg, w, 3)
    try:
        _pass_after(torch, ctx, w, W, cache, pos)
    finally:
        ctx.close()


def test_commit_f32_then_pass(torch, dg):
    w = dataclasses.replace(C1, prompt_len=64)
    ctx, W, cache, pos = _run_commits(torch, dg, w, 2)
    try:
        _pass_after(torch, ctx, w, W, cache, pos)
    finally:
        ctx.close()


def test_prefill_from_empty_cache_bf16(torch, dg):
    # the prompt KV built from token ids by successive commits
    ctx, W, cache, pos = _run_commits(torch, dg, COMMIT_BF16, 3, prefill_from_empty=True)
    ctx.close()


def test_prefill_ragged_prompt_then_pass_bf16(torch, dg):
    # a 107-token prompt from an empty cache: chunks of 32, 32, 32 and 11
    # (the window of 64 truncates the local layer's cache along the way),
    # then a denoise pass at positions 107 + i
    ctx, W, cache, pos = _run_commits(torch, dg, COMMIT_BF16, 4, prefill_from_empty=True, counts=[32, 32, 32, 11])
    try:
        assert pos == 107
        _pass_after(torch, ctx, dataclasses.replace(COMMIT_BF16, prompt_len=0), W, cache, pos)
    finally:
        ctx.close()


def test_commit_one_token_at_a_time_f32(torch, dg):
    w = dataclasses.replace(C1, prompt_len=64)
    ctx, W, cache, pos = _run_commits(torch, dg, w, 3, counts=[1, 5, 1])
    try:
        _pass_after(torch, ctx, w, W, cache, pos)
    finally:
        ctx.close()


def test_prefill_helper_equals_commits(torch, dg):
    # Context.prefill (chunked dg_commit_tokens) gives the same caches as the
    # explicit commits of the test above, bit for bit
    w = COMMIT_BF16
    m = w.model
    rng = np.random.default_rng(w.seed + 1000)
    toks = [rng.integers(0, m.vocab, size=(1, m.canvas_len)) for _ in range(4)]
    counts = [32, 32, 32, 11]
    prompt = np.concatenate([t[:, :n] for t, n in zip(toks, counts)], axis=1).astype(np.int32)
    caches = []
    for mode in ("prefill", "commits"):
        with dg.Context(m, max_batch=1, max_prompt_len=107) as ctx:
            upload.load_context(ctx, dataclasses.replace(w, prompt_len=0))
            if mode == "prefill":
                ctx.prefill(torch.from_numpy(prompt).cuda())
            else:
                for t, n in zip(toks, counts):
                    ctx.commit_tokens(torch.from_numpy(t.astype(np.int32)).cuda(), n)
            torch.cuda.synchronize()
            caches.append([_gpu_cache(torch, ctx, m, l) for l in range(m.n_layers)])
    for l in range(m.n_layers):
        assert np.array_equal(caches[0][l][0], caches[1][l][0]) and np.array_equal(caches[0][l][1], caches[1][l][1])


def test_commit_rejects_overflow(torch, dg):
    w = COMMIT_BF16
    m = w.model
    with dg.Context(m, max_batch=1, max_prompt_len=w.prompt_len + m.canvas_len - 16) as ctx:
        upload.load_context(ctx, w)
        toks = torch.zeros((1, m.canvas_len), dtype=torch.int32, device="cuda")
        with pytest.raises(Exception, match="exceeds max_prompt_len"):
            ctx.commit_block(toks)
        assert ctx.prompt_kv_len(0, 1) == w.prompt_len  # nothing changed
        for bad in (0, m.canvas_len + 1):
            with pytest.raises(Exception, match="outside"):
                ctx.commit_tokens(toks, bad)
        ctx.commit_tokens(toks, 16)  # fits
        assert ctx.prompt_kv_len(0, 1) == w.prompt_len + 16
