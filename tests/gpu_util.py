"""Shared helpers of the GPU parity tests (plumbing only)."""
import os
import sys

import numpy as np
import pytest

from oracle import model as om
from oracle.inputs import prompt_kv_fn, weights_for
from synth import gen


def gpu_ok() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


needs_gpu = pytest.mark.skipif(not gpu_ok(), reason="needs a GPU")


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| over the tensor."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(gpu - ref))) / max(den, 1e-30) if ref.size else 0.0


def host64(t) -> np.ndarray:
    """torch tensor (bf16 / f32 / int) -> float64 numpy on the host."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_tensor_to_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# tolerances (max relative error, per tensor) for the two storage formats
TOL = {"bf16": 2e-2, "f32": 1e-4}
# shadowed comparison: a discrete decision whose oracle margin is below delta
# (relative to the RMS of the compared quantity) may follow the GPU's choice
DELTA_REL = {"f32": 1e-3, "bf16": 1e-2}


# ------------------------------------------------ block-level parity helpers

def run_block_stepwise(torch, ctx, w, steps=None):
    m = w.model
    B, N = w.batch, m.canvas_len
    tok0, lk0 = gen.canvas(w)
    tokens = torch.from_numpy(tok0).cuda()
    locked = torch.from_numpy(lk0).cuda()
    trace = torch.empty((m.n_layers, B * N, m.top_k), dtype=torch.int32, device="cuda")
    ctx.set_trace(trace)
    conf = torch.empty((B, N), dtype=torch.float32, device="cuda")
    pred = torch.empty((B, N), dtype=torch.int32, device="cuda")
    passes = []
    for t in range(w.n_steps if steps is None else steps):
        ctx.denoise_step(tokens, locked, [w.n_steps - t] * B, conf, pred)
        torch.cuda.synchronize()
        passes.append(dict(trace=trace.cpu().numpy().copy(), conf=conf.cpu().numpy().copy(),
                           pred=pred.cpu().numpy().copy(), tokens=tokens.cpu().numpy().copy(),
                           locked=locked.cpu().numpy().copy()))
    ctx.set_trace(None)
    return tok0, lk0, passes


def shadow_compare(w, tok0, lk0, passes, delta_rel, conf_tol, weights=None, route_delta=None):
    m = w.model
    W = weights if weights is not None else weights_for(w, cache_layers=True)
    kvf = prompt_kv_fn(w)
    t_o, l_o = tok0, lk0
    report = {"route": 0, "pred": 0, "lock": 0}
    worst_conf = 0.0
    for t, p in enumerate(passes):
        # deltas relative to the RMS of the quantity a decision compares
        sh = om.Shadow(route_idx=[p["trace"][l] for l in range(m.n_layers)], pred=p["pred"],
                       locked_after=p["locked"])
        trace = []
        # router logits have unit-order RMS in these workloads unless the caller
        # scales the delta to its own logit RMS
        sh.delta_route = delta_rel if route_delta is None else route_delta
        sh.delta_logit = delta_rel
        sh.delta_conf = delta_rel * float(np.sqrt(np.mean(p["conf"].astype(np.float64) ** 2)))
        t_o, l_o, pred_o, conf_o, _ = om.denoise_pass(t_o, l_o, [w.n_steps - t] * w.batch, W, m, kvf,
                                                       [w.prompt_len] * w.batch, shadow=sh, trace=trace)
        assert not sh.failures, (t, sh.failures[:5])
        for k in report:
            report[k] += sh.adopted[k]
        ce = float(np.max(np.abs(p["conf"] - conf_o) / conf_o))
        worst_conf = max(worst_conf, ce)
        assert ce <= conf_tol, (t, ce)
        assert np.array_equal(p["tokens"], t_o), t
        assert np.array_equal(p["locked"], l_o), t
    return report, worst_conf



# ----------------------------------------- per-pass comparison from a state ---

def rms(a) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def oracle_head_step(x_final, W, m, tokens, locked, steps_left, gpu, logit_delta, conf_delta_rel):
    """The end of a pass in the oracle from a given final residual stream
    ``x_final [B*N, H]``: final norm, tied LM head, argmax and confidence,
    lock step, with the GPU pass's argmax and lock set (``gpu``: its
    ``pred``, ``locked`` after the pass) adopted at near-ties.  Returns the
    oracle's new ``tokens, locked``, its ``pred, conf`` and the shadow."""
    B, N = tokens.shape
    rnd = om.bf16_round if m.dtype == "bf16" else (lambda z: z)
    h = rnd(om.rmsnorm(x_final, W.norm_final(), m.rms_eps))
    logits = om.lm_logits(h, W.embed())
    pred, conf = om.argmax_conf(logits)
    pred, conf = pred.reshape(B, N), conf.reshape(B, N)
    sh = om.Shadow(pred=gpu["pred"], locked_after=gpu["locked"], delta_logit=logit_delta,
                   delta_conf=conf_delta_rel * rms(gpu["conf"]))
    om.adopt_pred(logits.reshape(B, N, -1), pred, conf, sh)
    del logits
    t_o, l_o, chosen = om.lock_select(conf, pred, tokens, locked, steps_left)
    om.adopt_locks(conf, pred, tokens, locked, t_o, l_o, chosen, sh)
    return t_o, l_o, pred, conf, sh


def gpu_layer_states(torch, ctx, w, tokens):
    """The GPU's residual stream before and after every layer of a pass over
    ``tokens [B, N]``, and the routing of each layer: the embedded canvas
    (bf16 rows widened exactly) through ``dg_forward_layers`` one layer at a
    time, which equals the pass's own stack bit for bit."""
    from synth import gen
    m = w.model
    L, M = m.n_layers, tokens.size
    E = gen.embed(w)[tokens.reshape(-1)]
    x0 = om.bf16_bits_to_f64(E) if m.dtype == "bf16" else np.asarray(E, dtype=np.float64)
    xd = torch.from_numpy(x0.astype(np.float32)).cuda()
    trace = torch.zeros((L, M, m.top_k), dtype=torch.int32, device="cuda")
    ctx.set_trace(trace)
    xs = [x0]
    for l in range(L):
        xn = torch.empty_like(xd)
        ctx.forward_layers(l, 1, xd, xn)
        torch.cuda.synchronize()
        xs.append(host64(xn))
        xd = xn
    ctx.set_trace(None)
    return xs, trace.cpu().numpy()


class _KeptExperts:
    """One expert stack of a layer whose matrices, once widened to float64,
    are kept for the other passes compared with that layer."""

    def __init__(self, stack):
        self.stack, self.shape, self.kept = stack, stack.shape, {}

    def __getitem__(self, e):
        if e not in self.kept:
            self.kept[e] = self.stack[e]
        return self.kept[e]


class _OneLayer:
    """Layer ``l`` of oracle weights with its expert matrices kept once
    widened (the oracle widens each used expert on every call, most of its
    time at the full sizes); the same float64 values as ``W.layer(l)``."""

    def __init__(self, W, l):
        self.l = l
        self.d = {k: (_KeptExperts(v) if isinstance(v, om._ExpertStack) else v) for k, v in W.layer(l).items()}

    def layer(self, l):
        assert l == self.l
        return self.d


def anchored_passes_compare(torch, ctx, w, W, kvf, t0, t1, tokens, locked, passes, route_delta, logit_delta,
                            conf_delta_rel, tag):
    """Passes ``t0 .. t1 - 1`` of a block (``passes[t]``: the GPU pass's
    ``tokens``, ``locked``, ``pred``, ``conf``, ``trace``; ``tokens``,
    ``locked``: the canvas before pass ``t0``), each checked exactly as
    :func:`anchored_pass_compare` checks one pass, with the oracle run layer
    by layer across the passes so that a layer's expert matrices are widened
    once for all of them.  Returns the per-pass (worst layer error, conf
    error, adopted counts)."""
    m = w.model
    L = m.n_layers
    tol = TOL[m.dtype]
    runs = []
    for t in range(t0, t1):
        gpu = passes[t]
        say(tag, "pass", t, "layer states")
        xs, tr = gpu_layer_states(torch, ctx, w, tokens)
        diff = [l for l in range(L) if not np.array_equal(tr[l], gpu["trace"][l])]
        assert not diff, (tag, t, f"the layer-by-layer replay routes differently from the pass from layer {diff[0]} "
                                  f"on ({int((tr[diff[0]] != gpu['trace'][diff[0]]).any(axis=1).sum())} rows)")
        runs.append({"t": t, "tokens": tokens, "locked": locked, "xs": xs, "tr": tr, "gpu": gpu, "worst": 0.0,
                     "adopted": {"route": 0, "pred": 0, "lock": 0}})
        tokens, locked = gpu["tokens"], gpu["locked"]
    lens = [w.prompt_len] * w.batch
    for l in range(L):
        Wl = _OneLayer(W, l)
        for r in runs:
            route = [None] * L
            route[l] = r["tr"][l]
            sh = om.Shadow(route_idx=route, delta_route=route_delta)
            ref = om.forward_hidden(r["xs"][l], Wl, m, kvf, lens, layers=[l], shadow=sh)
            e = rel_err(r["xs"][l + 1], ref)
            r["worst"] = max(r["worst"], e)
            assert not sh.failures, (tag, r["t"], l, sh.failures[:5])
            assert e <= tol, (tag, r["t"], l, e)
            r["adopted"]["route"] += sh.adopted["route"]
        del Wl
    out = []
    for r in runs:
        t, gpu = r["t"], r["gpu"]
        steps = [w.n_steps - t] * w.batch
        t_o, l_o, pred_o, conf_o, sh = oracle_head_step(r["xs"][L], W, m, r["tokens"], r["locked"], steps, gpu,
                                                        logit_delta, conf_delta_rel)
        assert not sh.failures, (tag, t, sh.failures[:5])
        ce = rel_err(gpu["conf"], conf_o)
        assert ce <= tol, (tag, t, ce)
        assert np.array_equal(gpu["tokens"], t_o), (tag, t)
        assert np.array_equal(gpu["locked"], l_o), (tag, t)
        r["adopted"]["pred"] += sh.adopted["pred"]
        r["adopted"]["lock"] += sh.adopted["lock"]
        print(f"{tag} pass {t}: every layer from the GPU's own input within {r['worst']:.3e}; conf rel err "
              f"{ce:.3e}; adopted {r['adopted']}", flush=True)
        out.append((r["worst"], ce, r["adopted"]))
    return out


def anchored_pass_compare(torch, ctx, w, W, kvf, t, tokens, locked, gpu, route_delta, logit_delta,
                          conf_delta_rel, tag):
    """Pass ``t`` of a block compared with the oracle layer by layer: every
    layer of the oracle starts from the GPU's own residual stream at that
    layer's input (so each layer is held to the one-layer tolerance and its
    routing to the one-layer decision delta), then the oracle's head and lock
    step run from the GPU's final residual stream with the GPU's argmax and
    lock set adopted at near-ties.  The oracle's tokens and locked mask after
    the pass must equal the GPU's (``gpu``: the pass's ``tokens``,
    ``locked``, ``pred``, ``conf``).  Returns (worst layer error, conf error,
    adopted counts)."""
    m = w.model
    L = m.n_layers
    tol = TOL[m.dtype]
    say(tag, "pass", t, "layer states")
    xs, tr = gpu_layer_states(torch, ctx, w, tokens)
    # the replay is the pass's own stack: same kernels, same inputs, so the
    # same routing at every layer (every kernel is deterministic)
    if "trace" in gpu:
        diff = [l for l in range(L) if not np.array_equal(tr[l], gpu["trace"][l])]
        assert not diff, (tag, t, f"the layer-by-layer replay routes differently from the pass from layer {diff[0]} "
                                  f"on ({int((tr[diff[0]] != gpu['trace'][diff[0]]).any(axis=1).sum())} rows)")
    lens = [w.prompt_len] * w.batch
    worst, adopted = 0.0, {"route": 0, "pred": 0, "lock": 0}
    for l in range(L):
        route = [None] * L
        route[l] = tr[l]
        sh = om.Shadow(route_idx=route, delta_route=route_delta)
        ref = om.forward_hidden(xs[l], W, m, kvf, lens, layers=[l], shadow=sh)
        e = rel_err(xs[l + 1], ref)
        worst = max(worst, e)
        assert not sh.failures, (tag, t, l, sh.failures[:5])
        assert e <= tol, (tag, t, l, e)
        adopted["route"] += sh.adopted["route"]
    steps = [w.n_steps - t] * w.batch
    t_o, l_o, pred_o, conf_o, sh = oracle_head_step(xs[L], W, m, tokens, locked, steps, gpu, logit_delta,
                                                    conf_delta_rel)
    assert not sh.failures, (tag, t, sh.failures[:5])
    ce = rel_err(gpu["conf"], conf_o)
    assert ce <= tol, (tag, t, ce)
    assert np.array_equal(gpu["tokens"], t_o), (tag, t)
    assert np.array_equal(gpu["locked"], l_o), (tag, t)
    adopted["pred"] += sh.adopted["pred"]
    adopted["lock"] += sh.adopted["lock"]
    print(f"{tag} pass {t}: every layer from the GPU's own input within {worst:.3e}; conf rel err "
          f"{ce:.3e}; adopted {adopted}", flush=True)
    return worst, ce, adopted
