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

