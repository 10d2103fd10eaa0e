"""Move seeded host inputs into torch device tensors (plumbing only)."""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import gen
from .configs import BF16, Workload


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """bf16 bits (uint16) -> torch.bfloat16; float32 -> torch.float32."""
    import torch
    if dtype == BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device, non_blocking=False)


def layer_to_device(w: Workload, layer: int, device="cuda") -> Dict[str, "object"]:
    return {k: to_device(v, w.model.dtype, device) for k, v in gen.layer_weights(w, layer).items()}


def prompt_kv_to_device(w: Workload, canvas: int, device="cuda"):
    ks, vs = [], []
    for l in range(w.model.n_layers):
        k, v = gen.prompt_kv(w, l, canvas)
        ks.append(to_device(k, w.model.dtype, device))
        vs.append(to_device(v, w.model.dtype, device))
    return ks, vs


def load_context(ctx, w: Workload, device="cuda", layers=None, progress: bool = False):
    """Upload every weight and prompt KV of workload ``w`` into ``ctx`` (one
    layer at a time so the caller-side staging stays one layer large)."""
    import sys
    import time

    import torch
    m = w.model
    t0 = time.perf_counter()

    def note(msg):
        if progress:
            print(f"[load {time.perf_counter() - t0:6.1f}s] {msg}", file=sys.stderr, flush=True)
    if m.has_lm_head:
        e = to_device(gen.embed(w), m.dtype, device)
        nf = to_device(gen.norm_final(w), m.dtype, device)
        ctx.set_embedding(e, nf)
        torch.cuda.synchronize()
        del e, nf
    for l in (range(m.n_layers) if layers is None else layers):
        lw = layer_to_device(w, l, device)
        ctx.set_layer_weights(l, lw)
        torch.cuda.synchronize()
        del lw
        note(f"layer {l} weights")
    for b in range(w.batch):
        ks, vs = prompt_kv_to_device(w, b, device)
        ctx.load_prompt_kv(b, w.prompt_len, ks, vs)
        torch.cuda.synchronize()
        del ks, vs
