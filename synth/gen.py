"""Seeded synthetic inputs: random-init weights, prompt KV, canvases.

Recipe (identical for every consumer):

* every tensor is cut into fixed chunks of ``CHUNK`` elements in C order;
  chunk ``c`` of tensor ``code`` of layer ``layer_id`` (``layer + 1`` for
  per-layer tensors, 0 for global ones) for canvas ``sub`` is drawn from
  ``numpy.random.default_rng([seed, layer_id, code, sub, c])`` as
  ``standard_normal(float32) * std``;
* bf16 workloads round those float32 draws to bf16 with round-to-nearest-even
  (torch's float32 -> bfloat16 conversion) and hand out the raw uint16 bits;
* canvases are ``integers(0, vocab)`` draws, pre-locked positions the first
  ``n_b`` entries of a seeded permutation of the canvas slots.

Nothing here computes any step of the method; it only produces inputs.
Large tensors are generated chunk-parallel on a thread pool (numpy's generators
release the GIL), so a 30-layer workload's ~35 GB of bf16 weights takes tens
of seconds rather than minutes.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Tuple

import numpy as np

from .configs import BF16, F32, Workload

CHUNK = 1 << 22

# per-layer tensor codes
WQ, WK, WV, WO, ROUTER, W_GATE, W_UP, W_DOWN, SH_GATE, SH_UP, SH_DOWN = range(1, 12)
NORM_IN, NORM_PA, NORM_PF, NORM_PF2 = 12, 13, 14, 15
KCACHE, VCACHE = 16, 17
# global tensor codes (layer_id 0)
EMBED, NORM_FINAL, CANVAS, PRELOCK_PERM, X_IN = 1, 2, 3, 4, 5

LAYER_TENSORS = ("wq", "wk", "wv", "wo", "router", "w_gate", "w_up", "w_down",
                 "sh_gate", "sh_up", "sh_down", "norm_in", "norm_pa", "norm_pf", "norm_pf2")


def n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=n_threads())
    return _POOL


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32 (input plumbing for uploads)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, layer_id: int, code: int, sub: int, shape, std: float,
           dtype: str) -> np.ndarray:
    """N(0, std^2) tensor; float32 for ``f32``, bf16 bits (uint16) for ``bf16``."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    std32 = np.float32(std)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng([seed, layer_id, code, sub, c])
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        x *= std32
        if dtype == BF16:
            out[lo:hi] = f32_to_bf16_bits(x)
        else:
            out[lo:hi] = x

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        list(_pool().map(fill, range(nchunks)))
    return out.reshape(shape)


def layer_shapes(w: Workload) -> Dict[str, Tuple[int, ...]]:
    m = w.model
    H, F, E = m.hidden, m.expert_ffn, m.n_experts
    return {
        "wq": (H, m.q_dim), "wk": (H, m.kv_dim), "wv": (H, m.kv_dim), "wo": (m.q_dim, H),
        "router": (H, E), "w_gate": (E, H, F), "w_up": (E, H, F), "w_down": (E, F, H),
        "sh_gate": (H, F), "sh_up": (H, F), "sh_down": (F, H),
        "norm_in": (H,), "norm_pa": (H,), "norm_pf": (H,), "norm_pf2": (H,),
    }


_CODES = {"wq": WQ, "wk": WK, "wv": WV, "wo": WO, "router": ROUTER, "w_gate": W_GATE,
          "w_up": W_UP, "w_down": W_DOWN, "sh_gate": SH_GATE, "sh_up": SH_UP,
          "sh_down": SH_DOWN, "norm_in": NORM_IN, "norm_pa": NORM_PA, "norm_pf": NORM_PF,
          "norm_pf2": NORM_PF2}


def layer_tensor(w: Workload, layer: int, name: str) -> np.ndarray:
    std = w.router_std if name == "router" else w.weight_std
    return normal(w.seed, layer + 1, _CODES[name], 0, layer_shapes(w)[name], std, w.model.dtype)


def layer_weights(w: Workload, layer: int) -> Dict[str, np.ndarray]:
    return {name: layer_tensor(w, layer, name) for name in LAYER_TENSORS}


def embed(w: Workload) -> np.ndarray:
    m = w.model
    return normal(w.seed, 0, EMBED, 0, (m.vocab, m.hidden), w.weight_std, m.dtype)


def norm_final(w: Workload) -> np.ndarray:
    m = w.model
    if not w.final_norm_shift:
        return normal(w.seed, 0, NORM_FINAL, 0, (m.hidden,), w.weight_std, m.dtype)
    x = normal(w.seed, 0, NORM_FINAL, 0, (m.hidden,), w.weight_std, F32) + np.float32(w.final_norm_shift)
    return f32_to_bf16_bits(x) if m.dtype == BF16 else x


def prompt_kv(w: Workload, layer: int, canvas: int) -> Tuple[np.ndarray, np.ndarray]:
    """Cached prompt K and V of one layer for one canvas, ``[len, Hkv, D]``.

    ``len`` is the number of prompt positions the layer reads (the last
    ``window`` positions on sliding-window layers).  K is taken to be already
    position-encoded, as a cache written by the prompt encoder would be."""
    m = w.model
    L = m.kv_len(layer, w.prompt_len)
    shape = (L, m.n_kv_heads, m.head_dim)
    k = normal(w.seed, layer + 1, KCACHE, canvas, shape, w.kv_std, m.dtype)
    v = normal(w.seed, layer + 1, VCACHE, canvas, shape, w.kv_std, m.dtype)
    return k, v


def canvas(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Initial canvas tokens ``int32 [B, N]`` (uniform over the vocabulary) and
    the locked mask ``uint8 [B, N]`` (pre-locked positions set)."""
    m = w.model
    B, N = w.batch, m.canvas_len
    tokens = np.empty((B, N), dtype=np.int32)
    locked = np.zeros((B, N), dtype=np.uint8)
    pre = w.prelock_counts()
    for b in range(B):
        rng = np.random.default_rng([w.seed, 0, CANVAS, b, 0])
        tokens[b] = rng.integers(0, m.vocab, size=N, dtype=np.int64).astype(np.int32)
        if pre[b]:
            prng = np.random.default_rng([w.seed, 0, PRELOCK_PERM, b, 0])
            perm = prng.permutation(N)
            locked[b, perm[: pre[b]]] = 1
    return tokens, locked


def x_in(w: Workload) -> np.ndarray:
    """Residual-stream input ``float32 [B*N, H]`` ~ N(0, 1) for the
    hidden-only (no embedding, no LM head) workload."""
    m = w.model
    return normal(w.seed, 0, X_IN, 0, (w.batch * m.canvas_len, m.hidden), 1.0, "f32")


def router_logits(seed: int, rows: int, n_experts: int, std: float = 1.0) -> np.ndarray:
    """Gate logits ``float32 [rows, E]`` for routing tests."""
    return normal(seed, 0, 100, 0, (rows, n_experts), std, "f32")


def activations(seed: int, code: int, shape, std: float = 1.0, dtype: str = BF16) -> np.ndarray:
    """Generic activation-like tensor for kernel-level tests."""
    return normal(seed, 0, 200 + code, 0, shape, std, dtype)
