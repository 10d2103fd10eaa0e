"""Glue from the seeded synthetic inputs to the oracle's float64 view.

Test infrastructure only."""
from __future__ import annotations

from functools import lru_cache

import numpy as np

from synth import gen

from .model import OracleWeights, _to_f64


def weights_for(w, cache_layers: bool = False) -> OracleWeights:
    m = w.model
    return OracleWeights(
        dtype=m.dtype,
        layer_fn=lambda l: gen.layer_weights(w, l),
        embed_raw=gen.embed(w) if m.has_lm_head else None,
        norm_final_raw=gen.norm_final(w) if m.has_lm_head else None,
        cache_layers=cache_layers,
        expert_format=getattr(m, "expert_format", "native"),
    )


def prompt_kv_fn(w):
    """``fn(l, b) -> (K, V)`` float64 ``[len, Hkv, D]`` for layer ``l``,
    canvas ``b``."""
    dtype = w.model.dtype

    @lru_cache(maxsize=8)
    def fn(l, b):
        k, v = gen.prompt_kv(w, l, b)
        return _to_f64(k, dtype), _to_f64(v, dtype)

    return fn
