"""Model shapes and workloads of the five synthetic configurations.

Plain data only: no arithmetic of the method lives here.  Both the HIP path's
harness and the CPU oracle read these records; the shapes follow the pages'
specification of the DiffusionGemma decoder:

* canvas of 256 slots, 128 experts with 8 active + 1 shared, 1024-token
  sliding window, 262K vocabulary, 30 layers -- "DiffusionGemma: The Diffusion
  Era Begins with 4x Faster Text Generation", section "DiffusionGemma's
  Technical Architecture";
* 30 blocks arranged as five groups of (5 local + 1 global) attention layers,
  GELU-tanh gated MLP, RMS-style norm sandwich, tied embedding / LM head --
  "Hands-On with Diffusion Gemma", section "Detailed Specs".

The hidden size 2048, 16/8 query/KV heads of 128, expert FFN width 704 and the
per-workload sizes (prompt length, passes, batch, seeds, distributions) are the
benchmark workloads' own; the pages' 2,816 hidden size is context only.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Tuple

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class ModelConfig:
    """Architecture of one decoder stack (mirrors the C struct ``dg_config``)."""

    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_ffn: int
    vocab: int
    canvas_len: int
    window: int
    # layer l is global when bit l is set; the others are sliding-window layers
    global_layer_mask: int
    rope_theta: float = 10000.0
    # fraction of rotary pairs that p-RoPE rotates on global layers
    prope_frac: float = 0.25
    rms_eps: float = 1e-6
    dtype: str = BF16
    has_lm_head: bool = True
    n_shared: int = 1
    # norm of the MoE output before the residual add (symmetric with the
    # post-attention norm)
    post_ffn_norm: bool = True
    # storage of the routed and shared experts' matrices: "native" (dtype) or
    # "mxfp4" (4-bit blocks of 32 along the input dimension, bf16 only)
    expert_format: str = "native"

    def is_global(self, layer: int) -> bool:
        return bool((self.global_layer_mask >> layer) & 1)

    def kv_len(self, layer: int, prompt_len: int) -> int:
        """Prompt positions layer ``layer`` reads: all on global layers, the
        last ``window`` on sliding-window layers."""
        if self.is_global(layer):
            return prompt_len
        return min(prompt_len, self.window)

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim


def five_local_one_global(n_layers: int) -> int:
    """Global-layer bitmask for the (5 local + 1 global) x k pattern: layer l
    is global iff (l + 1) % 6 == 0."""
    m = 0
    for l in range(n_layers):
        if (l + 1) % 6 == 0:
            m |= 1 << l
    return m


def alternating(n_layers: int) -> int:
    """Global-layer bitmask for a strict local/global alternation."""
    m = 0
    for l in range(n_layers):
        if l % 2 == 1:
            m |= 1 << l
    return m


@dataclass(frozen=True)
class Workload:
    """One seeded synthetic workload: a model plus its inputs' recipe."""

    name: str
    model: ModelConfig
    batch: int
    prompt_len: int
    n_steps: int
    seed: int
    weight_std: float = 0.02
    # std of the router weight entries; logits of unit-RMS inputs then have a
    # std close to router_std * sqrt(hidden)
    router_std: float = 0.02
    kv_std: float = 1.0
    # added to every final-norm weight w (the norm scales by 1 + w): a value
    # of g - 1 scales the logits by about g, sharpening the output
    # distribution (low-entropy workloads for the entropy-bounded sampler)
    final_norm_shift: float = 0.0
    # number of positions pre-locked per canvas (len == batch)
    prelock: Tuple[int, ...] = field(default=())
    description: str = ""

    def prelock_counts(self) -> Tuple[int, ...]:
        return self.prelock if self.prelock else (0,) * self.batch

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_BIG = dict(hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128, n_experts=128,
            top_k=8, expert_ffn=704, canvas_len=256, window=1024)

C1 = Workload(
    name="C1-tiny-f32",
    model=ModelConfig(n_layers=2, hidden=256, n_heads=4, n_kv_heads=4, head_dim=64,
                      n_experts=16, top_k=2, expert_ffn=128, vocab=1024, canvas_len=32,
                      window=1024, global_layer_mask=0b10, dtype=F32),
    batch=1, prompt_len=64, n_steps=4, seed=0,
    description="2-layer fp32 decoder (local, global), hidden 256, 4x64 heads, "
                "16 experts top-2 + 1 shared, FFN 128, vocab 1024, 64-position "
                "prompt KV, 32-slot canvas, 4 passes")

C2 = Workload(
    name="C2-one-layer-bf16",
    model=ModelConfig(n_layers=1, vocab=0, global_layer_mask=0b1, has_lm_head=False,
                      dtype=BF16, **_BIG),
    batch=1, prompt_len=1024, n_steps=1, seed=1,
    router_std=1.0 / 2048 ** 0.5,
    description="one global bf16 decoder layer over a 256-slot canvas, "
                "1024-position prompt KV, router logits ~N(0,1), no LM head")

C3 = Workload(
    name="C3-30L-bf16-kv4096",
    model=ModelConfig(n_layers=30, vocab=262144, global_layer_mask=five_local_one_global(30),
                      dtype=BF16, **_BIG),
    batch=1, prompt_len=4096, n_steps=8, seed=2,
    description="30-layer bf16 stack (5 local : 1 global), 4096-position prompt "
                "KV (local layers read the last 1024), 256-slot canvas, tied "
                "LM head over 262144 tokens, 8 passes")

C4 = Workload(
    name="C4-30L-bf16-kv131072",
    model=C3.model,
    batch=1, prompt_len=131072, n_steps=8, seed=3,
    description="C3's stack with a 131072-position prompt KV on global layers")

C5 = Workload(
    name="C5-30L-bf16-4x256-kv32768",
    model=C3.model,
    batch=4, prompt_len=32768, n_steps=12, seed=4,
    router_std=2.0 / 2048 ** 0.5,
    prelock=(0, 64, 128, 192),
    description="4 independent canvases, each with its own 32768-position prompt "
                "KV, 12 passes, 0/25/50/75% of positions pre-locked, router "
                "logits ~N(0, 2^2)")

ALL = {w.name: w for w in (C1, C2, C3, C4, C5)}
BY_ID = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}


def shrink(w: Workload, **model_kw) -> Workload:
    """A copy of ``w`` with some model fields replaced (small test shapes)."""
    wkw = {k: model_kw.pop(k) for k in list(model_kw) if k in
           ("batch", "prompt_len", "n_steps", "seed", "prelock", "router_std", "name")}
    return dataclasses.replace(w, model=dataclasses.replace(w.model, **model_kw), **wkw)
