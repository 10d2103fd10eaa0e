"""Plain float64 reference of one canvas denoise pass and of a block of passes.

Test infrastructure only (see the package docstring for the sources and the
rounding points).  Every function follows one step of the method in the
order the pages give it; numpy's matmul, sort and exp are the only library
primitives used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Value of bf16 bit patterns: the bf16 word is the upper half of a
    float32 word with the lower 16 bits zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps float32's 8 exponent bits and 7 of its mantissa bits.  On the
    float64 bit pattern that means keeping the top 7 of the 52 mantissa bits
    and rounding on the 45 dropped ones (valid for normal numbers inside
    float32's exponent range; the method's values never leave it)."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64).copy()
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    bits = bits + (np.uint64((1 << 44) - 1) + lsb)
    bits &= ~np.uint64((1 << 45) - 1)
    out = bits.view(np.float64)
    return np.where(x == 0.0, x, out)


def _identity(x: np.ndarray) -> np.ndarray:
    return x


# --------------------------------------------------------------------------
# per-step functions
# --------------------------------------------------------------------------


def rmsnorm(z: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMS normalisation over the last axis with a (1 + w) scale.

    The norm sandwich (input_layernorm, post_attention_layernorm,
    pre_feedforward_layernorm, final norm) is listed in [HandsOn] "Detailed
    Specs"; the RMS form and the (1 + w) gain are the Gemma-family convention
    the decoder inherits."""
    ms = np.mean(z * z, axis=-1, keepdims=True)
    return z / np.sqrt(ms + eps) * (1.0 + w)


def rope(x: np.ndarray, pos: np.ndarray, theta: float, n_rot: int) -> np.ndarray:
    """Rotary position encoding, rotate-half pairing.

    ``x`` is ``[n, heads, D]``, ``pos`` is ``[n]``.  Pair ``(j, j + D/2)`` is
    rotated by the angle ``pos * theta**(-2j/D)`` for ``j < n_rot`` and left
    alone otherwise: ``n_rot = D/2`` is plain RoPE (local layers),
    ``n_rot < D/2`` is p-RoPE, which rotates only the highest-frequency
    fraction of the pairs (global layers) -- [HandsOn] "Detailed Specs",
    dual RoPE configuration."""
    n, h, D = x.shape
    half = D // 2
    out = x.copy()
    if n_rot <= 0:
        return out
    j = np.arange(n_rot, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]  # [n, n_rot]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[:, :, :n_rot]
    b = x[:, :, half:half + n_rot]
    out[:, :, :n_rot] = a * c - b * s
    out[:, :, half:half + n_rot] = b * c + a * s
    return out


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                      return_probs: bool = False, mask: Optional[np.ndarray] = None):
    """One head of scaled dot-product attention.

    ``q [nq, D]``, ``k [nk, D]``, ``v [nk, D]``.  Without ``mask`` every query
    sees every key: no causal mask ([4xFaster] "What is Diffusion...": every
    token of the block can access all other tokens).  ``mask [nq, nk]``
    (True = visible) hides keys from queries."""
    s = (q @ k.T) * scale
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    o = p @ v
    return (o, p) if return_probs else o


def attention_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Grouped-query attention over all heads.

    ``q [nq, Hq, D]``; ``k, v [nk, Hkv, D]``.  Query head ``h`` reads KV head
    ``h // (Hq / Hkv)`` ([HandsOn] "Detailed Specs": global attention uses
    group query attention).  Returns ``[nq, Hq, D]``."""
    nq, Hq, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    for h in range(Hq):
        g = h // group
        out[:, h, :] = softmax_attention(q[:, h, :], k[:, g, :], v[:, g, :], scale, mask=mask)
    return out


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh form (the activation named Gelu_Pytorch_tanh in [HandsOn]
    "Detailed Specs")."""
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def route(r: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k expert choice and gates.

    ``r [M, E]`` router logits.  Each row keeps the ``k`` experts with the
    largest logits, ordered by (logit descending, expert index ascending) so
    equal logits go to the lower index; gates are the softmax over the kept
    logits.  128 experts with 8 active per token: [4xFaster] "DiffusionGemma's
    Technical Architecture"."""
    M, E = r.shape
    order = np.argsort(-r, axis=1, kind="stable")  # stable: ties keep lower e first
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(r, idx.astype(np.int64), axis=1)
    e = np.exp(sel - sel[:, :1])
    return idx, e / e.sum(axis=1, keepdims=True)


def expert_ffn(f: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               rnd: Callable[[np.ndarray], np.ndarray]) -> np.ndarray:
    """Gated expert MLP: down(gelu_tanh(f @ gate) * (f @ up)).

    ``rnd`` rounds the gated activation to the storage format of the
    workload before the down projection."""
    u = rnd(gelu_tanh(f @ wg) * (f @ wu))
    return u @ wd


def moe_block(f: np.ndarray, lw: Dict[str, np.ndarray], top_k: int,
              rnd: Callable[[np.ndarray], np.ndarray],
              route_override: Optional[Callable] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Routed MoE with one always-on shared expert.

    For every token ``t``: ``m_t = sum_s g[t,s] * FFN_{idx[t,s]}(f_t) +
    FFN_shared(f_t)``, the routed terms summed in slot order.  Tokens are
    grouped by expert only so that each expert's matmul is one library call;
    every token's result is the per-token definition above.

    Returns ``(m, r, idx, gates)``."""
    M = f.shape[0]
    r = f @ lw["router"]
    idx, gates = route(r, top_k)
    if route_override is not None:
        idx, gates = route_override(r, idx, gates)
    E = lw["w_gate"].shape[0]
    H = lw["w_down"].shape[2]
    y = np.zeros((M, top_k, H))
    for e in range(E):
        tt, ss = np.nonzero(idx == e)
        if tt.size == 0:
            continue
        y[tt, ss] = expert_ffn(f[tt], lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e], rnd)
    m = np.zeros((M, H))
    for s in range(top_k):
        m = m + gates[:, s:s + 1] * y[:, s]
    m = m + expert_ffn(f, lw["sh_gate"], lw["sh_up"], lw["sh_down"], rnd)
    return m, r, idx, gates


def lm_logits(h: np.ndarray, embed: np.ndarray) -> np.ndarray:
    """Logits of the tied LM head: ``h @ embed.T`` (embed_tokens shared with
    lm_head.weight, [HandsOn] "Detailed Specs", weight sharing)."""
    return h @ embed.T


def argmax_conf(logits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row greedy prediction and its confidence.

    ``pred`` is the lowest vocabulary id with the largest logit; ``conf`` is
    that token's softmax probability at temperature 1, ``1 / sum_v
    exp(l_v - l_max)`` -- the probability distribution from which the model
    judges which tokens are final ([HandsOn] "Detailed Specs", decoder)."""
    logits = np.asarray(logits, dtype=np.float64)
    pred = np.argmax(logits, axis=1).astype(np.int32)  # first index of the maximum
    mx = logits.max(axis=1, keepdims=True)
    conf = 1.0 / np.exp(logits - mx).sum(axis=1)
    return pred, conf


def lock_count(remaining: int, steps_left: int) -> int:
    """Positions to lock in a pass: ``ceil(remaining / steps_left)``, so that a
    canvas is fully resolved after its fixed number of passes ([Experimental]
    "How Text Diffusion Actually Works": a small, fixed number of passes)."""
    if steps_left < 1:
        raise ValueError("steps_left must be >= 1")
    return -(-remaining // steps_left)


def lock_select(conf: np.ndarray, pred: np.ndarray, tokens: np.ndarray, locked: np.ndarray,
                steps_left: Sequence[int]) -> Tuple[np.ndarray, np.ndarray, List[np.ndarray]]:
    """Lock the most confident unlocked positions of every canvas; remask the rest.

    Per canvas: ``k = ceil(remaining / steps_left)`` unlocked positions with
    the highest (confidence, then lower position) take their predicted token
    and become locked; locked tokens never change and serve as context for the
    following passes ([4xFaster] "What is Diffusion...": correct tokens are
    locked in; [ParadigmShift] "Analysis of Implications": uncertain tokens
    are re-noised).  Unselected positions keep their placeholder token.

    ``conf, pred, tokens, locked`` are ``[B, N]``.  Returns new copies of
    ``tokens, locked`` and the selected positions of every canvas."""
    tokens = tokens.copy()
    locked = locked.copy()
    chosen = []
    for b in range(tokens.shape[0]):
        free = np.nonzero(locked[b] == 0)[0]
        k = lock_count(free.size, int(steps_left[b]))
        # sort unlocked positions by (conf descending, position ascending)
        order = sorted(free.tolist(), key=lambda i: (-float(conf[b, i]), i))
        sel = np.array(order[:k], dtype=np.int64)
        tokens[b, sel] = pred[b, sel]
        locked[b, sel] = 1
        chosen.append(sel)
    return tokens, locked, chosen


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------


def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


_EXPERT_STACKS = ("w_gate", "w_up", "w_down")


_SHARED = ("sh_gate", "sh_up", "sh_down")


def _expert_values(a: np.ndarray, expert_format: str) -> np.ndarray:
    """The values an expert matrix ``[in, out]`` stands for in its stored
    format: itself, or its MXFP4 quantisation along ``in``."""
    if expert_format == "mxfp4":
        from .quant import mxfp4_weight
        return mxfp4_weight(a)
    return a


class _ExpertStack:
    """``[E, in, out]`` expert weights kept in their stored form; indexing one
    expert returns its float64 matrix."""

    def __init__(self, raw: np.ndarray, dtype: str, expert_format: str = "native"):
        self.raw, self.dtype, self.shape, self.fmt = raw, dtype, raw.shape, expert_format

    def __getitem__(self, e: int) -> np.ndarray:
        return _expert_values(_to_f64(self.raw[e], self.dtype), self.fmt)

    def __array__(self, dtype=None, copy=None):
        a = np.stack([self[e] for e in range(self.shape[0])])
        return a if dtype is None else a.astype(dtype)


@dataclass
class OracleWeights:
    """Weights as float64 arrays, fetched layer by layer from a provider so
    that a 30-layer stack never has to be widened to float64 all at once.

    ``layer_fn(l)`` returns the raw per-layer dict (bf16 bits or float32) in
    the math layout ``y = x @ W``; ``embed`` and ``norm_final`` likewise."""

    dtype: str
    layer_fn: Callable[[int], Dict[str, np.ndarray]]
    embed_raw: Optional[np.ndarray] = None
    norm_final_raw: Optional[np.ndarray] = None
    _embed: Optional[np.ndarray] = None
    _cache: Dict[int, Dict[str, np.ndarray]] = field(default_factory=dict)
    cache_layers: bool = False
    # storage of the routed and shared experts' matrices: "native" (dtype) or
    # "mxfp4" (quantised along the input dimension, see quant.py)
    expert_format: str = "native"

    def layer(self, l: int) -> Dict[str, np.ndarray]:
        if l in self._cache:
            return self._cache[l]
        raw = self.layer_fn(l)
        # per-expert stacks are widened one expert at a time, when an expert is used
        out = {}
        for k, v in raw.items():
            if k in _EXPERT_STACKS:
                out[k] = _ExpertStack(v, self.dtype, self.expert_format)
            elif k in _SHARED:
                out[k] = _expert_values(_to_f64(v, self.dtype), self.expert_format)
            else:
                out[k] = _to_f64(v, self.dtype)
        if self.cache_layers:
            self._cache[l] = out
        return out

    def embed(self) -> np.ndarray:
        if self._embed is None:
            self._embed = _to_f64(self.embed_raw, self.dtype)
        return self._embed

    def embed_rows(self, ids: np.ndarray) -> np.ndarray:
        if self._embed is not None:
            return self._embed[ids]
        return _to_f64(self.embed_raw[ids], self.dtype)

    def norm_final(self) -> np.ndarray:
        return _to_f64(self.norm_final_raw, self.dtype)


# --------------------------------------------------------------------------
# decisions taken by the GPU, for the shadowed comparison
# --------------------------------------------------------------------------


@dataclass
class Shadow:
    """GPU decisions of one pass and the margins within which the oracle
    adopts them (a decision whose oracle margin is below ``delta`` has more
    than one correct outcome at the precision of the GPU path).

    ``route_idx[l]`` is the GPU's ``[M, k]`` expert choice at layer ``l``;
    ``pred`` its ``[B, N]`` argmax; ``locked_after`` its locked mask after
    the pass."""

    route_idx: Optional[Sequence[np.ndarray]] = None
    pred: Optional[np.ndarray] = None
    locked_after: Optional[np.ndarray] = None
    delta_route: float = 0.0
    delta_logit: float = 0.0
    delta_conf: float = 0.0
    adopted: Dict[str, int] = field(default_factory=lambda: {"route": 0, "pred": 0, "lock": 0})
    max_margin: Dict[str, float] = field(default_factory=lambda: {"route": 0.0, "pred": 0.0, "lock": 0.0})
    failures: List[str] = field(default_factory=list)


def _shadow_route(sh: Shadow, layer: int):
    gidx_all = sh.route_idx[layer]

    def override(r, idx, gates):
        idx = idx.copy()
        gates = gates.copy()
        k = idx.shape[1]
        for t in range(r.shape[0]):
            go = set(int(e) for e in gidx_all[t])
            if go == set(int(e) for e in idx[t]):
                continue
            gl = np.array(sorted(go), dtype=np.int64)
            rest = np.setdiff1d(np.arange(r.shape[1]), gl)
            margin = float(r[t, rest].max() - r[t, gl].min())
            if len(go) == k and margin <= sh.delta_route:
                sh.adopted["route"] += 1
                sh.max_margin["route"] = max(sh.max_margin["route"], margin)
                # gates are recomputed from the oracle's own logits
                order = sorted(gl.tolist(), key=lambda e: (-r[t, e], e))
                idx[t] = order
                sel = r[t, order]
                ex = np.exp(sel - sel.max())
                gates[t] = ex / ex.sum()
            else:
                sh.failures.append(f"route layer {layer} token {t}: gpu {sorted(go)} "
                                   f"oracle {sorted(idx[t].tolist())} margin {margin:.3e}")
        return idx, gates

    return override


def adopt_pred(logits: np.ndarray, pred: np.ndarray, conf: np.ndarray, sh: Shadow) -> None:
    """Shadowed argmax: where the GPU's token differs from the oracle's, the
    oracle takes it when its own logit margin for the GPU's token (its best
    logit minus the GPU token's logit) is at most ``sh.delta_logit``, and then
    reports that token's probability as the confidence; otherwise the
    difference is a failure.  ``logits [B, N, V]``; ``pred, conf [B, N]`` are
    updated in place."""
    B, N = pred.shape
    for b in range(B):
        for i in range(N):
            gp = int(sh.pred[b, i])
            if gp == int(pred[b, i]):
                continue
            margin = float(logits[b, i, pred[b, i]] - logits[b, i, gp])
            if margin <= sh.delta_logit:
                sh.adopted["pred"] += 1
                sh.max_margin["pred"] = max(sh.max_margin["pred"], margin)
                pred[b, i] = gp
                conf[b, i] = 1.0 / np.exp(logits[b, i] - logits[b, i, gp]).sum()
            else:
                sh.failures.append(f"pred canvas {b} pos {i}: gpu {gp} oracle "
                                   f"{int(pred[b, i])} margin {margin:.3e}")


def adopt_locks(conf: np.ndarray, pred: np.ndarray, tokens: np.ndarray, locked: np.ndarray,
                new_tokens: np.ndarray, new_locked: np.ndarray, chosen: Sequence[np.ndarray],
                sh: Shadow) -> None:
    """Shadowed lock step: where the GPU locked another set of positions than
    the oracle's ``chosen``, the oracle takes the GPU's set when it has the
    same size and the most confident position the GPU left unlocked beats the
    least confident one it locked by at most ``sh.delta_conf`` (by the oracle's
    confidences); otherwise the difference is a failure.  ``new_tokens,
    new_locked`` are updated in place."""
    B = tokens.shape[0]
    for b in range(B):
        gsel = set(np.nonzero((sh.locked_after[b] == 1) & (locked[b] == 0))[0].tolist())
        osel = set(chosen[b].tolist())
        if gsel == osel:
            continue
        free = np.nonzero(locked[b] == 0)[0]
        rest = [i for i in free.tolist() if i not in gsel]
        if gsel:
            worst_in = float(min(conf[b, list(gsel)]))
            best_out = float(max(conf[b, rest])) if rest else -np.inf
            margin = best_out - worst_in
        else:
            margin = np.inf
        if len(gsel) == len(osel) and margin <= sh.delta_conf:
            sh.adopted["lock"] += 1
            sh.max_margin["lock"] = max(sh.max_margin["lock"], float(margin))
            sel = np.array(sorted(gsel), dtype=np.int64)
            new_tokens[b] = tokens[b]
            new_locked[b] = locked[b]
            new_tokens[b, sel] = pred[b, sel]
            new_locked[b, sel] = 1
        else:
            sh.failures.append(f"lock canvas {b}: margin {margin:.3e}")


# --------------------------------------------------------------------------
# one layer, one pass, one block
# --------------------------------------------------------------------------


def qkv_rope(a: np.ndarray, lw: Dict[str, np.ndarray], cfg, layer: int,
             prompt_lens: Sequence[int], rnd: Callable[[np.ndarray], np.ndarray]):
    """q/k/v projections of the normalised input ``a [B*N, H]`` with RoPE at
    canvas positions ``prompt_len + i`` (p-RoPE on global layers), rounded to
    the storage format.  Returns ``q [B, N, Hq, D]``, ``k, v [B, N, Hkv, D]``."""
    N = cfg.canvas_len
    B = len(prompt_lens)
    D, Hq, Hkv = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    n_rot = int(cfg.prope_frac * (D // 2)) if cfg.is_global(layer) else D // 2
    q = a @ lw["wq"]
    k = a @ lw["wk"]
    v = a @ lw["wv"]
    qs, ks, vs = [], [], []
    for b in range(B):
        rows = slice(b * N, (b + 1) * N)
        pos = prompt_lens[b] + np.arange(N)
        qs.append(rnd(rope(q[rows].reshape(N, Hq, D), pos, cfg.rope_theta, n_rot)))
        ks.append(rnd(rope(k[rows].reshape(N, Hkv, D), pos, cfg.rope_theta, n_rot)))
        vs.append(rnd(v[rows].reshape(N, Hkv, D)))
    return np.stack(qs), np.stack(ks), np.stack(vs)


def canvas_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     prompt_kv: Sequence[Tuple[np.ndarray, np.ndarray]],
                     rnd: Callable[[np.ndarray], np.ndarray], canvas_keys: bool = True,
                     causal: bool = False) -> np.ndarray:
    """One softmax per canvas query over the keys [prompt KV ; all canvas
    positions]: the canvas attends to itself bidirectionally and to the
    cached prompt context ([4xFaster] "DiffusionGemma's Technical
    Architecture").  ``q [B, N, Hq, D]``; ``k, v [B, N, Hkv, D]``;
    ``prompt_kv[b] = (K, V)`` each ``[len, Hkv, D]``.  Returns ``o [B*N, Hq*D]``
    rounded to the storage format.

    ``causal``: canvas position i sees the prompt keys and canvas keys j <= i
    only -- the causal context building over a finished block ([HandsOn] "How
    Is This Different from Previous Models?", Figure 3)."""
    B, N, Hq, D = q.shape
    o = np.empty((B * N, Hq * D))
    for b in range(B):
        Kp, Vp = prompt_kv[b]
        if canvas_keys:
            keys = np.concatenate([Kp, k[b]], axis=0)
            vals = np.concatenate([Vp, v[b]], axis=0)
        else:
            keys, vals = Kp, Vp
        mask = None
        if causal and canvas_keys:
            Lp = Kp.shape[0]
            i = np.arange(N)[:, None]
            j = np.arange(Lp + N)[None, :]
            mask = (j < Lp) | (j - Lp <= i)
        o[b * N:(b + 1) * N] = rnd(attention_heads(q[b], keys, vals, mask)).reshape(N, Hq * D)
    return o


def layer_forward(x: np.ndarray, lw: Dict[str, np.ndarray], cfg, layer: int,
                  prompt_kv: Sequence[Tuple[np.ndarray, np.ndarray]],
                  prompt_lens: Sequence[int], rnd: Callable[[np.ndarray], np.ndarray],
                  route_override: Optional[Callable] = None,
                  canvas_keys: bool = True, causal: bool = False) -> Tuple[np.ndarray, dict]:
    """One decoder layer over every canvas position at once.

    ``x [B*N, H]`` residual stream; ``prompt_kv[b] = (K, V)``, each
    ``[len, Hkv, D]``, the cached prompt keys/values of canvas ``b`` visible to
    this layer (the whole prompt on global layers, its last ``window``
    positions on sliding-window layers).

    Steps, in order:
      1. a = RMSNorm(x) (input_layernorm), stored as bf16 in bf16 workloads;
      2. q, k, v = a @ Wq, a @ Wk, a @ Wv; RoPE at canvas positions
         ``prompt_len + i`` (p-RoPE on global layers);
      3. one softmax over the keys [prompt KV ; all canvas positions]
         (bidirectional canvas attention plus the encoder's cached context,
         with q/k/v/o shared between encoder and decoder, [HandsOn] "Detailed
         Specs");
      4. x += RMSNorm(o @ Wo) (post_attention_layernorm);
      5. f = RMSNorm(x) (pre_feedforward_layernorm);
      6. m = routed top-k MoE + shared expert;
      7. x += RMSNorm(m) (post-FFN norm; plain x += m when disabled).

    ``causal`` masks later canvas keys (block commit).  The returned info
    carries the canvas ``k, v [B, N, Hkv, D]`` as stored (after RoPE).
    """
    eps = cfg.rms_eps
    a = rnd(rmsnorm(x, lw["norm_in"], eps))
    q, k, v = qkv_rope(a, lw, cfg, layer, prompt_lens, rnd)
    o = canvas_attention(q, k, v, prompt_kv, rnd, canvas_keys, causal)
    x = x + rmsnorm(o @ lw["wo"], lw["norm_pa"], eps)
    f = rnd(rmsnorm(x, lw["norm_pf"], eps))
    m, r, idx, gates = moe_block(f, lw, cfg.top_k, rnd, route_override)
    if cfg.post_ffn_norm:
        x = x + rmsnorm(m, lw["norm_pf2"], eps)
    else:
        x = x + m
    return x, {"router_logits": r, "route_idx": idx, "gates": gates, "k": k, "v": v}


def _rounder(cfg):
    return bf16_round if cfg.dtype == "bf16" else _identity


def forward_hidden(x: np.ndarray, weights: OracleWeights, cfg, prompt_kv_fn, prompt_lens,
                   layers: Optional[Sequence[int]] = None, trace: Optional[list] = None,
                   shadow: Optional[Shadow] = None) -> np.ndarray:
    """Decoder layers only, on a given residual stream ``x [B*N, H]``.

    ``prompt_kv_fn(l, b)`` returns the float64 ``(K, V)`` of layer ``l``,
    canvas ``b``."""
    rnd = _rounder(cfg)
    B = len(prompt_lens)
    for l in (range(cfg.n_layers) if layers is None else layers):
        kv = [prompt_kv_fn(l, b) for b in range(B)]
        ov = _shadow_route(shadow, l) if (shadow is not None and shadow.route_idx is not None) else None
        x, info = layer_forward(x, weights.layer(l), cfg, l, kv, prompt_lens, rnd, ov)
        if trace is not None:
            trace.append(info)
    return x


def denoise_pass(tokens: np.ndarray, locked: np.ndarray, steps_left: Sequence[int],
                 weights: OracleWeights, cfg, prompt_kv_fn, prompt_lens: Sequence[int],
                 shadow: Optional[Shadow] = None, trace: Optional[list] = None):
    """One denoise pass over ``B`` canvases of ``N`` slots.

    embed -> decoder stack -> final norm -> tied LM head -> greedy prediction
    and confidence -> lock the most confident, remask the rest.

    Returns ``(tokens, locked, pred, conf, logits_hidden)`` where
    ``logits_hidden`` is the final normalised hidden state ``h``."""
    B, N = tokens.shape
    rnd = _rounder(cfg)
    # embedding lookup, no scale ([HandsOn] "Detailed Specs": embed_tokens)
    x = weights.embed_rows(tokens.reshape(-1).astype(np.int64)).copy()
    x = forward_hidden(x, weights, cfg, prompt_kv_fn, prompt_lens, trace=trace, shadow=shadow)
    h = rnd(rmsnorm(x, weights.norm_final(), cfg.rms_eps))
    logits = lm_logits(h, weights.embed())
    pred, conf = argmax_conf(logits)
    pred = pred.reshape(B, N)
    conf = conf.reshape(B, N)
    if shadow is not None and shadow.pred is not None:
        adopt_pred(logits.reshape(B, N, -1), pred, conf, shadow)
    new_tokens, new_locked, chosen = lock_select(conf, pred, tokens, locked, steps_left)
    if shadow is not None and shadow.locked_after is not None:
        adopt_locks(conf, pred, tokens, locked, new_tokens, new_locked, chosen, shadow)
    return new_tokens, new_locked, pred, conf, h


def generate_block(tokens: np.ndarray, locked: np.ndarray, n_steps: int,
                   weights: OracleWeights, cfg, prompt_kv_fn, prompt_lens: Sequence[int],
                   shadows: Optional[Sequence[Shadow]] = None, history: Optional[list] = None):
    """A fixed number of passes; pass ``t`` runs with ``steps_left = n_steps
    - t`` so that every position is locked after the last pass ([Experimental]
    "How Text Diffusion Actually Works"; [4xFaster] "What is Diffusion...")."""
    B = tokens.shape[0]
    for t in range(n_steps):
        sh = shadows[t] if shadows is not None else None
        tokens, locked, pred, conf, _ = denoise_pass(
            tokens, locked, [n_steps - t] * B, weights, cfg, prompt_kv_fn, prompt_lens, shadow=sh)
        if history is not None:
            history.append((tokens.copy(), locked.copy(), pred, conf))
    return tokens, locked


# --------------------------------------------------------------------------
# block continuation
# --------------------------------------------------------------------------


def commit_block(tokens: np.ndarray, weights: OracleWeights, cfg, prompt_kv_fn,
                 prompt_lens: Sequence[int], shadow: Optional[Shadow] = None,
                 trace: Optional[list] = None):
    """K/V of a finished block, to be appended to the prompt cache.

    After a block is resolved the model builds the context for the next
    canvas the way a causal model would ([HandsOn] "How Is This Different from
    Previous Models?", Figure 3): the decoder stack runs once over the block's
    tokens at positions ``prompt_len + i`` with the cached context visible and
    causal attention inside the block.  Returns, per layer, the block's
    ``(k, v)``, each ``[B, N, Hkv, D]`` as stored (k after RoPE)."""
    B, N = tokens.shape
    rnd = _rounder(cfg)
    x = weights.embed_rows(tokens.reshape(-1).astype(np.int64)).copy()
    out = []
    for l in range(cfg.n_layers):
        kv = [prompt_kv_fn(l, b) for b in range(B)]
        # layers whose GPU routing record is None keep the oracle's own routing
        shadowed = shadow is not None and shadow.route_idx is not None and shadow.route_idx[l] is not None
        ov = _shadow_route(shadow, l) if shadowed else None
        x, info = layer_forward(x, weights.layer(l), cfg, l, kv, prompt_lens, rnd, ov, causal=True)
        if trace is not None:
            trace.append(info)
        out.append((info["k"], info["v"]))
    return out


def append_kv(K_old: np.ndarray, V_old: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray,
              visible: int) -> Tuple[np.ndarray, np.ndarray]:
    """A layer's cache after a block: ``[old ; block]`` along positions
    (``[len, Hkv, D]``), of which the last ``visible`` positions stay (all of
    them on global layers, the last ``window`` on sliding-window layers,
    [HandsOn] "Detailed Specs")."""
    K = np.concatenate([K_old, k_blk], axis=0)
    V = np.concatenate([V_old, v_blk], axis=0)
    return K[K.shape[0] - visible:], V[V.shape[0] - visible:]
