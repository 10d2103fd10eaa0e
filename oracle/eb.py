"""Entropy-bounded (EB) denoising with a temperature schedule and adaptive
stopping: the sampler recommended for DiffusionGemma.

Test infrastructure only: the CPU oracle of the EB path.  Nothing in the
product imports it.

Sources (page title, section):
  [4xFaster] "DiffusionGemma: The Diffusion Era Begins with 4x Faster Text
      Generation" -- "Recommended Inference Settings": EB denoising, at most
      48 steps, temperature decaying linearly from 0.8 to 0.4, entropy bound
      0.1, adaptive stopping once the average canvas entropy is below 0.005
      and the high-probability tokens stay stable for 2 consecutive steps.
  [ParadigmShift] "DiffusionGemma: Exploring the Paradigm Shift in
      Non-Autoregressive Language Modeling" -- "Serving in Production: The
      Role of vLLM": the 0.005 entropy threshold halts a block once two
      consecutive passes agree.

The pages name the sampler and its parameters, not its steps; the readings
taken here:
  * pass t of at most T: tau_t = 0.8 + (0.4 - 0.8) t / (T - 1);
  * per position, p = softmax(logits / tau_t) and H = -sum_v p_v log p_v
    (nats); a sample x ~ p by the Gumbel-max rule, argmax_v (l_v / tau + g_v)
    with counter-based Gumbel noise g (ties: lower id);
  * EB step: the unlocked positions in order of increasing entropy (ties:
    lower position) are locked while the running sum of their entropies
    stays within the bound, and at least one is; a locked position takes its
    sample and never changes again;
  * adaptive stop, after each pass: the mean entropy over the canvas's
    positions is below 0.005 and every position's greedy token (the argmax
    of its logits) equals that of the previous pass; then every unlocked
    position takes its greedy token and the canvas is done;
  * the last allowed pass locks every remaining position with its sample.

Precision: the entropies, the softmax and the logits are float64; the
discrete decisions (the sampled id, the entropy order, the running sum
against the bound, the mean against the stop threshold) are taken in
float32, the precision of the GPU path, as the rule for decisions the
method leaves open: H is rounded to float32 and summed in float32 in the
stated order.

Noise: Philox4x32-10 (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011).  For canvas b with seed s_b,
block k, pass t, position i and vocabulary id v: key (s_b, k), counter
((v >> 6) * 16 + (v & 15), i, t, 0), output word (v >> 4) & 3; the word's
top 23 bits n give u = (2n + 1) 2^-24 in (0, 1), and g = -log(-log u),
rounded to float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

T_MAX = 48
TAU_FIRST, TAU_LAST = 0.8, 0.4
ENTROPY_BOUND = 0.1
STOP_ENTROPY = 0.005

# --------------------------------------------------------------------------
# Philox4xW-R (Salmon et al. 2011): W-bit words, R rounds of two
# multiply-high/low steps with a Weyl sequence of round keys
# --------------------------------------------------------------------------

PHILOX = {
    32: dict(M=(0xD2511F53, 0xCD9E8D57), W=(0x9E3779B9, 0xBB67AE85)),
    64: dict(M=(0xD2E7470EE14C6C93, 0xCA5A826395121157), W=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)),
}
_U32 = np.uint64(0xFFFFFFFF)


def _mulhilo(bits: int, a: int, b: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(high, low) words of the 2W-bit products a * b."""
    if bits == 32:  # the product of two 32-bit words fits in 64 bits
        p = np.uint64(a) * b
        return p >> np.uint64(32), p & _U32
    a0, a1 = np.uint64(a & 0xFFFFFFFF), np.uint64(a >> 32)
    b0, b1 = b & _U32, b >> np.uint64(32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> np.uint64(32)) + (p01 & _U32) + (p10 & _U32)
    lo = (p00 & _U32) | ((mid & _U32) << np.uint64(32))
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4(counter: np.ndarray, key: Sequence[int], bits: int = 32, rounds: int = 10) -> np.ndarray:
    """Philox4x``bits``-``rounds`` of ``counter [..., 4]`` under ``key``
    (two words); returns the four output words ``[..., 4]`` (uint64 holding
    W-bit values)."""
    p = PHILOX[bits]
    mask = (1 << bits) - 1
    x = [np.asarray(counter[..., j], dtype=np.uint64) for j in range(4)]
    k0, k1 = int(key[0]) & mask, int(key[1]) & mask
    with np.errstate(over="ignore"):
        for _ in range(rounds):
            hi0, lo0 = _mulhilo(bits, p["M"][0], x[0])
            hi1, lo1 = _mulhilo(bits, p["M"][1], x[2])
            x = [hi1 ^ x[1] ^ np.uint64(k0), lo1, hi0 ^ x[3] ^ np.uint64(k1), lo0]
            k0 = (k0 + p["W"][0]) & mask
            k1 = (k1 + p["W"][1]) & mask
    return np.stack(x, axis=-1)


def uniform_from_bits(word: np.ndarray) -> np.ndarray:
    """u = (2n + 1) 2^-24 from the top 23 bits n of a 32-bit word: exact in
    float32, strictly inside (0, 1)."""
    n = (np.asarray(word, dtype=np.uint64) >> np.uint64(9)).astype(np.float64)
    return ((2.0 * n + 1.0) * 2.0 ** -24).astype(np.float32)


def gumbel_noise(seed: int, block: int, t: int, positions: Sequence[int], V: int) -> np.ndarray:
    """Gumbel noise ``[len(positions), V]`` (float32) of one canvas and pass."""
    v = np.arange(V, dtype=np.uint64)
    call = (v >> np.uint64(6)) * np.uint64(16) + (v & np.uint64(15))
    word = ((v >> np.uint64(4)) & np.uint64(3)).astype(np.int64)
    pos = np.asarray(positions, dtype=np.uint64).reshape(-1)
    g = np.empty((pos.size, V), dtype=np.float32)
    step = max(1, (1 << 22) // max(V, 1))  # positions per chunk, to bound the memory
    for p0 in range(0, pos.size, step):
        pc = pos[p0:p0 + step]
        ctr = np.zeros((pc.size, V, 4), dtype=np.uint64)
        ctr[..., 0] = call[None, :]
        ctr[..., 1] = pc[:, None]
        ctr[..., 2] = np.uint64(t)
        out = philox4(ctr, (seed, block), bits=32)
        bits = np.take_along_axis(out, word[None, :, None], axis=2)[..., 0]
        u = uniform_from_bits(bits).astype(np.float64)
        g[p0:p0 + step] = -np.log(-np.log(u))
    return g


# --------------------------------------------------------------------------
# the sampler's quantities
# --------------------------------------------------------------------------

def temperature(t: int, t_max: int = T_MAX) -> float:
    """Linear decay from 0.8 at the first pass to 0.4 at the last allowed one."""
    if t_max <= 1:
        return TAU_FIRST
    return TAU_FIRST + (TAU_LAST - TAU_FIRST) * t / (t_max - 1)


def _softmax_z(logits: np.ndarray, tau: float) -> Tuple[np.ndarray, np.ndarray]:
    z = np.asarray(logits, dtype=np.float64) / tau
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=1, keepdims=True), z


def entropy(logits: np.ndarray, tau: float) -> np.ndarray:
    """Entropy (nats) of softmax(logits / tau) per row, from its definition."""
    p, _ = _softmax_z(logits, tau)
    with np.errstate(divide="ignore", invalid="ignore"):
        return -np.where(p > 0, p * np.log(p), 0.0).sum(axis=1)


def entropy_slack(logits: np.ndarray, tau: float, dlogit: float) -> np.ndarray:
    """First-order bound on how far each row's entropy moves when every logit
    moves by at most ``dlogit``: dH/dz_v = -p_v (z_v - E_p[z]), so |dH| <=
    (dlogit / tau) E_p|z - E_p[z]|."""
    p, z = _softmax_z(logits, tau)
    mean = (p * z).sum(axis=1, keepdims=True)
    return (dlogit / tau) * (p * np.abs(z - mean)).sum(axis=1)


def sample_scores(logits: np.ndarray, tau: float, noise: np.ndarray) -> np.ndarray:
    """l_v * f32(1/tau) + g_v in float32, the product and the sum rounded
    separately."""
    inv = np.float32(1.0 / tau)
    return (np.asarray(logits, dtype=np.float64).astype(np.float32) * inv).astype(np.float32) + noise


def sample(logits: np.ndarray, tau: float, noise: np.ndarray) -> np.ndarray:
    """Gumbel-max sample per row: the argmax of the scores (ties: lower id)."""
    return np.argmax(sample_scores(logits, tau, noise), axis=1).astype(np.int32)


def eb_select(H: np.ndarray, free: Sequence[int], bound: float = ENTROPY_BOUND) -> np.ndarray:
    """Positions an EB step locks: the unlocked positions ``free`` in order of
    increasing entropy (ties: lower position), while the float32 running sum
    of their entropies stays within ``bound``; at least one."""
    H32 = np.asarray(H, dtype=np.float64).astype(np.float32)
    b32 = np.float32(bound)
    order = sorted((int(i) for i in free), key=lambda i: (H32[i], i))
    sel: List[int] = []
    run = np.float32(0.0)
    for i in order:
        run = np.float32(run + H32[i])
        if sel and run > b32:
            break
        sel.append(i)
    return np.array(sel, dtype=np.int64)


def mean_entropy32(H: np.ndarray) -> np.float32:
    """Mean entropy of a canvas in float32: the sum in position order, then
    one division by the number of positions."""
    s = np.float32(0.0)
    for h in np.asarray(H, dtype=np.float64).astype(np.float32):
        s = np.float32(s + h)
    return np.float32(s / np.float32(len(H)))


# --------------------------------------------------------------------------
# one EB update from logits, and the loop over passes
# --------------------------------------------------------------------------

@dataclass
class EBState:
    """Per canvas: the greedy tokens of the previous pass (None before the
    first) and whether the canvas is done."""
    B: int
    prev_pred: List[Optional[np.ndarray]] = field(default_factory=list)
    done: Optional[np.ndarray] = None

    def __post_init__(self):
        if not self.prev_pred:
            self.prev_pred = [None] * self.B
        if self.done is None:
            self.done = np.zeros(self.B, dtype=bool)


@dataclass
class EBShadow:
    """GPU decisions of one pass and the margins within which the oracle
    adopts them, for logits that differ from the oracle's by up to
    ``dlogit``: ``sample``/``pred`` ``[B, N]``, ``locked_after`` ``[B, N]``
    and the stop decisions ``stopped`` ``[B]``."""
    sample: Optional[np.ndarray] = None
    pred: Optional[np.ndarray] = None
    locked_after: Optional[np.ndarray] = None
    stopped: Optional[np.ndarray] = None
    dlogit: float = 0.0
    adopted: Dict[str, int] = field(default_factory=lambda: {"sample": 0, "pred": 0, "lock": 0, "stop": 0})
    failures: List[str] = field(default_factory=list)


def _adopt_argmax(score: np.ndarray, mine: np.ndarray, gpu: np.ndarray, delta: float, kind: str,
                  b: int, sh: EBShadow) -> np.ndarray:
    out = mine.copy()
    for i in np.nonzero(mine != gpu)[0]:
        margin = float(score[i, mine[i]]) - float(score[i, gpu[i]])
        if margin <= delta:
            sh.adopted[kind] += 1
            out[i] = gpu[i]
        else:
            sh.failures.append(f"{kind} canvas {b} pos {i}: gpu {int(gpu[i])} oracle {int(mine[i])} "
                               f"margin {margin:.3e}")
    return out


def eb_set_plausible(H: np.ndarray, d: np.ndarray, free: np.ndarray, g: np.ndarray) -> bool:
    """Could the EB rule give the lock set ``g`` when each entropy H_i may
    move by up to d_i?  Each condition of the rule is checked at its most
    favourable end of the intervals."""
    gs = set(int(i) for i in g)
    if not gs or not gs <= set(int(i) for i in free):
        return False
    out = [int(i) for i in free if int(i) not in gs]
    if out and min(H[i] + d[i] for i in out) < max(H[i] - d[i] for i in gs):
        return False  # not a prefix of any admissible order
    if len(gs) > 1 and sum(H[i] - d[i] for i in gs) > ENTROPY_BOUND:
        return False  # over the bound whatever the error
    if out and sum(H[i] + d[i] for i in gs) + min(H[i] + d[i] for i in out) <= ENTROPY_BOUND:
        return False  # room for one more whatever the error
    return True


def eb_apply(H: np.ndarray, xs: np.ndarray, pred: np.ndarray, tokens: np.ndarray, locked: np.ndarray, t: int,
             t_max: int, prev_pred: Optional[np.ndarray], sel: Optional[np.ndarray] = None,
             stop: Optional[bool] = None):
    """The lock step of one canvas that is not done, from its entropies ``H``,
    samples ``xs`` and greedy tokens ``pred`` ``[N]``: the EB locks (every
    unlocked position at the last pass), then the stop rule against the
    previous pass's greedy tokens ``prev_pred`` (None before the first pass).
    ``sel`` / ``stop`` replace the rule's own decisions (shadowed
    comparison).  Returns new ``(tokens, locked)``, the positions the EB rule
    locked, the stop flag and whether the canvas is done."""
    tokens, locked = tokens.copy(), locked.copy()
    free = np.nonzero(locked == 0)[0]
    if stop is None:
        stable = prev_pred is not None and bool(np.array_equal(prev_pred, pred))
        stop = bool(stable and mean_entropy32(H) < np.float32(STOP_ENTROPY))
    if sel is None:
        sel = free if t >= t_max - 1 else eb_select(H, free)
    tokens[sel] = xs[sel]
    locked[sel] = 1
    if stop:
        rest = np.nonzero(locked == 0)[0]
        tokens[rest] = pred[rest]
        locked[rest] = 1
    return tokens, locked, sel, stop, bool(stop or locked.all())


def eb_update(logits: np.ndarray, tokens: np.ndarray, locked: np.ndarray, t: int, state: EBState,
              seeds: Sequence[int], block: int = 0, t_max: int = T_MAX, shadow: Optional[EBShadow] = None):
    """The sampler's step after the LM head, for ``B`` canvases.

    ``logits [B, N, V]``; ``tokens, locked [B, N]``.  Canvases already done
    are left as they are.  Returns new ``(tokens, locked)`` and a dict of the
    pass's per-canvas values (H, sample, pred, the positions the EB rule
    locked, the stop flag)."""
    B, N, V = logits.shape
    tau = temperature(t, t_max)
    tokens, locked = tokens.copy(), locked.copy()
    info: Dict[str, list] = {"tau": tau, "H": [], "sample": [], "pred": [], "selected": [], "stopped": []}
    for b in range(B):
        lb = np.asarray(logits[b], dtype=np.float64)
        H = entropy(lb, tau)
        noise = gumbel_noise(int(seeds[b]), block, t, np.arange(N), V)
        xs = sample(lb, tau, noise)
        pred = np.argmax(lb, axis=1).astype(np.int32)
        d = np.zeros(N)
        if shadow is not None:
            d = entropy_slack(lb, tau, shadow.dlogit) + 1e-6 * (1.0 + H)
            if shadow.sample is not None:
                score = sample_scores(lb, tau, noise).astype(np.float64)
                slack = shadow.dlogit / tau + 2e-6 * (1.0 + float(np.abs(score).max()))
                xs = _adopt_argmax(score, xs, shadow.sample[b], slack, "sample", b, shadow)
            if shadow.pred is not None:
                pred = _adopt_argmax(lb, pred, shadow.pred[b], shadow.dlogit, "pred", b, shadow)
        info["H"].append(H)
        info["sample"].append(xs)
        info["pred"].append(pred)
        if state.done[b]:
            info["selected"].append(np.zeros(0, dtype=np.int64))
            info["stopped"].append(False)
            continue
        prev = state.prev_pred[b]
        state.prev_pred[b] = pred
        free = np.nonzero(locked[b] == 0)[0]
        stable = prev is not None and bool(np.array_equal(prev, pred))
        stop = bool(stable and mean_entropy32(H) < np.float32(STOP_ENTROPY))
        if shadow is not None and shadow.stopped is not None and bool(shadow.stopped[b]) != stop:
            # the GPU's stop decision where the mean entropy is within its error of the threshold
            if stable and abs(float(H.mean()) - STOP_ENTROPY) <= float(d.mean()):
                shadow.adopted["stop"] += 1
                stop = bool(shadow.stopped[b])
            else:
                shadow.failures.append(f"stop canvas {b} pass {t}: gpu {bool(shadow.stopped[b])} oracle {stop}")
        sel = free if t >= t_max - 1 else eb_select(H, free)
        if shadow is not None and shadow.locked_after is not None and not stop and t < t_max - 1:
            g = np.nonzero((shadow.locked_after[b] == 1) & (locked[b] == 0))[0]
            if set(g.tolist()) != set(sel.tolist()):
                if eb_set_plausible(H, d, free, g):
                    shadow.adopted["lock"] += 1
                    sel = g
                else:
                    shadow.failures.append(f"EB lock set canvas {b} pass {t}")
        tokens[b], locked[b], sel, stop, done = eb_apply(H, xs, pred, tokens[b], locked[b], t, t_max, prev,
                                                         sel=sel, stop=stop)
        state.done[b] = done
        info["selected"].append(sel)
        info["stopped"].append(stop)
    return tokens, locked, info


def generate_block_eb(logits_fn: Callable[[np.ndarray, int], np.ndarray], tokens: np.ndarray,
                      locked: np.ndarray, seeds: Sequence[int], block: int = 0, t_max: int = T_MAX,
                      history: Optional[list] = None):
    """EB passes until every canvas is done; at most ``t_max``.

    ``logits_fn(tokens, t)`` gives the ``[B, N, V]`` logits of a pass (the
    decoder stack and the tied LM head for the model, or any stand-in).
    Returns ``(tokens, locked, passes)``."""
    B = tokens.shape[0]
    state = EBState(B)
    t = 0
    while t < t_max and not state.done.all():
        tokens, locked, info = eb_update(logits_fn(tokens, t), tokens, locked, t, state, seeds, block, t_max)
        if history is not None:
            history.append((tokens.copy(), locked.copy(), info))
        t += 1
    return tokens, locked, t


def model_logits_fn(weights, cfg, prompt_kv_fn, prompt_lens: Sequence[int]):
    """``logits_fn`` of the model: embed, decoder stack, final norm and the
    tied LM head of one pass (the same steps as the greedy pass)."""
    from .model import _rounder, forward_hidden, lm_logits, rmsnorm

    def fn(tokens: np.ndarray, t: int) -> np.ndarray:
        B, N = tokens.shape
        x = weights.embed_rows(tokens.reshape(-1).astype(np.int64)).copy()
        x = forward_hidden(x, weights, cfg, prompt_kv_fn, prompt_lens)
        h = _rounder(cfg)(rmsnorm(x, weights.norm_final(), cfg.rms_eps))
        return lm_logits(h, weights.embed()).reshape(B, N, -1)

    return fn
