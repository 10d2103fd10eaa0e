"""Pins of the CPU oracle to facts independent of its own code.

Every check here compares the oracle with a closed form, an invariant the
pages state, a different library routine, a hand-worked fixture under
``tests/golden/`` or exhaustive enumeration on tiny inputs -- chosen so that a
dropped term, a wrong sign, index or transpose in the oracle fails one of them.
"""
import dataclasses
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import model as om
from oracle.inputs import prompt_kv_fn, weights_for
from synth import C1, C3, C5, configs, gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- bf16 -----

def test_bf16_round_matches_torch_conversion():
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even
    rng = _rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # add exact halfway cases: low 16 bits == 0x8000
    u = x.view(np.uint32).copy()
    u[:5000] = (u[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = u.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = om.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_hand_cases():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert om.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even mantissa is 1+2^-6
    assert om.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert om.bf16_round(np.array([-(1.0 + 2.0 ** -8 + 2.0 ** -30)]))[0] == -(1.0 + 2.0 ** -7)
    assert om.bf16_round(np.array([0.0]))[0] == 0.0
    bits = np.array([0x3F80, 0xC000, 0x3E80], dtype=np.uint16)  # 1, -2, 0.25
    assert np.array_equal(om.bf16_bits_to_f64(bits), [1.0, -2.0, 0.25])


# ------------------------------------------------------------- rmsnorm -----

def test_rmsnorm_unit_rms_and_gain():
    rng = _rng(2)
    z = rng.standard_normal((7, 64)) * 5.0
    eps = 1e-6
    out = om.rmsnorm(z, np.zeros(64), eps)
    ms = np.mean(z * z, axis=1)
    # closed form: mean(out^2) = ms / (ms + eps)
    assert np.allclose(np.mean(out * out, axis=1), ms / (ms + eps), rtol=1e-12)
    assert np.allclose(np.sqrt(np.mean(out * out, axis=1)), 1.0, atol=1e-6)
    # (1 + w) gain, per channel
    w = rng.standard_normal(64) * 0.1
    assert np.allclose(om.rmsnorm(z, w, eps), out * (1.0 + w), rtol=1e-12)
    # scale invariance up to eps
    assert np.allclose(om.rmsnorm(3.0 * z, w, 0.0), om.rmsnorm(z, w, 0.0), rtol=1e-12)


# ---------------------------------------------------------------- rope -----

def test_rope_worked_example():
    # D = 8, theta = 10000: pair j = 1 has frequency 10000^(-2/8) = 0.1, so at
    # position 3 its angle is 0.3 rad; pair (1, 5) of e_1 becomes (cos .3, sin .3)
    x = np.zeros((1, 1, 8))
    x[0, 0, 1] = 1.0
    out = om.rope(x, np.array([3]), 10000.0, 4)
    exp = np.zeros(8)
    exp[1], exp[5] = math.cos(0.3), math.sin(0.3)
    assert np.allclose(out[0, 0], exp, atol=1e-15)
    # the second element of a pair rotates the other way: e_5 -> (-sin, cos)
    y = np.zeros((1, 1, 8))
    y[0, 0, 5] = 1.0
    out = om.rope(y, np.array([3]), 10000.0, 4)
    exp = np.zeros(8)
    exp[1], exp[5] = -math.sin(0.3), math.cos(0.3)
    assert np.allclose(out[0, 0], exp, atol=1e-15)
    # pair j = 0 rotates by the position itself
    z = np.zeros((1, 1, 8))
    z[0, 0, 0] = 1.0
    out = om.rope(z, np.array([2]), 10000.0, 4)
    assert np.isclose(out[0, 0, 0], math.cos(2.0)) and np.isclose(out[0, 0, 4], math.sin(2.0))


def test_rope_invariants():
    rng = _rng(3)
    D, H = 16, 3
    q = rng.standard_normal((5, H, D))
    k = rng.standard_normal((5, H, D))
    pos = np.array([0, 7, 100, 4096, 131072])
    rq = om.rope(q, pos, 10000.0, D // 2)
    # rotation preserves norms
    assert np.allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-12)
    # scores depend only on the position difference (full RoPE)
    p1, p2, d = 37, 11, 1000
    a = om.rope(q[:1], np.array([p1]), 10000.0, D // 2)
    b = om.rope(k[:1], np.array([p2]), 10000.0, D // 2)
    a2 = om.rope(q[:1], np.array([p1 + d]), 10000.0, D // 2)
    b2 = om.rope(k[:1], np.array([p2 + d]), 10000.0, D // 2)
    assert np.allclose(np.sum(a * b, -1), np.sum(a2 * b2, -1), rtol=1e-9)
    # p-RoPE: n_rot = 0 is the identity; pairs at or beyond n_rot are untouched
    assert np.array_equal(om.rope(q, pos, 10000.0, 0), q)
    part = om.rope(q, pos, 10000.0, 2)
    full = om.rope(q, pos, 10000.0, D // 2)
    keep = [j for j in range(D) if not (j < 2 or D // 2 <= j < D // 2 + 2)]
    assert np.array_equal(part[:, :, keep], q[:, :, keep])
    rot = [0, 1, D // 2, D // 2 + 1]
    assert np.allclose(part[:, :, rot], full[:, :, rot], rtol=1e-15)


# ----------------------------------------------------------- attention -----

def test_attention_rows_sum_to_one():
    rng = _rng(4)
    q = rng.standard_normal((9, 16))
    k = rng.standard_normal((30, 16)) * 3
    v = rng.standard_normal((30, 16))
    _, p = om.softmax_attention(q, k, v, 0.25, return_probs=True)
    assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 30 * 2.0 ** -52 * 4)
    assert np.all(p >= 0)


def test_single_cached_kv_returns_value():
    # one key: the softmax weight is exactly 1, the output is that value
    rng = _rng(5)
    q = rng.standard_normal((4, 3, 8))
    k = rng.standard_normal((1, 3, 8))
    v = om.bf16_round(rng.standard_normal((1, 3, 8)))
    o = om.attention_heads(q, k, v)
    assert np.array_equal(om.bf16_round(o), np.broadcast_to(v, o.shape))


def test_attention_matches_torch_sdpa_with_gqa():
    rng = _rng(6)
    nq, nk, Hq, Hkv, D = 6, 11, 8, 2, 16
    q = rng.standard_normal((nq, Hq, D))
    k = rng.standard_normal((nk, Hkv, D))
    v = rng.standard_normal((nk, Hkv, D))
    o = om.attention_heads(q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(1, 0, 2)[None].repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=False)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = _rng(7)
    v = rng.standard_normal((5, 1, 4))
    # zero query: uniform weights, output is the mean of the values
    o = om.attention_heads(np.zeros((2, 1, 4)), rng.standard_normal((5, 1, 4)), v)
    assert np.allclose(o, v.mean(axis=0), atol=1e-14)
    # two keys with score difference d: weights are sigmoid(d) and 1 - sigmoid(d)
    D = 4
    q = np.array([[[2.0, 0, 0, 0]]])
    k = np.array([[[1.0, 0, 0, 0]], [[0.0, 0, 0, 0]]])
    vv = np.array([[[1.0, 0, 0, 0]], [[0.0, 1.0, 0, 0]]])
    o = om.attention_heads(q, k, vv)
    w0 = 1.0 / (1.0 + math.exp(-2.0 / math.sqrt(D)))
    assert np.allclose(o[0, 0, :2], [w0, 1 - w0], atol=1e-14)
    # GQA head mapping: query head h reads KV head h // 2 (distinct one-key heads)
    q = rng.standard_normal((3, 4, 4))
    k = rng.standard_normal((1, 2, 4))
    vh = np.stack([np.full(4, 1.0), np.full(4, 2.0)])[None]  # [1, 2, 4]
    o = om.attention_heads(q, k, vh)
    assert np.array_equal(o[:, :, 0], np.array([[1.0, 1.0, 2.0, 2.0]] * 3))


# --------------------------------------------------------------- gelu ------

def test_gelu_tanh_pins():
    z = np.linspace(-6, 6, 2001)
    g = om.gelu_tanh(z)
    assert om.gelu_tanh(np.array([0.0]))[0] == 0.0
    # gelu(z) - gelu(-z) = z exactly for the tanh form (tanh is odd)
    assert np.allclose(g - om.gelu_tanh(-z), z, atol=1e-12)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-13, atol=1e-13)
    # close to the exact GELU z * Phi(z)
    exact = z * 0.5 * (1 + scipy.special.erf(z / math.sqrt(2)))
    assert np.max(np.abs(g - exact)) < 1e-3


# --------------------------------------------------------------- routing ---

def _dominates(r, i, j):
    return r[i] > r[j] or (r[i] == r[j] and i < j)


def test_route_exhaustive_with_ties():
    rng = _rng(8)
    for E, k in [(4, 1), (5, 2), (6, 3), (8, 3), (8, 2)]:
        for _ in range(60):
            r = rng.integers(-2, 3, size=E).astype(np.float64)  # many ties
            idx, gates = om.route(r[None], k)
            chosen = set(idx[0].tolist())
            valid = [set(S) for S in itertools.combinations(range(E), k)
                     if all(_dominates(r, i, j) for i in S for j in range(E) if j not in S)]
            assert len(valid) == 1 and valid[0] == chosen
            # slot order is (logit desc, index asc)
            sl = idx[0].tolist()
            assert sl == sorted(sl, key=lambda e: (-r[e], e))
            assert np.allclose(gates[0], scipy.special.softmax(r[sl]), rtol=1e-14)


def test_moe_identical_experts_equal_dense_ffn():
    rng = _rng(9)
    M, H, F, E, k = 12, 16, 8, 6, 3
    f = rng.standard_normal((M, H))
    wg, wu, wd = rng.standard_normal((H, F)), rng.standard_normal((H, F)), rng.standard_normal((F, H))
    sg, su, sd = rng.standard_normal((H, F)), rng.standard_normal((H, F)), rng.standard_normal((F, H))
    lw = {"router": rng.standard_normal((H, E)),
          "w_gate": np.stack([wg] * E), "w_up": np.stack([wu] * E), "w_down": np.stack([wd] * E),
          "sh_gate": sg, "sh_up": su, "sh_down": sd}
    m, *_ = om.moe_block(f, lw, k, lambda x: x)
    dense = (om.gelu_tanh(f @ wg) * (f @ wu)) @ wd + (om.gelu_tanh(f @ sg) * (f @ su)) @ sd
    assert np.allclose(m, dense, rtol=1e-12, atol=1e-12)


def test_moe_single_live_expert_carries_its_gate():
    rng = _rng(10)
    M, H, F, E, k = 20, 8, 4, 5, 2
    f = rng.standard_normal((M, H))
    lw = {"router": rng.standard_normal((H, E)),
          "w_gate": np.zeros((E, H, F)), "w_up": np.zeros((E, H, F)), "w_down": np.zeros((E, F, H)),
          "sh_gate": np.zeros((H, F)), "sh_up": np.zeros((H, F)), "sh_down": np.zeros((F, H))}
    e0 = 3
    lw["w_gate"][e0] = rng.standard_normal((H, F))
    lw["w_up"][e0] = rng.standard_normal((H, F))
    lw["w_down"][e0] = rng.standard_normal((F, H))
    m, r, idx, gates = om.moe_block(f, lw, k, lambda x: x)
    ffn = (om.gelu_tanh(f @ lw["w_gate"][e0]) * (f @ lw["w_up"][e0])) @ lw["w_down"][e0]
    for t in range(M):
        sl = list(idx[t])
        g = gates[t, sl.index(e0)] if e0 in sl else 0.0
        assert np.allclose(m[t], g * ffn[t], atol=1e-12)
    # the router logits are f @ router with router [H, E] (not its transpose)
    assert np.allclose(r, f @ lw["router"])


# ------------------------------------------------------- argmax / conf -----

def test_argmax_conf_against_softmax_and_first_max():
    rng = _rng(11)
    logits = rng.standard_normal((6, 300)) * 2
    logits[2, 17] = logits[2, 200] = logits[2].max() + 1.0  # tie -> lower id
    pred, conf = om.argmax_conf(logits)
    sm = scipy.special.softmax(logits, axis=1)
    for i in range(6):
        first = next(v for v in range(300) if logits[i, v] == logits[i].max())
        assert pred[i] == first
        assert np.isclose(conf[i], sm[i, first], rtol=1e-13)
    assert pred[2] == 17


# ------------------------------------------------------------ lock rule ----

def test_lock_worked_examples():
    for c in _gold("lock_worked.json")["cases"]:
        tok = np.array([c["tokens"]], dtype=np.int32)
        lk = np.array([c["locked"]], dtype=np.uint8)
        t2, l2, _ = om.lock_select(np.array([c["conf"]]), np.array([c["pred"]]), tok, lk, [c["steps_left"]])
        assert t2[0].tolist() == c["tokens_after"], c["why"]
        assert l2[0].tolist() == c["locked_after"], c["why"]


def test_lock_rule_exhaustive():
    rng = _rng(12)
    for N in range(1, 9):
        for _ in range(40):
            conf = rng.integers(0, 3, size=N).astype(np.float64)  # ties
            locked = (rng.random(N) < 0.3).astype(np.uint8)
            tokens = rng.integers(0, 50, size=N).astype(np.int32)
            pred = rng.integers(50, 100, size=N).astype(np.int32)
            s = int(rng.integers(1, 5))
            t2, l2, ch = om.lock_select(conf[None], pred[None], tokens[None], locked[None], [s])
            free = [i for i in range(N) if not locked[i]]
            k = -(-len(free) // s)
            valid = [set(S) for S in itertools.combinations(free, k)
                     if all(_dominates(conf, i, j) for i in S for j in free if j not in S)]
            assert len(valid) == 1 and set(ch[0].tolist()) == valid[0]
            for i in range(N):
                if locked[i]:
                    assert t2[0, i] == tokens[i] and l2[0, i] == 1
                elif i in valid[0]:
                    assert t2[0, i] == pred[i] and l2[0, i] == 1
                else:  # remasked: keeps its placeholder
                    assert t2[0, i] == tokens[i] and l2[0, i] == 0


def _tiny(**kw):
    base = dict(n_layers=2, hidden=32, n_heads=4, n_kv_heads=2, head_dim=8, n_experts=6,
                top_k=2, expert_ffn=16, vocab=64, canvas_len=12, window=1024,
                global_layer_mask=0b10, dtype="f32")
    base.update(kw)
    return configs.ModelConfig(**base)


def _tiny_workload(model, **kw):
    d = dict(name="tiny", model=model, batch=1, prompt_len=5, n_steps=3, seed=21)
    d.update(kw)
    return configs.Workload(**d)


def _counts(hist, locked0):
    prev = locked0
    out = []
    for tokens, locked, _, _ in hist:
        out.append((locked.astype(int) - prev.astype(int)).sum(axis=1).tolist())
        prev = locked
    return np.array(out).T.tolist()


@pytest.mark.parametrize("cid", ["C1", "C3", "C4", "C5"])
def test_lock_schedule_closed_form(cid):
    g = _gold("lock_schedules.json")[cid]
    # a tiny model with the workload's canvas length, pass count and pre-locks:
    # the schedule depends only on those
    w = _tiny_workload(_tiny(canvas_len=g["canvas_len"], vocab=32, hidden=16, head_dim=4,
                             n_heads=2, n_kv_heads=1, expert_ffn=4, n_experts=4, n_layers=1,
                             global_layer_mask=1),
                       batch=len(g["prelock"]), n_steps=g["n_steps"], prelock=tuple(g["prelock"]))
    W = weights_for(w, cache_layers=True)
    tok, lk = gen.canvas(w)
    assert lk.sum(axis=1).tolist() == g["prelock"]
    hist = []
    t_end, l_end = om.generate_block(tok, lk, w.n_steps, W, w.model, prompt_kv_fn(w),
                                     [w.prompt_len] * w.batch, history=hist)
    assert _counts(hist, lk) == g["counts"]
    assert l_end.all()  # fully resolved after the fixed number of passes
    # a locked token never changes afterwards
    prev_t, prev_l = tok, lk
    for t_i, l_i, _, _ in hist:
        assert np.array_equal(t_i[prev_l == 1], prev_t[prev_l == 1])
        prev_t, prev_l = t_i, l_i


def test_c1_block_end_to_end_invariants():
    w = C1
    W = weights_for(w, cache_layers=True)
    tok, lk = gen.canvas(w)
    hist = []
    t_end, l_end = om.generate_block(tok, lk, w.n_steps, W, w.model, prompt_kv_fn(w),
                                     [w.prompt_len], history=hist)
    assert _counts(hist, lk) == _gold("lock_schedules.json")["C1"]["counts"]
    assert l_end.all()
    # every locked token is the pass's prediction at the moment it locked
    prev_l = lk
    for t_i, l_i, pred, conf in hist:
        new = (l_i == 1) & (prev_l == 0)
        assert np.array_equal(t_i[new], pred[new])
        assert np.all(conf > 0) and np.all(conf <= 1)
        prev_l = l_i


# ---------------------------------------------------- layer invariants -----

def _layer_setup(model, seed=30, prompt_len=5, batch=1):
    w = _tiny_workload(model, seed=seed, prompt_len=prompt_len, batch=batch)
    W = weights_for(w, cache_layers=True)
    return w, W, prompt_kv_fn(w)


def test_permuting_the_canvas_permutes_outputs_without_positions():
    # NoPE on every layer (all global, p = 0): bidirectional attention is
    # permutation-equivariant over the canvas; a causal mask would break this
    m = _tiny(global_layer_mask=0b11, prope_frac=0.0)
    w, W, kvf = _layer_setup(m)
    rng = _rng(13)
    x = rng.standard_normal((m.canvas_len, m.hidden))
    perm = rng.permutation(m.canvas_len)
    y = om.forward_hidden(x, W, m, kvf, [w.prompt_len])
    yp = om.forward_hidden(x[perm], W, m, kvf, [w.prompt_len])
    assert np.allclose(yp, y[perm], rtol=1e-11, atol=1e-11)


def test_later_canvas_positions_influence_earlier_ones():
    m = _tiny()
    w, W, kvf = _layer_setup(m)
    rng = _rng(14)
    x = rng.standard_normal((m.canvas_len, m.hidden))
    x2 = x.copy()
    x2[-1] += 1.0
    y = om.forward_hidden(x, W, m, kvf, [w.prompt_len], layers=[0])
    y2 = om.forward_hidden(x2, W, m, kvf, [w.prompt_len], layers=[0])
    assert np.abs(y2[0] - y[0]).max() > 1e-6


def test_window_at_least_prompt_makes_local_equal_global():
    rng = _rng(15)
    x = rng.standard_normal((12, 32))
    outs = []
    for mask in (0b00, 0b11):
        m = _tiny(global_layer_mask=mask, prope_frac=1.0, window=1024)
        w, W, kvf = _layer_setup(m, prompt_len=5)
        assert m.kv_len(0, 5) == 5 and m.kv_len(1, 5) == 5
        outs.append(om.forward_hidden(x, W, m, kvf, [5]))
    assert np.array_equal(outs[0], outs[1])
    # a window shorter than the prompt keeps its last positions only
    m = _tiny(window=3)
    assert m.kv_len(0, 5) == 3 and m.kv_len(1, 5) == 5


def test_zero_sublayers_leave_residual_unchanged():
    m = _tiny()
    w, W, kvf = _layer_setup(m)
    base = W.layer(0)
    zero = {k: (np.zeros_like(np.asarray(v)) if k in ("wo", "w_down", "sh_down") else v) for k, v in base.items()}
    W0 = om.OracleWeights(dtype="f32", layer_fn=None)
    W0._cache = {0: zero}
    x = _rng(16).standard_normal((m.canvas_len, m.hidden))
    y = om.forward_hidden(x, W0, m, kvf, [w.prompt_len], layers=[0])
    # RMSNorm of a zero vector is zero, so both residual branches add nothing
    assert np.array_equal(y, x)


def test_batch_independence():
    m = _tiny(vocab=40)
    w2 = _tiny_workload(m, batch=2, seed=31)
    W = weights_for(w2, cache_layers=True)
    kv2 = prompt_kv_fn(w2)
    tok, lk = gen.canvas(w2)
    t_all, l_all, p_all, c_all, _ = om.denoise_pass(tok, lk, [3, 3], W, m, kv2, [5, 5])
    t_1, l_1, p_1, c_1, _ = om.denoise_pass(tok[1:], lk[1:], [3], W, m,
                                            lambda l, b: kv2(l, b + 1), [5])
    assert np.array_equal(t_all[1:], t_1) and np.array_equal(p_all[1:], p_1)
    assert np.allclose(c_all[1:], c_1, rtol=1e-12)


def test_resume_invariance():
    m = _tiny(vocab=40)
    w = _tiny_workload(m, n_steps=5, seed=32)
    W = weights_for(w, cache_layers=True)
    kvf = prompt_kv_fn(w)
    tok, lk = gen.canvas(w)
    t_full, l_full = om.generate_block(tok, lk, 5, W, m, kvf, [5])
    # stop after 2 passes (steps_left 5, 4), keep (tokens, locked), resume
    # with a block of the 3 remaining passes
    t, l = tok, lk
    for s in (5, 4):
        t, l, *_ = om.denoise_pass(t, l, [s], W, m, kvf, [5])
    t_res, l_res = om.generate_block(t, l, 3, W, m, kvf, [5])
    assert np.array_equal(t_res, t_full) and np.array_equal(l_res, l_full)


def test_architecture_constants_match_pages():
    g = _gold("architecture.json")
    m = C3.model
    assert m.canvas_len == g["canvas_len"]["value"]
    assert m.n_experts == g["n_experts"]["value"] and m.top_k == g["top_k"]["value"]
    assert m.n_shared == g["n_shared"]["value"] and m.window == g["window"]["value"]
    assert m.n_layers == g["n_layers"]["value"]
    assert abs(m.vocab - g["vocab_approx"]["value"]) <= g["vocab_approx"]["tolerance"]
    pattern = [m.is_global(l) for l in range(m.n_layers)]
    per = g["local_per_group"]["value"] + g["global_per_group"]["value"]
    assert len(pattern) == per * g["n_groups"]["value"]
    for gi in range(g["n_groups"]["value"]):
        grp = pattern[gi * per:(gi + 1) * per]
        assert grp.count(False) == g["local_per_group"]["value"] and grp[-1]
    assert C5.batch == 4 and C5.prelock == (0, 64, 128, 192)


def test_each_branch_is_normalised():
    # RMSNorm is scale-invariant, so scaling Wo (post-attention norm) or the
    # expert down projections (post-FFN norm) by c > 0 leaves the layer output
    # unchanged up to eps; a dropped norm would scale the branch by c.
    # a tiny eps keeps RMSNorm(0) = 0 for silenced branches
    m = _tiny(rms_eps=1e-20)
    w, W, kvf = _layer_setup(m)
    base = W.layer(0)
    x = _rng(17).standard_normal((m.canvas_len, m.hidden))

    def run(lw, xx):
        Wx = om.OracleWeights(dtype="f32", layer_fn=None)
        Wx._cache = {0: lw}
        return om.forward_hidden(xx, Wx, m, kvf, [w.prompt_len], layers=[0])

    y = run(base, x)
    s_o = dict(base, wo=base["wo"] * 7.0)
    assert np.allclose(run(s_o, x), y, rtol=1e-10, atol=1e-10)
    s_d = dict(base, w_down=np.asarray(base["w_down"]) * 5.0, sh_down=base["sh_down"] * 5.0)
    assert np.allclose(run(s_d, x), y, rtol=1e-10, atol=1e-10)
    # input norm: with the FFN branch silenced, y - x is invariant under x -> c x
    nf = dict(base, w_down=np.zeros_like(np.asarray(base["w_down"])), sh_down=np.zeros_like(base["sh_down"]))
    assert np.allclose(run(nf, 3.0 * x) - 3.0 * x, run(nf, x) - x, rtol=1e-10, atol=1e-10)
    # the post-attention branch has unit RMS times (1 + w_pa) per channel
    zf = dict(nf, norm_pa=np.zeros_like(base["norm_pa"]))
    d = run(zf, x) - x
    assert np.allclose(np.sqrt(np.mean(d * d, axis=1)), 1.0, rtol=1e-10)
