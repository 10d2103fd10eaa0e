"""Pins of the oracle's block commit (causal context building over a finished
block and the KV-cache append) to facts independent of its own code: closed
forms of a one-key softmax, invariants of causal attention, the equality of
chunked and whole causal processing, and the sliding-window rule."""
import dataclasses

import numpy as np
import pytest

from oracle import model as om
from oracle.inputs import prompt_kv_fn, weights_for
from synth import C1, configs, gen

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _qkv(seed, N, Hq=4, Hkv=2, D=8):
    r = _rng(seed)
    return (r.standard_normal((1, N, Hq, D)), r.standard_normal((1, N, Hkv, D)),
            r.standard_normal((1, N, Hkv, D)))


def test_causal_first_position_sees_only_its_own_key():
    # no cached context: position 0 has one visible key, whose softmax weight is 1
    q, k, v = _qkv(1, 6)
    empty = [(np.zeros((0, 2, 8)), np.zeros((0, 2, 8)))]
    o = om.canvas_attention(q, k, v, empty, lambda x: x, causal=True).reshape(6, 4, 8)
    for h in range(4):
        assert np.array_equal(o[0, h], v[0, 0, h // 2])


def test_causal_last_position_equals_bidirectional():
    # the last position sees every key either way
    q, k, v = _qkv(2, 7)
    r = _rng(3)
    ctx = [(r.standard_normal((5, 2, 8)), r.standard_normal((5, 2, 8)))]
    oc = om.canvas_attention(q, k, v, ctx, lambda x: x, causal=True).reshape(7, -1)
    ob = om.canvas_attention(q, k, v, ctx, lambda x: x, causal=False).reshape(7, -1)
    assert np.allclose(oc[6], ob[6], rtol=0, atol=1e-13)
    assert not np.allclose(oc[0], ob[0])  # earlier positions do differ


def test_causal_outputs_ignore_later_positions():
    # changing the keys / values of positions > i leaves position i's output unchanged
    N = 9
    q, k, v = _qkv(4, N)
    r = _rng(5)
    ctx = [(r.standard_normal((3, 2, 8)), r.standard_normal((3, 2, 8)))]
    base = om.canvas_attention(q, k, v, ctx, lambda x: x, causal=True).reshape(N, -1)
    for i in range(N - 1):
        k2, v2 = k.copy(), v.copy()
        k2[0, i + 1:] += r.standard_normal(k2[0, i + 1:].shape)
        v2[0, i + 1:] += r.standard_normal(v2[0, i + 1:].shape)
        got = om.canvas_attention(q, k2, v2, ctx, lambda x: x, causal=True).reshape(N, -1)
        assert np.array_equal(got[:i + 1], base[:i + 1])
        assert not np.allclose(got[i + 1:], base[i + 1:])


def test_causal_matches_per_prefix_softmax():
    # position i's output equals a bidirectional softmax over [context ; keys 0..i]
    N = 5
    q, k, v = _qkv(6, N)
    r = _rng(7)
    Kp, Vp = r.standard_normal((4, 2, 8)), r.standard_normal((4, 2, 8))
    oc = om.canvas_attention(q, k, v, [(Kp, Vp)], lambda x: x, causal=True).reshape(N, 4, 8)
    for i in range(N):
        keys = np.concatenate([Kp, k[0, :i + 1]], axis=0)
        vals = np.concatenate([Vp, v[0, :i + 1]], axis=0)
        for h in range(4):
            s = keys[:, h // 2] @ q[0, i, h] / np.sqrt(8.0)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ vals[:, h // 2]
            assert np.allclose(oc[i, h], ref, rtol=0, atol=1e-13)


def test_append_keeps_the_last_visible_positions():
    r = _rng(8)
    Ko, Vo = r.standard_normal((6, 2, 3)), r.standard_normal((6, 2, 3))
    kb, vb = r.standard_normal((4, 2, 3)), r.standard_normal((4, 2, 3))
    K, V = om.append_kv(Ko, Vo, kb, vb, 10)  # global: everything
    assert np.array_equal(K[:6], Ko) and np.array_equal(K[6:], kb) and np.array_equal(V[6:], vb)
    K, V = om.append_kv(Ko, Vo, kb, vb, 7)  # window 7: drop the 3 oldest
    assert K.shape[0] == 7 and np.array_equal(K[:3], Ko[3:]) and np.array_equal(K[3:], kb)
    assert np.array_equal(V[:3], Vo[3:]) and np.array_equal(V[3:], vb)
    K, V = om.append_kv(Ko[:0], Vo[:0], kb, vb, 4)  # from an empty cache
    assert np.array_equal(K, kb) and np.array_equal(V, vb)


# a tiny fp32 model; the window covers every position so chunked and whole
# processing see the same keys
TINY = dataclasses.replace(
    C1, name="commit-tiny",
    model=configs.ModelConfig(n_layers=2, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16,
                              n_experts=8, top_k=2, expert_ffn=32, vocab=97, canvas_len=8,
                              window=1024, global_layer_mask=0b10, dtype="f32"),
    batch=1, prompt_len=0, n_steps=1, seed=21)


def _commit_chain(w, tokens, chunk):
    """Commit ``tokens`` in chunks of ``chunk`` (the last one shorter when the
    length is not a multiple) from an empty cache; returns the per-layer
    caches."""
    W = weights_for(w)
    L = w.model.n_layers
    Hkv, D = w.model.n_kv_heads, w.model.head_dim
    cache = [(np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D))) for _ in range(L)]
    pos = 0
    for c0 in range(0, tokens.shape[1], chunk):
        part = tokens[:, c0:c0 + chunk]
        n = part.shape[1]
        m = dataclasses.replace(w.model, canvas_len=n)
        blk = om.commit_block(part, W, m, lambda l, b: cache[l], [pos])
        for l in range(L):
            vis = pos + n if m.is_global(l) else min(pos + n, m.window)
            cache[l] = om.append_kv(cache[l][0], cache[l][1], blk[l][0][0], blk[l][1][0], vis)
        pos += n
    return cache


def test_chunked_commits_equal_one_causal_pass():
    # causal attention makes prefix processing order-free: 24 tokens committed
    # as three 8-token blocks, as two 12-token blocks and as one 24-token
    # block give the same cache at every layer
    tokens = _rng(9).integers(0, TINY.model.vocab, size=(1, 24))
    whole = _commit_chain(TINY, tokens, 24)
    for chunk in (8, 12, 7, 5):  # 7 and 5 leave a shorter last chunk (3 and 4)
        got = _commit_chain(TINY, tokens, chunk)
        for l in range(TINY.model.n_layers):
            assert np.allclose(got[l][0], whole[l][0], rtol=0, atol=1e-10), (chunk, l)
            assert np.allclose(got[l][1], whole[l][1], rtol=0, atol=1e-10), (chunk, l)


def test_commit_layer0_keys_follow_token_positions():
    # layer 0's keys depend only on each token and its position: the same
    # token at the same absolute position gives the same key whatever the
    # rest of the block holds, and RoPE makes it differ at another position
    w = TINY
    m = w.model
    W = weights_for(w)
    Hkv, D = m.n_kv_heads, m.head_dim
    empty = [(np.zeros((0, Hkv, D)), np.zeros((0, Hkv, D)))] * m.n_layers
    t1 = _rng(10).integers(0, m.vocab, size=(1, 8))
    t2 = t1.copy()
    t2[0, 3:] = (t2[0, 3:] + 5) % m.vocab
    k1 = om.commit_block(t1, W, m, lambda l, b: empty[l], [16])[0][0]
    k2 = om.commit_block(t2, W, m, lambda l, b: empty[l], [16])[0][0]
    assert np.array_equal(k1[0, :3], k2[0, :3])
    k3 = om.commit_block(t1, W, m, lambda l, b: empty[l], [17])[0][0]
    assert not np.allclose(k1[0, :3], k3[0, :3])
