"""Pins of the EB sampler's oracle to facts independent of its own code: the
published known-answer vectors of Philox4x32-10, numpy's Philox4x64-10 (the
same round structure at 64-bit width), the Gumbel distribution, the
Gumbel-max sampling law, scipy's entropy, closed forms, exhaustive
enumeration of the EB lock set on tiny inputs, and the adaptive stop rule on
stand-in logit sources whose entropies are known."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import eb

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# the generator
# --------------------------------------------------------------------------

def test_philox4x32_known_answers():
    for case in _gold("philox4x32_10_kat.json")["cases"]:
        ctr = np.array([[int(w, 16) for w in case["counter"]]], dtype=np.uint64)
        key = [int(w, 16) for w in case["key"]]
        out = eb.philox4(ctr, key, bits=32)[0]
        assert [int(w) for w in out] == [int(w, 16) for w in case["out"]]


def test_philox4x64_matches_numpy():
    # numpy's Philox is Philox4x64-10; it advances the 256-bit counter by one
    # before each block of four words
    for key in ([1, 2], [0xDEADBEEF, 7], [2 ** 64 - 1, 2 ** 63]):
        for start in (0, 5, 2 ** 64 - 2):
            ref = np.random.Philox(key=np.array(key, dtype=np.uint64),
                                   counter=np.array([start, 0, 0, 0], dtype=np.uint64))
            raw = ref.random_raw(8)
            ctr = np.zeros((2, 4), dtype=np.uint64)
            for j in range(2):
                c = start + 1 + j
                ctr[j, 0] = c % 2 ** 64
                ctr[j, 1] = c // 2 ** 64
            got = eb.philox4(ctr, key, bits=64).reshape(-1)
            assert [int(w) for w in got] == [int(w) for w in raw], (key, start)


def test_uniform_mapping_is_exact_and_open():
    words = np.array([0, 511, 512, 0x7FFFFFFF, 0xFFFFFE00, 0xFFFFFFFF], dtype=np.uint64)
    u = eb.uniform_from_bits(words)
    assert u.dtype == np.float32
    assert float(u[0]) == 2.0 ** -24 and float(u[1]) == 2.0 ** -24  # low 9 bits ignored
    assert float(u[2]) == 3 * 2.0 ** -24
    assert float(u[-1]) == 1.0 - 2.0 ** -24 and float(u[-2]) == float(u[-1])
    assert np.all((u > 0) & (u < 1))
    # every one of the 2^23 levels is distinct and exactly representable
    n = np.arange(0, 2 ** 23, 4099, dtype=np.uint64)
    uu = eb.uniform_from_bits(n << np.uint64(9)).astype(np.float64)
    assert np.array_equal(uu, (2.0 * n.astype(np.float64) + 1.0) * 2.0 ** -24)


def test_gumbel_noise_follows_the_gumbel_law():
    g = eb.gumbel_noise(seed=11, block=0, t=0, positions=np.arange(64), V=1024).astype(np.float64).ravel()
    ks = stats.kstest(g, lambda x: np.exp(-np.exp(-x)))
    assert ks.pvalue > 1e-3, ks
    assert abs(g.mean() - np.euler_gamma) < 0.02
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05


def test_gumbel_noise_uses_every_word_once_and_depends_on_every_counter_field():
    V, N = 1024, 8
    v = np.arange(V)
    call = (v >> 6) * 16 + (v & 15)
    word = (v >> 4) & 3
    assert len(set(zip(call.tolist(), word.tolist()))) == V  # no word reused within a row
    base = eb.gumbel_noise(3, 1, 2, np.arange(N), V)
    for other in (eb.gumbel_noise(4, 1, 2, np.arange(N), V), eb.gumbel_noise(3, 2, 2, np.arange(N), V),
                  eb.gumbel_noise(3, 1, 3, np.arange(N), V), eb.gumbel_noise(3, 1, 2, np.arange(1, N + 1), V)):
        assert np.mean(other != base) > 0.99
    # rows of different positions are not shifted copies of each other, and
    # no row repeats a value beyond the rare collision of 23-bit levels
    assert np.mean(base[0] != base[1]) > 0.99
    for i in range(N):
        assert len(np.unique(base[i])) >= V - 3
    # positions are independent of the other rows requested with them
    assert np.array_equal(eb.gumbel_noise(3, 1, 2, [5], V)[0], base[5])


def test_gumbel_max_sampling_law():
    # frequencies of argmax(l / tau + g) over many independent counters follow softmax(l / tau)
    rng = np.random.default_rng(5)
    V, tau, n = 64, 0.8, 20000
    logits = rng.normal(0, 1.0, size=V)
    noise = eb.gumbel_noise(seed=99, block=0, t=0, positions=np.arange(n), V=V)
    xs = eb.sample(np.broadcast_to(logits, (n, V)), tau, noise)
    p = np.exp(logits / tau - (logits / tau).max())
    p /= p.sum()
    counts = np.bincount(xs, minlength=V)
    big = p * n >= 10
    obs, exp = counts[big], p[big] * n
    if (~big).any():
        obs, exp = np.append(obs, counts[~big].sum()), np.append(exp, p[~big].sum() * n)
    chi = stats.chisquare(obs, exp)
    assert chi.pvalue > 1e-3, chi


def test_sample_is_argmax_when_the_gap_dwarfs_the_noise():
    # g lies in [-log(-log 2^-24), -log(-log(1 - 2^-24))] = [-2.81, 16.64]
    g = eb.gumbel_noise(1, 0, 0, np.arange(32), 256)
    assert g.min() >= -2.82 and g.max() <= 16.64
    rng = np.random.default_rng(6)
    logits = rng.normal(0, 0.1, size=(32, 256))
    top = rng.integers(0, 256, size=32)
    logits[np.arange(32), top] += 17.0  # gap / tau > 16.64 + 2.81 at every tau <= 0.8
    for tau in (0.8, 0.4):
        assert np.array_equal(eb.sample(logits, tau, g), top)


# --------------------------------------------------------------------------
# temperature, entropy
# --------------------------------------------------------------------------

def test_temperature_schedule_endpoints():
    s = _gold("eb_settings.json")
    T = s["max_steps"]
    assert eb.T_MAX == T
    assert eb.temperature(0, T) == pytest.approx(s["tau_first"], abs=1e-15)
    assert eb.temperature(T - 1, T) == pytest.approx(s["tau_last"], abs=1e-15)
    taus = np.array([eb.temperature(t, T) for t in range(T)])
    assert np.allclose(np.diff(taus), (s["tau_last"] - s["tau_first"]) / (T - 1), atol=1e-15)
    assert eb.temperature(0, 1) == s["tau_first"]
    assert (eb.ENTROPY_BOUND, eb.STOP_ENTROPY) == (s["entropy_bound"], s["stop_entropy"])


def test_entropy_matches_scipy_and_closed_forms():
    rng = np.random.default_rng(7)
    lg = rng.normal(0, 3, size=(16, 300))
    for tau in (0.8, 0.55, 0.4):
        z = lg / tau
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.allclose(eb.entropy(lg, tau), stats.entropy(p, axis=1), rtol=1e-12, atol=1e-14)
    # uniform: log V; two tokens: the binary entropy; one dominant token: -> 0
    assert eb.entropy(np.zeros((1, 1000)), 0.8)[0] == pytest.approx(math.log(1000), rel=1e-13)
    a = 1.3
    q = 1 / (1 + math.exp(a / 0.5))
    two = np.full((1, 2), 0.0)
    two[0, 1] = a
    assert eb.entropy(two, 0.5)[0] == pytest.approx(-(q * math.log(q) + (1 - q) * math.log(1 - q)), rel=1e-13)
    one = np.zeros((1, 50))
    one[0, 3] = 200.0
    assert eb.entropy(one, 0.4)[0] < 1e-200


def test_entropy_slack_bounds_the_change():
    rng = np.random.default_rng(8)
    lg = rng.normal(0, 4, size=(64, 500))
    for tau in (0.8, 0.4):
        d = 1e-4
        s = eb.entropy_slack(lg, tau, d)
        h0 = eb.entropy(lg, tau)
        for _ in range(5):
            dh = np.abs(eb.entropy(lg + rng.uniform(-d, d, size=lg.shape), tau) - h0)
            assert np.all(dh <= s * 1.01 + 1e-12)
        # and it is tight to first order in the direction of its gradient
        p, z = eb._softmax_z(lg, tau)
        mean = (p * z).sum(axis=1, keepdims=True)
        worst = lg - d * np.sign(z - mean)
        dh = eb.entropy(worst, tau) - h0
        assert np.all(np.abs(dh) >= s * 0.98)


# --------------------------------------------------------------------------
# the EB lock set
# --------------------------------------------------------------------------

def _eb_brute(H, free, bound):
    """The lock set by enumeration: the nonempty subset S of the free
    positions that is downward closed in (H, position) order, has a sum
    within the bound when |S| > 1, and is maximal.  H on a dyadic grid so
    every sum is exact."""
    best = None
    for r in range(1, len(free) + 1):
        for S in itertools.combinations(free, r):
            rest = [j for j in free if j not in S]
            if rest and max((H[i], i) for i in S) > min((H[j], j) for j in rest):
                continue
            if len(S) > 1 and sum(H[i] for i in S) > bound:
                continue
            if best is None or len(S) > len(best):
                best = S
    return sorted(best)


def test_eb_select_against_enumeration():
    rng = np.random.default_rng(9)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        H = rng.integers(0, 12, size=n) / 64.0  # ties on purpose
        locked = rng.random(n) < 0.3
        free = [i for i in range(n) if not locked[i]]
        if not free:
            continue
        got = sorted(eb.eb_select(H, free, 0.1).tolist())
        assert got == _eb_brute(H, free, 0.1), (H, free)


def test_eb_select_keeps_at_least_one_and_takes_all_below_the_bound():
    assert eb.eb_select(np.array([5.0, 3.0, 4.0]), [0, 1, 2]).tolist() == [1]
    assert sorted(eb.eb_select(np.full(10, 0.001), range(10)).tolist()) == list(range(10))
    assert eb.eb_select(np.array([0.0, 0.0]), [1]).tolist() == [1]


def test_eb_select_running_sum_is_float32():
    # two entropies of f32(0.05): their float32 sum is exactly f32(0.1), within
    # the bound taken in float32; a float64 sum against 0.1 would reject it
    h = float(np.float32(0.05))
    assert h + h > 0.1
    assert sorted(eb.eb_select(np.array([h, h, 1.0]), [0, 1, 2]).tolist()) == [0, 1]


def test_mean_entropy_float32():
    rng = np.random.default_rng(10)
    H = rng.random(256) * 0.01
    m = eb.mean_entropy32(H)
    assert isinstance(m, np.float32)
    assert abs(float(m) - math.fsum(H) / 256) <= 256 * 2.0 ** -24 * float(m) + 1e-9


# --------------------------------------------------------------------------
# the loop: EB locks, the stop rule, the last pass
# --------------------------------------------------------------------------

def _peaked(N, V, target, gap):
    """Logits with one token per position above the others by ``gap``."""
    lg = np.zeros((N, V))
    lg[np.arange(N), target] = gap
    return lg


def _gap_for_entropy(V, tau, h):
    """Gap g at which one token above V-1 equal ones has entropy h at tau."""
    lo, hi = 0.0, 200.0
    for _ in range(200):
        mid = (lo + hi) / 2
        if eb.entropy(_peaked(1, V, [0], mid), tau)[0] > h:
            lo = mid
        else:
            hi = mid
    return hi


def test_confident_canvas_locks_everything_in_one_pass():
    N, V = 32, 128
    tgt = np.arange(N) % V
    fn = lambda toks, t: _peaked(N, V, tgt, 60.0)[None]
    tok0 = np.full((1, N), 7)
    toks, lk, passes = eb.generate_block_eb(fn, tok0, np.zeros((1, N), np.uint8), seeds=[1])
    assert passes == 1 and lk.all() and np.array_equal(toks[0], tgt)


def test_stop_rule_needs_two_agreeing_passes_and_locks_the_rest_greedily():
    # every position has entropy ~0.004 at every tau: the mean is below 0.005,
    # but 64 x 0.004 exceeds the bound, so the first pass locks only part of
    # the canvas; the second pass agrees with the first and stops
    N, V = 64, 128
    tgt = (np.arange(N) * 5) % V
    gaps = [_gap_for_entropy(V, eb.temperature(t), 0.004) for t in range(2)]
    fn = lambda toks, t: _peaked(N, V, tgt, gaps[min(t, 1)])[None]
    hist = []
    toks, lk, passes = eb.generate_block_eb(fn, np.full((1, N), 9), np.zeros((1, N), np.uint8), seeds=[2],
                                            history=hist)
    first = hist[0][2]
    assert 0 < len(first["selected"][0]) < N and not first["stopped"][0]
    assert passes == 2 and hist[1][2]["stopped"][0] and lk.all()
    second_sel = set(hist[1][2]["selected"][0].tolist())
    rest = [i for i in range(N) if i not in set(first["selected"][0].tolist()) | second_sel]
    assert rest and np.array_equal(toks[0, rest], hist[1][2]["pred"][0][rest])  # the rest took the greedy token
    assert np.array_equal(toks[0, rest], tgt[rest])


def test_no_stop_while_predictions_change():
    # same low entropies, but the greedy token moves every pass: no stop, the
    # EB rule alone resolves the canvas
    N, V = 32, 128
    gap = _gap_for_entropy(V, 0.4, 0.004)
    fn = lambda toks, t: _peaked(N, V, (np.arange(N) + t) % V, gap)[None]
    hist = []
    toks, lk, passes = eb.generate_block_eb(fn, np.full((1, N), 9), np.zeros((1, N), np.uint8), seeds=[3],
                                            history=hist)
    assert lk.all() and passes >= 2 and not any(h[2]["stopped"][0] for h in hist)


def test_no_stop_above_the_entropy_threshold():
    N, V = 32, 128
    gap = _gap_for_entropy(V, 0.8, 0.02)  # stable predictions, mean entropy > 0.005 at every tau
    fn = lambda toks, t: _peaked(N, V, np.arange(N), gap)[None]
    hist = []
    eb.generate_block_eb(fn, np.full((1, N), 9), np.zeros((1, N), np.uint8), seeds=[4], history=hist)
    assert not any(h[2]["stopped"][0] for h in hist)
    for h in hist:
        assert float(np.mean(h[2]["H"][0])) > 0.005


def test_high_entropy_canvas_runs_to_the_last_pass():
    # every entropy > 0.1: one lock per pass; pass 47 locks the remaining 17
    # with their samples; locked tokens never change
    N, V = 64, 256
    rng = np.random.default_rng(11)
    lg = rng.normal(0, 0.5, size=(1, N, V))
    hist = []
    tok0 = np.full((1, N), 1)
    lk0 = np.zeros((1, N), np.uint8)
    toks, lk, passes = eb.generate_block_eb(lambda t_, t: lg, tok0, lk0, seeds=[5], history=hist)
    assert passes == eb.T_MAX and lk.all()
    for t, (tk, l, info) in enumerate(hist):
        assert len(info["selected"][0]) == (1 if t < eb.T_MAX - 1 else N - (eb.T_MAX - 1))
        if t:
            was = hist[t - 1][1][0] == 1
            assert np.array_equal(tk[0, was], hist[t - 1][0][0, was])
        # a position locked in pass t holds that pass's sample
        sel = info["selected"][0]
        assert np.array_equal(tk[0, sel], info["sample"][0][sel])


def test_prelocked_positions_and_done_canvases_are_left_alone():
    N, V = 32, 128
    tgt = np.arange(N)
    conf = _peaked(N, V, tgt, 60.0)
    rng = np.random.default_rng(12)
    vague = rng.normal(0, 0.5, size=(N, V))
    fn = lambda toks, t: np.stack([conf, vague])
    tok0 = np.full((2, N), 3)
    lk0 = np.zeros((2, N), np.uint8)
    lk0[:, ::4] = 1
    hist = []
    toks, lk, passes = eb.generate_block_eb(fn, tok0, lk0, seeds=[6, 7], t_max=6, history=hist)
    assert passes == 6 and lk.all()
    assert np.array_equal(toks[:, ::4], tok0[:, ::4])  # pre-locked never change
    # canvas 0 finished in pass 0; nothing of it moves afterwards
    for tk, l, info in hist[1:]:
        assert np.array_equal(tk[0], hist[0][0][0]) and len(info["selected"][0]) == 0
