"""Pins of the oracle's adjudicator: the rules by which a shadowed comparison
lets the oracle take a discrete decision of the GPU path.

A decision whose oracle margin lies within the error of the compared quantity
has more than one correct outcome; the oracle then takes the GPU's outcome,
but only if that outcome is itself within the margin of the oracle's best.
Every bf16 pass-level parity test leans on these rules, so each is pinned
here on hand-built logits, confidences and entropies, at the ends of its
interval: a decision exactly at the margin is taken, one a hair beyond it
fails, and cases that a flipped sign, a comparison with the wrong neighbour
or a missing size check would accept fail.

The rules follow what the pages fix about the decisions: the probability
distribution of the decoder's output judges which tokens are final ("Hands-On
with Diffusion Gemma", section "Detailed Specs"); 8 of 128 experts are
active per token ("DiffusionGemma: The Diffusion Era Begins with 4x Faster
Text Generation", section "DiffusionGemma's Technical Architecture"); the EB
sampler locks low-entropy positions within a bound and stops on a stable,
low-entropy canvas (same page, section "Recommended Inference Settings").
"""
import math

import numpy as np
import pytest
from scipy.optimize import brentq

from oracle import eb
from oracle import model as om

TINY = 2.0 ** -30


# --------------------------------------------------------------- routing ---

def _route_case(r, gpu_rows, k, delta):
    r = np.asarray(r, dtype=np.float64)
    idx, gates = om.route(r, k)
    sh = om.Shadow(route_idx=[np.asarray(gpu_rows, dtype=np.int32)], delta_route=delta)
    idx2, gates2 = om._shadow_route(sh, 0)(r, idx, gates)
    return sh, idx, idx2, gates2


R6 = [1.0, 0.75, 0.5, 0.0, -1.0, -2.0]


def test_route_adopts_at_the_margin_and_recomputes_gates():
    # oracle top-2 {0, 1}; the GPU took {0, 2}: the best expert it left out
    # (1, logit 0.75) beats the worst it took (2, logit 0.5) by 0.25
    sh, idx, idx2, g2 = _route_case([R6], [[0, 2]], 2, 0.25)
    assert not sh.failures
    assert sh.adopted["route"] == 1 and sh.max_margin["route"] == 0.25
    assert idx2[0].tolist() == [0, 2]
    # gates: softmax over the oracle's own logits of the adopted set, in
    # (logit descending, expert ascending) order
    e = np.exp(np.array([1.0, 0.5]) - 1.0)
    np.testing.assert_allclose(g2[0], e / e.sum(), rtol=0, atol=1e-15)


def test_route_fails_just_beyond_the_margin():
    sh, idx, idx2, _ = _route_case([R6], [[0, 2]], 2, 0.25 - TINY)
    assert sh.adopted["route"] == 0 and len(sh.failures) == 1
    assert idx2[0].tolist() == idx[0].tolist() == [0, 1]


def test_route_far_choice_fails():
    # {4, 5} is 3.0 below the oracle's best excluded expert: a flipped margin
    # sign (worst taken minus best left out = -3.0) would accept it
    sh, _, _, _ = _route_case([R6], [[4, 5]], 2, 0.5)
    assert sh.adopted["route"] == 0 and len(sh.failures) == 1
    assert "margin 3.000e+00" in sh.failures[0]


def test_route_margin_uses_the_best_expert_the_gpu_left_out():
    # oracle top-2 {0, 1}, third 0.74 close behind; the GPU took {0, 3}.  Its
    # best excluded expert is 1 (0.75), not the oracle's runner-up 2: the
    # margin is 0.75 - 0.0, so the choice fails at delta 0.1 (a margin taken
    # from the oracle's own ranking, 0.75 - 0.74, would accept it)
    r = [1.0, 0.75, 0.74, 0.0, -1.0, -2.0]
    sh, _, _, _ = _route_case([r], [[0, 3]], 2, 0.1)
    assert sh.adopted["route"] == 0 and len(sh.failures) == 1


def test_route_set_of_wrong_size_fails():
    # a repeated expert is a set of one: never a valid top-2, whatever delta
    sh, _, _, _ = _route_case([R6], [[0, 0]], 2, 100.0)
    assert sh.adopted["route"] == 0 and len(sh.failures) == 1


def test_route_same_set_in_another_order_is_no_decision():
    sh, idx, idx2, g2 = _route_case([R6], [[1, 0]], 2, 0.0)
    assert not sh.failures and sh.adopted["route"] == 0
    assert idx2[0].tolist() == idx[0].tolist()


def test_route_exact_tie_adopted_at_zero_delta():
    # equal logits: the oracle takes the lower expert (1); the GPU's 2 is
    # just as large, margin 0
    r = [[1.0, 1.0, 1.0, 0.0, -1.0, -2.0]]
    sh, idx, idx2, _ = _route_case(r, [[0, 2]], 2, 0.0)
    assert idx[0].tolist() == [0, 1]
    assert not sh.failures and sh.adopted["route"] == 1 and sh.max_margin["route"] == 0.0
    assert idx2[0].tolist() == [0, 2]


def test_route_rows_are_judged_one_by_one():
    r = [R6, R6, R6]
    sh, _, idx2, _ = _route_case(r, [[0, 1], [0, 2], [4, 5]], 2, 0.25)
    assert sh.adopted["route"] == 1 and len(sh.failures) == 1
    assert "token 2" in sh.failures[0]
    assert idx2[1].tolist() == [0, 2]


# ------------------------------------------------------------ prediction ---

def _pred_case(logits, gpu, delta):
    lg = np.asarray(logits, dtype=np.float64)[None]  # [1, N, V]
    pred, conf = om.argmax_conf(lg[0])
    pred, conf = pred[None].copy(), conf[None].copy()
    sh = om.Shadow(pred=np.asarray(gpu, dtype=np.int32)[None], delta_logit=delta)
    om.adopt_pred(lg, pred, conf, sh)
    return sh, pred[0], conf[0]


L5 = [0.0, 2.0, 1.5, 1.0, -1.0]


def test_pred_adopts_at_the_margin_with_the_token_probability():
    sh, pred, conf = _pred_case([L5], [2], 0.5)
    assert not sh.failures and sh.adopted["pred"] == 1 and sh.max_margin["pred"] == 0.5
    assert pred[0] == 2
    p = np.exp(np.array(L5)) / np.exp(np.array(L5)).sum()
    assert abs(conf[0] - p[2]) <= 1e-15


def test_pred_fails_just_beyond_the_margin():
    sh, pred, conf = _pred_case([L5], [2], 0.5 - TINY)
    assert sh.adopted["pred"] == 0 and len(sh.failures) == 1
    assert pred[0] == 1


def test_pred_far_choice_fails():
    # token 4 is 3.0 below the best: a flipped sign would accept it
    sh, _, _ = _pred_case([L5], [4], 1.0)
    assert sh.adopted["pred"] == 0 and len(sh.failures) == 1


def test_pred_equal_is_no_decision_and_ties_adopt_at_zero():
    sh, pred, _ = _pred_case([L5, [1.0, 3.0, 3.0, 0.0, 0.0]], [1, 2], 0.0)
    assert not sh.failures and sh.adopted["pred"] == 1
    assert pred.tolist() == [1, 2]


# ----------------------------------------------------------------- locks ---

C6 = np.array([0.9, 0.8, 0.7, 0.65, 0.1, 0.05])


def _lock_case(conf, locked, gpu_new, steps_left, delta):
    conf = np.asarray(conf, dtype=np.float64)[None]
    locked = np.asarray(locked, dtype=np.uint8)[None]
    N = conf.shape[1]
    pred = (100 + np.arange(N, dtype=np.int32))[None]
    tokens = np.arange(N, dtype=np.int32)[None]
    new_t, new_l, chosen = om.lock_select(conf, pred, tokens, locked, [steps_left])
    g_after = locked.copy()
    g_after[0, list(gpu_new)] = 1
    sh = om.Shadow(locked_after=g_after, delta_conf=delta)
    om.adopt_locks(conf, pred, tokens, locked, new_t, new_l, chosen, sh)
    return sh, chosen[0], new_t[0], new_l[0]


def test_lock_adopts_at_the_margin():
    # k = ceil(6 / 3) = 2: the oracle locks {0, 1}; the GPU locked {0, 2},
    # leaving position 1 (0.8) out for position 2 (0.7): margin 0.1
    d = C6[1] - C6[2]
    sh, chosen, t, l = _lock_case(C6, [0] * 6, [0, 2], 3, d)
    assert sorted(chosen.tolist()) == [0, 1]
    assert not sh.failures and sh.adopted["lock"] == 1 and sh.max_margin["lock"] == d
    assert l.tolist() == [1, 0, 1, 0, 0, 0]
    assert t.tolist() == [100, 1, 102, 3, 4, 5]  # locked take the prediction, the rest keep theirs


def test_lock_fails_just_beyond_the_margin():
    d = C6[1] - C6[2]
    sh, _, t, l = _lock_case(C6, [0] * 6, [0, 2], 3, d - TINY)
    assert sh.adopted["lock"] == 0 and len(sh.failures) == 1
    assert l.tolist() == [1, 1, 0, 0, 0, 0]


def test_lock_margin_uses_the_best_position_the_gpu_left_out():
    # the GPU locked {0, 3}: it left out position 1 (0.8), which beats 3
    # (0.65) by 0.15; measured against the positions outside the oracle's own
    # set (best 0.7) the margin would be 0.05 and pass at delta 0.1
    sh, _, _, _ = _lock_case(C6, [0] * 6, [0, 3], 3, 0.1)
    assert sh.adopted["lock"] == 0 and len(sh.failures) == 1


def test_lock_far_choice_fails():
    # {4, 5} against {0, 1}: a flipped sign would accept it
    sh, _, _, _ = _lock_case(C6, [0] * 6, [4, 5], 3, 0.5)
    assert sh.adopted["lock"] == 0 and len(sh.failures) == 1


def test_lock_set_of_wrong_size_fails():
    # three positions where the schedule locks two, however close the confidences
    conf = [0.5, 0.5, 0.5, 0.5, 0.5, 0.5]
    sh, _, _, _ = _lock_case(conf, [0] * 6, [0, 1, 2], 3, 1.0)
    assert sh.adopted["lock"] == 0 and len(sh.failures) == 1
    sh, _, _, _ = _lock_case(conf, [0] * 6, [], 3, 1.0)
    assert sh.adopted["lock"] == 0 and len(sh.failures) == 1


def test_lock_pre_locked_positions_are_not_decisions():
    # position 0 is locked before the pass; 5 free, k = ceil(5 / 3) = 2: the
    # oracle locks {1, 2}; the GPU {1, 3} with 3 = 0.65 against 2 = 0.7
    pre = [1, 0, 0, 0, 0, 0]
    sh, chosen, t, l = _lock_case(C6, pre, [1, 3], 3, 0.05 + 1e-12)
    assert sorted(chosen.tolist()) == [1, 2]
    assert not sh.failures and sh.adopted["lock"] == 1
    assert l.tolist() == [1, 1, 0, 1, 0, 0]
    assert t[0] == 0  # a pre-locked position keeps its token


# ------------------------------------------------------ EB: argmax rules ---

def test_eb_adopt_argmax_interval_ends():
    score = np.array([[0.0, 2.0, 1.5, -1.0]])
    mine = np.array([1])
    sh = eb.EBShadow()
    out = eb._adopt_argmax(score, mine, np.array([2]), 0.5, "sample", 0, sh)
    assert out.tolist() == [2] and sh.adopted["sample"] == 1 and not sh.failures
    sh = eb.EBShadow()
    out = eb._adopt_argmax(score, mine, np.array([2]), 0.5 - TINY, "sample", 0, sh)
    assert out.tolist() == [1] and sh.adopted["sample"] == 0 and len(sh.failures) == 1
    # 3.0 below the best: a flipped sign would accept it
    sh = eb.EBShadow()
    out = eb._adopt_argmax(score, mine, np.array([3]), 1.0, "pred", 0, sh)
    assert out.tolist() == [1] and len(sh.failures) == 1


# ------------------------------------------------------ EB: lock-set rule ---

def _plaus(H, d, g, free=None):
    H = np.asarray(H, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    free = np.arange(H.size) if free is None else np.asarray(free)
    return eb.eb_set_plausible(H, d, free, np.asarray(g, dtype=np.int64))


def test_eb_plausible_prefix_condition_at_its_end():
    H = [0.01, 0.02, 0.03, 0.5]
    assert _plaus(H, [0] * 4, [0, 1, 2])
    # {0, 2} skips position 1 (0.02 < 0.03): no admissible order has it as a prefix
    assert not _plaus(H, [0] * 4, [0, 2])
    # with errors of 1/256 on positions 1 and 2 (binary fractions, so the
    # ends meet exactly) 1 and 2 become exchangeable exactly at the end
    Hd = [8 / 256, 10 / 256, 12 / 256, 128 / 256]
    d_end = [0.0, 1 / 256, 1 / 256, 0.0]
    assert (Hd[1] + d_end[1]) == (Hd[2] - d_end[2])
    assert not _plaus(Hd, [0] * 4, [0, 2])
    assert _plaus(Hd, d_end, [0, 2]) and _plaus(Hd, d_end, [0, 1])
    d_short = [0.0, 1 / 256, 1 / 256 - 2 ** -40, 0.0]
    assert not _plaus(Hd, d_short, [0, 2])


def test_eb_plausible_bound_condition_at_its_end():
    # two positions summing to exactly the bound are admissible; a hair more is not
    assert 0.05 + 0.05 == eb.ENTROPY_BOUND
    assert _plaus([0.05, 0.05, 0.9], [0] * 3, [0, 1])
    assert not _plaus([0.05, 0.05 + 1e-12, 0.9], [0] * 3, [0, 1])
    # the error may bring an over-the-bound pair back to it
    assert _plaus([0.05, 0.05 + 1e-12, 0.9], [0.0, 1e-12, 0.0], [0, 1])
    # one position is always admissible, however large its entropy
    assert _plaus([0.5, 0.6], [0, 0], [0])
    assert not _plaus([0.5, 0.6], [0, 0], [1])


def test_eb_plausible_room_condition_at_its_end():
    # {0} with 0.05 and the next one 0.05: the pair fits the bound exactly,
    # so a set that stops at one position is not admissible
    assert not _plaus([0.05, 0.05, 0.9], [0] * 3, [0])
    # the next one a hair over: stopping at one is admissible
    assert _plaus([0.05, 0.05 + 1e-12, 0.9], [0] * 3, [0])
    # the error may push the next one over
    assert _plaus([0.05, 0.05, 0.9], [0.0, 1e-12, 0.0], [0])


def test_eb_plausible_set_membership():
    assert not _plaus([0.01, 0.02], [0, 0], [])
    assert not _plaus([0.01, 0.02, 0.03], [0, 0, 0], [0], free=[1, 2])  # 0 is locked already
    assert _plaus([0.01, 0.02, 0.03], [0, 0, 0], [1, 2], free=[1, 2])


# ---------------------------------------------- EB: decisions inside a pass ---

def _row_with_entropy(target: float, V: int, tau: float) -> np.ndarray:
    """Logits [a, 0, ..., 0] whose softmax(l / tau) has entropy ``target``."""
    def f(a):
        return float(eb.entropy(np.array([[a] + [0.0] * (V - 1)]), tau)[0]) - target
    a = brentq(f, 0.0, 200.0, xtol=1e-14)
    return np.array([a] + [0.0] * (V - 1))


def test_eb_update_lock_adoption_follows_the_plausibility_rule():
    tau = eb.temperature(0)
    V, N = 8, 4
    # entropies 0.03, 0.031, 0.5, 0.6: the oracle locks {0, 1} (0.061 <= 0.1)
    Hs = [0.03, 0.031, 0.5, 0.6]
    lg = np.stack([_row_with_entropy(h, V, tau) for h in Hs])[None]
    tokens = np.zeros((1, N), dtype=np.int32)
    locked = np.zeros((1, N), dtype=np.uint8)
    # the GPU locked {0} only: with these logits' slack that is not admissible
    # (room for position 1 whatever the error) -> a failure
    g_after = np.array([[1, 0, 0, 0]], dtype=np.uint8)
    sh = eb.EBShadow(locked_after=g_after, dlogit=1e-3)
    _, l_o, info = eb.eb_update(lg, tokens, locked, 0, eb.EBState(1), [7], 0, shadow=sh)
    assert sorted(info["selected"][0].tolist()) == [0, 1]
    assert len(sh.failures) == 1 and sh.adopted["lock"] == 0
    # a pair at 0.05 + 0.0501: over the bound by 1e-4; a logit error large
    # enough to move each entropy by 1e-4 makes the GPU's pair admissible
    Hs = [0.05, 0.0501, 0.5, 0.6]
    lg = np.stack([_row_with_entropy(h, V, tau) for h in Hs])[None]
    g_after = np.array([[1, 1, 0, 0]], dtype=np.uint8)
    slack = eb.entropy_slack(lg[0], tau, 1.0)  # dH per unit of logit error
    dlogit = 2e-4 / float(slack[:2].min())
    sh = eb.EBShadow(locked_after=g_after, dlogit=dlogit)
    t_o, l_o, info = eb.eb_update(lg, tokens, locked, 0, eb.EBState(1), [7], 0, shadow=sh)
    assert not sh.failures and sh.adopted["lock"] == 1
    assert l_o[0].tolist() == [1, 1, 0, 0]
    # without that error the same pair fails
    sh = eb.EBShadow(locked_after=g_after, dlogit=0.0)
    eb.eb_update(lg, tokens, locked, 0, eb.EBState(1), [7], 0, shadow=sh)
    assert len(sh.failures) == 1


def test_eb_update_stop_adoption_interval():
    tau = eb.temperature(3)
    V, N = 8, 4
    tokens = np.zeros((1, N), dtype=np.int32)
    locked = np.zeros((1, N), dtype=np.uint8)

    def run(mean_h, gpu_stop, dlogit):
        lg = np.stack([_row_with_entropy(mean_h, V, tau) for _ in range(N)])[None]
        st = eb.EBState(1)
        st.prev_pred[0] = np.zeros(N, dtype=np.int32)  # the greedy tokens are stable
        sh = eb.EBShadow(stopped=np.array([gpu_stop]), dlogit=dlogit)
        _, l_o, info = eb.eb_update(lg, tokens, locked, 3, st, [7], 0, shadow=sh, t_max=48)
        return sh, info["stopped"][0], lg

    # mean entropy 0.0051, just above the threshold: the oracle does not stop
    sh, stop, lg = run(0.0051, True, 0.0)
    assert len(sh.failures) == 1 and not stop
    # with a logit error whose entropy slack covers the 1e-4 gap, the GPU's stop is taken
    slack = float(eb.entropy_slack(lg[0], tau, 1.0).mean())
    sh, stop, _ = run(0.0051, True, 1.5e-4 / slack)
    assert not sh.failures and sh.adopted["stop"] == 1 and stop
    # far above the threshold no error of that size makes a stop plausible
    sh, stop, _ = run(0.05, True, 1.5e-4 / slack)
    assert len(sh.failures) == 1 and not stop


def test_eb_update_stop_needs_stable_tokens():
    # below the threshold but no previous pass: the oracle cannot stop, and a
    # GPU stop is a failure whatever the error
    tau = eb.temperature(0)
    V, N = 8, 4
    lg = np.stack([_row_with_entropy(0.001, V, tau) for _ in range(N)])[None]
    sh = eb.EBShadow(stopped=np.array([True]), dlogit=10.0)
    eb.eb_update(lg, np.zeros((1, N), np.int32), np.zeros((1, N), np.uint8), 0, eb.EBState(1), [7], 0,
                 shadow=sh)
    assert len(sh.failures) == 1 and sh.adopted["stop"] == 0
