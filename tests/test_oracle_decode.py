"""Pins of the oracle's vocab statistics and commit rules (no GPU)."""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

from oracle.decode import (candidates, credit_update, run_midpoints, select_commits,
                           smoothing_state, soft_embedding, vocab_stats)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(99)


# ----------------------------------------------------------------- vocab stats
def test_softmax_rows_sum_to_one_and_lse_closed_form():
    z = RNG.standard_normal((6, 500)) * 3
    pid = np.array([-1, 5, -1, 499, 17, -1])
    st = vocab_stats(z, pid, 4.0, mask_id=499, k=8)
    biased = z.copy()
    for r in range(6):
        if pid[r] >= 0:
            biased[r, pid[r]] += 4.0
    b32 = biased.astype(np.float32).astype(np.float64)
    b32[:, 499] = -np.inf
    lse = scipy.special.logsumexp(b32, axis=1)
    assert np.allclose(st["lse"], lse, rtol=0, atol=1e-12)
    probs = np.exp(b32 - st["lse"][:, None])
    assert np.all(np.abs(probs.sum(1) - 1.0) <= 1e-6)
    assert np.allclose(st["conf"], probs.max(1).astype(np.float32), rtol=1e-7)


def _bruteforce_topk(row, k):
    idx = sorted(range(len(row)), key=lambda i: (-row[i], i))
    return idx[:k]


def test_argmax_and_topk_bruteforce_with_ties_and_mask():
    V = 40
    z = np.round(RNG.standard_normal((8, V)) * 2, 1)      # many exact ties after rounding
    z[:, V - 1] = 100.0                                   # MASK would win if not excluded
    z[3, :] = 0.5                                         # a row of all-equal values
    st = vocab_stats(z, np.full(8, -1), 0.0, mask_id=V - 1, k=8)
    for r in range(8):
        row = [float(np.float32(v)) if i != V - 1 else -np.inf for i, v in enumerate(z[r])]
        want = _bruteforce_topk(row, 8)
        assert st["argmax"][r] == want[0]
        assert st["topk_id"][r].tolist() == want
        assert V - 1 not in st["topk_id"][r]
        # reported gaps, from the brute-force order: k-th minus (k+1)-th, and
        # the smallest consecutive gap among the k+1 largest
        top9 = sorted(row, reverse=True)[:9]
        assert st["kth_gap"][r] == pytest.approx(top9[7] - top9[8], abs=1e-12)
        assert st["rank_gap"][r] == pytest.approx(min(a - b for a, b in zip(top9, top9[1:])),
                                                  abs=1e-12)


def test_planted_confidence_closed_form():
    # All logits 0 and one planted id with bias b: the MASK entry is excluded,
    # so p = e^b / (e^b + V - 2).
    V, b = 1000, 6.0
    z = np.zeros((1, V))
    st = vocab_stats(z, np.array([123]), b, mask_id=V - 1, k=8)
    want = np.exp(np.float64(np.float32(b))) / (np.exp(np.float64(np.float32(b))) + V - 2)
    assert st["argmax"][0] == 123
    assert abs(float(st["conf"][0]) - want) <= 1e-7 * want
    # the other top-k entries are the lowest ids (all tied at 0)
    assert st["topk_id"][0].tolist() == [123, 0, 1, 2, 3, 4, 5, 6]


# ----------------------------------------------------------------------- credit
def test_credit_closed_form_for_constant_confidence():
    lam, gam = 1.0, 0.7
    for p in [0.8, 0.5, 0.3, 0.95]:
        c = np.zeros(1, np.float32)
        t = np.array([-1])
        for n in range(1, 15):
            c, t = credit_update(c, t, np.array([42]), np.array([p], np.float32), np.array([True]),
                                 gam, lam)
            want = lam * np.float32(p) * (1 - gam ** n) / (1 - gam)
            assert abs(float(c[0]) - want) <= 4e-7 * want * n


def test_credit_resets_on_argmax_change_and_ignores_unmasked():
    c = np.array([1.0, 1.0, 1.0], np.float32)
    t = np.array([5, 5, 5])
    c2, t2 = credit_update(c, t, np.array([5, 6, 6]), np.array([0.5, 0.5, 0.5], np.float32),
                           np.array([True, True, False]), 0.7, 1.0)
    assert c2[0] == np.float32(np.float32(0.7) * np.float32(1.0)) + np.float32(0.5)
    assert c2[1] == np.float32(0.5)          # argmax changed -> decayed part dropped
    assert c2[2] == np.float32(1.0) and t2[2] == 5   # not masked -> untouched
    assert t2[1] == 6


def test_credit_golden_commit_steps():
    g = json.load(open(os.path.join(GOLDEN, "credit_examples.json")))
    for case in g["cases"]:
        masked = np.ones(1, bool)
        c, t = np.zeros(1, np.float32), np.array([-1])
        step = None
        for n in range(1, 40):
            c, t = credit_update(c, t, np.array([7]), np.array([case["p"]], np.float32), masked,
                                 g["gamma"], g["lambda"])
            T, fb = select_commits(np.array([True, True]), np.array([case["p"], 0.0], np.float32),
                                   np.array([c[0], 0.0], np.float32), 0.9, g["kappa"], False)
            if not fb:
                step = n
                break
        assert step == case["commit_step"], case


# -------------------------------------------------------------------- selection
def _recursive_levels(B):
    levels = {}

    def rec(lo, hi, depth):
        if lo >= hi:
            return
        mid = lo + (hi - lo - 1) // 2
        levels.setdefault(depth, []).append(mid)
        rec(lo, mid, depth + 1)
        rec(mid + 1, hi, depth + 1)

    rec(0, B, 0)
    return [sorted(levels[k]) for k in sorted(levels)]


def _simulate_all_pass(B):
    masked = np.ones(B, bool)
    out = []
    while masked.any():
        T, fb = select_commits(masked, np.ones(B, np.float32), np.zeros(B, np.float32), 0.9, 1.5,
                               True)
        out.append(sorted(T.tolist()))
        masked[T] = False
    return out


def test_hierarchical_golden_levels():
    g = json.load(open(os.path.join(GOLDEN, "hierarchical_order.json")))
    for case in g["cases"]:
        assert _simulate_all_pass(case["block_len"]) == case["levels"]


@pytest.mark.parametrize("B", list(range(1, 17)))
def test_hierarchical_matches_recursive_midpoints(B):
    assert _simulate_all_pass(B) == _recursive_levels(B)


def _runs_by_groupby(masked):
    mids, i = [], 0
    for key, grp in itertools.groupby(masked):
        n = len(list(grp))
        if key:
            mids.append(i + (n - 1) // 2)
        i += n
    return mids


@pytest.mark.parametrize("B", [1, 2, 3, 7, 12])
def test_hierarchical_candidates_all_patterns(B):
    for bits in range(1 << B):
        masked = [(bits >> i) & 1 == 1 for i in range(B)]
        assert run_midpoints(np.array(masked)).tolist() == _runs_by_groupby(masked)


def test_select_invariants_bruteforce_small_blocks():
    tau, kappa = np.float32(0.9), np.float32(1.5)
    for B in [1, 3, 6]:
        for bits in range(1, 1 << B):
            masked = np.array([(bits >> i) & 1 == 1 for i in range(B)])
            conf = RNG.choice(np.float32([0.2, 0.5, 0.9, 0.95, 0.5]), size=B)
            credit = RNG.choice(np.float32([0.0, 1.4, 1.5, 2.0]), size=B)
            for hier in (False, True):
                T, fb = select_commits(masked, conf, credit, tau, kappa, hier)
                C = set(candidates(masked, hier).tolist())
                assert len(T) >= 1 and set(T.tolist()) <= C and all(masked[T])
                passing = {i for i in C if conf[i] >= tau or credit[i] >= kappa}
                if passing:
                    assert set(T.tolist()) == passing and not fb
                else:
                    best = max(C, key=lambda i: (conf[i], -i))
                    assert T.tolist() == [best] and fb


def test_zero_credit_weight_is_plain_threshold():
    # Credit starts at 0 at every block start; with lambda = 0 it stays 0 along
    # any trajectory, so the commits are those of plain threshold decoding.
    B = 8
    for _ in range(50):
        c = np.zeros(B, np.float32)
        t = np.full(B, -1)
        masked = np.ones(B, bool)
        while masked.any():
            conf = RNG.random(B).astype(np.float32)
            am = RNG.integers(0, 3, B)
            c, t = credit_update(c, t, am, conf, masked, 0.7, 0.0)
            assert np.all(c == 0)
            T1, _ = select_commits(masked, conf, c, 0.9, 1.5, False)
            T2, _ = select_commits(masked, conf, np.zeros(B, np.float32), 0.9, np.inf, False)
            assert T1.tolist() == T2.tolist()
            masked[T1] = False


# -------------------------------------------------------------------- smoothing
def test_smoothing_reductions():
    d, k = 16, 8
    E = RNG.standard_normal((50, d))
    ids = RNG.integers(0, 49, (3, k))
    ids, pt = smoothing_state(ids, RNG.random((3, k)))
    assert np.allclose(pt.sum(1), 1.0, atol=1e-15)
    # alpha = 0: the plain MASK embedding
    e = soft_embedding(E[49], E[ids], pt, 0.0)
    assert np.array_equal(e, np.broadcast_to(E[49], e.shape))
    # alpha = 1 with a one-hot distribution: the token's own embedding
    oh = np.zeros((3, k))
    oh[:, 0] = 1.0
    e = soft_embedding(E[49], E[ids], oh, 1.0)
    assert np.allclose(e, E[ids[:, 0]], atol=1e-15)
    # convexity: the mixture lies in the hull, so its distance to E[MASK] is
    # at most alpha * the farthest top-k embedding
    e = soft_embedding(E[49], E[ids], pt, 0.3)
    far = np.max(np.linalg.norm(E[ids] - E[49], axis=-1), axis=1)
    assert np.all(np.linalg.norm(e - E[49], axis=-1) <= 0.3 * far + 1e-12)
