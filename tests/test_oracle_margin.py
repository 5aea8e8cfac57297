"""Pins of oracle.run.decision_margin, the band the GPU lockstep uses to tell a
genuine near-tie from a wrong decision (no GPU).

Soundness by brute force: on small random blocks every decision of a step --
commit set, fallback flag, committed ids, the tracked ids handed to the credit
state, the kept smoothing id sets -- is recomputed from perturbed logits with
|perturbation| <= 0.45 * margin (random and adversarial directions: the top
logit up or down against the rest, adjacent pairs of the top nine squeezed);
none may change.  A margin that leaves out a decision fails here.

Tightness by hand-worked cases: each kind of decision is made the only close
one, and the margin must equal its closed form.  A margin that counts a
decision the step did not take (the fallback gap when a candidate passed a
gate, the order inside a kept top-8 set) fails here."""
import math

import numpy as np
import pytest

from oracle.decode import credit_update, select_commits, vocab_stats
from oracle.run import decision_margin
import synth


def _dcfg(tau=0.9, credit=1.0, alpha=0.3, hier=False, kappa=1.5, gamma=0.7):
    return synth.DecodeCfg(block_len=8, vicinity_w=0, tau=tau, credit_weight=credit,
                           credit_decay=gamma, credit_kappa=kappa, smooth_alpha=alpha,
                           hierarchical=hier)


def _decide(z, masked, c_prev, t_prev, d, mask_id):
    """Every integer outcome of one step, recomputed from the logits."""
    R = z.shape[0]
    st = vocab_stats(z, np.full(R, -1), 0.0, mask_id, 8)
    c, t = credit_update(c_prev, t_prev, st["argmax"], st["conf"], masked, d.credit_decay,
                         d.credit_weight)
    T, fb = select_commits(masked, st["conf"], c, d.tau, d.credit_kappa, d.hierarchical)
    still = masked.copy()
    still[T] = False
    out = [tuple(int(x) for x in T), bool(fb), tuple(int(st["argmax"][i]) for i in T)]
    if d.credit_weight != 0.0:
        out.append(tuple(int(x) for x in t))
    if d.smooth_alpha != 0.0:
        out.append(tuple(tuple(sorted(int(x) for x in st["topk_id"][i])) for i in np.nonzero(still)[0]))
    margin = decision_margin(st, masked, c, d, T, still, fb)
    return tuple(out), margin


def _case(rng):
    B, V = 8, 14
    mask_id = V - 1
    d = _dcfg(tau=float(rng.choice([0.3, 0.5, 0.9])), credit=float(rng.choice([0.0, 1.0])),
              alpha=float(rng.choice([0.0, 0.3])), hier=bool(rng.random() < 0.3),
              kappa=float(rng.choice([0.6, 1.5])))
    scale = rng.choice([0.5, 1.5, 3.0])
    z = rng.standard_normal((B, V)) * scale
    # some rows get a clear favourite so gates pass, some near-even rows
    lift = rng.random(B) < 0.4
    z[lift, rng.integers(0, V - 1, B)[lift]] += rng.uniform(1.0, 5.0, lift.sum())
    masked = rng.random(B) < 0.8
    masked[rng.integers(0, B)] = True
    # prior credit as the method leaves it: none at all with credit off
    c_prev = np.where(rng.random(B) < 0.5, rng.uniform(0, 1.4, B), 0.0).astype(np.float32)
    c_prev *= np.float32(d.credit_weight != 0.0)
    am = np.argmax(np.where(np.arange(V) == mask_id, -np.inf, z), axis=1)
    t_prev = np.where(rng.random(B) < 0.6, am, rng.integers(-1, V - 1, B))
    return z, masked, c_prev, t_prev, d, mask_id


def _adversarial(z, delta, rng):
    """Perturbations of at most delta per logit that push decisions hardest:
    the row's top logit against all others (moves its log-probability by up
    to 2 delta), or two adjacent logits among its top nine squeezed together."""
    R, V = z.shape
    eps = np.zeros_like(z)
    for r in range(R):
        kind = rng.integers(0, 4)
        order = np.argsort(-z[r], kind="stable")
        if kind == 0:
            eps[r] = -delta
            eps[r, order[0]] = delta
        elif kind == 1:
            eps[r] = delta
            eps[r, order[0]] = -delta
        elif kind == 2:
            k = rng.integers(0, 9)
            eps[r, order[k]] = -delta
            eps[r, order[k + 1]] = delta
        else:
            eps[r] = rng.uniform(-delta, delta, V)
    return eps


def test_margin_is_sound_against_perturbed_recomputation():
    rng = np.random.default_rng(2024)
    checked = 0
    for _ in range(400):
        z, masked, c_prev, t_prev, d, mask_id = _case(rng)
        base, m = _decide(z, masked, c_prev, t_prev, d, mask_id)
        if not np.isfinite(m) or m < 1e-4:       # fp32 rounding of the logits dominates
            continue
        delta = 0.45 * m
        for _ in range(30):
            got, _ = _decide(z + _adversarial(z, delta, rng), masked, c_prev, t_prev, d, mask_id)
            assert got == base, (d, m)
        checked += 1
    assert checked > 250


def _row(V, top, rest=0.0, mask_id=None):
    z = np.full(V, rest, dtype=np.float64)
    for i, v in enumerate(top):
        z[i] = v
    if mask_id is not None:
        z[mask_id] = 0.0
    return z


def _st(z, mask_id):
    return vocab_stats(z, np.full(z.shape[0], -1), 0.0, mask_id, 8)


def test_fallback_gap_halved_and_counted_only_when_taken():
    # Two masked rows, nothing passes tau = 0.99: the fallback commits row 0;
    # its margin against row 1 is half their log-confidence gap.
    V, mask_id = 16, 15
    z = np.stack([_row(V, [2.0]), _row(V, [1.99])])      # confidences about 0.345, 0.343
    st = _st(z, mask_id)
    d = _dcfg(tau=0.99, credit=0.0, alpha=0.0)
    masked = np.array([True, True])
    T, fb = select_commits(masked, st["conf"], np.zeros(2, np.float32), d.tau, d.credit_kappa, False)
    assert fb and list(T) == [0]
    p = st["conf"].astype(np.float64)
    want = 0.5 * (math.log(p[0]) - math.log(p[1]))
    gates = np.abs(np.log(p) - math.log(0.99))
    assert want < gates.min() and want < st["topk_p"][0, 0]   # the fallback gap decides
    assert decision_margin(st, masked, np.zeros(2, np.float32), d, T, None, fb) == pytest.approx(want, rel=1e-9)
    # Now tau = 0.3: both rows pass, no fallback; their near-equal
    # confidences decide nothing.
    d2 = _dcfg(tau=0.3, credit=0.0, alpha=0.0)
    T2, fb2 = select_commits(masked, st["conf"], np.zeros(2, np.float32), 0.3, 1.5, False)
    assert not fb2 and list(T2) == [0, 1]
    m2 = decision_margin(st, masked, np.zeros(2, np.float32), d2, T2, None, fb2)
    want2 = min(float(np.min(np.abs(np.log(p) - math.log(0.3)))),
                float(np.min(np.log(st["topk_p"][:, 0]) - np.log(st["topk_p"][:, 1]))))
    assert m2 == pytest.approx(want2, rel=1e-9)
    assert m2 > 10 * want


def test_tracked_id_gap_counts_only_with_credit():
    # Row 0 commits with a wide gap; row 1 stays masked with its top two logits
    # 0.003 apart.  With credit on, its argmax feeds the credit state.
    V, mask_id = 16, 15
    z = np.full((2, V), -6.0)
    z[0, 3] = 8.0
    z[1, 4], z[1, 5] = 0.003, 0.0
    st = _st(z, mask_id)
    masked = np.array([True, True])
    credit = np.array([0.0, 0.0], np.float32)
    for lam, want_small in ((1.0, True), (0.0, False)):
        d = _dcfg(tau=0.9, credit=lam, alpha=0.0, kappa=1.5)
        c, _ = credit_update(credit, np.array([-1, -1]), st["argmax"], st["conf"], masked,
                             d.credit_decay, d.credit_weight)
        T, fb = select_commits(masked, st["conf"], c, d.tau, d.credit_kappa, False)
        assert list(T) == [0] and not fb
        m = decision_margin(st, masked, c, d, T, masked & (np.arange(2) != 0), fb)
        if want_small:
            assert m == pytest.approx(0.003, rel=1e-4)
        else:
            assert m > 0.1


def test_smoothing_margin_is_the_set_boundary_not_the_order():
    # A still-masked row whose top eight logits sit 1e-6 apart but whose 8th
    # and 9th are 0.004 apart: the kept set is decided with margin 0.004.
    V, mask_id = 32, 31
    z = np.full((2, V), -8.0)
    z[0, 0] = 9.0                                   # row 0 commits (tau 0.9)
    top8 = 1.0 - 1e-6 * np.arange(8)
    z[1, 10:18] = top8
    z[1, 18] = top8[-1] - 0.004
    st = _st(z, mask_id)
    d = _dcfg(tau=0.9, credit=0.0, alpha=0.3)
    masked = np.array([True, True])
    T, fb = select_commits(masked, st["conf"], np.zeros(2, np.float32), d.tau, d.credit_kappa, False)
    assert list(T) == [0] and not fb
    still = np.array([False, True])
    m = decision_margin(st, masked, np.zeros(2, np.float32), d, T, still, fb)
    gates = float(np.min(np.abs(np.log(st["conf"].astype(np.float64)) - math.log(0.9))))
    assert m == pytest.approx(min(0.004, gates), rel=1e-3)
    assert m > 1e-3


def test_gate_margins_closed_form():
    # One masked row, confidence tau * e^0.01: the threshold gate decides.
    V, mask_id = 16, 15
    tau = 0.6
    # p = e^a / (e^a + 14): choose a so that ln p = ln tau + 0.01
    p = tau * math.exp(0.01)
    a = math.log(14.0 * p / (1.0 - p))
    z = np.zeros((1, V))
    z[0, 0] = a
    st = _st(z, mask_id)
    d = _dcfg(tau=tau, credit=0.0, alpha=0.0)
    masked = np.array([True])
    T, fb = select_commits(masked, st["conf"], np.zeros(1, np.float32), tau, 1.5, False)
    assert list(T) == [0] and not fb
    m = decision_margin(st, masked, np.zeros(1, np.float32), d, T, None, fb)
    assert m == pytest.approx(0.01, abs=2e-6)          # fp32 rounding of the confidence
    # the credit gate: credit kappa * e^-0.02 with credit on
    d2 = _dcfg(tau=0.99, credit=1.0, alpha=0.0, kappa=1.5)
    c = np.array([1.5 * math.exp(-0.02)], np.float32)
    T2, fb2 = select_commits(masked, st["conf"], c, 0.99, 1.5, False)
    m2 = decision_margin(st, masked, c, d2, T2, None, fb2)
    assert m2 == pytest.approx(0.02, abs=2e-6)
