"""Pins of the deficit token-budget scheduler oracle (Sangam abstract): a
hand-worked schedule, its two limits (unbounded budget: every waiting refresh
admitted at once; zero budget: one refresh per round with no decode) and a
cumulative-credit formulation of one busy period that shares no step with the
oracle's running counter."""
import numpy as np
import pytest

from oracle.sched import DeficitScheduler


def test_hand_worked_schedule():
    # budget 100 tokens per round, three slots
    s = DeficitScheduler(100, 3)
    rounds = [
        # (decode rows, refresh rows) -> (admitted, counter after the round)
        # idle round: queue [0, 1]; 0 + 100 = 100 < 150 but nothing decodes, so
        # the head is admitted anyway (100 - 150 = -50); -50 < 50 stops slot 1
        (([0, 0, 0], [150, 50, 0]), ([1, 0, 0], -50)),
        # -50 + 100 - 30 = 20 < 50
        (([30, 0, 0], [0, 50, 0]), ([0, 0, 0], 20)),
        # slot 2 joins behind slot 1: 20 + 70 = 90 -> admit 1 (40); 40 < 80
        (([30, 0, 0], [0, 50, 80]), ([0, 1, 0], 40)),
        # 40 + 100 - 60 = 80 -> admit 2 (0); queue empty -> 0
        (([30, 30, 0], [0, 0, 80]), ([0, 0, 1], 0)),
        # nothing waits: 100 - 90 = 10 is not banked
        (([30, 30, 30], [0, 0, 0]), ([0, 0, 0], 0)),
        # 100 - 60 = 40 -> admit 2 exactly
        (([30, 30, 0], [0, 0, 40]), ([0, 0, 1], 0)),
        # decode overload: 100 - 120 = -20 < 10
        (([120, 0, 0], [0, 10, 10]), ([0, 0, 0], -20)),
        # slot 0 joins behind 1, 2; idle: -20 + 100 = 80 -> 1 (70), 2 (60), 0 (0)
        (([0, 0, 0], [60, 10, 10]), ([1, 1, 1], 0)),
        (([10, 10, 10], [0, 0, 0]), ([0, 0, 0], 0)),
        # head-of-line: slot 1 (200) blocks slot 2 (10) although 2 would fit
        (([50, 0, 0], [0, 200, 10]), ([0, 0, 0], 50)),
        (([50, 0, 0], [0, 200, 10]), ([0, 0, 0], 100)),
        (([50, 0, 0], [0, 200, 10]), ([0, 0, 0], 150)),
        # 150 + 50 = 200 -> admit 1 (0); 0 < 10
        (([50, 0, 0], [0, 200, 10]), ([0, 1, 0], 0)),
        # 0 + 100 - 90 = 10 -> admit 2 (0)
        (([50, 40, 0], [0, 0, 10]), ([0, 0, 1], 0)),
    ]
    for i, ((dec, ref), (want, deficit)) in enumerate(rounds):
        got = s.round(dec, ref)
        assert got == want, (i, got, want)
        assert s.deficit == deficit, (i, s.deficit, deficit)


def test_withdrawn_slot_leaves_the_queue():
    s = DeficitScheduler(10, 2)
    assert s.round([5, 0], [0, 100]) == [0, 0]          # 5 < 100
    assert s.round([5, 0], [0, 0]) == [0, 0]            # slot 1 no longer waits
    assert s.queue == [] and s.deficit == 0
    assert s.round([5, 0], [0, 5]) == [0, 1]            # a fresh wait starts from zero


def test_unbounded_budget_admits_every_waiting_refresh_at_once():
    rng = np.random.default_rng(1)
    n = 6
    s = DeficitScheduler(1 << 60, n)
    for _ in range(200):
        state = rng.integers(0, 3, size=n)              # 0 idle, 1 decoding, 2 waiting
        dec = np.where(state == 1, rng.integers(1, 200, size=n), 0)
        ref = np.where(state == 2, rng.integers(1, 5000, size=n), 0)
        assert s.round(dec, ref) == [int(x) for x in (state == 2)]


def test_zero_budget_admits_one_refresh_per_round_without_decodes():
    rng = np.random.default_rng(2)
    n = 5
    s = DeficitScheduler(0, n)
    waiting = []
    for _ in range(300):
        state = rng.integers(0, 3, size=n)
        dec = np.where(state == 1, rng.integers(1, 200, size=n), 0)
        ref = np.where(state == 2, rng.integers(1, 5000, size=n), 0)
        waiting = [r for r in waiting if state[r] == 2] + \
                  [r for r in range(n) if state[r] == 2 and r not in waiting]
        got = s.round(dec, ref)
        if dec.sum() == 0 and waiting:
            assert got == [int(r == waiting[0]) for r in range(n)]
            waiting.pop(0)
        else:
            assert not any(got)


@pytest.mark.parametrize("seed", range(20))
def test_busy_period_matches_cumulative_credit(seed):
    """Every slot starts waiting in round 0 and some slot decodes in every
    round: the k-th slot (slot order) is admitted in the first round t at which
    the credit of rounds 0..t, sum(budget - decode rows), covers the first k
    refreshes together."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 8))
    budget = int(rng.integers(50, 500))
    costs = rng.integers(1, 2000, size=n)
    # decoding happens on a separate set of slots; only their total matters
    T = 400
    dec_tot = rng.integers(1, budget + 100, size=T)
    credit = np.cumsum(budget - dec_tot)
    need = np.cumsum(costs)
    want = []
    for k in range(n):
        t_ok = np.nonzero(credit >= need[k])[0]
        want.append(int(t_ok[0]) if len(t_ok) else None)
    s = DeficitScheduler(budget, n + 1)
    ref = list(costs) + [0]
    got = [None] * n
    for t in range(T):
        dec = [0] * n + [int(dec_tot[t])]
        adm = s.round(dec, ref)
        for r in range(n):
            if adm[r]:
                got[r] = t
                ref[r] = 0
    assert got == want


def test_rejects_bad_rounds():
    s = DeficitScheduler(10, 2)
    with pytest.raises(ValueError):
        s.round([1, 0], [1, 0])                         # decodes and waits at once
    with pytest.raises(ValueError):
        s.round([-1, 0], [0, 0])
    with pytest.raises(ValueError):
        s.round([0], [0])
    with pytest.raises(ValueError):
        DeficitScheduler(-1, 2)
