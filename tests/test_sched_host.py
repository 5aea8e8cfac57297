"""The library's deficit token-budget scheduler (dinfer_sched_*, host code,
no GPU) against the oracle scheduler: admissions and counter identical,
round by round, on seeded sequences of rounds that mix decoding, waiting,
idle and withdrawn slots and rounds with no decode."""
import numpy as np
import pytest

from diffusion_vicinity_kv_amd import binding as B
from oracle.sched import DeficitScheduler as OracleSched


def _rounds(rng, n, T):
    """Per round: each slot decodes, waits (a refresh of fixed rows until it is
    admitted or withdrawn) or idles; about one round in six has no decode."""
    waiting = {}
    for _ in range(T):
        dec = [0] * n
        ref = [0] * n
        no_decode = rng.random() < 1 / 6
        for r in range(n):
            if r in waiting:
                if rng.random() < 0.05:
                    del waiting[r]                      # withdrawn
                else:
                    ref[r] = waiting[r]
                    continue
            u = rng.random()
            if u < 0.25:
                waiting[r] = int(rng.integers(1, 3000))
                ref[r] = waiting[r]
            elif u < 0.8 and not no_decode:
                dec[r] = int(rng.integers(1, 400))
        yield dec, ref, waiting


@pytest.mark.parametrize("budget", [0, 1, 97, 640, 4096, 1 << 40])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_library_scheduler_matches_oracle(budget, seed):
    rng = np.random.default_rng(1000 * seed + 7)
    n = int(rng.integers(1, 17))
    lib_s = B.DeficitScheduler(budget, n)
    ora = OracleSched(budget, n)
    admitted = 0
    for t, (dec, ref, waiting) in enumerate(_rounds(rng, n, 400)):
        got, deficit = lib_s.round(dec, ref)
        want = ora.round(dec, ref)
        assert got == want, (t, dec, ref, got, want)
        assert deficit == ora.deficit, (t, deficit, ora.deficit)
        for r in range(n):
            if got[r]:
                waiting.pop(r, None)
        admitted += sum(got)
    assert admitted > 0
    lib_s.close()


def test_library_scheduler_rejects_bad_rounds_and_keeps_its_state():
    s = B.DeficitScheduler(100, 2)
    # idle round: the head is admitted; the queue is then empty, the counter 0
    assert s.round([0, 0], [0, 500]) == ([0, 1], 0)
    with pytest.raises(B.DinferError):
        s.round([1, 0], [1, 0])
    with pytest.raises(B.DinferError):
        s.round([0, -1], [0, 0])
    # state unchanged by the rejected rounds: 100 - 50 = 50 < 60 stays queued
    assert s.round([50, 0], [0, 60]) == ([0, 0], 50)
    s.close()
    for budget, n in [(-1, 2), ((1 << 62) + 1, 2), (10, 0)]:
        with pytest.raises(B.DinferError):
            B.DeficitScheduler(budget, n)
