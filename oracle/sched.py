"""Oracle of the deficit token-budget admission of whole KV refreshes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Sangam: Efficiently Serving Diffusion LLMs with the AR Stack"
(abstract).  With cached decoding a request alternates between decodes (one
denoising step over its block and the neighbouring window) and prefills (a
whole refresh of its KV cache, which recurs at every block start and cannot be
split into chunks because attention is bidirectional).  The scheduler gives
each scheduling round a token budget, lets the in-flight decodes spend it
first, admits waiting prefills only as whole units and only once the budget
accumulated so far covers them, and carries what is left to later rounds.

Readings where the abstract leaves a step open (the plainest ones that agree
with the rest of it):
  * tokens are rows the model computes: a decode costs its window rows, a
    prefill the request's full length;
  * waiting prefills are served first-come first-served; slots that start to
    wait in the same round queue in slot order; the head of the queue blocks
    the ones behind it (no smaller prefill overtakes a larger one, so none
    starves);
  * the counter runs only while a prefill waits: when the queue is empty at
    the end of a round it returns to zero (the rule of deficit round robin for
    an idle flow), so budget left over while nothing waits is not banked for
    a later burst, and decode overload while nothing waits is not a debt;
  * liveness: in a round with no decode, the head of the queue is admitted
    even if the counter does not cover it, and the counter goes negative by
    the difference (otherwise nothing would run).
"""
from __future__ import annotations


class DeficitScheduler:
    """State: the FIFO queue of waiting slots and the deficit counter."""

    def __init__(self, budget: int, n_slots: int):
        if budget < 0 or n_slots < 1:
            raise ValueError("budget must be >= 0 and n_slots >= 1")
        self.budget = int(budget)
        self.n = int(n_slots)
        self.queue: list[int] = []
        self.deficit = 0

    def round(self, decode_rows, refresh_rows):
        """One scheduling round.  decode_rows[r] > 0: slot r decodes in this
        round (its rows); refresh_rows[r] > 0: slot r waits for a whole refresh
        of that many rows.  Returns the list of admitted flags."""
        dec = [int(x) for x in decode_rows]
        ref = [int(x) for x in refresh_rows]
        if len(dec) != self.n or len(ref) != self.n:
            raise ValueError("one entry per slot")
        for r in range(self.n):
            if dec[r] < 0 or ref[r] < 0 or (dec[r] > 0 and ref[r] > 0):
                raise ValueError("a slot decodes or waits, with non-negative rows")
        # arrivals join the tail (slot order within the round); slots that no
        # longer wait leave the queue
        self.queue = [r for r in self.queue if ref[r] > 0]
        for r in range(self.n):
            if ref[r] > 0 and r not in self.queue:
                self.queue.append(r)
        # this round's budget, spent by the decodes first
        self.deficit += self.budget - sum(dec)
        decoding = any(d > 0 for d in dec)
        admit = [0] * self.n
        while self.queue:
            head = self.queue[0]
            idle = not decoding and not any(admit)
            if self.deficit >= ref[head] or idle:
                admit[head] = 1
                self.deficit -= ref[head]
                self.queue.pop(0)
            else:
                break
        if not self.queue:
            self.deficit = 0
        return admit
