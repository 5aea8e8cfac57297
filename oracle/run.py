"""Oracle iteration manager: blocks, refreshes and denoising steps of one request.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Structure (dInfer abstract: model, diffusion iteration manager, decoding
strategy, KV-cache manager; Sangam abstract: a masked response is denoised
block by block, cached KV is refreshed and reused across the decodes in
between; dInfer news article, section "削减计算成本：邻近KV缓存刷新": each
iteration recomputes KV only for the current block and a small neighbourhood
and leaves distant entries as they are):

  for each block [bs, be) of the response, left to right, while the
  response holds MASK (an end-of-sequence token fills the rest; see
  decode.eos_fill):
      full refresh: every position's K, V recomputed from hard embeddings
      credit, tracked ids and smoothing state reset
      while the block holds MASK:
          window [max(0, bs-w), min(L, be+w)) runs through every layer with its
          K, V scattered into the cache first; block rows -> final norm -> LM
          head -> vocab stats -> credit -> commit -> smoothing state

Requests are independent; a batch is a loop over requests.
"""
from __future__ import annotations

import numpy as np

from .decode import (F32, vocab_stats, credit_update, select_commits, smoothing_state,
                     soft_embedding, eos_fill)
from .model import OracleModel


class OracleRun:
    """Decode state of one request driven step by step."""

    def __init__(self, model: OracleModel, dcfg, tokens, prompt_len, gen_len, plant_id,
                 plant_bias, router_bias=None, kv_round=None):
        self.model = model
        self.m = model.m
        self.d = dcfg
        self.P = int(prompt_len)
        self.G = int(gen_len)
        self.L = self.P + self.G
        self.tokens = np.array(tokens[: self.L], dtype=np.int64)
        self.plant_id = np.array(plant_id[: self.L], dtype=np.int64)
        self.plant_bias = float(plant_bias)
        self.router_bias = None if router_bias is None else np.asarray(router_bias, dtype=np.float64)
        self.B = dcfg.block_len
        self.n_blocks = self.G // self.B
        self.cache = model.new_cache(self.L, kv_round)
        self.block = -1
        self.steps = []            # steps per finished block
        self.records = []          # per-step details
        self.complete = False      # no MASK left in the response (end-of-sequence)
        self._k = dcfg.smooth_topk
        self.refresh_route_margin = np.inf        # MoE routing near-ties (reported)
        self.step_route_margin_rows = None
        self.step_route_margin_window = np.inf
        self.refresh_record = self.step_record = None   # MoE: experts, route_margin per layer

    # --- block bookkeeping ------------------------------------------------
    @property
    def bs(self):
        return self.P + self.block * self.B

    @property
    def be(self):
        return self.bs + self.B

    def window(self):
        w = self.d.vicinity_w
        return max(0, self.bs - w), min(self.L, self.be + w)

    def _router_bias_block(self):
        if self.router_bias is None:
            return None
        return self.router_bias[:, self.block, :]

    def block_masked(self):
        return self.tokens[self.bs:self.be] == self.m.mask_id

    def start_block(self, k):
        """Full refresh at the block start, then reset the per-block decode state."""
        self.block = k
        pos = np.arange(self.L)
        e = self.model.embed(self.tokens[pos])
        rec = {} if self.m.is_moe else None
        self.model.forward_rows(self.cache, pos, e, self.L, self._router_bias_block(), rec)
        # routing near-ties of layers whose output feeds a later layer's cache
        self.refresh_route_margin = _min_route_margin(rec, self.model.layer_ids[:-1])
        self.refresh_record = rec
        B, kk = self.B, self._k
        self.credit = np.zeros(B, dtype=F32)
        self.tracked = np.full(B, -1, dtype=np.int64)
        self.smooth_valid = np.zeros(B, dtype=bool)
        self.smooth_ids = np.zeros((B, kk), dtype=np.int64)
        self.smooth_p = np.zeros((B, kk), dtype=np.float64)
        self.block_steps = 0

    # --- one denoising step ------------------------------------------------
    def window_embeddings(self, lo, hi):
        """Hard embeddings, except soft ones for still-masked block rows with state."""
        e = self.model.embed(self.tokens[lo:hi])
        alpha = self.d.smooth_alpha
        if alpha != 0.0:
            masked = self.block_masked()
            soft = np.nonzero(masked & self.smooth_valid)[0]
            if len(soft):
                e_mask = self.model.embed([self.m.mask_id])[0]
                e_ids = self.model.embed(self.smooth_ids[soft].reshape(-1)).reshape(
                    len(soft), self._k, -1)
                e[soft + (self.bs - lo)] = soft_embedding(e_mask, e_ids, self.smooth_p[soft], alpha)
        return e

    def denoise_logits(self):
        """Vicinity step over the current window; returns fp64 logits of the block rows."""
        lo, hi = self.window()
        pos = np.arange(lo, hi)
        e = self.window_embeddings(lo, hi)
        rec = {} if self.m.is_moe else None
        h = self.model.forward_rows(self.cache, pos, e, self.L, self._router_bias_block(), rec)
        if rec is not None:
            # per block row: its own routing in every layer; any window row's
            # routing below the last layer also reaches every row through the cache
            own = np.min(np.stack([rec["route_margin"][li] for li in self.model.layer_ids]), axis=0)
            self.step_route_margin_rows = own[self.bs - lo: self.be - lo]
            self.step_route_margin_window = _min_route_margin(rec, self.model.layer_ids[:-1])
            self.step_record = rec
        hb = h[self.bs - lo: self.be - lo]
        return self.model.logits(hb)

    def stats(self, logits):
        return vocab_stats(logits, self.plant_id[self.bs:self.be], self.plant_bias,
                           self.m.mask_id, self._k)

    def commit(self, st):
        """Credit update, selection, token writes and smoothing state for one step."""
        d = self.d
        masked = self.block_masked()
        self.credit, self.tracked = credit_update(self.credit, self.tracked, st["argmax"],
                                                  st["conf"], masked, d.credit_decay,
                                                  d.credit_weight)
        T, fallback = select_commits(masked, st["conf"], self.credit, d.tau, d.credit_kappa,
                                     d.hierarchical)
        self.tokens[self.bs + T] = st["argmax"][T]
        self.complete = eos_fill(self.tokens, self.P, self.L, self.m.mask_id,
                                 getattr(d, "eos_id", -1))
        still = self.block_masked()
        ids, pt = smoothing_state(st["topk_id"], st["topk_p"])
        self.smooth_ids = np.where(still[:, None], ids, self.smooth_ids)
        self.smooth_p = np.where(still[:, None], pt, self.smooth_p)
        self.smooth_valid = still.copy()
        self.block_steps += 1
        rec = {"block": self.block, "commits": T.copy(), "fallback": fallback,
               "margin": decision_margin(st, masked, self.credit, d, T, still, fallback)}
        self.records.append(rec)
        return T, fallback

    def step(self):
        logits = self.denoise_logits()
        st = self.stats(logits)
        self.commit(st)
        return logits, st

    def run(self, max_steps_per_block=None):
        cap = self.B if max_steps_per_block is None else max_steps_per_block
        self.complete = False
        for k in range(self.n_blocks):
            self.start_block(k)
            while self.block_masked().any():
                if self.block_steps >= cap:
                    raise RuntimeError("block did not finish within its step cap")
                self.step()
            self.steps.append(self.block_steps)
            if self.complete:      # end-of-sequence: nothing masked is left
                break
        return self.tokens


def _min_route_margin(rec, layer_ids):
    if not rec or not layer_ids:
        return np.inf
    return float(min(np.min(rec["route_margin"][li]) for li in layer_ids))


def decision_margin(st, masked, credit, d, committed, still=None, fallback=False):
    """How far this step's float-to-integer decisions are from flipping, as a
    band on the block rows' logits: if two computations of the same step differ
    by at most e in every logit, each decision below is taken alike by both
    whenever the returned margin exceeds 2e.  Reported, not used by the method.

    Under a logit error of at most e a row's log max-probability moves by at most
    2e (its top logit and its log-sum-exp each by e), a difference of two logits
    of one row by at most 2e, and a difference of two rows' log-probabilities
    by at most 4e.  The decisions of a step and their margins:
      * the threshold gate of every candidate: |ln p - ln tau|;
      * the credit gate of every candidate (credit on): |ln c - ln kappa| --
        c = gamma*c_prev + lambda*p moves by at most the factor p does;
      * the fallback, only when it was taken (no candidate passed a gate): the
        best against the second-best candidate, (ln p1 - ln p2) / 2;
      * the id of each committed row, and with credit on the id every masked
        row passes to the credit state (stable or reset): the row's top-1 minus
        top-2 logit;
      * with smoothing on, the set of ids each still-masked row keeps (the soft
        embedding sums over the set, so the order inside it decides nothing):
        the row's 8th minus 9th largest logit."""
    from .decode import candidates
    C = candidates(masked, d.hierarchical)
    if len(C) == 0:
        return np.inf
    tiny = 1e-300
    conf = np.maximum(st["conf"][C].astype(np.float64), tiny)
    m = float(np.min(np.abs(np.log(conf) - np.log(d.tau))))
    if d.credit_weight != 0.0:
        c = np.maximum(credit[C].astype(np.float64), tiny)
        m = min(m, float(np.min(np.abs(np.log(c) - np.log(d.credit_kappa)))))
    if fallback and len(C) > 1:
        s = np.sort(conf)[::-1]
        m = min(m, 0.5 * float(np.log(s[0]) - np.log(s[1])))
    tp = np.maximum(np.asarray(st["topk_p"], dtype=np.float64), tiny)
    top_gap = np.log(tp[:, 0]) - np.log(tp[:, 1])
    rows = np.zeros(len(masked), dtype=bool)
    rows[np.asarray(committed, dtype=np.int64)] = True
    if d.credit_weight != 0.0:
        rows |= np.asarray(masked, dtype=bool)
    if rows.any():
        m = min(m, float(np.min(top_gap[rows])))
    if d.smooth_alpha != 0.0 and still is not None and np.any(still):
        m = min(m, float(np.min(st["kth_gap"][np.asarray(still, dtype=bool)])))
    return float(m)


def run_request(mcfg, dcfg, weights, req, r=0, model=None):
    """Run request r of a synth request batch to completion; returns the OracleRun."""
    model = model or OracleModel(mcfg, weights)
    rb = None if req.get("router_bias") is None else req["router_bias"][r].numpy()
    run = OracleRun(model, dcfg, req["tokens"][r].numpy(), int(req["prompt_len"][r]),
                    int(req["gen_len"][r]), req["plant_id"][r].numpy(),
                    float(req["plant_bias"][r]), rb)
    run.run()
    return run
