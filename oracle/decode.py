"""Oracle decoding strategy: vocab statistics and the parallel-decode commit.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: dInfer news article (aigc.bar), section "扩散模型的“理论翅膀”与“现实枷锁”"
(classic decoding keeps only the most confident token per iteration, throwing
the rest of the distribution away) and section "解码的艺术" (the art of
decoding: hierarchical decoding, credit decoding, iteration smoothing); Sangam
abstract (several positions commit per invocation).

Readings where the pages are silent:
  * MASK can never be predicted: its logit is -inf before softmax/argmax.
  * Planting adds a bias to the raw logit of a row's planted target id.
  * Ties: argmax and top-k by (logit desc, id asc); fallback by (confidence
    desc, position asc).
  * Threshold and credit gates are inclusive (p >= tau, c >= kappa).
  * Credit: every still-masked block position accumulates
    c <- (argmax == tracked ? gamma*c : 0) + lambda*p, then tracked <- argmax;
    update first, then gate.  lambda = 0 gives plain threshold decoding.
  * Fallback: if nothing passes, the single candidate with the highest
    confidence commits (the "top-1" rule of classic decoding).
  * Hierarchical: candidates are the midpoints lo + (hi-lo-1)//2 of the
    maximal masked runs [lo, hi) inside the block; only they may commit.
  * Smoothing: a still-masked position keeps its top-k ids with probabilities
    renormalised to sum 1; its next input embedding is
    (1-alpha) E[MASK] + alpha * sum_j p~_j E[id_j].
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def vocab_stats(z, plant_id, plant_bias, mask_id, k=8):
    """Per-row vocab statistics of logits z [R, V].

    Returns dict: argmax [R] int64, conf [R] float32 (max softmax probability),
    lse [R] float64, topk_id [R,k] int64, topk_p [R,k] float64, kth_gap [R]:
    the k-th largest minus the (k+1)-th largest biased logit (how far the
    top-k set is from changing), and rank_gap [R]: the smallest gap between
    consecutive logits among the k+1 largest (how far the top-k set or its
    order is from changing); both reported, not used by the method.
    The biased logits are rounded to fp32 before any order decision; the
    probabilities are then computed in fp64 from those fp32 values.
    """
    z = np.array(z, dtype=np.float64)
    R, V = z.shape
    pid = np.asarray(plant_id, dtype=np.int64)
    pb = np.broadcast_to(np.asarray(plant_bias, dtype=np.float64), (R,))
    rows = np.nonzero(pid >= 0)[0]
    z[rows, pid[rows]] += pb[rows]
    z32 = z.astype(np.float32)
    z32[:, mask_id] = -np.inf
    argmax = np.argmax(z32, axis=1)                      # first max = lowest id
    zd = z32.astype(np.float64)
    zmax = zd[np.arange(R), argmax]
    e = np.exp(zd - zmax[:, None])
    Z = e.sum(axis=1)
    conf = (1.0 / Z).astype(np.float32)
    lse = zmax + np.log(Z)
    order = np.argsort(-z32, axis=1, kind="stable")[:, :k + 1]   # value desc, id asc
    kth_gap = (np.take_along_axis(zd, order[:, k - 1:k], axis=1)
               - np.take_along_axis(zd, order[:, k:k + 1], axis=1))[:, 0]
    ztop = np.take_along_axis(zd, order, axis=1)
    rank_gap = np.min(ztop[:, :-1] - ztop[:, 1:], axis=1)
    order = order[:, :k]
    topk_p = np.take_along_axis(e, order, axis=1) / Z[:, None]
    return {"argmax": argmax, "conf": conf, "lse": lse, "topk_id": order, "topk_p": topk_p,
            "logit_max": zmax, "kth_gap": kth_gap, "rank_gap": rank_gap}


def credit_update(credit, tracked, argmax, conf, masked, gamma, lam):
    """One credit step for a block (credit decoding bullet of the decoding section).

    All float arithmetic in fp32 with one rounding per operation.  Positions
    that are not masked keep their state.
    """
    credit = np.asarray(credit, dtype=F32)
    conf = np.asarray(conf, dtype=F32)
    stable = np.asarray(argmax) == np.asarray(tracked)
    decayed = np.where(stable, F32(gamma) * credit, F32(0.0)).astype(F32)
    new_c = (decayed + (F32(lam) * conf).astype(F32)).astype(F32)
    new_t = np.where(masked, argmax, tracked)
    return np.where(masked, new_c, credit).astype(F32), new_t


def run_midpoints(masked):
    """Midpoints of the maximal runs of True in `masked` (hierarchical decoding)."""
    masked = np.asarray(masked, dtype=bool)
    padded = np.concatenate([[False], masked, [False]]).astype(np.int8)
    edges = np.diff(padded)
    starts = np.nonzero(edges == 1)[0]
    ends = np.nonzero(edges == -1)[0]
    return starts + (ends - starts - 1) // 2


def candidates(masked, hierarchical):
    """Block offsets that may commit this step."""
    masked = np.asarray(masked, dtype=bool)
    if hierarchical:
        return run_midpoints(masked)
    return np.nonzero(masked)[0]


def select_commits(masked, conf, credit, tau, kappa, hierarchical):
    """Block offsets committed this step (threshold / credit gate, top-1 fallback).

    Returns (commit offsets, used_fallback).
    """
    C = candidates(masked, hierarchical)
    if len(C) == 0:
        return C, False
    conf = np.asarray(conf, dtype=F32)
    credit = np.asarray(credit, dtype=F32)
    passed = C[(conf[C] >= F32(tau)) | (credit[C] >= F32(kappa))]
    if len(passed):
        return passed, False
    best = C[np.argmax(conf[C])]                         # first max = lowest position
    return np.array([best]), True


def smoothing_state(topk_id, topk_p):
    """Top-k ids with probabilities renormalised to sum 1 (iteration smoothing)."""
    p = np.asarray(topk_p, dtype=np.float64)
    return np.asarray(topk_id), p / p.sum(axis=-1, keepdims=True)


def soft_embedding(e_mask, e_ids, p_tilde, alpha):
    """(1-alpha) E[MASK] + alpha * sum_j p~_j E[id_j]; e_ids [n, k, d], p_tilde [n, k]."""
    return (1.0 - alpha) * e_mask[None, :] + alpha * np.einsum("nk,nkd->nd", p_tilde, e_ids)


def eos_fill(tokens, P, L, mask_id, eos_id):
    """Early stop at the end-of-sequence token (dInfer news article, section
    "系统级压榨": computation after EOS is skipped).  Reading: once the
    response [P, L) holds eos_id at some position, every response position
    after the first such position that is still MASK becomes eos_id; the
    positions before it are decoded as usual.  tokens is changed in place;
    returns True when no MASK is left in the response."""
    resp = tokens[P:L]
    if eos_id >= 0:
        at = np.nonzero(resp == eos_id)[0]
        if len(at):
            tail = resp[at[0] + 1:]
            tail[tail == mask_id] = eos_id
    return not bool((resp == mask_id).any())
