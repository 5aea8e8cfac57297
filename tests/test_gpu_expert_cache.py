"""TIDE-style interval expert placement (TIDE abstract: expert activations are
stable within a block; the placement is refreshed per interval, losslessly):
an HBM cache of a few expert slots per layer over a pinned host store of
every expert.  Lossless means bit-identical: the grouped projection reads the
same bytes from a slot or from the host store.

  * runs to completion with 3 of 8 experts per layer in HBM (placement at
    block starts, and every 4 steps) give the oracle's tokens, and step logits
    bit-identical to the all-in-HBM context on the same weights;
  * the accounting: every row assignment is a hit or a miss, as many as the
    passes route (refreshes stop before the last layer's FFN; idle graph
    steps route nothing); with every expert in a slot nothing misses after
    the first placement;
  * bf16 with 16 experts top-4."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import build, note, small_workload

pytestmark = pytest.mark.gpu

TINY = dict(F=0, experts=8, top_k=2, Fe=128, Fs=256, pref_bias=1.0, pref_count=2)


def _expected_assignments(wc, runs):
    """Row assignments the passes of the runs route: per block a refresh of
    every position through all but the last layer, then the block's steps over
    its window through every layer."""
    m, d = wc.model, wc.decode
    tot = 0
    for run in runs:
        for k, n_steps in enumerate(run.steps):
            bs = run.P + k * run.B
            lo, hi = max(0, bs - d.vicinity_w), min(run.L, bs + run.B + d.vicinity_w)
            tot += run.L * (m.n_layers - 1) * m.top_k + n_steps * (hi - lo) * m.n_layers * m.top_k
    return tot


@pytest.mark.parametrize("unroll,interval", [(0, 0), (4, 0), (4, 4)])
def test_offloaded_run_matches_oracle_and_accounts_every_row(unroll, interval):
    note(f"expert cache 3 of 8, unroll {unroll}, interval {interval}")
    # batch 1: graph steps past the block's end route no rows at all
    wc = small_workload(**TINY, batch=1, prompt=(70, 70), gen=96, alpha=0.3,
                        bias=6.0 + float(np.log(4094.0)) - 2.0, prob=(0.7, 0.7), seed=31)
    eng, w, req, tokens = build(wc, graph_unroll=unroll)
    eng.expert_offload(3, interval)
    stats = eng.run_to_completion()
    torch.cuda.synchronize()
    runs = [oracle.run_request(wc.model, wc.decode, w, req, r=r) for r in range(wc.batch)]
    for r, run in enumerate(runs):
        assert np.array_equal(tokens.cpu().numpy()[r][: run.L], run.tokens), r
    rep = eng.expert_report()
    note(f"  {stats} {rep}")
    assert rep["row_hits"] + rep["row_misses"] == _expected_assignments(wc, runs)
    assert rep["row_misses"] > 0 and rep["row_hits"] > 0
    assert rep["placements"] >= len(runs[0].steps)        # one per block start at least
    assert rep["bytes_host_read"] == rep["expert_misses"] * 3 * 128 * 256 * 4
    eng.close()


def test_offloaded_steps_bit_identical_to_all_resident():
    note("expert cache 3 of 8: step logits bit-identical to the all-in-HBM context")
    wc = small_workload(**TINY, alpha=0.3, seed=32)
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    a, _, _, ta = build(wc, weights=w, req=req)
    b, _, _, tb = build(wc, weights=w, req=req)
    b.expert_offload(3, 0)
    for eng in (a, b):
        eng.refresh_kv()
    b.expert_place()                    # the refresh's routing picks the residents
    for step in range(6):
        for eng in (a, b):
            eng.denoise_step()
        torch.cuda.synchronize()
        la, lb = a.view()["logits"].clone(), b.view()["logits"].clone()
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), step
        for eng in (a, b):
            eng.commit()
        if step == 2:
            b.expert_place()            # a placement mid-block changes no bit
        torch.cuda.synchronize()
        assert torch.equal(ta, tb), step
    rep = b.expert_report()
    note(f"  {rep}")
    assert rep["expert_misses"] > 0
    for eng in (a, b):
        eng.close()


def test_all_slots_resident_never_misses_after_placement():
    wc = small_workload(**TINY, alpha=0.0, seed=33)
    eng, w, req, tokens = build(wc)
    eng.expert_offload(8, 0)
    eng.run_to_completion()
    rep = eng.expert_report()
    assert rep["row_misses"] == 0 and rep["expert_misses"] == 0
    assert rep["bytes_placed"] == wc.model.n_layers * 8 * 3 * 128 * 256 * 4   # the initial fill
    eng.close()


def test_bf16_sixteen_experts_matches_all_resident():
    note("bf16, 16 experts top-4, 6 slots: tokens equal to the all-in-HBM run")
    wc = small_workload(dtype="bf16", d=512, H=4, hd=128, F=0, V=4096, experts=16, top_k=4,
                        Fe=256, Fs=512, pref_bias=2.0, pref_count=4, batch=2, prompt=(60, 100),
                        gen=64, bias=8.0 + float(np.log(4095.0)), prob=(0.6, 0.8), alpha=0.3,
                        seed=34)
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    a, _, _, ta = build(wc, graph_unroll=4, weights=w, req=req)
    b, _, _, tb = build(wc, graph_unroll=4, weights=w, req=req)
    b.expert_offload(6, 8)
    sa, sb = a.run_to_completion(), b.run_to_completion()
    torch.cuda.synchronize()
    assert torch.equal(ta, tb)
    assert sa["committed"] == sb["committed"] and sa["steps"] == sb["steps"]
    rep = b.expert_report()
    note(f"  {rep}")
    assert rep["row_misses"] > 0
    for eng in (a, b):
        eng.close()
