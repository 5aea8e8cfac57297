"""MoE FFN through the C ABI against the oracle: router (logits + per-block
preference bias, top-k, renormalised gates), per-expert row lists, grouped
expert projections, shared expert and combine.

Routing is a float-to-integer decision inside the forward pass, taken by the
two sides on router inputs that differ by the path's rounding.  The library
reports the router logits of the last routed layer; their largest difference
e from the oracle's bounds how far the two sides can disagree on any choice:
a row whose gap between its top_k-th and next oracle logit exceeds the band
2e must pick the same experts, and every row's choice must be a top-k of the
oracle's logits up to the band.  Gates are a softmax over the selection, so
each differs by at most 2e * gate <= 2e."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import build, cache_rows, lockstep, note, oracle_runs, small_workload

pytestmark = pytest.mark.gpu

# tiny fp32 MoE: 8 experts, top-2, expert FFN 128, shared FFN 256
TINY = dict(F=0, experts=8, top_k=2, Fe=128, Fs=256, pref_bias=1.0, pref_count=2)


def check_routing(eng, rec, layer, n, top_k, min_safe=0.0, clean=None):
    """Routing of the last routed layer (rows [0, n) of the last pass) against
    the oracle record of the same pass; returns (band, safe rows).  clean:
    rows whose router input can differ by rounding only (no earlier routing
    flip reaches them); the band is measured on those, and only those rows
    are held to the exact comparison."""
    v = eng.view()
    sel = v["moe_sel"][:n].cpu().numpy()
    gate = v["moe_gate"][:n].cpu().numpy()
    glog = v["moe_logits"][:n].cpu().numpy().astype(np.float64)
    olog = np.asarray(rec["router_logits"][layer])
    want = np.asarray(rec["experts"][layer])
    margin = np.asarray(rec["route_margin"][layer])
    clean = np.ones(n, dtype=bool) if clean is None else clean
    band = 2.0 * float(np.max(np.abs(glog - olog)[clean])) + 1e-6
    # every choice is a top-k of the library's own logits, and of the
    # oracle's up to the band where only rounding separates the two
    kth_g = -np.sort(-glog, axis=1)[:, top_k - 1]
    assert np.all(np.take_along_axis(glog, sel.astype(np.int64), axis=1) >= kth_g[:, None])
    kth = -np.sort(-olog, axis=1)[:, top_k - 1]
    chosen = np.take_along_axis(olog, sel.astype(np.int64), axis=1)
    assert np.all((chosen >= kth[:, None] - band)[clean]), "a selected expert is not a top-k choice"
    assert np.all(np.sort(sel, axis=1)[:, 1:] != np.sort(sel, axis=1)[:, :-1]), "duplicate expert"
    safe = (margin >= band) & clean
    note(f"  layer {layer}: router logit band {band:.2e}, {int(safe.sum())}/{n} rows unique")
    assert safe.mean() >= min_safe
    got_sets = np.sort(sel[safe], axis=1)
    want_sets = np.sort(want[safe], axis=1)
    bad = np.nonzero((got_sets != want_sets).any(axis=1))[0]
    assert len(bad) == 0, f"layer {layer}: {len(bad)} rows chose other experts"
    g_got = np.take_along_axis(gate[safe], np.argsort(sel[safe], axis=1), axis=1)
    g_want = np.take_along_axis(np.asarray(rec["gates"][layer])[safe],
                                np.argsort(want[safe], axis=1), axis=1)
    assert np.allclose(gate.sum(axis=1), 1.0, atol=1e-5)
    if safe.any():
        assert float(np.max(np.abs(g_got - g_want))) <= band
    return band, safe


@pytest.mark.parametrize("variant", ["credit_smooth", "hier"])
def test_tiny_moe_lockstep(variant):
    note(f"tiny fp32 MoE lockstep {variant}")
    kw = dict(alpha=0.3) if variant == "credit_smooth" else dict(alpha=0.0, hier=True, credit=0.0)
    wc = small_workload(**TINY, **kw, seed=11)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=1e-5, check_cache=True, route_band=1e-4)
    note(f"  {rep}")
    assert rep["diverged"] is None
    assert all(getattr(r, "_finished", False) for r in runs)


@pytest.mark.parametrize("unroll", [0, 4])
def test_tiny_moe_run_to_completion_matches_oracle(unroll):
    note(f"tiny fp32 MoE run_to_completion unroll={unroll}")
    wc = small_workload(**TINY, alpha=0.3, seed=12)
    eng, w, req, tokens = build(wc, graph_unroll=unroll)
    stats = eng.run_to_completion()
    torch.cuda.synchronize()
    run = oracle.run_request(wc.model, wc.decode, w, req)
    assert np.array_equal(tokens.cpu().numpy()[0][: run.L], run.tokens)
    assert stats["committed"] == wc.gen_len


def test_tiny_moe_batched_ragged_lockstep():
    """Three requests of different lengths: the expert row lists mix rows of
    every request, and each request reads its own block's router bias."""
    note("tiny fp32 MoE batch 3 lockstep")
    wc = small_workload(**TINY, batch=3, prompt=(40, 90), gen=64, bias=8.0, prob=(0.5, 0.9),
                        alpha=0.3, seed=13)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=1e-5, route_band=1e-4)
    note(f"  {rep}")
    # The kept smoothing ids are compared as a set (the soft embedding sums
    # over it), so a tie inside a row's top eight decides nothing.  The run
    # ends with every decision identical unless a decision inside the
    # numerical band (logged) parts the two.
    d = rep["diverged"]
    assert d is None or d.get("margin", 0.0) < d.get("band", 1.0), rep
    assert d is not None or all(getattr(r, "_finished", False) for r in runs)


def test_tiny_moe_routing_of_refresh_and_step():
    """Expert choice and gates of every row, after the refresh (layer 0 of 2)
    and after a step (layer 1)."""
    note("tiny fp32 MoE routing tables")
    wc = small_workload(**TINY, seed=14)
    eng, w, req, tokens = build(wc)
    run = oracle_runs(wc, w, req)[0]
    run.start_block(0)
    eng.refresh_kv()
    torch.cuda.synchronize()
    band, _ = check_routing(eng, run.refresh_record, 0, run.L, 2, min_safe=0.95)
    assert band < 1e-4
    eng.denoise_step()
    torch.cuda.synchronize()
    run.denoise_logits()
    lo, hi = run.window()
    band, _ = check_routing(eng, run.step_record, 1, hi - lo, 2, min_safe=0.95)
    assert band < 1e-4


@pytest.mark.parametrize("n_layers", [1, 2])
def test_full_width_moe(n_layers):
    """The MoE shape at full width (d 2048, 16 heads, 64 experts top-8, expert
    FFN 1024, shared FFN 2048, V 157184, bf16) on the benchmark's request
    (prompt 1024, response 1024, block 64, window +-32) with n_layers layers:
    refresh, then one step, every kernel in the benchmark's launch shapes.

    Two layers: the refresh routes all 2048 positions in layer 0, and layer
    1's K, V of a position depend on that position's routing only, so the
    layer-1 cache is compared at positions whose choice is unique.  The step:
    block-row logits within 2e-2 * RMS on rows whose own routing is unique in
    every layer (a flipped window row reaches other rows only as one of the
    2048 keys of their layer-1 attention).  The block's rows all hold MASK,
    so their layer-0 routing is nearly the same; when it sits within the
    band of a flip no block row's logits are unique and only the routing
    checks apply."""
    note(f"full-width MoE, {n_layers} layer(s): refresh + step")
    wc = synth.preset("moe_b1").with_model(n_layers=n_layers).with_decode(smooth_alpha=0.0)
    K = wc.model.top_k
    eng, w, req, tokens = build(wc)
    run = oracle_runs(wc, w, req)[0]
    note("  oracle refresh")
    run.start_block(0)
    eng.refresh_kv()
    torch.cuda.synchronize()
    band0 = 0.0
    if n_layers > 1:
        band0, safe_pos = check_routing(eng, run.refresh_record, 0, run.L, K, min_safe=0.5)
        v = eng.view()
        for key in ("k", "v"):
            g = cache_rows(v, key, 1, 0, run.L)
            o = run.cache[key][1]
            rms = np.sqrt(np.mean(o ** 2))
            excess = (np.abs(g - o) - 2e-2 * rms - 2.0 ** -8 * np.abs(o))[safe_pos]
            assert np.max(excess) <= 0, f"layer-1 cache {key}: exceeds bound by {np.max(excess):.2e}"
    note("  oracle step")
    eng.denoise_step()
    torch.cuda.synchronize()
    v = eng.view()
    glog = v["logits"].cpu().numpy()
    ol = run.denoise_logits()
    lo, hi = run.window()
    # layer-0 routing of the step, with the refresh's band (same layer, same
    # kind of input); rows that may have flipped there are not clean in layer 1
    m0 = np.asarray(run.step_record["route_margin"][0])
    clean = m0 >= band0 if n_layers > 1 else None
    band1, _ = check_routing(eng, run.step_record, n_layers - 1, hi - lo, K, clean=clean)
    band = max(band0, band1)
    own = np.min(np.stack([run.step_record["route_margin"][li] for li in range(n_layers)]), axis=0)
    safe = own[run.bs - lo: run.be - lo] >= band
    rms = float(np.sqrt(np.mean(ol ** 2)))
    row_err = np.max(np.abs(glog - ol), axis=1) / rms
    note(f"  block rows with unique routing {int(safe.sum())}/{len(safe)}; max rel logit err "
         f"{row_err[safe].max() if safe.any() else float('nan'):.3e} (all rows {row_err.max():.3e})")
    if n_layers == 1:
        assert safe.sum() >= 16
    if safe.any():
        assert row_err[safe].max() <= 2e-2


def test_tiny_moe_long_refresh_wide_plan():
    """A refresh with more expert assignments than the plan stages in LDS
    (2112 positions x top-8 of 8 experts = 16896 > 16384) takes the per-expert
    ballot plan; with every expert chosen by every row there is no routing
    decision, so the layer-1 cache after the refresh (which every expert's
    row list feeds) and the next step's logits match the oracle to fp32
    rounding.  The step's 48 window rows take the staged plan."""
    note("tiny fp32 MoE, all 8 experts chosen, 2112 positions: wide plan in the refresh")
    wc = small_workload(F=0, experts=8, top_k=8, Fe=128, Fs=256, pref_bias=1.0, pref_count=2,
                        prompt=(2080, 2080), gen=32, seed=16)
    eng, w, req, tokens = build(wc)
    run = oracle_runs(wc, w, req)[0]
    assert run.L * wc.model.top_k > 16384
    run.start_block(0)
    eng.refresh_kv()
    torch.cuda.synchronize()
    v = eng.view()
    for key in ("k", "v"):
        g = cache_rows(v, key, 1, 0, run.L)
        o = run.cache[key][1]
        rms = float(np.sqrt(np.mean(o ** 2)))
        err = float(np.max(np.abs(g - o))) / rms
        note(f"  layer-1 cache {key}: max rel err {err:.2e}")
        assert err <= 1e-5
    eng.denoise_step()
    torch.cuda.synchronize()
    glog = eng.view()["logits"].cpu().numpy()
    ol = run.denoise_logits()
    rms = float(np.sqrt(np.mean(ol ** 2)))
    err = float(np.max(np.abs(glog[: ol.shape[0]] - ol))) / rms
    note(f"  step logits: max rel err {err:.2e}")
    assert err <= 1e-5


def test_full_width_moe_graph_replays_equal_eager_steps():
    """The shared expert runs on a second stream, forked and joined with
    events inside each layer.  At the benchmark shape (2 layers, bf16), 32
    steps replayed from a step graph of 4 (eight replays, the host
    synchronising and reading the tokens between them) give the same tokens,
    bit for bit, as 32 eager steps from the same refresh -- the join leaves
    no race between the shared and the routed experts."""
    note("full-width MoE, 2 layers: graph replays against eager steps")
    wc = synth.preset("moe_b1").with_model(n_layers=2)
    eager, w, req, tok_e = build(wc, graph_unroll=0)
    graph, _, _, tok_g = build(wc, graph_unroll=4, weights=w, req=req)
    for e in (eager, graph):
        e.refresh_kv()
    for r in range(8):
        for _ in range(4):
            eager.denoise_step()
            eager.commit()
        graph.step_graph(4)
        torch.cuda.synchronize()
        assert torch.equal(tok_e, tok_g), f"tokens differ after replay {r}"
    n = int((tok_g[0] != wc.model.mask_id).sum())
    note(f"  32 steps: {n} unmasked positions, identical")
    for e in (eager, graph):
        e.close()
