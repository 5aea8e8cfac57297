"""Helpers of the GPU parity tests: build an engine on synth inputs, drive the
HIP library and the oracle in lockstep, compare.  The oracle only ever sees
synth inputs and its own state; nothing computed by the HIP path is fed to it."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from diffusion_vicinity_kv_amd.engine import Engine
from oracle.model import OracleModel


def note(msg):
    print(msg, flush=True)


def small_workload(name="small", *, n_layers=2, d=256, H=4, hd=64, F=768, V=4096, dtype="f32",
                   batch=1, prompt=(64, 64), gen=64, B=32, w=8, tau=0.9, credit=1.0,
                   alpha=0.3, hier=False, bias=6.0, prob=(0.7, 0.7), seed=0,
                   experts=0, top_k=0, Fe=0, Fs=0, pref_bias=0.0, pref_count=0):
    m = synth.ModelCfg(n_layers=n_layers, d_model=d, n_heads=H, head_dim=hd, ffn_dim=F, vocab=V,
                       mask_id=V - 1, dtype=dtype, n_experts=experts, top_k=top_k,
                       expert_ffn=Fe, shared_ffn=Fs)
    dc = synth.DecodeCfg(block_len=B, vicinity_w=w, tau=tau, credit_weight=credit,
                         smooth_alpha=alpha, hierarchical=hier)
    return synth.WorkloadCfg(name=name, model=m, decode=dc, batch=batch, prompt_len=prompt,
                             gen_len=gen, plant_bias=bias, plant_prob=prob, seed=seed,
                             router_pref_bias=pref_bias, router_pref_count=pref_count or top_k)


def build(wc, graph_unroll=0, weights=None, req=None):
    w = weights if weights is not None else synth.make_weights(wc.model, wc.seed, device="cuda")
    req = req if req is not None else synth.make_requests(wc)
    max_len = req["tokens"].shape[1]
    eng = Engine(wc.model, wc.decode, w, wc.batch, max_len, graph_unroll=graph_unroll,
                 keep_logits=True)
    tokens = req["tokens"].cuda().contiguous()
    rb = req.get("router_bias")
    eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                  req["plant_id"].cuda().contiguous(), req["plant_bias"].cuda().contiguous(),
                  None if rb is None else rb.cuda().contiguous())
    return eng, w, req, tokens


def oracle_runs(wc, w, req, layers=None):
    om = OracleModel(wc.model, w, layers=layers)
    runs = []
    for r in range(wc.batch):
        rb = req.get("router_bias")
        runs.append(oracle.OracleRun(om, wc.decode, req["tokens"][r].numpy(),
                                     int(req["prompt_len"][r]), int(req["gen_len"][r]),
                                     req["plant_id"][r].numpy(), float(req["plant_bias"][r]),
                                     None if rb is None else rb[r].numpy()))
    return runs


def lockstep(wc, eng, tokens, runs, logit_tol, max_steps=10_000, max_blocks=None,
             check_cache=False, route_band=0.0):
    """Drive GPU and oracle step by step.  Per step: block-row logits within
    logit_tol * RMS(oracle logits); commits, tokens, tracked ids (credit on)
    and the kept smoothing id sets identical.  Every decision of a step
    (committed ids, threshold/credit gates, fallback choice, tracked ids, kept
    top-8 set) is a float-to-integer decision taken on different logits by the
    two sides; oracle.run.decision_margin states how far each is from flipping
    in units where the observed max |logit difference| e moves it by at most
    2e: when the oracle's margin of some decision
    is below that band and the two sides decided differently, the trajectories
    part legitimately and the lockstep stops there (reported as "diverged");
    near-ties decided alike are counted and the lockstep goes on.  Decisions
    that differ with a margin above the band fail the test.

    MoE routing is such a decision too, taken inside the forward pass: the
    oracle reports each row's gap between its top_k-th and next router logit.
    route_band bounds the router-logit error of the HIP path.  A block row
    whose logits miss logit_tol is accepted only when its own routing, or any
    routing that reaches it through the cache (a window row below the last
    layer, or the block's refresh), was within route_band of flipping: the
    lockstep then stops there as "diverged"."""
    B = wc.decode.block_len
    batch = wc.batch
    rep = {"steps": 0, "max_rel_logit_err": 0.0, "diverged": None, "min_margin": np.inf,
           "near_ties_same": 0}
    for r, run in enumerate(runs):
        run.start_block(0)
    eng.refresh_kv()
    steps = 0
    blocks_done = 0
    while True:
        active = [r for r in range(batch) if not getattr(runs[r], "_finished", False)]
        if not active:
            break
        if steps >= max_steps:
            break
        eng.denoise_step()
        torch.cuda.synchronize()
        v = eng.view()
        glog = v["logits"].cpu().numpy().reshape(batch, B, -1)
        ostats = {}
        err_step = {}
        for r in active:
            run = runs[r]
            if getattr(run, "_waiting", False):
                continue
            ol = run.denoise_logits()
            rms = float(np.sqrt(np.mean(ol ** 2)))
            row_err = np.max(np.abs(glog[r] - ol), axis=1) / rms
            if wc.model.is_moe:
                shared = min(run.refresh_route_margin, run.step_route_margin_window)
                near = (run.step_route_margin_rows < route_band) | (shared < route_band)
                rep["route_near_ties"] = rep.get("route_near_ties", 0) + int(near.sum())
                bad = row_err > logit_tol
                if bad.any():
                    assert near[bad].all(), (
                        f"request {r} step {steps}: logits rel err {row_err.max():.3e} > "
                        f"{logit_tol} on rows {np.nonzero(bad & ~near)[0].tolist()} whose "
                        f"routing margins are >= {route_band}")
                    rep["diverged"] = {"request": r, "step": steps, "route_rows":
                                       np.nonzero(bad)[0].tolist(), "row_err": float(row_err.max())}
                    rep["steps"] = steps
                    return rep
            err = float(row_err.max())
            err_step[r] = err * rms
            rep["max_rel_logit_err"] = max(rep["max_rel_logit_err"], err)
            assert err <= logit_tol, f"request {r} step {steps}: logits rel err {err:.3e} > {logit_tol}"
            ostats[r] = run.stats(ol)
        eng.commit()
        torch.cuda.synchronize()
        gtok = tokens.cpu().numpy()
        gmask = v["commit_mask"].cpu().numpy().reshape(batch, B)
        gsid = v["smooth_id"].cpu().numpy().reshape(batch, B, -1)
        gsv = v["smooth_valid"].cpu().numpy().reshape(batch, B).astype(bool)
        gtr = v["tracked"].cpu().numpy().reshape(batch, B)
        unsafe = None
        for r, st in ostats.items():
            run = runs[r]
            T, fb = run.commit(st)
            margin = run.records[-1]["margin"]
            rep["min_margin"] = min(rep["min_margin"], margin)
            band = 2.0 * err_step[r] + 1e-6
            om = np.zeros(B, dtype=np.uint8)
            om[T] = 1
            same = np.array_equal(om, gmask[r]) and np.array_equal(gtok[r][: run.L], run.tokens)
            if same and wc.decode.credit_weight != 0.0:
                # the argmax each masked row hands to the credit state
                same = np.array_equal(gtr[r], run.tracked)
            if same and wc.decode.smooth_alpha != 0.0:
                # the soft embedding sums over the kept ids: their set is the
                # decision, not the order they are stored in
                sv = run.smooth_valid
                same = (np.array_equal(gsv[r], sv)
                        and np.array_equal(np.sort(gsid[r][sv], axis=1),
                                           np.sort(run.smooth_ids[sv], axis=1)))
            if margin < band:
                if same:
                    rep["near_ties_same"] += 1
                else:
                    unsafe = {"request": r, "step": steps, "margin": margin, "band": band}
            elif not same:
                raise AssertionError(f"request {r} step {steps}: decisions differ "
                                     f"(oracle commits {sorted(T.tolist())}, gpu "
                                     f"{np.nonzero(gmask[r])[0].tolist()}), margin {margin:.3e} "
                                     f">= band {band:.3e}")
        steps += 1
        rep["steps"] = steps
        if unsafe is not None:
            rep["diverged"] = unsafe
            return rep
        need, unfinished = eng.advance_blocks()
        for r in active:
            run = runs[r]
            if getattr(run, "_waiting", False):
                continue
            if not run.block_masked().any():
                run.steps.append(run.block_steps)
                if run.block + 1 >= run.n_blocks:
                    run._finished = True
                else:
                    run._waiting = True
        if any(need):
            blocks_done += 1
            if max_blocks is not None and blocks_done >= max_blocks:
                break
            for r in range(batch):
                if need[r]:
                    runs[r].start_block(runs[r].block + 1)
                    runs[r]._waiting = False
            eng.refresh_kv(need)
            if check_cache:
                compare_cache(wc, eng, runs)
        if unfinished == 0:
            break
    return rep


def cache_rows(v, key, layer, r, L):
    """K or V cache of request r in one layer as [L][H][hd] float32 numpy
    (K is stored [H][Lp][hd], V in transposed tiles [H][Lp/32][hd][32])."""
    if key == "k":
        return v["kv_k"][layer, r, :, :L].float().cpu().numpy().transpose(1, 0, 2)
    t = v["kv_v"][layer, r].float().cpu().numpy()            # [H][nb][hd][32]
    H, nb, hd, _ = t.shape
    return t.transpose(1, 3, 0, 2).reshape(nb * 32, H, hd)[:L]


def compare_cache(wc, eng, runs, tol=None, layers=None):
    """K, V caches of every request against the oracle's.  fp32 caches: max
    |diff| <= tol * RMS.  bf16 caches store each value rounded to bf16, so an
    element may differ by its own rounding (at most 2^-8 of its magnitude) on
    top of the tol * RMS allowance; against an oracle that also stores bf16,
    the two roundings of nearly equal values may land one bf16 step apart
    (at most 2^-7 of the magnitude)."""
    torch.cuda.synchronize()
    v = eng.view()
    m = wc.model
    f32 = m.dtype == "f32"
    tol = tol if tol is not None else (1e-5 if f32 else 2e-2)
    items = runs.items() if isinstance(runs, dict) else enumerate(runs)
    for r, run in items:
        for li in (run.cache["k"] if layers is None else layers):
            for key in ("k", "v"):
                g = cache_rows(v, key, li, r, run.L)
                o = run.cache[key][li]
                rms = np.sqrt(np.mean(o ** 2))
                own = 2.0 ** -7 if run.cache.get("round") == "bf16" else 2.0 ** -8
                bound = tol * rms + (0.0 if f32 else own * np.abs(o))
                excess = np.max(np.abs(g - o) - bound)
                assert excess <= 0, f"cache {key} layer {li} req {r}: exceeds bound by {excess:.2e}"


def _gpu_block_state(v, batch, B):
    return {"credit": v["credit"].cpu().numpy().reshape(batch, B).copy(),
            "tracked": v["tracked"].cpu().numpy().reshape(batch, B).copy()}


def selector_check(wc, req, tok_before, state_before, v, tok_after, blk, active, band=1e-3):
    """The decoding strategy against the oracle selector, on the GPU's own step.

    (1) vocab statistics: the oracle's vocab_stats of the GPU's fp32 logits
        gives the same argmax and top-8 ids (exact comparisons on the same
        numbers) and confidences within 2e-5 relative;
    (2) the oracle selector fed the GPU's statistics (argmax, confidence,
        top-8) and the GPU's credit state before the step: commit mask, tokens,
        credit bits, tracked ids, kept smoothing ids bit-exact, smoothing
        probabilities within 1e-6 relative;
    (3) fed the oracle statistics of (1) instead, the commit decisions are the
        same except where a candidate's confidence lies within `band` of tau
        or its credit within `band` of kappa (excluded and counted), or the
        fallback's best two confidences lie within `band` relative.
    Returns the counts of (3)."""
    d = wc.decode
    m = wc.model
    B = d.block_len
    V = m.vocab
    batch = tok_before.shape[0]
    glog = v["logits"].cpu().numpy().reshape(batch, B, V)
    g = {k: v[k].cpu().numpy() for k in ("argmax", "conf", "topk_id", "topk_p", "credit",
                                         "tracked", "smooth_id", "smooth_p", "smooth_valid",
                                         "commit_mask")}
    tau, kappa = np.float32(d.tau), np.float32(d.credit_kappa)
    excluded = 0
    P = req["prompt_len"].tolist()
    for r in active:
        sl = slice(r * B, (r + 1) * B)
        bs = P[r] + blk[r] * B
        masked = tok_before[r, bs:bs + B] == m.mask_id
        pid = req["plant_id"][r, bs:bs + B].numpy()
        st = oracle.vocab_stats(glog[r], pid, float(req["plant_bias"][r]), m.mask_id, 8)
        assert np.array_equal(g["argmax"][sl], st["argmax"]), f"request {r}: argmax"
        assert np.array_equal(g["topk_id"][sl], st["topk_id"]), f"request {r}: top-8 ids"
        assert np.allclose(g["conf"][sl], st["conf"], rtol=2e-5, atol=0), f"request {r}: conf"
        # (2) on the GPU's statistics
        c2, t2 = oracle.credit_update(state_before["credit"][r], state_before["tracked"][r],
                                      g["argmax"][sl], g["conf"][sl], masked, d.credit_decay,
                                      d.credit_weight)
        T, fb = oracle.select_commits(masked, g["conf"][sl], c2, tau, kappa, d.hierarchical)
        om = np.zeros(B, np.uint8)
        om[T] = 1
        assert np.array_equal(g["commit_mask"][sl], om), f"request {r}: commit mask"
        want_tok = tok_before[r, bs:bs + B].copy()
        want_tok[T] = g["argmax"][sl][T]
        assert np.array_equal(tok_after[r, bs:bs + B], want_tok), f"request {r}: tokens"
        assert np.array_equal(g["credit"][sl].view(np.uint32), c2.view(np.uint32)), f"request {r}: credit"
        assert np.array_equal(g["tracked"][sl], t2), f"request {r}: tracked"
        still = masked.copy()
        still[T] = False
        if d.smooth_alpha != 0.0:
            assert np.array_equal(g["smooth_valid"][sl].astype(bool), still)
            ids, pt = oracle.smoothing_state(g["topk_id"][sl], g["topk_p"][sl])
            assert np.array_equal(g["smooth_id"][sl][still], ids[still])
            assert np.allclose(g["smooth_p"][sl][still], pt[still], rtol=1e-6)
        # (3) on the oracle's own statistics of the same logits
        c3, _ = oracle.credit_update(state_before["credit"][r], state_before["tracked"][r],
                                     st["argmax"], st["conf"], masked, d.credit_decay,
                                     d.credit_weight)
        T3, fb3 = oracle.select_commits(masked, st["conf"], c3, tau, kappa, d.hierarchical)
        C = oracle.candidates(masked, d.hierarchical)
        near = (np.abs(st["conf"][C] - tau) < band).any()
        if d.credit_weight != 0.0:
            near = near or (np.abs(c3[C] - kappa) < band).any()
        if fb3 and len(C) > 1:
            s = np.sort(st["conf"][C].astype(np.float64))[::-1]
            near = near or (s[0] - s[1]) < band * s[0]
        if near:
            excluded += 1
        else:
            assert np.array_equal(np.sort(T3), np.sort(T)) and fb3 == fb, f"request {r}: selector"
    return excluded


def teacher_forced(wc, eng, tokens, req, runs, n_steps, logit_tol, check_cache_layers=None,
                   shadow=None):
    """Refresh, then n_steps denoise+commit steps of the first block.  Each
    step: the block-row logits of every request in `runs` (request index ->
    OracleRun) within logit_tol * RMS of the oracle's, and selector_check on
    every active request.  After each step the oracle runs take over the
    GPU's decode state (tokens, credit, tracked ids, smoothing state), so the
    two never part and each step is compared on the same inputs.

    shadow (request index -> OracleRun with an fp64 cache), when `runs` store
    their caches in bf16: the GPU's logits must also lie within logit_tol *
    RMS of the shadow's plus the cache storage's own effect, the largest
    difference between the two oracles' logits (both on the CPU)."""
    B = wc.decode.block_len
    batch = wc.batch
    shadow = shadow or {}
    rep = {"steps": 0, "max_rel_logit_err": 0.0, "excluded": 0, "cache_err": None,
           "max_rel_logit_err_fp64_cache": 0.0, "max_rel_storage_effect": 0.0}
    for r, run in list(runs.items()) + list(shadow.items()):
        note(f"  oracle refresh of request {r} ({run.L} positions)")
        run.start_block(0)
    eng.refresh_kv()
    torch.cuda.synchronize()
    if check_cache_layers is not None:
        compare_cache(wc, eng, runs, layers=check_cache_layers)
    blk = [0] * batch
    for step in range(n_steps):
        v = eng.view()
        tok0 = tokens.cpu().numpy()
        st0 = _gpu_block_state(v, batch, B)
        eng.denoise_step()
        torch.cuda.synchronize()
        glog = v["logits"].cpu().numpy().reshape(batch, B, -1)
        for r, run in runs.items():
            ol = run.denoise_logits()
            rms = float(np.sqrt(np.mean(ol ** 2)))
            err = float(np.max(np.abs(glog[r] - ol))) / rms
            rep["max_rel_logit_err"] = max(rep["max_rel_logit_err"], err)
            note(f"  step {step} request {r}: max |dlogit| / RMS = {err:.3e}")
            assert err <= logit_tol, f"step {step} request {r}: {err:.3e} > {logit_tol}"
            if r in shadow:
                o64 = shadow[r].denoise_logits()
                e64 = float(np.max(np.abs(glog[r] - o64))) / rms
                store = float(np.max(np.abs(ol - o64))) / rms
                rep["max_rel_logit_err_fp64_cache"] = max(rep["max_rel_logit_err_fp64_cache"], e64)
                rep["max_rel_storage_effect"] = max(rep["max_rel_storage_effect"], store)
                note(f"  step {step} request {r}: against an fp64 cache {e64:.3e} "
                     f"(the bf16 storage alone moves the oracle by {store:.3e})")
                assert e64 <= logit_tol + store, f"step {step} request {r}: fp64-cache oracle"
        eng.commit()
        torch.cuda.synchronize()
        tok1 = tokens.cpu().numpy()
        rep["excluded"] += selector_check(wc, req, tok0, st0, v, tok1, blk, range(batch))
        # teacher forcing: the oracle takes the GPU's decode state
        g_sid = v["smooth_id"].cpu().numpy().reshape(batch, B, -1)
        g_sp = v["smooth_p"].cpu().numpy().reshape(batch, B, -1).astype(np.float64)
        g_sv = v["smooth_valid"].cpu().numpy().reshape(batch, B).astype(bool)
        st1 = _gpu_block_state(v, batch, B)
        for r, run in list(runs.items()) + list(shadow.items()):
            run.tokens[:] = tok1[r, :run.L]
            run.credit = st1["credit"][r].copy()
            run.tracked = st1["tracked"][r].astype(np.int64)
            run.smooth_ids = g_sid[r].astype(np.int64)
            run.smooth_p = g_sp[r]
            run.smooth_valid = g_sv[r].copy()
            run.block_steps += 1
        rep["steps"] = step + 1
        if not any(run.block_masked().any() for run in runs.values()):
            break
    return rep
