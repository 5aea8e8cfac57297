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
    eng = Engine(wc.model, wc.decode, w, wc.batch, max_len, graph_unroll=graph_unroll)
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
    logit_tol * RMS(oracle logits); commits, tokens and smoothing ids identical.
    Every decision of a step (committed ids, threshold/credit gates, fallback
    choice, kept top-8) is a float-to-integer decision taken on different
    logits by the two sides.  Each is a difference of two log-probabilities or
    logits, so the observed max |logit difference| e bounds how far the two
    sides can disagree on it by 2e: when the oracle's margin of some decision
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
            if same and wc.decode.smooth_alpha != 0.0:
                same = (np.array_equal(gsv[r], run.smooth_valid)
                        and np.array_equal(gsid[r][run.smooth_valid], run.smooth_ids[run.smooth_valid]))
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


def compare_cache(wc, eng, runs, tol=None):
    """K, V caches of every request against the oracle's.  fp32 caches: max
    |diff| <= tol * RMS.  bf16 caches store each value rounded to bf16, so an
    element may differ by its own rounding (at most 2^-8 of its magnitude) on
    top of the tol * RMS allowance."""
    torch.cuda.synchronize()
    v = eng.view()
    m = wc.model
    f32 = m.dtype == "f32"
    tol = tol if tol is not None else (1e-5 if f32 else 2e-2)
    for r, run in enumerate(runs):
        for li in run.cache["k"]:
            for key in ("k", "v"):
                g = cache_rows(v, key, li, r, run.L)
                o = run.cache[key][li]
                rms = np.sqrt(np.mean(o ** 2))
                bound = tol * rms + (0.0 if f32 else 2.0 ** -8 * np.abs(o))
                excess = np.max(np.abs(g - o) - bound)
                assert excess <= 0, f"cache {key} layer {li} req {r}: exceeds bound by {excess:.2e}"
