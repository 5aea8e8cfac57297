"""GPU parity: the HIP library through its C ABI against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from diffusion_vicinity_kv_amd.engine import Engine
from diffusion_vicinity_kv_amd import binding as B
from oracle.sched import DeficitScheduler as OracleSched
from oracle.decode import credit_update, select_commits, smoothing_state, vocab_stats

from gpu_util import build, compare_cache, lockstep, note, oracle_runs, small_workload

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------- vocab stats (K3)
@pytest.mark.parametrize("rows,V,ties", [(32, 4096, 0), (37, 4096, 3), (32, 126464, 0),
                                         (512, 126464, 2), (64, 157184, 0), (5, 1000, 0)])
def test_vocab_stats_parity(rows, V, ties):
    note(f"vocab_stats rows={rows} V={V} ties={ties}")
    z = synth.make_logits(rows, V, seed=rows + V, ties=ties, device="cuda")
    g = torch.Generator().manual_seed(rows)
    pid = torch.where(torch.rand(rows, generator=g) < 0.6,
                      torch.randint(0, V - 1, (rows,), generator=g), torch.full((rows,), -1))
    pid = pid.to(torch.int32)
    pb = torch.full((rows,), 8.0)
    pb[::3] = 2.5
    mask_id = V - 1
    z[:, mask_id] = 50.0                     # the MASK column must never win
    lib = B.load()
    scratch = torch.empty(lib.dinfer_vocab_stats_scratch_bytes(rows, V), dtype=torch.uint8,
                          device="cuda")
    out = {"argmax": torch.empty(rows, dtype=torch.int32, device="cuda"),
           "conf": torch.empty(rows, device="cuda"), "lse": torch.empty(rows, device="cuda"),
           "topk_id": torch.empty(rows, 8, dtype=torch.int32, device="cuda"),
           "topk_p": torch.empty(rows, 8, device="cuda")}
    B.vocab_stats(z, pid.cuda(), pb.cuda(), mask_id, out, scratch)
    torch.cuda.synchronize()
    want = vocab_stats(z.cpu().numpy(), pid.numpy(), pb.numpy(), mask_id, 8)
    assert np.array_equal(out["argmax"].cpu().numpy(), want["argmax"])
    assert np.array_equal(out["topk_id"].cpu().numpy(), want["topk_id"])
    assert np.allclose(out["conf"].cpu().numpy(), want["conf"], rtol=2e-5, atol=0)
    assert np.allclose(out["lse"].cpu().numpy(), want["lse"], rtol=0, atol=2e-5 * np.abs(want["lse"]).max())
    assert np.allclose(out["topk_p"].cpu().numpy(), want["topk_p"], rtol=2e-5, atol=1e-12)


# --------------------------------------------------------------- commit (K8)
@pytest.mark.parametrize("hier", [False, True])
@pytest.mark.parametrize("B_len", [32, 64, 7])
def test_commit_parity_on_synthetic_stats(hier, B_len):
    """Selector bit-exactness: both sides get the same synthetic stats, credit,
    tracked ids and masked patterns (exact threshold values and ties included)."""
    note(f"commit hier={hier} B={B_len}")
    wc = small_workload(batch=3, B=B_len, gen=B_len * 2, prompt=(70, 70), hier=hier, w=4)
    eng, w, req, tokens = build(wc)
    rng = np.random.default_rng(B_len + 10 * hier)
    tau, kappa = np.float32(wc.decode.tau), np.float32(wc.decode.credit_kappa)
    mask_id = wc.model.mask_id
    for trial in range(25):
        eng.refresh_kv()
        eng.denoise_step()
        torch.cuda.synchronize()
        v = eng.view()
        R = wc.batch * B_len
        masked = rng.random((wc.batch, B_len)) < rng.choice([0.2, 0.6, 1.0])
        if trial % 5 == 0:
            masked[0] = False                  # a block with nothing left
        am = rng.integers(0, 5, R).astype(np.int32)
        choices = np.float32([tau, np.nextafter(tau, np.float32(0)), 0.5, 0.3, 0.95, 0.05, 0.3])
        conf = rng.choice(choices, R).astype(np.float32)
        credit = rng.choice(np.float32([0.0, 1.2, kappa, np.nextafter(kappa, np.float32(0)), 0.8]),
                            R).astype(np.float32)
        tracked = np.where(rng.random(R) < 0.5, am, rng.integers(-1, 5, R)).astype(np.int32)
        tid = rng.integers(0, wc.model.vocab - 1, (R, 8)).astype(np.int32)
        tp = np.sort(rng.random((R, 8)).astype(np.float32), axis=1)[:, ::-1].copy()
        bs = 70
        tok = tokens.cpu().numpy()
        blk = np.where(masked, mask_id, rng.integers(0, 100, masked.shape)).astype(np.int32)
        tok[:, bs:bs + B_len] = blk
        tokens.copy_(torch.from_numpy(tok))
        v["argmax"].copy_(torch.from_numpy(am))
        v["conf"].copy_(torch.from_numpy(conf))
        v["credit"].copy_(torch.from_numpy(credit))
        v["tracked"].copy_(torch.from_numpy(tracked))
        v["topk_id"].copy_(torch.from_numpy(tid))
        v["topk_p"].copy_(torch.from_numpy(tp))
        ds0 = v["decode_stats"].cpu().numpy().copy()
        eng.commit()
        torch.cuda.synchronize()
        gt = tokens.cpu().numpy()
        dds = v["decode_stats"].cpu().numpy() - ds0
        for r in range(wc.batch):
            sl = slice(r * B_len, (r + 1) * B_len)
            c2, t2 = credit_update(credit[sl], tracked[sl], am[sl], conf[sl], masked[r],
                                   wc.decode.credit_decay, wc.decode.credit_weight)
            T, fb = select_commits(masked[r], conf[sl], c2, tau, kappa, hier)
            want_tok = blk[r].copy()
            want_tok[T] = am[sl][T]
            assert np.array_equal(gt[r, bs:bs + B_len], want_tok), (trial, r)
            gm = v["commit_mask"].cpu().numpy()[sl]
            om = np.zeros(B_len, np.uint8)
            om[T] = 1
            assert np.array_equal(gm, om), (trial, r)
            assert np.array_equal(v["credit"].cpu().numpy()[sl].view(np.uint32),
                                  c2.view(np.uint32)), (trial, r)
            assert np.array_equal(v["tracked"].cpu().numpy()[sl], t2), (trial, r)
            still = masked[r].copy()
            still[T] = False
            assert np.array_equal(v["smooth_valid"].cpu().numpy()[sl].astype(bool), still)
            ids, pt = smoothing_state(tid[sl], tp[sl])
            gs = v["smooth_p"].cpu().numpy()[sl]
            gi = v["smooth_id"].cpu().numpy()[sl]
            assert np.array_equal(gi[still], ids[still])
            assert np.allclose(gs[still], pt[still], rtol=1e-6)
            done = int(v["block_done"].cpu().numpy()[r])
            assert done == int(not still.any())
            # accounting: threshold / credit-only / fallback commits, one step
            # in the histogram bin of its commit count
            want = np.zeros(dds.shape[1], np.int64)
            if fb:
                want[2] = len(T)
            else:
                want[0] = int(np.sum(conf[sl][T] >= tau))
                want[1] = len(T) - want[0]
            want[4 + len(T)] = 1
            assert np.array_equal(dds[r], want), (trial, r, dds[r][:8], want[:8])


# ----------------------------------------------------- one step and full runs
def test_tiny_refresh_cache_and_first_step_logits():
    note("tiny fp32: refresh cache + first step")
    wc = synth.preset("tiny_f32")
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    runs[0].start_block(0)
    eng.refresh_kv()
    compare_cache(wc, eng, runs)
    eng.denoise_step()
    torch.cuda.synchronize()
    ol = runs[0].denoise_logits()
    gl = eng.view()["logits"].cpu().numpy()
    err = np.max(np.abs(gl - ol)) / np.sqrt(np.mean(ol ** 2))
    note(f"  first step: max |dlogit| / RMS = {err:.3e}")
    assert err < 1e-5, err
    compare_cache(wc, eng, runs)


@pytest.mark.parametrize("variant", ["literal", "confident", "credit", "hier"])
def test_tiny_lockstep_run(variant):
    note(f"tiny fp32 lockstep {variant}")
    wc = synth.preset("tiny_f32")
    if variant == "confident":       # planted p ~ 0.99: the threshold fires
        wc = wc.with_(plant_bias=6.0 + float(np.log(4094.0)))
    elif variant == "credit":        # planted p in the credit band below tau
        wc = wc.with_(plant_bias=6.0 + float(np.log(4094.0)) - 3.3)
    elif variant == "hier":
        wc = wc.with_(plant_bias=6.0 + float(np.log(4094.0))).with_decode(hierarchical=True)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=1e-5, check_cache=True)
    note(f"  {rep}")
    assert rep["diverged"] is None
    assert np.array_equal(tokens.cpu().numpy()[0][: runs[0].L], runs[0].tokens)


@pytest.mark.parametrize("shape", ["one_key_step", "many_key_splits", "hd128_ragged_length"])
def test_attention_edge_lockstep(shape):
    """Attention layouts at the edges of the kernel's tiling, fp32 so every
    decision must match: a sequence shorter than one key step (the second key
    group of the workgroup has no step); a long sequence whose window is split
    over several key ranges merged afterwards, with a ragged last range (the
    refresh splits too); head dim 128 with a length that is not a multiple of
    the 32-key V tiles."""
    note(f"tiny fp32 attention edge case {shape}")
    if shape == "one_key_step":
        wc = small_workload(prompt=(4, 4), gen=8, B=8, w=2, bias=6.0 + float(np.log(4094.0)),
                            seed=21)
    elif shape == "many_key_splits":
        wc = small_workload(prompt=(1000, 1000), gen=32, B=16, w=4, alpha=0.3, seed=22)
    else:
        wc = small_workload(H=2, hd=128, prompt=(301, 301), gen=32, B=16, w=3, alpha=0.3,
                            bias=6.0 + float(np.log(4094.0)), seed=23)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=1e-5, check_cache=True,
                   max_steps=16 if shape == "many_key_splits" else 10_000)
    note(f"  {rep}")
    assert rep["diverged"] is None
    if shape == "many_key_splits":
        assert rep["steps"] >= 16                     # the whole first block
    else:
        assert all(getattr(r, "_finished", False) for r in runs)


@pytest.mark.parametrize("unroll", [0, 1, 4])
def test_tiny_run_to_completion_matches_oracle(unroll):
    note(f"tiny fp32 run_to_completion unroll={unroll}")
    wc = synth.preset("tiny_f32")
    eng, w, req, tokens = build(wc, graph_unroll=unroll)
    stats = eng.run_to_completion()
    torch.cuda.synchronize()
    run = oracle.run_request(wc.model, wc.decode, w, req)
    assert np.array_equal(tokens.cpu().numpy()[0][: run.L], run.tokens)
    assert stats["committed"] == wc.gen_len
    assert stats["refreshes"] == wc.gen_len // wc.decode.block_len
    assert stats["steps"] >= sum(run.steps)


def test_batched_tiny_run_matches_per_request_oracle():
    note("tiny fp32 batch 3, ragged prompts, graph")
    wc = small_workload(batch=3, prompt=(40, 90), gen=64, bias=6.0 + float(np.log(4094.0)) - 2.0,
                        prob=(0.5, 0.9), seed=3)
    eng, w, req, tokens = build(wc, graph_unroll=3)
    eng.run_to_completion()
    torch.cuda.synchronize()
    for r in range(wc.batch):
        run = oracle.run_request(wc.model, wc.decode, w, req, r=r)
        assert np.array_equal(tokens.cpu().numpy()[r][: run.L], run.tokens), r


@pytest.mark.parametrize("unroll", [0, 3])
def test_eos_early_stop_matches_oracle(unroll):
    """End-of-sequence early stop: the EOS id is the first token request 0's
    plain run commits, so that request stops inside its first block (the rest
    of its response filled with EOS, no further refresh); every request's
    tokens equal its oracle run with the same EOS id, and the refreshes are
    the blocks the oracle runs."""
    note(f"tiny fp32 batch 3 with an EOS id, unroll={unroll}")
    wc = small_workload(batch=3, prompt=(40, 90), gen=64, bias=6.0 + float(np.log(4094.0)) - 2.0,
                        prob=(0.5, 0.9), seed=3)
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    plain = oracle.run_request(wc.model, wc.decode, w, req, r=0)
    eos = int(plain.tokens[plain.P + int(plain.records[0]["commits"][0])])
    wce = wc.with_decode(eos_id=eos)
    eng, _, _, tokens = build(wce, graph_unroll=unroll, weights=w, req=req)
    stats = eng.run_to_completion()
    torch.cuda.synchronize()
    runs = [oracle.run_request(wce.model, wce.decode, w, req, r=r) for r in range(wce.batch)]
    for r, run in enumerate(runs):
        assert np.array_equal(tokens.cpu().numpy()[r][: run.L], run.tokens), r
    assert len(runs[0].steps) < len(plain.steps)
    assert stats["refreshes"] == sum(len(run.steps) for run in runs)
    note(f"  refreshes {stats['refreshes']} (oracle blocks {[len(x.steps) for x in runs]})")


@pytest.mark.parametrize("unroll", [0, 3])
def test_continuous_batching_refill_matches_oracle(unroll):
    """Six requests through two slots: a finished slot takes the next queued
    request (dinfer_refill) while the other keeps decoding.  Requests are
    independent, so every response equals its own oracle run."""
    note(f"tiny fp32: 6 requests through 2 slots, unroll={unroll}")
    wc = small_workload(batch=6, prompt=(40, 90), gen=64, bias=6.0 + float(np.log(4094.0)) - 2.0,
                        prob=(0.5, 0.9), seed=5)
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    max_len = req["tokens"].shape[1]
    eng = Engine(wc.model, wc.decode, w, 2, max_len, graph_unroll=unroll)
    tokens = req["tokens"][:2].cuda().contiguous()
    plant_id = req["plant_id"][:2].cuda().contiguous()
    plant_bias = req["plant_bias"][:2].cuda().contiguous()
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    eng.set_batch(tokens, P[:2], G[:2], plant_id, plant_bias)
    queue = [{"tokens": req["tokens"][i].cuda(), "prompt_len": P[i], "gen_len": G[i],
              "plant_id": req["plant_id"][i].cuda(), "plant_bias": float(req["plant_bias"][i])}
             for i in range(2, 6)]
    res = eng.run_queue(queue)
    torch.cuda.synchronize()
    got = sorted(i for i, _ in res["outputs"])
    assert got == list(range(6)), got
    for i, row in res["outputs"]:
        run = oracle.run_request(wc.model, wc.decode, w, req, r=i)
        assert np.array_equal(row.cpu().numpy()[: run.L], run.tokens), i
    note(f"  steps {res['steps']}, refreshes {res['refreshes']}")


def test_pending_rows_report_window_and_refresh_rows():
    """dinfer_pending_rows: a waiting request costs its full length, a
    refreshed one its block with the +-w window clipped to the request, a
    finished one nothing."""
    note("pending rows of three requests")
    wc = small_workload(batch=3, prompt=(4, 90), gen=64, w=8, seed=9)
    eng, w, req, tokens = build(wc)
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    Bl, wv = wc.decode.block_len, wc.decode.vicinity_w
    dec, ref = eng.pending_rows()
    assert dec == [0, 0, 0] and ref == [P[r] + G[r] for r in range(3)]
    eng.refresh_kv([True, False, True])
    dec, ref = eng.pending_rows()
    for r in range(3):
        L, bs = P[r] + G[r], P[r]
        want = min(L, bs + Bl + wv) - max(0, bs - wv)
        assert dec[r] == (want if r != 1 else 0), (r, dec)
        assert ref[r] == (0 if r != 1 else L), (r, ref)
    eng.run_to_completion()
    torch.cuda.synchronize()
    assert eng.pending_rows() == ([0, 0, 0], [0, 0, 0])


@pytest.mark.parametrize("unroll,budget", [(0, 200), (3, 64)])
def test_deficit_budget_admission_matches_oracle(unroll, budget):
    """Six requests through three slots with the deficit token budget deciding
    which waiting refreshes (new requests and block starts) run in each round:
    responses equal their own oracle runs, the library's admissions equal the
    oracle scheduler's on the same rounds, and the budget defers some refresh
    that the unbudgeted loop would have run at once."""
    note(f"tiny fp32: 6 requests through 3 slots, unroll={unroll}, budget={budget} rows/step")
    wc = small_workload(batch=6, prompt=(40, 90), gen=64, bias=6.0 + float(np.log(4094.0)) - 2.0,
                        prob=(0.5, 0.9), seed=6)
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    max_len = req["tokens"].shape[1]
    S = 3
    eng = Engine(wc.model, wc.decode, w, S, max_len, graph_unroll=unroll)
    tokens = req["tokens"][:S].cuda().contiguous()
    plant_id = req["plant_id"][:S].cuda().contiguous()
    plant_bias = req["plant_bias"][:S].cuda().contiguous()
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    eng.set_batch(tokens, P[:S], G[:S], plant_id, plant_bias)
    queue = [{"tokens": req["tokens"][i].cuda(), "prompt_len": P[i], "gen_len": G[i],
              "plant_id": req["plant_id"][i].cuda(), "plant_bias": float(req["plant_bias"][i])}
             for i in range(S, 6)]
    res = eng.run_queue(queue, token_budget=budget)
    torch.cuda.synchronize()
    assert sorted(i for i, _ in res["outputs"]) == list(range(6))
    for i, row in res["outputs"]:
        run = oracle.run_request(wc.model, wc.decode, w, req, r=i)
        assert np.array_equal(row.cpu().numpy()[: run.L], run.tokens), i
    per_round = max(unroll, 1)
    ora = OracleSched(budget * per_round, S)
    deferred = 0
    for dec, ref, admit, deficit in res["rounds"]:
        assert ora.round(dec, ref) == admit
        assert ora.deficit == deficit
        deferred += sum(1 for r in range(S) if ref[r] > 0 and not admit[r])
    note(f"  rounds {len(res['rounds'])}, steps {res['steps']}, refreshes {res['refreshes']}, "
         f"deferred waits {deferred}")
    assert deferred > 0


@pytest.mark.parametrize("unroll,budget", [(0, 200), (3, 64)])
def test_eos_refill_and_budget_admission_match_oracle(unroll, budget):
    """End-of-sequence stop, slot refill and budgeted admission together: six
    requests through three slots with an EOS id that ends request 0 inside its
    first block; a slot freed early takes the next request, whose first
    refresh waits for the budget like every other.  Every response equals its
    own oracle run with the same EOS id."""
    note(f"tiny fp32: EOS + 6 requests through 3 slots, unroll={unroll}, budget={budget}")
    wc = small_workload(batch=6, prompt=(40, 90), gen=64, bias=6.0 + float(np.log(4094.0)) - 2.0,
                        prob=(0.5, 0.9), seed=3)
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    plain = oracle.run_request(wc.model, wc.decode, w, req, r=0)
    eos = int(plain.tokens[plain.P + int(plain.records[0]["commits"][0])])
    wce = wc.with_decode(eos_id=eos)
    max_len = req["tokens"].shape[1]
    S = 3
    eng = Engine(wce.model, wce.decode, w, S, max_len, graph_unroll=unroll)
    tokens = req["tokens"][:S].cuda().contiguous()
    plant_id = req["plant_id"][:S].cuda().contiguous()
    plant_bias = req["plant_bias"][:S].cuda().contiguous()
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    eng.set_batch(tokens, P[:S], G[:S], plant_id, plant_bias)
    queue = [{"tokens": req["tokens"][i].cuda(), "prompt_len": P[i], "gen_len": G[i],
              "plant_id": req["plant_id"][i].cuda(), "plant_bias": float(req["plant_bias"][i])}
             for i in range(S, 6)]
    res = eng.run_queue(queue, token_budget=budget)
    torch.cuda.synchronize()
    assert sorted(i for i, _ in res["outputs"]) == list(range(6))
    runs = {}
    for i, row in res["outputs"]:
        runs[i] = oracle.run_request(wce.model, wce.decode, w, req, r=i)
        assert np.array_equal(row.cpu().numpy()[: runs[i].L], runs[i].tokens), i
    assert len(runs[0].steps) < len(plain.steps)
    assert res["refreshes"] == sum(len(r.steps) for r in runs.values())
    ora = OracleSched(budget * max(unroll, 1), S)
    for dec, ref, admit, deficit in res["rounds"]:
        assert ora.round(dec, ref) == admit and ora.deficit == deficit
    note(f"  rounds {len(res['rounds'])}, steps {res['steps']}, refreshes {res['refreshes']}")


@pytest.mark.parametrize("alpha", [0.0, 0.3])
def test_bf16_small_lockstep(alpha):
    note(f"bf16 small lockstep alpha={alpha}")
    wc = small_workload(dtype="bf16", d=256, H=2, hd=128, F=768, V=4096, batch=2,
                        prompt=(60, 100), gen=64, w=8, bias=8.0, prob=(0.75, 0.75), seed=5,
                        alpha=alpha)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=2e-2, check_cache=True)
    note(f"  {rep}")
    # every step until the run ends matched, unless a genuine near-tie (a
    # decision inside the numerical band, logged) parts the two earlier
    assert rep["diverged"] is not None or all(getattr(r, "_finished", False) for r in runs)


def test_bf16_batch16_fat_step_path_lockstep():
    note("bf16 batch 16 (fat GEMM in the step) lockstep")
    wc = small_workload(dtype="bf16", d=512, H=4, hd=128, F=1024, V=8192, batch=16,
                        prompt=(16, 96), gen=64, B=32, w=16, bias=8.0, prob=(0.5, 0.9), seed=7,
                        alpha=0.0)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=2e-2, max_steps=40)
    note(f"  {rep}")
    # at least the first block (32 steps of one fallback commit each), unless a
    # logged near-tie parts the two earlier
    assert rep["diverged"] is not None or rep["steps"] >= 32


@pytest.mark.parametrize("preset", ["dense8b_b1"])
def test_full_width_two_layer_parity(preset):
    """Full width of the dense 8B shape (d 4096, 32 heads, F 12288, V 126464),
    two layers: every per-layer kernel runs in the launch configuration of the
    32-layer benchmark.  Refresh cache and two steps against the oracle."""
    note(f"full-width 2-layer {preset}")
    wc = synth.preset(preset).with_model(n_layers=2)
    eng, w, req, tokens = build(wc)
    runs = oracle_runs(wc, w, req)
    rep = lockstep(wc, eng, tokens, runs, logit_tol=2e-2, max_steps=8, check_cache=False)
    note(f"  {rep}")
    compare_cache(wc, eng, runs)
    assert rep["diverged"] is not None or rep["steps"] == 8


# --------------------------------------------------------------- linear (K1)
@pytest.mark.parametrize("shape,dt", [((48, 256), "bf16"), ((3, 32, 96), "bf16"),
                                      ((4096, 4096), "bf16"), ((384, 128), "bf16"),
                                      ((2, 400, 64), "bf16"), ((32, 48), "f32"),
                                      ((2, 272, 64), "f32")])
def test_pack_linear_layout(shape, dt):
    """Packed weight layout, bit for bit, against the layout written out with
    reshapes: 1 KB blocks of 16 rows x one vector step (32 bf16 / 16 f32
    columns), slot 16q + c = row c of the group, columns [q*VEC, (q+1)*VEC);
    blocks stored step-major (every group of step 0, then of step 1, ...);
    each matrix of a stack on its own."""
    note(f"pack_linear {shape} {dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    vec = 8 if dt == "bf16" else 4
    g = torch.Generator(device="cuda").manual_seed(len(shape) * 100 + shape[-1])
    W = torch.randn(*shape, device="cuda", generator=g).to(tdt)
    P = B.pack_linear(W)
    torch.cuda.synchronize()
    N, K = shape[-2], shape[-1]
    ks = K // (4 * vec)
    want = []
    for w in W.reshape(-1, N, K).cpu():
        # blocks[g][s] = the (group, step) block in slot order
        blocks = w.reshape(N // 16, 16, ks, 4, vec).permute(0, 2, 3, 1, 4).reshape(N // 16, ks, -1)
        want.append(blocks.permute(1, 0, 2).reshape(-1))   # step-major
    assert torch.equal(P.reshape(-1).cpu(), torch.cat(want))


@pytest.mark.parametrize("M,N,K,dt", [(64, 24576, 4096, "bf16"), (64, 12288, 4096, "bf16"),
                                      (48, 4096, 12288, "bf16"), (37, 4096, 4096, "bf16"),
                                      (128, 1024, 2048, "bf16"), (100, 512, 1024, "bf16"),
                                      (96, 768, 512, "bf16"), (300, 384, 512, "bf16"),
                                      (1024, 1536, 1024, "bf16"), (48, 768, 256, "f32"),
                                      (200, 256, 768, "f32")])
def test_linear_parity(M, N, K, dt):
    """Projection = A W^T (plain fp64 matmul as the reference), skinny and fat
    kernels, ragged row counts.  A is fp32; with bf16 weights it enters the
    MFMAs as hi + lo bf16 (two roundings to nearest, each within 2^-8), which
    leaves at most 2^-16 of each element behind: about 2.5e-6 of the output
    RMS per output, 1.1e-5 at the largest of 0.5 M outputs (fp64 emulation of
    the split at 64 x 8192 x 4096), plus fp32 accumulation; 3e-5 keeps a
    margin over that."""
    note(f"linear M={M} N={N} K={K} {dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(M * 7 + N)
    A = torch.randn(M, K, device="cuda", generator=g)
    W = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(tdt)
    lib = B.load()
    n_out = lib.dinfer_linear_out_elems(M, N, K, B.BF16 if dt == "bf16" else B.F32)
    out = torch.full((n_out,), float("nan"), device="cuda")
    S = B.linear(A, B.pack_linear(W), out)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(S, M, N).sum(0)
    want = A.cpu().double().numpy() @ W.cpu().double().numpy().T
    err = np.max(np.abs(got - want)) / np.sqrt(np.mean(want ** 2))
    assert err < 3e-5, err


@pytest.mark.parametrize("unroll", [0, 4])
def test_empty_prompt_matches_oracle(unroll):
    """A request with no prompt at all (prompt_len 0: the first block starts
    at position 0, its vicinity window clipped at the sequence start, and
    the cache holds only MASK rows at the first refresh), fp32: step by step
    against the oracle (logits at 1e-5 * RMS, every decision), then a whole
    run, eager and from step graphs."""
    note(f"tiny fp32, empty prompt, unroll={unroll}")
    wc = small_workload(prompt=(0, 0), gen=96, alpha=0.3, seed=21)
    eng, w, req, tokens = build(wc, graph_unroll=unroll)
    assert int(req["prompt_len"][0]) == 0
    if unroll == 0:
        runs = oracle_runs(wc, w, req)
        rep = lockstep(wc, eng, tokens, runs, logit_tol=1e-5, check_cache=True)
        note(f"  {rep}")
        assert rep["diverged"] is None and all(getattr(r, "_finished", False) for r in runs)
    else:
        stats = eng.run_to_completion()
        torch.cuda.synchronize()
        run = oracle.run_request(wc.model, wc.decode, w, req)
        assert np.array_equal(tokens.cpu().numpy()[0][: run.L], run.tokens)
        assert stats["committed"] == wc.gen_len
    eng.close()
