"""Properties of the full dense 8B-shaped model (32 layers, bf16, batch 1) in
the launch configuration the benchmark times, checked at every step of a
block or a run without an oracle forward pass (test_gpu_fullshape.py runs the
oracle's forward at this size for a refresh and two steps): the vicinity
scatter writes only the window, the vocab statistics agree with the step's own
logits, the oracle selector fed the step's own statistics takes the GPU's
decisions bit for bit, the commit rules hold, and graph replays are
bit-deterministic."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import build, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dense8b():
    note("full-size dense 8B: drawing weights on the GPU")
    wc = synth.preset("dense8b_b1")
    eng, w, req, tokens = build(wc, graph_unroll=8)
    yield wc, eng, w, req, tokens
    eng.close()
    del w
    torch.cuda.empty_cache()


def test_vicinity_scatter_writes_only_the_window(dense8b):
    wc, eng, w, req, tokens = dense8b
    note("full-size: vicinity scatter footprint")
    eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                  req["plant_id"].cuda(), req["plant_bias"].cuda())
    eng.refresh_kv()
    torch.cuda.synchronize()
    v = eng.view()
    before = {li: (v["kv_k"][li, 0].clone(), v["kv_v"][li, 0].clone()) for li in (0, 13, 31)}
    eng.denoise_step()
    torch.cuda.synchronize()
    P, B, wv = int(req["prompt_len"][0]), wc.decode.block_len, wc.decode.vicinity_w
    lo, hi = max(0, P - wv), min(P + wc.gen_len, P + B + wv)
    for li, (k0, v0) in before.items():
        # K [H][Lp][hd] and V [H][Lp/32][hd][32]: positions whose entries changed
        for changed in ((v["kv_k"][li, 0] != k0).any(dim=-1).any(dim=0),
                        (v["kv_v"][li, 0] != v0).any(dim=2).any(dim=0).flatten()):
            idx = changed.nonzero().flatten().cpu().numpy()
            assert len(idx) > 0
            assert idx.min() >= lo and idx.max() < hi, (li, idx.min(), idx.max())


def test_vocab_stats_agree_with_step_logits(dense8b):
    wc, eng, w, req, tokens = dense8b
    note("full-size: vocab stats vs the step's logits")
    eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                  req["plant_id"].cuda(), req["plant_bias"].cuda())
    eng.refresh_kv()
    eng.denoise_step()
    torch.cuda.synchronize()
    v = eng.view()
    z = v["logits"].double().clone()
    P, B = int(req["prompt_len"][0]), wc.decode.block_len
    pid = req["plant_id"][0, P:P + B].cuda().long()
    rows = (pid >= 0).nonzero().flatten()
    z[rows, pid[rows]] = (v["logits"][rows, pid[rows]] + float(req["plant_bias"][0])).double()
    z[:, wc.model.mask_id] = -float("inf")
    p = torch.softmax(z, dim=-1)
    conf = p.max(dim=-1).values
    assert torch.equal(v["argmax"].long(), torch.argmax(z, dim=-1))
    assert torch.allclose(v["conf"].double(), conf, rtol=2e-5, atol=0)
    assert torch.allclose(v["lse"].double(), torch.logsumexp(z, dim=-1), rtol=0, atol=1e-4)
    top = torch.topk(z, 8, dim=-1)
    assert torch.equal(v["topk_id"].long(), top.indices)


def test_commit_rules_and_graph_determinism(dense8b):
    wc, eng, w, req, tokens = dense8b
    note("full-size: commit rules over one block, twice, from graph replays")
    results = []
    for rep in range(2):
        tokens.copy_(req["tokens"].cuda())
        eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                      req["plant_id"].cuda(), req["plant_bias"].cuda())
        eng.refresh_kv()
        P, B = int(req["prompt_len"][0]), wc.decode.block_len
        prev = tokens[0, P:P + B].clone()
        for s in range(B // 8):
            eng.step_graph(8)
            torch.cuda.synchronize()
            cur = tokens[0, P:P + B]
            changed = (cur != prev)
            assert bool((prev[changed] == wc.model.mask_id).all())      # never re-masked
            assert int(changed.sum()) >= 1
            prev = cur.clone()
        v = eng.view()
        results.append((tokens.clone(), v["logits"].clone(), v["credit"].clone()))
    assert torch.equal(results[0][0], results[1][0])
    assert torch.equal(results[0][1].view(torch.int32), results[1][1].view(torch.int32))
    assert torch.equal(results[0][2].view(torch.int32), results[1][2].view(torch.int32))


def test_full_run_commits_every_position(dense8b):
    wc, eng, w, req, tokens = dense8b
    note("full-size: run to completion")
    tokens.copy_(req["tokens"].cuda())
    eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                  req["plant_id"].cuda(), req["plant_bias"].cuda())
    stats = eng.run_to_completion()
    P = int(req["prompt_len"][0])
    t = tokens[0].cpu().numpy()
    assert stats["committed"] == wc.gen_len
    assert not np.any(t[P:P + wc.gen_len] == wc.model.mask_id)
    assert np.array_equal(t[:P], req["tokens"][0, :P].numpy())
    note(f"  {stats}")


def test_selector_bit_exact_on_the_steps_own_statistics(dense8b):
    """A whole block of the 32-layer model, eager steps: after each step the
    oracle selector, fed the step's own statistics and the credit state before
    it, must give the GPU's commit mask, tokens, credit bits, tracked ids and
    smoothing state; fed the oracle's vocab statistics of the step's logits it
    must take the same commits except at confidences or credits within 1e-3 of
    tau or kappa (excluded and counted)."""
    from gpu_util import _gpu_block_state, selector_check
    wc, eng, w, req, tokens = dense8b
    note("full-size: selector on the step's own statistics, one block")
    tokens.copy_(req["tokens"].cuda())
    eng.set_batch(tokens, req["prompt_len"].tolist(), req["gen_len"].tolist(),
                  req["plant_id"].cuda(), req["plant_bias"].cuda())
    eng.refresh_kv()
    B = wc.decode.block_len
    excluded = 0
    for s in range(B):
        v = eng.view()
        tok0 = tokens.cpu().numpy()
        st0 = _gpu_block_state(v, 1, B)
        eng.denoise_step()
        eng.commit()
        torch.cuda.synchronize()
        excluded += selector_check(wc, req, tok0, st0, v, tokens.cpu().numpy(), [0], [0])
        if not (tokens[0, int(req["prompt_len"][0]):int(req["prompt_len"][0]) + B]
                == wc.model.mask_id).any():
            break
    note(f"  {s + 1} steps, {excluded} excluded near tau/kappa")
    assert s + 1 == B       # one commit per step under the literal planting
