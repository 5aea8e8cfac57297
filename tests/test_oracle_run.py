"""Run-level invariants of the oracle's iteration manager (no GPU)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.model import OracleModel


def _small_workload(hier=False, smooth=0.3, bias=2.0, credit=1.0, moe=False, batch=2):
    m = synth.ModelCfg(n_layers=2, d_model=32, n_heads=2, head_dim=16, ffn_dim=0 if moe else 48,
                       vocab=64, mask_id=63, dtype="f32", n_experts=4 if moe else 0,
                       top_k=2 if moe else 0, expert_ffn=12 if moe else 0,
                       shared_ffn=16 if moe else 0)
    dc = synth.DecodeCfg(block_len=8, vicinity_w=3, tau=0.5, credit_weight=credit,
                         smooth_alpha=smooth, hierarchical=hier)
    return synth.WorkloadCfg(name="small", model=m, decode=dc, batch=batch, prompt_len=(6, 12),
                             gen_len=24, plant_bias=bias, plant_prob=(0.6, 0.9),
                             router_pref_bias=2.0 if moe else 0.0, seed=11)


@pytest.mark.parametrize("hier,smooth,moe", [(False, 0.3, False), (True, 0.3, False),
                                             (False, 0.0, True), (True, 0.0, False)])
def test_run_invariants(hier, smooth, moe):
    wc = _small_workload(hier=hier, smooth=smooth, moe=moe)
    w = synth.make_weights(wc.model, wc.seed)
    req = synth.make_requests(wc)
    for r in range(wc.batch):
        run = oracle.OracleRun(OracleModel(wc.model, w), wc.decode, req["tokens"][r].numpy(),
                               int(req["prompt_len"][r]), wc.gen_len, req["plant_id"][r].numpy(),
                               float(req["plant_bias"][r]),
                               None if req["router_bias"] is None else req["router_bias"][r].numpy())
        P = run.P
        prompt = run.tokens[:P].copy()
        history = []
        for k in range(run.n_blocks):
            run.start_block(k)
            while run.block_masked().any():
                before = run.tokens.copy()
                run.step()
                rec = run.records[-1]
                after = run.tokens
                changed = np.nonzero(before != after)[0]
                # at least one commit per step, only masked positions of the block change,
                # nothing is ever re-masked
                assert len(changed) >= 1
                assert np.all(before[changed] == wc.model.mask_id)
                assert np.all(after[changed] != wc.model.mask_id)
                assert np.all((changed >= run.bs) & (changed < run.be))
                assert sorted((changed - run.bs).tolist()) == sorted(rec["commits"].tolist())
                history.append(len(changed))
            assert 1 <= run.block_steps <= wc.decode.block_len
        assert np.array_equal(run.tokens[:P], prompt)
        assert not np.any(run.tokens == wc.model.mask_id)
        assert sum(history) == wc.gen_len


def test_threshold_and_credit_commit_several_per_step_when_confident():
    # A strong planting bias puts planted rows above tau; those commit together.
    wc = _small_workload(bias=12.0, batch=1)
    w = synth.make_weights(wc.model, wc.seed)
    req = synth.make_requests(wc)
    run = oracle.run_request(wc.model, wc.decode, w, req)
    assert max(len(r["commits"]) for r in run.records) > 1
    assert sum(run.steps) < wc.gen_len


def test_credit_commits_below_threshold():
    # Confidence in [0.45, tau) for planted rows: credit lets them commit before
    # the plain rule would; with lambda = 0 the same run needs more steps.
    wc = _small_workload(bias=5.0, batch=1).with_decode(tau=0.95)
    w = synth.make_weights(wc.model, wc.seed)
    req = synth.make_requests(wc)
    with_credit = oracle.run_request(wc.model, wc.decode, w, req)
    no_credit = oracle.run_request(wc.model, wc.with_decode(credit_weight=0.0).decode, w, req)
    credit_only = [r for r in with_credit.records if not r["fallback"] and len(r["commits"])]
    assert sum(with_credit.steps) < sum(no_credit.steps)
    assert credit_only


def test_batch_requests_are_independent():
    wc = _small_workload(batch=3)
    w = synth.make_weights(wc.model, wc.seed)
    req = synth.make_requests(wc)
    r1 = oracle.run_request(wc.model, wc.decode, w, req, r=1)
    # the same request alone, with the other requests' data scrambled
    req2 = {k: (v.clone() if v is not None else None) for k, v in req.items()}
    req2["tokens"][0] = 5
    req2["tokens"][2] = 7
    r1b = oracle.run_request(wc.model, wc.decode, w, req2, r=1)
    assert np.array_equal(r1.tokens, r1b.tokens) and r1.steps == r1b.steps


def test_eos_fill_cases():
    """End-of-sequence fill against a brute-force rewrite of the rule: after
    the first EOS of the response every MASK becomes EOS; MASKs before it,
    other tokens, and EOS ids in the prompt are left alone."""
    from oracle.decode import eos_fill
    M, E, P = 9, 5, 4
    cases = [[1, 5, 2, 3, M, M, 7, M, M, M],       # EOS only in the prompt
             [1, 2, 3, 4, M, 5, M, 7, M, 5],       # first response EOS at 5
             [1, 2, 3, 4, 5, M, M, M, M, M],       # EOS at the response start
             [1, 2, 3, 4, M, M, M, M, M, M],       # no EOS
             [1, 2, 3, 4, 6, 7, 8, 5, 1, 2]]       # nothing masked
    for c in cases:
        t = np.array(c)
        want = t.copy()
        first = next((i for i in range(P, len(c)) if c[i] == E), None)
        if first is not None:
            for i in range(first + 1, len(c)):
                if c[i] == M:
                    want[i] = E
        done = eos_fill(t, P, len(c), M, E)
        assert t.tolist() == want.tolist()
        assert done == (M not in want[P:].tolist())
        t2 = np.array(c)
        eos_fill(t2, P, len(c), M, -1)                # no EOS id: unchanged
        assert t2.tolist() == c


def test_eos_run_stops_after_the_first_eos():
    """A run whose EOS id is a token the plain run commits early: the run
    ends once nothing is masked, every response position after the first EOS
    holds EOS, none before it is MASK, and no block after the EOS's block is
    run; an EOS id the plain run never commits leaves the run unchanged."""
    import dataclasses
    wc = _small_workload(batch=1)
    w = synth.make_weights(wc.model, wc.seed)
    req = synth.make_requests(wc)

    def run_with(eos):
        dc = dataclasses.replace(wc.decode, eos_id=eos)
        run = oracle.OracleRun(OracleModel(wc.model, w), dc, req["tokens"][0].numpy(),
                               int(req["prompt_len"][0]), wc.gen_len, req["plant_id"][0].numpy(),
                               float(req["plant_bias"][0]))
        run.run()
        return run

    plain = run_with(-1)
    P, L = plain.P, plain.L
    # the first token committed by the plain run (block 0, step 0)
    T0 = plain.records[0]["commits"]
    eos = int(plain.tokens[P + int(T0[0])])
    run = run_with(eos)
    resp = run.tokens[P:L]
    first = int(np.nonzero(resp == eos)[0][0])
    assert (resp[first + 1:] == eos).all()
    assert (resp[:first] != wc.model.mask_id).all()
    assert len(run.steps) == first // wc.decode.block_len + 1
    assert sum(run.steps) < sum(plain.steps)
    unused = next(i for i in range(wc.model.vocab - 1) if i not in plain.tokens[P:L])
    same = run_with(unused)
    assert np.array_equal(same.tokens, plain.tokens) and same.steps == plain.steps
