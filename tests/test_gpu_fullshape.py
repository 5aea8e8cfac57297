"""Oracle parity at the shapes the benchmark runs, in its launch configuration.

Each test is teacher-forced (gpu_util.teacher_forced): after a block-start
refresh, denoise+commit steps whose block-row logits must lie within
2e-2 * RMS of the oracle's (bf16 weights and cache against fp64), with the
decoding strategy checked bit-exact against the oracle selector on the GPU's
own statistics, and the oracle taking over the GPU's decode state after each
step so both sides see the same inputs.

  * the dense 8B shape at batch 1 with all 32 layers (the headline workload):
    refresh caches of five layers, then two steps, against an oracle that
    stores its cache in bf16 like the model and one that keeps it in fp64;
  * the batch-16 request mix at full width (d 4096, V 126464, sixteen ragged
    prompts of 128..1024 positions) with two layers: all sixteen requests run
    the batched step, four of them (the shortest, the longest and two more)
    are followed by the oracle, the selector is checked on all sixteen;
  * the long-context shape (prompt 8192 + 1024 generated, batch 4, blocks of
    64, w 32, hierarchical order, tau 0.85) with two layers: request 0 is
    followed by the oracle, the selector is checked on all four."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import build, note, teacher_forced
from oracle.model import OracleModel

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _runs(wc, w, req, which, layers=None, model=None, kv_round=None):
    om = model or OracleModel(wc.model, w, layers=layers)
    rb = req.get("router_bias")
    return {r: oracle.OracleRun(om, wc.decode, req["tokens"][r].numpy(), int(req["prompt_len"][r]),
                                int(req["gen_len"][r]), req["plant_id"][r].numpy(),
                                float(req["plant_bias"][r]), None if rb is None else rb[r].numpy(),
                                kv_round=kv_round)
            for r in which}


def test_dense8b_32_layers_refresh_and_two_steps():
    """All 32 layers.  The cache of a bf16 model is stored in bf16, and that
    rounding, written at the refresh and read at every step through 32
    layers, moves the logits by about 5e-2 * RMS on its own (measured between
    two fp64 oracles, one storing its cache in bf16): no bf16-cache
    implementation can meet 2e-2 against an oracle that keeps an fp64 cache.
    So the gate is taken against the oracle that stores its cache like the
    model (all arithmetic fp64), and against the fp64-cache oracle with the
    storage effect added to the tolerance; the caches are compared with each
    element's own bf16 rounding allowed on top of 2e-2 * RMS."""
    note("dense 8B, 32 layers, batch 1: refresh + 2 teacher-forced steps")
    wc = synth.preset("dense8b_b1")
    eng, w, req, tokens = build(wc)
    note("  upcasting the 32 layers for the oracle")
    om = OracleModel(wc.model, w)
    runs = _runs(wc, w, req, [0], model=om, kv_round="bf16")
    shadow = _runs(wc, w, req, [0], model=om)
    rep = teacher_forced(wc, eng, tokens, req, runs, n_steps=2, logit_tol=TOL,
                         check_cache_layers=[0, 7, 15, 23, 31], shadow=shadow)
    note(f"  {rep}")
    assert rep["steps"] == 2
    eng.close()


def test_dense8b_batch16_mix_full_width_two_layers():
    note("dense 8B batch-16 mix at full width, 2 layers: 4 teacher-forced steps")
    wc = synth.preset("dense8b_b16").with_model(n_layers=2)
    eng, w, req, tokens = build(wc)
    P = req["prompt_len"].tolist()
    order = np.argsort(P, kind="stable")
    which = sorted({int(order[0]), int(order[-1]), int(order[5]), int(order[10])})
    note(f"  prompts {P}; oracle on requests {which}")
    runs = _runs(wc, w, req, which)
    rep = teacher_forced(wc, eng, tokens, req, runs, n_steps=4, logit_tol=TOL,
                         check_cache_layers=[1])
    note(f"  {rep}")
    assert rep["steps"] == 4
    eng.close()


def test_long_context_shape_two_layers_hierarchical():
    note("long-context shape (8192 + 1024, batch 4, B 64, w 32, hierarchical), 2 layers")
    wc = synth.preset("dense8b_long_b4").with_model(n_layers=2)
    assert wc.decode.hierarchical and wc.decode.block_len == 64 and wc.decode.vicinity_w == 32
    eng, w, req, tokens = build(wc)
    runs = _runs(wc, w, req, [0])
    rep = teacher_forced(wc, eng, tokens, req, runs, n_steps=4, logit_tol=TOL,
                         check_cache_layers=[1])
    note(f"  {rep}")
    assert rep["steps"] == 4
    eng.close()
