"""The LM head's fused vocab statistics (per-(row, column tile) records in the
projection kernel's epilogue, merged per row) against the oracle's vocab
statistics of the very logits the same kernel stores when the inspection
switch is on, and against the standalone vocab pass over them; the switch
itself changes no result.

Shapes: the tiny fp32 model (fp32 skinny kernel, 128-column tiles), the dense
8B shape at batch 1 (bf16 skinny, 256-column tiles, 494 tiles per row), the
MoE vocabulary 157184 with 64 block rows (bf16 skinny, 614 tiles), the
batch-16 mix (512 rows: the fat kernel's epilogue, two row halves per tile);
two layers where the model is large (the epilogue sees only the LM head)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from diffusion_vicinity_kv_amd import binding as B
from gpu_util import build, note

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_f32": lambda: synth.preset("tiny_f32"),
    "dense8b_b1_2l": lambda: synth.preset("dense8b_b1").with_model(n_layers=2),
    "moe_b1_1l": lambda: synth.preset("moe_b1").with_model(n_layers=1),
    "dense8b_b16_2l": lambda: synth.preset("dense8b_b16").with_model(n_layers=2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_fused_vocab_stats(case):
    wc = CASES[case]()
    note(f"fused LM-head statistics: {case} ({wc.batch * wc.decode.block_len} rows, V {wc.model.vocab})")
    eng, w, req, tokens = build(wc)          # keep_logits on
    eng.refresh_kv()
    eng.denoise_step()
    torch.cuda.synchronize()
    v = eng.view()
    keys = ("argmax", "conf", "lse", "topk_id", "topk_p")
    got = {k: v[k].clone() for k in keys}
    z = v["logits"].clone()
    R, V = z.shape
    Bl = wc.decode.block_len
    # each block row's planting, as the step applies it
    P = req["prompt_len"].tolist()
    pid = torch.stack([req["plant_id"][r, P[r]:P[r] + Bl] for r in range(wc.batch)]).reshape(-1)
    pb = torch.repeat_interleave(req["plant_bias"], Bl)
    mask_id = wc.model.mask_id
    # the oracle's statistics of the same fp32 logits
    want = oracle.vocab_stats(z.cpu().numpy(), pid.numpy(), pb.numpy(), mask_id, 8)
    assert np.array_equal(got["argmax"].cpu().numpy(), want["argmax"])
    assert np.array_equal(got["topk_id"].cpu().numpy(), want["topk_id"])
    assert np.allclose(got["conf"].cpu().numpy(), want["conf"], rtol=2e-5, atol=0)
    assert np.allclose(got["topk_p"].cpu().numpy(), want["topk_p"], rtol=2e-5, atol=1e-12)
    assert np.allclose(got["lse"].cpu().numpy(), want["lse"], rtol=0,
                       atol=2e-5 * np.abs(want["lse"]).max())
    # the standalone vocab pass over the stored logits: same ids
    lib = B.load()
    scratch = torch.empty(lib.dinfer_vocab_stats_scratch_bytes(R, V), dtype=torch.uint8,
                          device="cuda")
    sep = {"argmax": torch.empty(R, dtype=torch.int32, device="cuda"),
           "conf": torch.empty(R, device="cuda"), "lse": torch.empty(R, device="cuda"),
           "topk_id": torch.empty(R, 8, dtype=torch.int32, device="cuda"),
           "topk_p": torch.empty(R, 8, device="cuda")}
    B.vocab_stats(z, pid.to(torch.int32).cuda(), pb.cuda(), mask_id, sep, scratch)
    torch.cuda.synchronize()
    assert torch.equal(sep["argmax"], got["argmax"]) and torch.equal(sep["topk_id"], got["topk_id"])
    # the inspection switch off: the same statistics, bit for bit
    eng.keep_logits(False)
    v["logits"].fill_(float("nan"))
    eng.denoise_step()
    torch.cuda.synchronize()
    for k in keys:
        assert torch.equal(v[k].view(torch.int32), got[k].view(torch.int32)), k
    assert torch.isnan(v["logits"]).all()    # nothing stored
    eng.close()


@pytest.mark.parametrize("mask,lo,hi", [(15, 1e-3, 1e-1), (16, 1e-4, 2e-2)])
def test_activation_precision_option_and_default(mask, lo, hi):
    """dinfer_set_activation_precision: with every projection taking bf16
    activations alone (mask 15) the logits move by the activations' own
    rounding (measured 4.1e-2 * RMS on two full-width layers), with the
    attention's probabilities in bf16 alone (mask 16) by theirs (measured
    7.2e-3 * RMS), and back at the default they are bit-identical to a
    context that never changed it."""
    wc = synth.preset("dense8b_b1").with_model(n_layers=2)
    eng, w, req, tokens = build(wc)
    ref, _, _, _ = build(wc, weights=w, req=req)
    out = {}
    for name, e, m in (("ref", ref, None), ("option", eng, mask), ("back", eng, 0)):
        if m is not None:
            e.set_activation_precision(m, m)
        e.refresh_kv()
        e.denoise_step()
        torch.cuda.synchronize()
        out[name] = e.view()["logits"].clone()
    z = out["ref"].double()
    rms = float(z.pow(2).mean().sqrt())
    err = float((out["option"].double() - z).abs().max()) / rms
    note(f"  precision mask {mask}: max |dlogit| / RMS = {err:.3e}")
    assert lo < err < hi
    assert torch.equal(out["back"].view(torch.int32), out["ref"].view(torch.int32))
    for e in (eng, ref):
        e.close()
