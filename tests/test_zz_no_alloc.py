"""dinfer_vocab_stats_noalloc (scratch in the library's fixed device array,
no allocation) against dinfer_vocab_stats (caller scratch) on the same
inputs: two calls in a row, the second smaller, each bit-identical to the
allocating entry point (same kernels, same partial layout and merge order);
and sizes beyond the fixed array rejected before any launch."""
import pytest
import torch

import synth
from diffusion_vicinity_kv_amd import binding as B

pytestmark = pytest.mark.gpu


def _outs(rows):
    return {"argmax": torch.empty(rows, dtype=torch.int32, device="cuda"),
            "conf": torch.empty(rows, device="cuda"), "lse": torch.empty(rows, device="cuda"),
            "topk_id": torch.empty(rows, 8, dtype=torch.int32, device="cuda"),
            "topk_p": torch.empty(rows, 8, device="cuda")}


def _inputs(rows, V, seed):
    z = synth.make_logits(rows, V, seed=seed, ties=2, device="cuda")
    g = torch.Generator().manual_seed(seed)
    pid = torch.where(torch.rand(rows, generator=g) < 0.5,
                      torch.randint(0, V - 1, (rows,), generator=g),
                      torch.full((rows,), -1)).to(torch.int32).cuda()
    pb = torch.full((rows,), 8.0, device="cuda")
    return z, pid, pb


def test_noalloc_matches_the_allocating_entry_point_twice():
    lib = B.load()
    for rows, V, seed in [(512, 126464, 1), (32, 126464, 2), (5, 4096, 3)]:
        print(f"no-alloc vocab stats rows={rows} V={V}", flush=True)
        z, pid, pb = _inputs(rows, V, seed)
        ref = _outs(rows)
        scratch = torch.empty(lib.dinfer_vocab_stats_scratch_bytes(rows, V), dtype=torch.uint8,
                              device="cuda")
        B.vocab_stats(z, pid, pb, V - 1, ref, scratch)
        got = _outs(rows)
        B.vocab_stats_noalloc(z, pid, pb, V - 1, got)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k].view(torch.int32), ref[k].view(torch.int32)), (rows, k)


def test_noalloc_rejects_sizes_beyond_its_array():
    lib = B.load()
    rows, V = 40000, 126464
    assert lib.dinfer_vocab_stats_scratch_bytes(rows, V) > (2 << 20)
    z = torch.empty(1, device="cuda")        # never read: the size check comes first
    o = torch.empty(8, device="cuda")
    st = lib.dinfer_vocab_stats_noalloc(B.ptr(z), rows, V, None, None, V - 1, B.ptr(o), B.ptr(o),
                                        B.ptr(o), B.ptr(o), B.ptr(o), B.stream_handle())
    assert st == B.E_UNSUPPORTED
    assert b"no-allocation" in lib.dinfer_last_error()
