"""Call-order and workspace errors on a live context (the C ABI's contract:
step_init -> set_batch -> refresh_kv -> (denoise_step -> commit)*).  Each
rejected call returns its status and leaves the context usable: after the
errors the same context runs a request to completion, token for token equal
to the oracle's run."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import synth
from diffusion_vicinity_kv_amd import binding as B
from diffusion_vicinity_kv_amd.engine import Engine, _decode_struct, _model_struct
from gpu_util import note

pytestmark = pytest.mark.gpu


def _status(fn, *args):
    try:
        fn(*args)
    except B.DinferError as e:
        return e.status
    return B.OK


@pytest.mark.parametrize("unroll", [0, 2])
def test_call_order_errors_leave_the_context_usable(unroll):
    note(f"call-order errors, graph_unroll={unroll}")
    wc = synth.preset("tiny_f32")
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    req = synth.make_requests(wc)
    eng = Engine(wc.model, wc.decode, w, 1, req["tokens"].shape[1], graph_unroll=unroll)
    # before set_batch
    assert _status(eng.denoise_step) == B.E_STATE
    assert _status(eng.commit) == B.E_STATE
    assert _status(eng.refresh_kv) == B.E_STATE
    if unroll:
        assert _status(eng.step_graph, unroll) == B.E_STATE
    tokens = req["tokens"].cuda().contiguous()
    P, G = req["prompt_len"].tolist(), req["gen_len"].tolist()
    pid, pb = req["plant_id"].cuda().contiguous(), req["plant_bias"].cuda().contiguous()
    eng.set_batch(tokens, P, G, pid, pb)
    # precision options: bits above 4 are rejected; an fp32 model has no
    # bf16-only option (both leave the default precision in place)
    assert _status(eng.set_activation_precision, 32, 0) == B.E_ARG
    assert _status(eng.set_activation_precision, 0, 1 << 31) == B.E_ARG
    assert _status(eng.set_activation_precision, 16, 16) == B.E_UNSUPPORTED
    eng.set_activation_precision(0, 0)
    # bound but nothing refreshed
    assert _status(eng.denoise_step) == B.E_STATE
    assert _status(eng.commit) == B.E_STATE
    if unroll:
        assert _status(eng.step_graph, unroll) == B.E_STATE
    eng.refresh_kv()
    # commit with no denoise_step since the refresh
    assert _status(eng.commit) == B.E_STATE
    eng.denoise_step()
    # a refresh in between makes the step's statistics stale
    eng.refresh_kv()
    assert _status(eng.commit) == B.E_STATE
    eng.denoise_step()
    eng.commit()
    assert _status(eng.commit) == B.E_STATE          # one commit per denoise_step
    torch.cuda.synchronize()
    # the context is still usable: a fresh run from the same prompt
    tokens.copy_(req["tokens"].cuda())
    eng.set_batch(tokens, P, G, pid, pb)
    stats = eng.run_to_completion()
    torch.cuda.synchronize()
    run = oracle.run_request(wc.model, wc.decode, w, req)
    assert np.array_equal(tokens.cpu().numpy()[0][: run.L], run.tokens)
    assert stats["committed"] == wc.gen_len
    eng.close()


def test_workspace_errors_on_device_memory():
    """Undersized and misaligned device workspaces are rejected; a correct one
    on the same arguments then initialises."""
    note("workspace errors with real device memory")
    wc = synth.preset("tiny_f32")
    w = synth.make_weights(wc.model, wc.seed, device="cuda")
    eng = Engine(wc.model, wc.decode, w, 1, wc.max_len)     # packs the weights
    lib = B.load()
    mc, dc = _model_struct(wc.model), _decode_struct(wc.decode, 0)
    need = lib.dinfer_workspace_bytes(C.byref(mc), C.byref(dc), 1, wc.max_len)
    raw = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    base = B.ptr(raw) + (-B.ptr(raw)) % 256
    st = torch.cuda.current_stream()
    ctx = C.c_void_p()
    for ws, nbytes in [(base, need - 256), (base + 64, need), (base + 4, need)]:
        s = lib.dinfer_step_init(C.byref(mc), C.byref(dc), C.byref(eng._w), 1, wc.max_len, ws,
                                 nbytes, B.stream_handle(st), C.byref(ctx))
        assert s == B.E_WORKSPACE and not ctx.value, (ws - base, nbytes, s)
    s = lib.dinfer_step_init(C.byref(mc), C.byref(dc), C.byref(eng._w), 1, wc.max_len, base,
                             need, B.stream_handle(st), C.byref(ctx))
    assert s == B.OK and ctx.value
    lib.dinfer_destroy(ctx)
    eng.close()
