"""Host-only checks of the C ABI: the library loads, exports every function
include/dinfer.h declares, and rejects bad configurations before touching a
GPU (no compute call runs here)."""
import ctypes as C
import os
import re

import pytest

import synth
from diffusion_vicinity_kv_amd import binding as B
from diffusion_vicinity_kv_amd.engine import _decode_struct, _model_struct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(dinfer_\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    lib = B.load()
    declared = _declared_functions()
    assert {"dinfer_step_init", "dinfer_refresh_kv", "dinfer_denoise_step", "dinfer_commit",
            "dinfer_run_to_completion"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(B.EXPORTS)


def test_status_strings():
    for s, name in [(0, "DINFER_OK"), (1, "DINFER_E_ARG"), (2, "DINFER_E_WORKSPACE"),
                    (3, "DINFER_E_STATE"), (4, "DINFER_E_HIP"), (5, "DINFER_E_UNSUPPORTED")]:
        assert B.status_name(s) == name


def _structs(name="tiny_f32", **mkw):
    wc = synth.preset(name)
    m = wc.model if not mkw else wc.with_model(**mkw).model
    return _model_struct(m), _decode_struct(wc.decode, 0), wc


@pytest.mark.parametrize("name", synth.PRESET_ORDER)
def test_workspace_bytes_positive_for_presets(name):
    mc, dc, wc = _structs(name)
    n = B.load().dinfer_workspace_bytes(C.byref(mc), C.byref(dc), wc.batch, wc.max_len)
    assert n > 0 and n % 256 == 0
    # the KV cache alone: 2 * layers * batch * heads * max_len * hd * element size
    m = wc.model
    es = 4 if m.dtype == "f32" else 2
    kv = 2 * m.n_layers * wc.batch * m.n_heads * wc.max_len * m.head_dim * es
    assert n >= kv
    if m.is_moe:
        # plus the packed expert activations: rows * top_k * (2 Fe + Fe + d) floats
        rows = wc.batch * wc.max_len
        assert n >= kv + rows * m.top_k * (3 * m.expert_ffn + m.d_model) * 4


def test_workspace_bytes_rejects_bad_shapes():
    lib = B.load()
    for kw in [dict(head_dim=96, d_model=4 * 96), dict(vocab=4098, mask_id=4097),
               dict(n_heads=3)]:
        mc, dc, wc = _structs(**kw)
        assert lib.dinfer_workspace_bytes(C.byref(mc), C.byref(dc), 1, 128) == 0
    mc, dc, wc = _structs()
    dc.block_len = 65
    assert lib.dinfer_workspace_bytes(C.byref(mc), C.byref(dc), 1, 128) == 0
    moe = dict(n_experts=64, top_k=8, expert_ffn=1024, shared_ffn=2048)
    for kw in [dict(moe, n_experts=65), dict(moe, top_k=9), dict(moe, top_k=0),
               dict(moe, expert_ffn=1000)]:
        mc, dc, wc = _structs(**kw)
        assert lib.dinfer_workspace_bytes(C.byref(mc), C.byref(dc), 1, 128) == 0, kw


def test_step_init_argument_errors_without_gpu():
    lib = B.load()
    mc, dc, wc = _structs()
    w = B.Weights()
    ctx = C.c_void_p()
    # null out pointer
    assert lib.dinfer_step_init(C.byref(mc), C.byref(dc), C.byref(w), 1, 128, None, 0, None,
                                None) == B.E_ARG
    # more experts or a wider top-k than the router kernel handles
    mc2, dc2, _ = _structs(n_experts=128, top_k=8, expert_ffn=1024, shared_ffn=2048)
    assert lib.dinfer_step_init(C.byref(mc2), C.byref(dc2), C.byref(w), 1, 128, None, 0, None,
                                C.byref(ctx)) == B.E_UNSUPPORTED
    # MoE model with dense FFN weights only
    mc3, dc3, _ = _structs(n_experts=64, top_k=8, expert_ffn=1024, shared_ffn=2048)
    nl = mc3.n_layers
    arr = (C.c_void_p * nl)(*([16] * nl))
    w3 = B.Weights()
    w3.tok_emb = w3.final_norm = w3.lm_head = 16
    for k in ("attn_norm", "wqkv", "wo", "ffn_norm", "w_gate_up", "w_down"):
        setattr(w3, k, C.cast(arr, B._PP))
    assert lib.dinfer_step_init(C.byref(mc3), C.byref(dc3), C.byref(w3), 1, 128, None, 0, None,
                                C.byref(ctx)) == B.E_ARG
    assert b"FFN weight" in lib.dinfer_last_error()
    # missing weights
    assert lib.dinfer_step_init(C.byref(mc), C.byref(dc), C.byref(w), 1, 128, None, 0, None,
                                C.byref(ctx)) == B.E_ARG
    assert b"weight" in lib.dinfer_last_error()


def test_vocab_stats_argument_errors_without_gpu():
    lib = B.load()
    assert lib.dinfer_vocab_stats(None, 4, 4096, None, None, -1, None, None, None, None, None,
                                  None, 0, None) == B.E_ARG
    assert lib.dinfer_vocab_stats_scratch_bytes(32, 126464) > 0
    assert lib.dinfer_vocab_stats_scratch_bytes(0, 126464) == 0


def test_pack_linear_argument_errors_without_gpu():
    """Every rejection happens before a launch (addresses are never touched)."""
    lib = B.load()
    a, b = 1 << 20, 1 << 40
    assert lib.dinfer_pack_linear(None, b, 1, 64, 128, B.BF16, None) == B.E_ARG
    assert lib.dinfer_pack_linear(a, a, 1, 64, 128, B.BF16, None) == B.E_ARG
    assert lib.dinfer_pack_linear(a, a + 64 * 128, 1, 64, 128, B.BF16, None) == B.E_ARG  # overlap
    assert lib.dinfer_pack_linear(a, a + 64 * 128 * 2, 2, 64, 128, B.BF16, None) == B.E_ARG
    assert lib.dinfer_pack_linear(a, b, 1, 40, 128, B.BF16, None) == B.E_ARG            # rows % 16
    assert lib.dinfer_pack_linear(a, b, 1, 0, 128, B.BF16, None) == B.E_ARG
    assert lib.dinfer_pack_linear(a, b, 0, 64, 128, B.BF16, None) == B.E_ARG            # n_mats
    assert lib.dinfer_pack_linear(a, b, 1, 64, 48, B.BF16, None) == B.E_ARG             # K % 32
    assert lib.dinfer_pack_linear(a, b, 1, 64, 24, B.F32, None) == B.E_ARG              # K % 16
    assert lib.dinfer_pack_linear(a, b, 1, 64, 128, 7, None) == B.E_ARG
    assert b"dtype" in lib.dinfer_last_error()


def test_calls_on_null_context_fail_cleanly():
    lib = B.load()
    assert lib.dinfer_denoise_step(None) == B.E_ARG
    assert lib.dinfer_commit(None) == B.E_ARG
    assert lib.dinfer_refresh_kv(None, None) == B.E_ARG
    assert lib.dinfer_run_to_completion(None, 1, None) == B.E_ARG
    lib.dinfer_destroy(None)


def test_pending_rows_and_scheduler_argument_errors_without_gpu():
    lib = B.load()
    a = (C.c_int32 * 4)()
    assert lib.dinfer_pending_rows(None, a, a) == B.E_ARG
    h = C.c_void_p()
    assert lib.dinfer_sched_create(10, 4, None) == B.E_ARG
    assert lib.dinfer_sched_create(10, 4, C.byref(h)) == B.OK and h.value
    adm = (C.c_uint8 * 4)()
    assert lib.dinfer_sched_round(h, None, a, adm, None) == B.E_ARG
    assert lib.dinfer_sched_round(h, a, a, None, None) == B.E_ARG
    assert lib.dinfer_sched_round(h, a, a, adm, None) == B.OK   # nothing decodes or waits
    lib.dinfer_sched_destroy(h)
    lib.dinfer_sched_destroy(None)


def test_step_init_workspace_errors_without_gpu():
    """An absent, misaligned or undersized workspace is rejected before any
    device call (the weight pointers are placeholders, never dereferenced)."""
    lib = B.load()
    mc, dc, wc = _structs()
    nl = mc.n_layers
    arr = (C.c_void_p * nl)(*([4096] * nl))
    w = B.Weights()
    w.tok_emb = w.final_norm = w.lm_head = 4096
    for k in ("attn_norm", "wqkv", "wo", "ffn_norm", "w_gate_up", "w_down"):
        setattr(w, k, C.cast(arr, B._PP))
    need = lib.dinfer_workspace_bytes(C.byref(mc), C.byref(dc), 1, wc.max_len)
    assert need > 0
    ctx = C.c_void_p(1234)
    base = 1 << 40
    for ws, nbytes, why in [(None, need, b"null"), (base + 8, need, b"aligned"),
                            (base + 128, need, b"aligned"), (base, need - 256, b"too small"),
                            (base, 0, b"too small")]:
        st = lib.dinfer_step_init(C.byref(mc), C.byref(dc), C.byref(w), 1, wc.max_len, ws,
                                  nbytes, None, C.byref(ctx))
        assert st == B.E_WORKSPACE, (ws, nbytes, st)
        assert why in lib.dinfer_last_error(), lib.dinfer_last_error()
        assert ctx.value is None            # *out cleared on every failure
        ctx = C.c_void_p(1234)
