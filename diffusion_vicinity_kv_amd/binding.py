"""ctypes binding of libdinfer.so (include/dinfer.h), argument marshalling only.

Every call here forwards to the HIP library; nothing of the method is computed
in Python.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdinfer.so")

OK, E_ARG, E_WORKSPACE, E_STATE, E_HIP, E_UNSUPPORTED = range(6)
F32, BF16 = 0, 1

EXPORTS = [
    "dinfer_workspace_bytes", "dinfer_step_init", "dinfer_set_batch", "dinfer_refresh_kv",
    "dinfer_denoise_step", "dinfer_commit", "dinfer_advance_blocks", "dinfer_run_to_completion",
    "dinfer_get_step_view", "dinfer_vocab_stats_scratch_bytes", "dinfer_vocab_stats",
    "dinfer_step_graph", "dinfer_pack_linear", "dinfer_linear_out_elems", "dinfer_linear",
    "dinfer_status_str", "dinfer_last_error", "dinfer_destroy", "dinfer_refill", "dinfer_finished",
    "dinfer_pending_rows", "dinfer_sched_create", "dinfer_sched_destroy", "dinfer_sched_round",
    "dinfer_vocab_stats_noalloc", "dinfer_keep_logits", "dinfer_expert_slot_bytes",
    "dinfer_expert_offload", "dinfer_expert_place", "dinfer_expert_cache_report",
    "dinfer_set_activation_precision",
]


class ModelCfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_heads", "head_dim", "ffn_dim",
                                          "vocab", "mask_id", "n_experts", "top_k", "expert_ffn",
                                          "shared_ffn")] + [
        ("rope_theta", C.c_float), ("rms_eps", C.c_float), ("dtype", C.c_int32)]


class DecodeCfg(C.Structure):
    _fields_ = [("block_len", C.c_int32), ("vicinity_w", C.c_int32), ("tau", C.c_float),
                ("credit_weight", C.c_float), ("credit_decay", C.c_float),
                ("credit_kappa", C.c_float), ("smooth_alpha", C.c_float),
                ("smooth_topk", C.c_int32), ("hierarchical", C.c_int32),
                ("graph_unroll", C.c_int32), ("eos_id", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class Weights(C.Structure):
    _fields_ = [("tok_emb", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p)] + [
        (n, _PP) for n in ("attn_norm", "wqkv", "wo", "ffn_norm", "w_gate_up", "w_down", "router",
                           "exp_gate_up", "exp_down", "shared_gate_up", "shared_down")]


class RunStats(C.Structure):
    _fields_ = [("steps", C.c_int64), ("refreshes", C.c_int64), ("committed", C.c_int64),
                ("wall_ms", C.c_double), ("refresh_ms", C.c_double)]


class StepView(C.Structure):
    _fields_ = [("batch", C.c_int32), ("block_len", C.c_int32), ("vocab", C.c_int32),
                ("topk", C.c_int32)] + [
        (n, C.c_void_p) for n in ("logits", "argmax", "conf", "lse", "topk_id", "topk_p", "credit",
                                  "tracked", "smooth_id", "smooth_p", "smooth_valid",
                                  "commit_mask", "block_done", "step_count", "commit_count",
                                  "kv_k", "kv_v")] + [
        ("moe_top_k", C.c_int32), ("moe_sel", C.c_void_p), ("moe_gate", C.c_void_p),
        ("moe_experts", C.c_int32), ("moe_logits", C.c_void_p), ("ffn_in", C.c_void_p),
        ("kv_len", C.c_int32), ("decode_stats", C.c_void_p), ("decode_stat_words", C.c_int32)]


class ExpertCacheStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("expert_hits", "expert_misses", "row_hits", "row_misses",
                                          "bytes_placed", "bytes_host_read", "placements")] + [
        ("slots", C.c_int32), ("interval", C.c_int32)]


class DinferError(RuntimeError):
    def __init__(self, status, what, detail):
        super().__init__(f"{what}: {status_name(status)}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libdinfer.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc for gfx950) before using the library")
    lib = C.CDLL(path)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    sig = {
        "dinfer_workspace_bytes": (sz, [C.POINTER(ModelCfg), C.POINTER(DecodeCfg), i32, i32]),
        "dinfer_step_init": (i32, [C.POINTER(ModelCfg), C.POINTER(DecodeCfg), C.POINTER(Weights),
                                   i32, i32, vp, sz, vp, C.POINTER(vp)]),
        "dinfer_set_batch": (i32, [vp, i32, vp, C.POINTER(i32), C.POINTER(i32), vp, vp, vp]),
        "dinfer_refresh_kv": (i32, [vp, C.POINTER(C.c_uint8)]),
        "dinfer_denoise_step": (i32, [vp]),
        "dinfer_commit": (i32, [vp]),
        "dinfer_advance_blocks": (i32, [vp, C.POINTER(C.c_uint8), C.POINTER(i32)]),
        "dinfer_run_to_completion": (i32, [vp, i32, C.POINTER(RunStats)]),
        "dinfer_get_step_view": (i32, [vp, C.POINTER(StepView)]),
        "dinfer_keep_logits": (i32, [vp, i32]),
        "dinfer_set_activation_precision": (i32, [vp, C.c_uint32, C.c_uint32]),
        "dinfer_expert_slot_bytes": (sz, [C.POINTER(ModelCfg)]),
        "dinfer_expert_offload": (i32, [vp, C.POINTER(vp), C.POINTER(vp), i32, i32, vp, sz]),
        "dinfer_expert_place": (i32, [vp]),
        "dinfer_expert_cache_report": (i32, [vp, C.POINTER(ExpertCacheStats), i32]),
        "dinfer_vocab_stats_scratch_bytes": (sz, [i32, i32]),
        "dinfer_vocab_stats": (i32, [vp, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "dinfer_vocab_stats_noalloc": (i32, [vp, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp]),
        "dinfer_step_graph": (i32, [vp, i32]),
        "dinfer_pack_linear": (i32, [vp, vp, i32, i32, i32, i32, vp]),
        "dinfer_linear_out_elems": (sz, [i32, i32, i32, i32]),
        "dinfer_linear": (i32, [vp, vp, vp, i32, i32, i32, i32, C.POINTER(i32), vp]),
        "dinfer_status_str": (C.c_char_p, [i32]),
        "dinfer_last_error": (C.c_char_p, []),
        "dinfer_destroy": (None, [vp]),
        "dinfer_refill": (i32, [vp, i32, i32, i32]),
        "dinfer_finished": (i32, [vp, C.POINTER(C.c_uint8)]),
        "dinfer_pending_rows": (i32, [vp, C.POINTER(i32), C.POINTER(i32)]),
        "dinfer_sched_create": (i32, [C.c_int64, i32, C.POINTER(vp)]),
        "dinfer_sched_destroy": (None, [vp]),
        "dinfer_sched_round": (i32, [vp, C.POINTER(i32), C.POINTER(i32), C.POINTER(C.c_uint8),
                                     C.POINTER(C.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def status_name(s: int) -> str:
    return load().dinfer_status_str(int(s)).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        detail = load().dinfer_last_error().decode()
        raise DinferError(status, what, detail)


def ptr(t) -> int:
    """Device (or host) address of a torch tensor, or 0 for None."""
    return 0 if t is None else int(t.data_ptr())


def stream_handle(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def pack_linear(W, stream=None):
    """dinfer_pack_linear on a contiguous torch device tensor W [N][K] or
    [E][N][K] (f32 or bf16); returns a new tensor of the same shape and dtype
    holding the packed layout the projection kernels read."""
    import torch
    lib = load()
    assert W.is_contiguous() and W.dtype in (torch.float32, torch.bfloat16)
    assert W.dim() in (2, 3)
    out = torch.empty_like(W)
    n_mats = W.shape[0] if W.dim() == 3 else 1
    check(lib.dinfer_pack_linear(ptr(W), ptr(out), n_mats, W.shape[-2], W.shape[-1],
                                 F32 if W.dtype == torch.float32 else BF16,
                                 stream_handle(stream)), "dinfer_pack_linear")
    return out


def linear(A, W, out, stream=None) -> int:
    """dinfer_linear on torch device tensors; returns the split count.
    A fp32 [M][K], W [N][K] (f32 or bf16) packed by pack_linear, out fp32 with
    at least dinfer_linear_out_elems(M, N, K, dtype) elements."""
    import torch
    lib = load()
    assert A.dtype == torch.float32
    M, K = A.shape
    N = W.shape[0]
    dt = F32 if W.dtype == torch.float32 else BF16
    need = lib.dinfer_linear_out_elems(M, N, K, dt)
    if need == 0 or out.numel() < need:
        raise DinferError(E_ARG, "dinfer_linear", f"out needs {need} floats")
    s = C.c_int32()
    check(lib.dinfer_linear(ptr(A), ptr(W), ptr(out), M, N, K, dt, C.byref(s),
                            stream_handle(stream)), "dinfer_linear")
    return int(s.value)


def vocab_stats(logits, plant_id, plant_bias, mask_id, out, scratch, stream=None):
    """dinfer_vocab_stats on torch device tensors; `out` holds argmax, conf, lse,
    topk_id, topk_p tensors."""
    lib = load()
    rows, vocab = logits.shape
    st = lib.dinfer_vocab_stats(ptr(logits), rows, vocab, ptr(plant_id), ptr(plant_bias), mask_id,
                                ptr(out["argmax"]), ptr(out["conf"]), ptr(out["lse"]),
                                ptr(out["topk_id"]), ptr(out["topk_p"]), ptr(scratch),
                                scratch.numel() * scratch.element_size(), stream_handle(stream))
    check(st, "dinfer_vocab_stats")


def vocab_stats_noalloc(logits, plant_id, plant_bias, mask_id, out, stream=None):
    """dinfer_vocab_stats_noalloc (no scratch argument, no allocation)."""
    lib = load()
    rows, vocab = logits.shape
    st = lib.dinfer_vocab_stats_noalloc(ptr(logits), rows, vocab, ptr(plant_id), ptr(plant_bias),
                                        mask_id, ptr(out["argmax"]), ptr(out["conf"]),
                                        ptr(out["lse"]), ptr(out["topk_id"]), ptr(out["topk_p"]),
                                        stream_handle(stream))
    check(st, "dinfer_vocab_stats_noalloc")


class DeficitScheduler:
    """dinfer_sched_* (deficit token-budget admission of whole refreshes):
    owns the host object; round() marshals one round's per-slot rows."""

    def __init__(self, budget: int, n_slots: int):
        lib = load()
        h = C.c_void_p()
        check(lib.dinfer_sched_create(int(budget), int(n_slots), C.byref(h)), "dinfer_sched_create")
        self._lib, self._h, self.n = lib, h, int(n_slots)

    def round(self, decode_rows, refresh_rows):
        n = self.n
        assert len(decode_rows) == n and len(refresh_rows) == n
        dec = (C.c_int32 * n)(*[int(x) for x in decode_rows])
        ref = (C.c_int32 * n)(*[int(x) for x in refresh_rows])
        adm = (C.c_uint8 * n)()
        deficit = C.c_int64()
        check(self._lib.dinfer_sched_round(self._h, dec, ref, adm, C.byref(deficit)),
              "dinfer_sched_round")
        return [int(adm[i]) for i in range(n)], int(deficit.value)

    def close(self):
        if self._h:
            self._lib.dinfer_sched_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
