"""Engine: one libdinfer context over torch-owned device memory.

PyTorch only allocates device memory and provides the stream; every step of
the method runs in the HIP library behind the C ABI.
"""
from __future__ import annotations

import ctypes as C
import time

import torch

from . import binding as B


def _model_struct(m) -> B.ModelCfg:
    s = B.ModelCfg()
    for f in ("n_layers", "d_model", "n_heads", "head_dim", "ffn_dim", "vocab", "mask_id",
              "n_experts", "top_k", "expert_ffn", "shared_ffn"):
        setattr(s, f, int(getattr(m, f)))
    s.rope_theta = float(m.rope_theta)
    s.rms_eps = float(m.rms_eps)
    s.dtype = B.F32 if m.dtype == "f32" else B.BF16
    return s


def _decode_struct(d, graph_unroll: int) -> B.DecodeCfg:
    s = B.DecodeCfg()
    s.block_len = int(d.block_len)
    s.vicinity_w = int(d.vicinity_w)
    s.tau = float(d.tau)
    s.credit_weight = float(d.credit_weight)
    s.credit_decay = float(d.credit_decay)
    s.credit_kappa = float(d.credit_kappa)
    s.smooth_alpha = float(d.smooth_alpha)
    s.smooth_topk = int(d.smooth_topk)
    s.hierarchical = int(bool(d.hierarchical))
    s.graph_unroll = int(graph_unroll)
    s.eos_id = int(getattr(d, "eos_id", -1))
    return s


class Engine:
    """A denoising-step context.

    weights: dict of row-major device tensors (synth.make_weights layout).  The
    projection matrices are packed once, at construction, into the layout the
    library reads (dinfer_pack_linear); the engine holds the packed copies.
    """

    PACKED = ("wqkv", "wo", "w_gate_up", "w_down", "exp_gate_up", "exp_down",
              "shared_gate_up", "shared_down")

    def __init__(self, model_cfg, decode_cfg, weights, max_batch, max_len, graph_unroll=0,
                 stream=None, keep_logits=False):
        self.lib = B.load()
        self.m = model_cfg
        self.d = decode_cfg
        self.max_batch = int(max_batch)
        self.max_len = int(max_len)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._mc = _model_struct(model_cfg)
        self._dc = _decode_struct(decode_cfg, graph_unroll)
        self._weights = weights
        nl = model_cfg.n_layers
        arr = C.c_void_p * nl
        # packed projection weights, per layer (None where the layer is absent)
        self.packed_layers = [
            {k: B.pack_linear(L[k], self.stream) for k in self.PACKED if L.get(k) is not None}
            if L else None for L in weights["layers"]]
        lm = weights.get("lm_head")
        self.packed_lm_head = None if lm is None else B.pack_linear(lm, self.stream)

        def per_layer(key):
            src = self.packed_layers if key in self.PACKED else weights["layers"]
            vals = [B.ptr(src[i].get(key)) if src[i] else 0 for i in range(nl)]
            return arr(*vals)

        keys = ["attn_norm", "wqkv", "wo", "ffn_norm"]
        if int(model_cfg.n_experts) > 0:
            keys += ["router", "exp_gate_up", "exp_down", "shared_gate_up", "shared_down"]
        else:
            keys += ["w_gate_up", "w_down"]
        self._arrays = {k: per_layer(k) for k in keys}
        w = B.Weights()
        w.tok_emb = B.ptr(weights["tok_emb"])
        w.final_norm = B.ptr(weights["final_norm"])
        w.lm_head = B.ptr(self.packed_lm_head)
        for k, a in self._arrays.items():
            setattr(w, k, C.cast(a, B._PP))
        self._w = w
        nbytes = self.lib.dinfer_workspace_bytes(C.byref(self._mc), C.byref(self._dc),
                                                 self.max_batch, self.max_len)
        if nbytes == 0:
            raise B.DinferError(B.E_ARG, "dinfer_workspace_bytes", "configuration rejected")
        self.ws_bytes = int(nbytes)
        raw = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device="cuda")
        off = (-raw.data_ptr()) % 256
        self._raw = raw
        self.workspace = raw[off: off + self.ws_bytes]
        ctx = C.c_void_p()
        st = self.lib.dinfer_step_init(C.byref(self._mc), C.byref(self._dc), C.byref(self._w),
                                       self.max_batch, self.max_len, B.ptr(self.workspace),
                                       self.ws_bytes, B.stream_handle(self.stream), C.byref(ctx))
        B.check(st, "dinfer_step_init")
        self.ctx = ctx
        self.batch = 0
        self.keep_logits(keep_logits)

    def expert_offload(self, slots, interval=0):
        """dinfer_expert_offload: every expert of every layer in a pinned host
        store (copies of the packed expert weights), `slots` experts per layer
        also in an HBM slot buffer; placement after each block-start refresh
        and every `interval` steps (0: block starts only)."""
        import torch
        nl = self.m.n_layers
        gu = [torch.empty(L["exp_gate_up"].shape, dtype=L["exp_gate_up"].dtype, pin_memory=True)
              for L in self.packed_layers]
        dn = [torch.empty(L["exp_down"].shape, dtype=L["exp_down"].dtype, pin_memory=True)
              for L in self.packed_layers]
        for i, L in enumerate(self.packed_layers):
            gu[i].copy_(L["exp_gate_up"])
            dn[i].copy_(L["exp_down"])
        torch.cuda.synchronize()
        one = self.lib.dinfer_expert_slot_bytes(C.byref(self._mc))
        nbytes = nl * int(slots) * one
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        off = (-raw.data_ptr()) % 256
        arr = C.c_void_p * nl
        self._expert_store = (gu, dn, raw, arr(*[B.ptr(t) for t in gu]), arr(*[B.ptr(t) for t in dn]))
        B.check(self.lib.dinfer_expert_offload(self.ctx, self._expert_store[3],
                                               self._expert_store[4], int(slots), int(interval),
                                               raw.data_ptr() + off, nbytes),
                "dinfer_expert_offload")

    def expert_place(self):
        B.check(self.lib.dinfer_expert_place(self.ctx), "dinfer_expert_place")

    def expert_report(self, reset=False):
        r = B.ExpertCacheStats()
        B.check(self.lib.dinfer_expert_cache_report(self.ctx, C.byref(r), 1 if reset else 0),
                "dinfer_expert_cache_report")
        return {k: getattr(r, k) for k, _ in B.ExpertCacheStats._fields_}

    def set_activation_precision(self, step_mask=0, refresh_mask=0):
        """dinfer_set_activation_precision: bit i (0 QKV, 1 O, 2 gate|up, 3 down)
        = that projection takes bf16 activations alone instead of hi + lo; bit
        4 = the attention's probabilities likewise in its P V product."""
        B.check(self.lib.dinfer_set_activation_precision(self.ctx, int(step_mask),
                                                         int(refresh_mask)),
                "dinfer_set_activation_precision")

    def keep_logits(self, on=True):
        """dinfer_keep_logits: also store the block rows' fp32 logits (inspection)."""
        B.check(self.lib.dinfer_keep_logits(self.ctx, 1 if on else 0), "dinfer_keep_logits")

    # -- calls ---------------------------------------------------------------
    def set_batch(self, tokens, prompt_len, gen_len, plant_id=None, plant_bias=None,
                  router_bias=None):
        """tokens: device int32 [batch][max_len] (updated in place).

        router_bias (MoE): device float32 [batch][n_layers][n_blocks][E].
        """
        assert tokens.dtype == torch.int32 and tokens.is_cuda and tokens.is_contiguous()
        if router_bias is not None:
            assert router_bias.dtype == torch.float32 and router_bias.is_cuda
            assert router_bias.is_contiguous() and router_bias.dim() == 4
            assert router_bias.shape[0] == tokens.shape[0]
        assert tokens.shape[1] == self.max_len
        batch = tokens.shape[0]
        P = (C.c_int32 * batch)(*[int(x) for x in prompt_len])
        G = (C.c_int32 * batch)(*[int(x) for x in gen_len])
        self._batch_refs = (tokens, plant_id, plant_bias, router_bias)
        st = self.lib.dinfer_set_batch(self.ctx, batch, B.ptr(tokens), P, G, B.ptr(plant_id),
                                       B.ptr(plant_bias), B.ptr(router_bias))
        B.check(st, "dinfer_set_batch")
        self.batch = batch
        self.tokens = tokens

    def refresh_kv(self, mask=None):
        m = None if mask is None else (C.c_uint8 * self.batch)(*[1 if x else 0 for x in mask])
        B.check(self.lib.dinfer_refresh_kv(self.ctx, m), "dinfer_refresh_kv")

    def denoise_step(self):
        B.check(self.lib.dinfer_denoise_step(self.ctx), "dinfer_denoise_step")

    def commit(self):
        B.check(self.lib.dinfer_commit(self.ctx), "dinfer_commit")

    def advance_blocks(self):
        need = (C.c_uint8 * max(self.batch, 1))()
        unf = C.c_int32()
        B.check(self.lib.dinfer_advance_blocks(self.ctx, need, C.byref(unf)),
                "dinfer_advance_blocks")
        return [bool(need[i]) for i in range(self.batch)], int(unf.value)

    def step_graph(self, n_steps):
        B.check(self.lib.dinfer_step_graph(self.ctx, int(n_steps)), "dinfer_step_graph")

    def run_to_completion(self, max_steps=1 << 30):
        s = B.RunStats()
        B.check(self.lib.dinfer_run_to_completion(self.ctx, int(max_steps), C.byref(s)),
                "dinfer_run_to_completion")
        return {"steps": s.steps, "refreshes": s.refreshes, "committed": s.committed,
                "wall_ms": s.wall_ms, "refresh_ms": s.refresh_ms}

    def refill(self, slot, prompt_len, gen_len):
        B.check(self.lib.dinfer_refill(self.ctx, int(slot), int(prompt_len), int(gen_len)),
                "dinfer_refill")

    def finished(self):
        f = (C.c_uint8 * max(self.batch, 1))()
        B.check(self.lib.dinfer_finished(self.ctx, f), "dinfer_finished")
        return [bool(f[i]) for i in range(self.batch)]

    def pending_rows(self):
        """dinfer_pending_rows: per slot, rows of its next step (decoding) and
        of a whole refresh (waiting)."""
        n = max(self.batch, 1)
        dec, ref = (C.c_int32 * n)(), (C.c_int32 * n)()
        B.check(self.lib.dinfer_pending_rows(self.ctx, dec, ref), "dinfer_pending_rows")
        return [int(dec[i]) for i in range(self.batch)], [int(ref[i]) for i in range(self.batch)]

    def run_queue(self, queue, max_steps=1 << 30, token_budget=None):
        """Continuous batching over the bound batch (set_batch holds the first
        requests): whenever a slot finishes, its response is taken and the next
        queued request is written into the slot's rows of the bound arrays and
        restarted (dinfer_refill).  queue: list of dicts with "tokens" (int32
        [max_len] row: prompt ids then mask_id), "prompt_len", "gen_len",
        "plant_id" (int32 [max_len] row) and "plant_bias" (float).

        Each round runs graph_unroll steps (one without graphs).  Without a
        token_budget every slot that waits for a refresh (a new request or a
        block start) is refreshed before the round; with one, the deficit
        scheduler (dinfer_sched_round, token_budget rows per step) decides
        which waiting slots are refreshed, and the others wait, not decoding,
        for a later round.

        Returns {"outputs": [(request index, tokens row copy)], "finish_step":
        {request index: steps run when it finished}, "finish_time": {request
        index: time.perf_counter() when it was taken}, "round_s": wall time of
        each round (its refreshes and steps), "steps", "refreshes",
        "rounds": [(decode rows, refresh rows, admitted, counter)] with a
        budget}; request index i >= batch is queue[i - batch]."""
        tokens, plant_id, plant_bias, router_bias = self._batch_refs
        assert router_bias is None, "refill of MoE router bias rows is the caller's"
        U = int(self._dc.graph_unroll)
        per_round = max(U, 1)
        sched = None
        if token_budget is not None:   # per round; the library caps budgets at 2^62 rows
            sched = B.DeficitScheduler(min(int(token_budget) * per_round, 1 << 62), self.batch)
        owner = list(range(self.batch))          # request index held by each slot
        nxt = self.batch
        outputs, finish_step, finish_time, log = [], {}, {}, []
        steps, refreshes = 0, 0
        need = [True] * self.batch               # set_batch: every slot waits
        round_end = [time.perf_counter()]
        while True:
            if sched is None:
                admit = need
            else:
                dec, ref = self.pending_rows()
                dec = [x * per_round for x in dec]
                admit, deficit = sched.round(dec, ref)
                log.append((dec, ref, admit, deficit))
            if any(admit):
                self.refresh_kv(admit)
                refreshes += sum(bool(a) for a in admit)
            if U > 0:
                self.step_graph(U)
            else:
                self.denoise_step()
                self.commit()
            steps += per_round
            if steps > max_steps:
                raise RuntimeError("run_queue: max_steps reached")
            self.advance_blocks()
            round_end.append(time.perf_counter())  # advance_blocks waited for the round
            for sl, done in enumerate(self.finished()):
                if not done or owner[sl] is None:
                    continue
                outputs.append((owner[sl], tokens[sl].clone()))
                finish_step[owner[sl]] = steps
                finish_time[owner[sl]] = time.perf_counter()   # advance_blocks waited
                if nxt - self.batch < len(queue):
                    q = queue[nxt - self.batch]
                    tokens[sl].copy_(q["tokens"])
                    if plant_id is not None:
                        plant_id[sl].copy_(q["plant_id"])
                    if plant_bias is not None:
                        plant_bias[sl] = float(q["plant_bias"])
                    self.refill(sl, q["prompt_len"], q["gen_len"])
                    owner[sl] = nxt
                    nxt += 1
                else:
                    owner[sl] = None
            need, unfinished = self.advance_blocks()
            if unfinished == 0:
                break
        if sched is not None:
            sched.close()
        return {"outputs": outputs, "finish_step": finish_step, "finish_time": finish_time,
                "round_s": [b - a for a, b in zip(round_end, round_end[1:])], "steps": steps,
                "refreshes": refreshes, "rounds": log}

    # -- state views -----------------------------------------------------------
    def view(self):
        """Torch views (no copies) of the context's state buffers."""
        v = B.StepView()
        B.check(self.lib.dinfer_get_step_view(self.ctx, C.byref(v)), "dinfer_get_step_view")
        base = self.workspace.data_ptr()
        R = self.batch * v.block_len
        K = v.topk

        def t(addr, n, dtype, shape):
            off = addr - base
            nb = n * torch.tensor([], dtype=dtype).element_size()
            return self.workspace[off: off + nb].view(dtype).view(*shape)

        es = 4 if self.m.dtype == "f32" else 2
        kvdt = torch.float32 if es == 4 else torch.bfloat16
        Lp = v.kv_len
        kv_n = self.m.n_layers * self.max_batch * self.m.n_heads * Lp * self.m.head_dim
        kv_shape = (self.m.n_layers, self.max_batch, self.m.n_heads, Lp, self.m.head_dim)
        # V: transposed tiles of 32 positions, [..][H][Lp/32][hd][32]
        vt_shape = (self.m.n_layers, self.max_batch, self.m.n_heads, Lp // 32, self.m.head_dim, 32)
        out = {}
        if v.moe_top_k > 0:
            # the last pass's rows; the widest pass is a refresh of max_batch * max_len rows
            n = self.max_batch * self.max_len
            out["moe_sel"] = t(v.moe_sel, n * v.moe_top_k, torch.int32, (n, v.moe_top_k))
            out["moe_gate"] = t(v.moe_gate, n * v.moe_top_k, torch.float32, (n, v.moe_top_k))
            out["moe_logits"] = t(v.moe_logits, n * v.moe_experts, torch.float32,
                                  (n, v.moe_experts))
        n = self.max_batch * self.max_len
        out["ffn_in"] = t(v.ffn_in, n * self.m.d_model, torch.float32, (n, self.m.d_model))
        return out | {
            "logits": t(v.logits, R * v.vocab, torch.float32, (R, v.vocab)),
            "argmax": t(v.argmax, R, torch.int32, (R,)),
            "conf": t(v.conf, R, torch.float32, (R,)),
            "lse": t(v.lse, R, torch.float32, (R,)),
            "topk_id": t(v.topk_id, R * K, torch.int32, (R, K)),
            "topk_p": t(v.topk_p, R * K, torch.float32, (R, K)),
            "credit": t(v.credit, R, torch.float32, (R,)),
            "tracked": t(v.tracked, R, torch.int32, (R,)),
            "smooth_id": t(v.smooth_id, R * K, torch.int32, (R, K)),
            "smooth_p": t(v.smooth_p, R * K, torch.float32, (R, K)),
            "smooth_valid": t(v.smooth_valid, R, torch.uint8, (R,)),
            "commit_mask": t(v.commit_mask, R, torch.uint8, (R,)),
            "block_done": t(v.block_done, self.batch, torch.int32, (self.batch,)),
            "step_count": t(v.step_count, self.batch, torch.int32, (self.batch,)),
            "commit_count": t(v.commit_count, self.batch, torch.int32, (self.batch,)),
            "decode_stats": t(v.decode_stats, self.batch * v.decode_stat_words, torch.int32,
                              (self.batch, v.decode_stat_words)),
            "kv_k": t(v.kv_k, kv_n, kvdt, kv_shape),
            "kv_v": t(v.kv_v, kv_n, kvdt, vt_shape),
        }

    def close(self):
        if getattr(self, "ctx", None) is not None and self.ctx.value:
            self.lib.dinfer_destroy(self.ctx)
            self.ctx = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
