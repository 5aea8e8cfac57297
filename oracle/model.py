"""Oracle model: the bidirectional transformer forward over a set of rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).  fp64 NumPy throughout.

Architecture readings (the pages name only a bidirectional transformer, dense or
MoE; the workloads name RoPE, RMSNorm and SwiGLU): pre-norm blocks, RMSNorm
x / sqrt(mean(x^2) + eps) * g, rotate-half RoPE pairing (j, j + hd/2) with
inverse frequencies theta^(-2j/hd) on absolute positions, attention scale
1/sqrt(hd), no biases, untied LM head after a final RMSNorm, SiLU(x) = x*sigmoid(x),
Linear weights stored [out][in].
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):          # torch tensor (bf16 upcasts exactly)
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _round_bf16(x):
    """x rounded to the nearest bfloat16 (ties to even), returned as fp64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def rmsnorm(x, g, eps):
    """RMSNorm over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """Rotary embedding of x [n, H, hd] at integer positions pos [n].

    Pair (j, j + hd/2) is rotated by the angle pos * theta^(-2j/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, K, V, scale):
    """Bidirectional softmax attention, no mask: q [n,H,hd], K,V [L,H,hd] -> [n,H,hd].

    Every query sees every cached key ([N] section on the bottlenecks: attention
    is bidirectional, so there is no causal mask).
    """
    # per head: S = q_h K_h^T (a batched matrix product), row softmax, P V_h
    s = np.matmul(q.transpose(1, 0, 2), K.transpose(1, 2, 0)) * scale      # [H, n, L]
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.matmul(p, V.transpose(1, 0, 2)).transpose(1, 0, 2)          # [n, H, hd]


def silu(x):
    return x / (1.0 + np.exp(-x))


def swiglu(f, w_gate_up, w_down):
    """SwiGLU FFN: (silu(f Wg^T) * (f Wu^T)) Wd^T with w_gate_up rows [gate | up]."""
    F = w_gate_up.shape[0] // 2
    gu = f @ w_gate_up.T
    return (silu(gu[:, :F]) * gu[:, F:]) @ w_down.T


def moe_ffn(f, router, bias, exp_gate_up, exp_down, shared_gate_up, shared_down, top_k):
    """MoE FFN ([A]: MoE model; [T]: expert activations per block).

    Router logits r = f W_r^T + bias; gates = softmax over all experts; the
    top_k experts by (logit desc, expert id asc) are kept and their gates
    renormalised to sum 1; output = sum of gated expert SwiGLUs + shared SwiGLU.
    """
    r = f @ router.T
    if bias is not None:
        r = r + bias[None, :]
    g = np.exp(r - r.max(axis=-1, keepdims=True))
    g = g / g.sum(axis=-1, keepdims=True)
    out = np.zeros_like(f)
    order = np.argsort(-r, axis=-1, kind="stable")[:, :top_k]     # ties -> lower id first
    gsel = np.take_along_axis(g, order, axis=-1)
    gsel = gsel / gsel.sum(axis=-1, keepdims=True)
    for e in np.unique(order):
        rows, slot = np.nonzero(order == e)
        out[rows] += gsel[rows, slot][:, None] * swiglu(f[rows], exp_gate_up[e], exp_down[e])
    if shared_gate_up is not None:
        out = out + swiglu(f, shared_gate_up, shared_down)
    return out, order, gsel


def router_logits(f, router, bias):
    """Router logits f W_r^T + bias of every row (reported alongside routing)."""
    r = f @ router.T
    return r if bias is None else r + bias[None, :]


def route_margin(f, router, bias, top_k):
    """Per row, the router-logit gap between the top_k-th and the next expert:
    how far the row's expert choice is from flipping.  Reported, not used by
    the method; inf when every expert is selected."""
    r = router_logits(f, router, bias)
    if top_k >= r.shape[1]:
        return np.full(r.shape[0], np.inf)
    s = -np.sort(-r, axis=-1)
    return s[:, top_k - 1] - s[:, top_k]


class OracleModel:
    """fp64 copy of the weights plus one request's KV cache.

    cache_k[l], cache_v[l]: [L, H, hd], K stored after RoPE.
    """

    def __init__(self, mcfg, weights, layers=None):
        self.m = mcfg
        self.n_layers = mcfg.n_layers
        self.layer_ids = list(range(mcfg.n_layers)) if layers is None else list(layers)
        emb = weights.get("tok_emb")              # gathered row by row, upcast on use
        if hasattr(emb, "detach"):
            emb = emb.detach().cpu()
        self.tok_emb = emb
        self.final_norm = _f64(weights["final_norm"])
        self.lm_head = _f64(weights.get("lm_head"))
        self.layers = {}
        for li in self.layer_ids:
            self.layers[li] = {k: _f64(v) for k, v in weights["layers"][li].items()}

    # --- embeddings -------------------------------------------------------
    def embed(self, ids):
        return _f64(self.tok_emb[np.asarray(ids, dtype=np.int64)])

    # --- forward ----------------------------------------------------------
    def new_cache(self, L, kv_round=None):
        """Zeroed K, V of L positions per layer.  kv_round="bf16" stores every
        cached K and V rounded to bfloat16 (nearest even), the storage of a
        bf16 model's cache; None keeps them in fp64."""
        m = self.m
        z = lambda: np.zeros((L, m.n_heads, m.head_dim))  # noqa: E731
        return {"k": {li: z() for li in self.layer_ids}, "v": {li: z() for li in self.layer_ids},
                "round": kv_round}

    def forward_rows(self, cache, pos, e, L, router_bias=None, record=None, rope_offset=0):
        """Run every layer over the rows at positions `pos` with inputs e [n, d].

        Per layer ([N] vicinity-refresh section): the rows' fresh K and V are
        written into the cache at their positions first, then the rows attend
        over all L cached positions -- fresh inside the row set, as left by the
        last write elsewhere.  Returns the final hidden states [n, d].
        router_bias: MoE only, [n_layers][E] for the current block.
        rope_offset: added to the positions for the rotary angles only (0 in the
        method; a check of the relative-position property uses it).
        """
        m = self.m
        H, hd, d = m.n_heads, m.head_dim, m.d_model
        n = len(pos)
        pos = np.asarray(pos, dtype=np.int64)
        h = np.array(e, dtype=np.float64)
        for li in self.layer_ids:
            W = self.layers[li]
            a = rmsnorm(h, W["attn_norm"], m.rms_eps)
            qkv = a @ W["wqkv"].T
            q = qkv[:, :d].reshape(n, H, hd)
            k = qkv[:, d:2 * d].reshape(n, H, hd)
            v = qkv[:, 2 * d:].reshape(n, H, hd)
            q = rope(q, pos + rope_offset, m.rope_theta)
            k = rope(k, pos + rope_offset, m.rope_theta)
            if cache.get("round") == "bf16":
                k, v = _round_bf16(k), _round_bf16(v)
            cache["k"][li][pos] = k
            cache["v"][li][pos] = v
            o = attention(q, cache["k"][li][:L], cache["v"][li][:L], 1.0 / np.sqrt(hd))
            h = h + o.reshape(n, d) @ W["wo"].T
            f = rmsnorm(h, W["ffn_norm"], m.rms_eps)
            if m.is_moe:
                rb = None if router_bias is None else np.asarray(router_bias[li], dtype=np.float64)
                y, order, gsel = moe_ffn(f, W["router"], rb, W["exp_gate_up"], W["exp_down"],
                                         W["shared_gate_up"], W["shared_down"], m.top_k)
                if record is not None:
                    record.setdefault("experts", {})[li] = order
                    record.setdefault("gates", {})[li] = gsel
                    record.setdefault("route_margin", {})[li] = route_margin(
                        f, W["router"], rb, m.top_k)
                    record.setdefault("router_logits", {})[li] = router_logits(f, W["router"], rb)
                h = h + y
            else:
                h = h + swiglu(f, W["w_gate_up"], W["w_down"])
        return h

    def logits(self, h):
        """LM head over final hidden states: RMSNorm(h) * g_f @ W_lm^T (fp64)."""
        return rmsnorm(h, self.final_norm, self.m.rms_eps) @ self.lm_head.T
