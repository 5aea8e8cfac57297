"""Seeded synthetic inputs: weights, requests, planting, router bias, logits.

Every tensor comes from its own torch.Generator, seeded from (workload seed,
tensor tag, layer) through SHA-256, so a tensor does not depend on which other
tensors were drawn before it.  Generators run on the device the caller names:
on "cpu" for host-only checks, on "cuda" for GPU runs (the oracle then takes a
host copy of the very same tensors).  This module holds none of the method's
arithmetic; the random numbers the method consumes (planting, router
preference) are drawn here and handed to both sides as inputs.

Weight distribution: every matrix and the embedding table N(0, 0.02); norm
gains 1; the MoE router N(0, 1/d) so router logits of a unit-RMS input are
about N(0, 1).  bf16 tensors are drawn in fp32 and rounded to nearest-even.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

from .configs import ModelCfg, WorkloadCfg

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DT[name]


def sub_seed(seed: int, tag: str, index: int = 0) -> int:
    h = hashlib.sha256(f"{seed}/{tag}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int, tag: str, index: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(sub_seed(seed, tag, index))
    return g


def normal(shape, std, dtype, device, seed, tag, index=0) -> torch.Tensor:
    g = _gen(device, seed, tag, index)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def make_weights(m: ModelCfg, seed: int, device="cpu", layers=None, with_embed=True,
                 with_head=True) -> dict:
    """Weights as row-major tensors (Linear storage [out][in]); the engine packs
    the projection matrices into the library's own layout.

    tok_emb [V][d], final_norm [d], lm_head [V][d]; per layer: attn_norm [d],
    wqkv [3d][d] (rows q | k | v, head-major inside each), wo [d][d],
    ffn_norm [d], then dense: w_gate_up [2F][d] (rows gate | up), w_down [d][F];
    or MoE: router [E][d], exp_gate_up [E][2Fe][d], exp_down [E][d][Fe],
    shared_gate_up [2Fs][d], shared_down [d][Fs].
    `layers` restricts which layer indices are drawn (others are None).
    """
    dt = torch_dtype(m.dtype)
    d, V = m.d_model, m.vocab
    w = {}
    if with_embed:
        w["tok_emb"] = normal((V, d), 0.02, dt, device, seed, "tok_emb")
    w["final_norm"] = torch.ones(d, dtype=dt, device=device)
    if with_head:
        w["lm_head"] = normal((V, d), 0.02, dt, device, seed, "lm_head")
    sel = range(m.n_layers) if layers is None else layers
    w["layers"] = [None] * m.n_layers
    for li in sel:
        L = {
            "attn_norm": torch.ones(d, dtype=dt, device=device),
            "wqkv": normal((3 * d, d), 0.02, dt, device, seed, "wqkv", li),
            "wo": normal((d, d), 0.02, dt, device, seed, "wo", li),
            "ffn_norm": torch.ones(d, dtype=dt, device=device),
        }
        if m.is_moe:
            E, Fe, Fs = m.n_experts, m.expert_ffn, m.shared_ffn
            L["router"] = normal((E, d), 1.0 / np.sqrt(d), dt, device, seed, "router", li)
            L["exp_gate_up"] = normal((E, 2 * Fe, d), 0.02, dt, device, seed, "exp_gate_up", li)
            L["exp_down"] = normal((E, d, Fe), 0.02, dt, device, seed, "exp_down", li)
            L["shared_gate_up"] = normal((2 * Fs, d), 0.02, dt, device, seed, "shared_gate_up", li)
            L["shared_down"] = normal((d, Fs), 0.02, dt, device, seed, "shared_down", li)
        else:
            F = m.ffn_dim
            L["w_gate_up"] = normal((2 * F, d), 0.02, dt, device, seed, "w_gate_up", li)
            L["w_down"] = normal((d, F), 0.02, dt, device, seed, "w_down", li)
        w["layers"][li] = L
    return w


def make_requests(wc: WorkloadCfg, seed=None) -> dict:
    """Requests of a workload, as host int32/float32 tensors.

    tokens [batch][max_len]: prompt ids U{0..V-2}, then gen_len MASK positions;
      positions past a request's length hold MASK and are never read.
    prompt_len, gen_len [batch] int32.
    plant_id [batch][max_len] int32: -1, or the planted target id of a generated
      position (planted with the request's probability p, target U{0..V-2}).
    plant_bias [batch] float32; plant_prob [batch] float32 (informational).
    router_bias [batch][n_layers][n_blocks][E] float32 for MoE, else None:
      per (request, layer, block) a seeded set of distinct preferred experts
      gets +router_pref_bias.
    """
    seed = wc.seed if seed is None else seed
    m = wc.model
    Bt = wc.batch
    g = torch.Generator(device="cpu")
    g.manual_seed(sub_seed(seed, "requests"))
    lo, hi = wc.prompt_len
    P = torch.randint(lo, hi + 1, (Bt,), generator=g, dtype=torch.int64)
    G = wc.gen_len
    max_len = int(P.max().item()) + G
    tokens = torch.full((Bt, max_len), m.mask_id, dtype=torch.int32)
    plant_id = torch.full((Bt, max_len), -1, dtype=torch.int32)
    plo, phi = wc.plant_prob
    prob = plo + (phi - plo) * torch.rand(Bt, generator=g, dtype=torch.float64)
    for r in range(Bt):
        pr = int(P[r])
        tokens[r, :pr] = torch.randint(0, m.vocab - 1, (pr,), generator=g, dtype=torch.int64).to(torch.int32)
        planted = torch.rand(G, generator=g, dtype=torch.float64) < prob[r]
        target = torch.randint(0, m.vocab - 1, (G,), generator=g, dtype=torch.int64).to(torch.int32)
        plant_id[r, pr:pr + G] = torch.where(planted, target, torch.full_like(target, -1))
    out = {
        "tokens": tokens,
        "prompt_len": P.to(torch.int32),
        "gen_len": torch.full((Bt,), G, dtype=torch.int32),
        "plant_id": plant_id,
        "plant_bias": torch.full((Bt,), wc.plant_bias, dtype=torch.float32),
        "plant_prob": prob.to(torch.float32),
        "router_bias": None,
    }
    if m.is_moe:
        nb = G // wc.decode.block_len
        rb = torch.zeros((Bt, m.n_layers, nb, m.n_experts), dtype=torch.float32)
        for r in range(Bt):
            for li in range(m.n_layers):
                for b in range(nb):
                    perm = torch.randperm(m.n_experts, generator=g)[: wc.router_pref_count]
                    rb[r, li, b, perm] = wc.router_pref_bias
        out["router_bias"] = rb
    return out


def make_logits(rows: int, vocab: int, seed: int, tag="logits", std=1.28, ties=0,
                device="cpu") -> torch.Tensor:
    """fp32 logits N(0, std) with optional forced exact ties at each row's maximum.

    With ties=k>0, k extra positions in every row are set equal to the row max
    (a tie on the value, so the lowest id must win).
    """
    g = _gen(device, seed, tag)
    z = torch.randn(rows, vocab, generator=g, device=device, dtype=torch.float32) * std
    if ties:
        gi = _gen("cpu", seed, tag + "/ties")
        for r in range(rows):
            mx = z[r].max()
            idx = torch.randint(0, vocab, (ties,), generator=gi)
            z[r, idx.to(z.device)] = mx
    return z
