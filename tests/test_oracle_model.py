"""Pins of the oracle's model forward against closed forms, library special cases
and invariants of the method (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.model import OracleModel, attention, moe_ffn, rmsnorm, rope, swiglu

RNG = np.random.default_rng(1234)


def test_rmsnorm_constant_row_closed_form():
    # A constant row c has mean square c^2, so RMSNorm gives c / sqrt(c^2 + eps) * g.
    for c in [0.5, -3.0, 1e-3]:
        x = np.full((1, 16), c)
        g = np.linspace(0.5, 2.0, 16)
        eps = 1e-5
        assert np.allclose(rmsnorm(x, g, eps), c / np.sqrt(c * c + eps) * g, rtol=1e-14)


def test_rope_matches_complex_rotation():
    # Rotate-half RoPE is multiplication of z_j = x_j + i x_{j+hd/2} by exp(i pos theta^(-2j/hd)).
    n, H, hd, theta = 7, 3, 16, 10000.0
    x = RNG.standard_normal((n, H, hd))
    pos = np.array([0, 1, 5, 100, 2047, 9000, 31])
    half = hd // 2
    z = x[..., :half] + 1j * x[..., half:]
    f = np.array([theta ** (-(2.0 * j) / hd) for j in range(half)])
    zr = z * np.exp(1j * pos[:, None, None] * f[None, None, :])
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.allclose(rope(x, pos, theta), want, atol=1e-12)


def test_rope_identity_at_zero_and_norm_and_relative():
    n, H, hd = 5, 2, 8
    x = RNG.standard_normal((n, H, hd))
    assert np.array_equal(rope(x, np.zeros(n, dtype=int), 10000.0), x)
    y = rope(x, np.arange(n) * 37, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # q(m).k(n) depends only on m - n
    q, k = RNG.standard_normal((1, 1, hd)), RNG.standard_normal((1, 1, hd))
    d1 = (rope(q, [10], 1e4) * rope(k, [3], 1e4)).sum()
    d2 = (rope(q, [1010], 1e4) * rope(k, [1003], 1e4)).sum()
    assert abs(d1 - d2) < 1e-10


def test_attention_matches_torch_sdpa():
    n, L, H, hd = 6, 11, 3, 8
    q, K, V = (RNG.standard_normal(s) for s in [(n, H, hd), (L, H, hd), (L, H, hd)])
    got = attention(q, K, V, 1.0 / np.sqrt(hd))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None]
    tv = torch.from_numpy(V).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0].permute(1, 0, 2).numpy()
    assert np.allclose(got, want, atol=1e-12)


def test_attention_single_key_returns_value_and_equal_keys_average():
    q = RNG.standard_normal((4, 2, 8))
    K = RNG.standard_normal((1, 2, 8))
    V = RNG.standard_normal((1, 2, 8))
    assert np.allclose(attention(q, K, V, 0.3), np.broadcast_to(V, (4, 2, 8)), atol=1e-15)
    K3 = np.repeat(K, 3, axis=0)
    V3 = RNG.standard_normal((3, 2, 8))
    assert np.allclose(attention(q, K3, V3, 0.3), np.broadcast_to(V3.mean(0), (4, 2, 8)), atol=1e-14)


def test_swiglu_matches_torch_silu():
    f = RNG.standard_normal((3, 8))
    wgu = RNG.standard_normal((10, 8))
    wd = RNG.standard_normal((8, 5))
    tf, tg, td = map(torch.from_numpy, (f, wgu, wd))
    gu = tf @ tg.T
    want = (torch.nn.functional.silu(gu[:, :5]) * gu[:, 5:]) @ td.T
    assert np.allclose(swiglu(f, wgu, wd), want.numpy(), atol=1e-12)


def _moe_bruteforce(f, router, bias, egu, ed, sgu, sd, k):
    out = np.zeros_like(f)
    for r in range(f.shape[0]):
        logits = [float(f[r] @ router[e] + bias[e]) for e in range(router.shape[0])]
        order = sorted(range(len(logits)), key=lambda e: (-logits[e], e))[:k]
        ex = [np.exp(logits[e] - max(logits)) for e in order]
        tot = sum(ex)
        for e, w in zip(order, ex):
            out[r] += (w / tot) * swiglu(f[r:r + 1], egu[e], ed[e])[0]
        out[r] += swiglu(f[r:r + 1], sgu, sd)[0]
    return out


def test_moe_matches_row_by_row_bruteforce_with_ties():
    E, d, Fe, k = 6, 8, 4, 3
    f = RNG.standard_normal((5, d))
    router = RNG.standard_normal((E, d))
    router[4] = router[1]             # exact tie between experts 1 and 4 on every row
    bias = np.zeros(E)
    bias[2] = 0.7
    egu = RNG.standard_normal((E, 2 * Fe, d))
    ed = RNG.standard_normal((E, d, Fe))
    sgu, sd = RNG.standard_normal((6, d)), RNG.standard_normal((d, 3))
    got, order, _ = moe_ffn(f, router, bias, egu, ed, sgu, sd, k)
    assert np.allclose(got, _moe_bruteforce(f, router, bias, egu, ed, sgu, sd, k), atol=1e-12)


def test_route_margin_is_gap_between_kept_and_first_dropped_expert():
    from oracle.model import route_margin
    E, d, k = 6, 8, 3
    f = RNG.standard_normal((7, d))
    router = RNG.standard_normal((E, d))
    bias = RNG.standard_normal(E)
    got = route_margin(f, router, bias, k)
    for r in range(f.shape[0]):
        logits = sorted((float(f[r] @ router[e] + bias[e]) for e in range(E)), reverse=True)
        assert abs(got[r] - (logits[k - 1] - logits[k])) < 1e-12
    # a tie at the boundary has margin 0; keeping every expert has no boundary
    router[4] = router[1]
    bias[:] = 0.0
    g2 = route_margin(f, router, bias, k)
    _, order, _ = moe_ffn(f, router, bias, RNG.standard_normal((E, 4, d)),
                          RNG.standard_normal((E, d, 2)), None, None, k)
    for r in range(f.shape[0]):
        if (1 in order[r]) != (4 in order[r]):
            assert g2[r] == 0.0
    assert np.all(np.isinf(route_margin(f, router, None, E)))


def test_moe_single_expert_is_dense_ffn():
    d, F = 8, 6
    f = RNG.standard_normal((4, d))
    egu = RNG.standard_normal((1, 2 * F, d))
    ed = RNG.standard_normal((1, d, F))
    got, _, _ = moe_ffn(f, RNG.standard_normal((1, d)), None, egu, ed, None, None, 1)
    assert np.allclose(got, swiglu(f, egu[0], ed[0]), atol=1e-13)


def _tiny_model(L_layers=2, d=32, H=2, hd=16, F=48, V=64, moe=False):
    m = synth.ModelCfg(n_layers=L_layers, d_model=d, n_heads=H, head_dim=hd,
                       ffn_dim=0 if moe else F, vocab=V, mask_id=V - 1, dtype="f32",
                       n_experts=4 if moe else 0, top_k=2 if moe else 0,
                       expert_ffn=12 if moe else 0, shared_ffn=16 if moe else 0)
    w = synth.make_weights(m, seed=7)
    # larger weights than N(0, 0.02) so that attention is far from uniform
    for L in w["layers"]:
        for key in ("wqkv", "wo", "w_gate_up", "w_down"):
            if key in L:
                L[key] = L[key] * 10
    return m, w


def test_single_position_layer_reduces_to_mlp_algebra():
    # With one cached position attention returns v, so a layer is
    # h + Wo Wv norm(h) followed by the FFN residual: no softmax involved.
    m, w = _tiny_model(L_layers=1)
    om = OracleModel(m, w)
    cache = om.new_cache(1)
    e = RNG.standard_normal((1, m.d_model))
    got = om.forward_rows(cache, [0], e, 1)
    W = {k: v.double().numpy() for k, v in w["layers"][0].items()}
    d = m.d_model
    a = e / np.sqrt((e ** 2).mean() + m.rms_eps)
    v = a @ W["wqkv"][2 * d:].T
    h = e + v @ W["wo"].T
    fa = h / np.sqrt((h ** 2).mean() + m.rms_eps)
    g = fa @ W["w_gate_up"][: m.ffn_dim].T
    u = fa @ W["w_gate_up"][m.ffn_dim:].T
    h = h + (g / (1 + np.exp(-g)) * u) @ W["w_down"].T
    assert np.allclose(got, h, atol=1e-12)


@pytest.mark.parametrize("moe", [False, True])
def test_forward_is_translation_invariant(moe):
    # RoPE carries only relative positions: shifting every position by the same
    # offset leaves all outputs unchanged (no absolute-position term anywhere).
    m, w = _tiny_model(moe=moe)
    om = OracleModel(m, w)
    L = 12
    e = RNG.standard_normal((L, m.d_model))
    rb = RNG.standard_normal((m.n_layers, 4)) if moe else None
    h0 = om.forward_rows(om.new_cache(L), np.arange(L), e, L, rb)
    h1 = om.forward_rows(om.new_cache(L), np.arange(L), e, L, rb, rope_offset=1000)
    assert np.allclose(h0, h1, atol=1e-10)
    # and the rotary angles do enter: a shift of one row's position alone changes the output
    pos = np.arange(L)
    pos2 = pos.copy()
    pos2[3] = 0
    pos2[0] = 3
    h2 = om.forward_rows(om.new_cache(L), pos2, e, L, rb)
    assert not np.allclose(h0, h2, atol=1e-6)


def _tiny_run(w_vic, smooth=0.0, moe=False, hier=False):
    m, w = _tiny_model(moe=moe)
    dc = synth.DecodeCfg(block_len=8, vicinity_w=w_vic, smooth_alpha=smooth, hierarchical=hier)
    wc = synth.WorkloadCfg(name="t", model=m, decode=dc, batch=1, prompt_len=(10, 10), gen_len=16,
                           plant_bias=2.0, plant_prob=(0.7, 0.7),
                           router_pref_bias=2.0 if moe else 0.0, seed=5)
    req = synth.make_requests(wc)
    om = OracleModel(m, w)
    rb = None if req["router_bias"] is None else req["router_bias"][0].numpy()
    run = oracle.OracleRun(om, dc, req["tokens"][0].numpy(), 10, 16, req["plant_id"][0].numpy(),
                           float(req["plant_bias"][0]), rb)
    return m, w, om, run


@pytest.mark.parametrize("moe", [False, True])
def test_vicinity_covering_everything_equals_full_recompute(moe):
    # With w >= L the window is every position: the step must reproduce a full
    # recompute from scratch, whatever stale values the cache held before
    # (K, V are scattered before anyone attends).
    m, w, om, run = _tiny_run(w_vic=1000, moe=moe)
    run.start_block(0)
    for li in run.cache["k"]:
        run.cache["k"][li][:] = RNG.standard_normal(run.cache["k"][li].shape) * 50
        run.cache["v"][li][:] = RNG.standard_normal(run.cache["v"][li].shape) * 50
    got = run.denoise_logits()
    fresh = om.new_cache(run.L)
    pos = np.arange(run.L)
    rb = run._router_bias_block()
    h = om.forward_rows(fresh, pos, om.embed(run.tokens), run.L, rb)
    want = om.logits(h[run.bs:run.be])
    assert np.allclose(got, want, atol=1e-12)
    for li in fresh["k"]:
        assert np.allclose(run.cache["k"][li], fresh["k"][li], atol=1e-12)
        assert np.allclose(run.cache["v"][li], fresh["v"][li], atol=1e-12)


def test_vicinity_zero_width_touches_only_block_rows():
    m, w, om, run = _tiny_run(w_vic=0)
    run.start_block(1)
    before = {li: run.cache["k"][li].copy() for li in run.cache["k"]}
    run.denoise_logits()
    for li in before:
        changed = np.nonzero(np.any(before[li] != run.cache["k"][li], axis=(1, 2)))[0]
        assert set(changed.tolist()) <= set(range(run.bs, run.be))


def test_vicinity_step_after_refresh_equals_refresh_outputs():
    # First step of a block (no smoothing state yet): window rows see the same
    # cache the refresh left, so block logits equal those of the full forward.
    m, w, om, run = _tiny_run(w_vic=3)
    run.start_block(0)
    pos = np.arange(run.L)
    h = om.forward_rows(om.new_cache(run.L), pos, om.embed(run.tokens), run.L)
    want = om.logits(h[run.bs:run.be])
    got = run.denoise_logits()
    assert np.allclose(got, want, atol=1e-10)


def test_bf16_cache_storage_rounds_to_nearest_even():
    """kv_round="bf16": the cache keeps K and V rounded to bfloat16 (8
    significant bits).  Worked cases: 1 + 2^-8 lies halfway between 1 and its
    neighbour 1 + 2^-7 and goes to the even one, 1; 1 + 3 * 2^-8 lies halfway
    between 1 + 2^-7 (odd) and 1 + 2^-6 (even) and goes up; anything past a
    halfway point goes to the nearer neighbour; representable values stay."""
    from oracle.model import _round_bf16
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                  -(1.0 + 2.0 ** -8 - 2.0 ** -20), 0.75, -96.0, 3.0 * 2.0 ** -130])
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0, 0.75, -96.0, 3.0 * 2.0 ** -130])
    assert np.array_equal(_round_bf16(x), want)


def test_bf16_cache_option_changes_only_the_stored_precision():
    wc = synth.preset("tiny_f32").with_model(n_layers=2, d_model=64, n_heads=2, head_dim=32,
                                             ffn_dim=96, vocab=256, mask_id=255)
    w = synth.make_weights(wc.model, 3)
    om = OracleModel(wc.model, w)
    pos = np.arange(40)
    e = om.embed(RNG.integers(0, 255, 40))
    c64, cbf = om.new_cache(40), om.new_cache(40, kv_round="bf16")
    om.forward_rows(c64, pos, e, 40)
    om.forward_rows(cbf, pos, e, 40)
    from oracle.model import _round_bf16
    # layer 0 sees the same inputs: its K, V are the fp64 ones rounded
    for key in ("k", "v"):
        assert np.array_equal(cbf[key][0], _round_bf16(c64[key][0]))
        # every stored value is a bfloat16: at most half an ulp (2^-8 relative) away
        rel = np.abs(cbf[key][0] - c64[key][0]) / np.maximum(np.abs(c64[key][0]), 1e-30)
        assert rel.max() <= 2.0 ** -8
    # deeper layers see the rounded cache through attention: close, not equal
    d = np.abs(cbf["k"][1] - c64["k"][1]).max() / np.sqrt(np.mean(c64["k"][1] ** 2))
    assert 0 < d < 5e-2
