"""Pins of the window input embedding and of the LM head (no GPU).

OracleRun.window_embeddings decides which window rows take the soft embedding
of iteration smoothing (dInfer news article, section "解码的艺术": the
distribution of a still-masked position from the previous iteration enters
the next one): only still-masked rows of the current block that carry a
smoothing state; every other row -- prompt, committed, and the MASK rows of
the next block that the window reaches -- takes its token's own embedding.
The expected rows are written out here one by one from an embedding table
whose rows are distinct, so a wrong row, a wrong offset between window and
block, or a soft row in the next block fails.

OracleModel.logits is the final RMSNorm with gain followed by the LM head:
scale invariance and an identity / permutation head pin the norm, the gain
and the orientation of the head."""
import numpy as np
import pytest

import oracle
import synth
from oracle.model import OracleModel


def _tiny(P, G, B, w, alpha, V=10, d=4):
    m = synth.ModelCfg(n_layers=0, d_model=d, n_heads=1, head_dim=d, ffn_dim=8, vocab=V,
                       mask_id=V - 1, dtype="f32")
    dc = synth.DecodeCfg(block_len=B, vicinity_w=w, smooth_alpha=alpha)
    # row v of the table = (v, 10 v, 100 v, 1): every row distinct
    emb = np.stack([[v, 10.0 * v, 100.0 * v, 1.0] for v in range(V)])
    wts = {"tok_emb": emb, "final_norm": np.ones(d), "lm_head": np.eye(V, d), "layers": []}
    model = OracleModel(m, wts, layers=[])
    M = V - 1
    tokens = np.array(list(range(1, P + 1)) + [M] * G)
    run = oracle.OracleRun(model, dc, tokens, P, G, np.full(P + G, -1), 0.0)
    return run, emb, M


def _set_state(run, block_tokens, valid, ids, probs):
    B = run.B
    run.tokens[run.bs:run.be] = block_tokens
    run.smooth_valid = np.array(valid, dtype=bool)
    run.smooth_ids = np.zeros((B, 8), dtype=np.int64)
    run.smooth_p = np.zeros((B, 8))
    for j in range(B):
        run.smooth_ids[j, :len(ids[j])] = ids[j]
        run.smooth_p[j, :len(probs[j])] = probs[j]


def _soft(emb, M, ids, probs, alpha):
    out = (1.0 - alpha) * emb[M].copy()
    for i, p in zip(ids, probs):
        out = out + alpha * p * emb[i]
    return out


@pytest.mark.parametrize("alpha", [0.3, 0.0])
def test_window_embeddings_rows_inside_the_window(alpha):
    # prompt 4, two blocks of 4, w = 2: block 0 is [4, 8), window [2, 10)
    run, emb, M = _tiny(P=4, G=8, B=4, w=2, alpha=alpha)
    run.start_block(0)
    ids = [[7, 2], [1, 2, 3], [5], [6, 8]]
    probs = [[0.5, 0.5], [0.5, 0.25, 0.25], [1.0], [0.75, 0.25]]
    # offset 0 committed to token 5 (with a stale state: still hard); 1 masked
    # with state (soft); 2 masked without state (hard MASK); 3 masked with state
    _set_state(run, [5, M, M, M], [True, True, False, True], ids, probs)
    lo, hi = run.window()
    assert (lo, hi) == (2, 10)
    got = run.window_embeddings(lo, hi)
    want = [emb[3], emb[4],                     # prompt positions 2, 3
            emb[5],                             # committed block position 4
            _soft(emb, M, ids[1], probs[1], alpha),
            emb[M],                             # masked, no state
            _soft(emb, M, ids[3], probs[3], alpha),
            emb[M], emb[M]]                     # next block's MASK rows 8, 9
    assert got.shape == (8, 4)
    for i, row in enumerate(want):
        assert np.allclose(got[i], row, rtol=0, atol=1e-12), (i, got[i], row)


def test_window_embeddings_clipped_at_the_sequence_start():
    # prompt 1, blocks of 4, w = 2: block 0 is [1, 5), window [0, 7) -- the
    # block starts one row into the window
    run, emb, M = _tiny(P=1, G=8, B=4, w=2, alpha=0.3)
    run.start_block(0)
    ids = [[2], [3, 4], [5], [6]]
    probs = [[1.0], [0.4, 0.6], [1.0], [1.0]]
    _set_state(run, [M, M, 8, M], [True, True, True, False], ids, probs)
    lo, hi = run.window()
    assert (lo, hi) == (0, 7)
    got = run.window_embeddings(lo, hi)
    want = [emb[1],
            _soft(emb, M, ids[0], probs[0], 0.3),
            _soft(emb, M, ids[1], probs[1], 0.3),
            emb[8],
            emb[M],
            emb[M], emb[M]]
    for i, row in enumerate(want):
        assert np.allclose(got[i], row, rtol=0, atol=1e-12), (i, got[i], row)


def test_window_embeddings_second_block():
    # block 1 of prompt 4 + blocks of 4, w = 3: block [8, 12), window [5, 12)
    # clipped at L = 12; rows 5..7 are block 0's committed tokens
    run, emb, M = _tiny(P=4, G=8, B=4, w=3, alpha=0.5)
    run.tokens[4:8] = [1, 2, 3, 4]
    run.start_block(1)
    ids = [[6], [7], [2, 3], [4]]
    probs = [[1.0], [1.0], [0.5, 0.5], [1.0]]
    _set_state(run, [M, 6, M, M], [True, False, True, False], ids, probs)
    lo, hi = run.window()
    assert (lo, hi) == (5, 12)
    got = run.window_embeddings(lo, hi)
    want = [emb[2], emb[3], emb[4],
            _soft(emb, M, ids[0], probs[0], 0.5),
            emb[6],
            _soft(emb, M, ids[2], probs[2], 0.5),
            emb[M]]
    for i, row in enumerate(want):
        assert np.allclose(got[i], row, rtol=0, atol=1e-12), (i, got[i], row)


def _head_model(d, V, g, W, eps):
    m = synth.ModelCfg(n_layers=0, d_model=d, n_heads=1, head_dim=d, ffn_dim=8, vocab=V,
                       mask_id=V - 1, dtype="f32", rms_eps=eps)
    return OracleModel(m, {"tok_emb": np.zeros((V, d)), "final_norm": g, "lm_head": W,
                           "layers": []}, layers=[])


def test_logits_final_norm_scale_invariance():
    rng = np.random.default_rng(5)
    d, V = 16, 40
    om = _head_model(d, V, rng.uniform(0.5, 2.0, d), rng.standard_normal((V, d)), eps=0.0)
    h = rng.standard_normal((5, d))
    base = om.logits(h)
    for k in (1e-3, 0.37, 12.0, 4096.0):
        assert np.allclose(om.logits(k * h), base, rtol=1e-12, atol=1e-12)


def test_logits_identity_and_permutation_head():
    rng = np.random.default_rng(6)
    d = 12
    h = rng.standard_normal((4, d)) * rng.uniform(0.1, 30.0, (4, 1))
    # identity head, unit gain: each row comes out with unit root mean square
    om = _head_model(d, d, np.ones(d), np.eye(d), eps=0.0)
    z = om.logits(h)
    assert np.allclose(np.sqrt(np.mean(z * z, axis=1)), 1.0, rtol=1e-12)
    assert np.allclose(z * np.sqrt(np.mean(h * h, axis=1, keepdims=True)), h, rtol=1e-12)
    # gain 2 doubles every logit
    om2 = _head_model(d, d, np.full(d, 2.0), np.eye(d), eps=0.0)
    assert np.allclose(om2.logits(h), 2.0 * z, rtol=1e-12)
    # head row v selects hidden unit perm[v]: logit v = normalised h[perm[v]]
    perm = rng.permutation(d)
    om3 = _head_model(d, d, np.ones(d), np.eye(d)[perm], eps=0.0)
    assert np.allclose(om3.logits(h), z[:, perm], rtol=1e-12)
