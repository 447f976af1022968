"""Pins of the first-generation (v1) oracle against things other than itself (CPU only).

Independent facts used: a 40-digit brute force with plain loops (mpmath); torch's
scaled_dot_product_attention with enable_gqa (its KV-head mapping is the standard GQA
one) and with explicit masks; a one-hot value matrix that turns attention outputs into
block probability masses; the probability-mass invariant; planted needles; tie rules.
A dropped head group, a transposed group mapping, a block off by one, a window off by
one or a swapped gate each fail at least one of these.
"""
import mpmath
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import hysparse_v1 as v1

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

H, G, GS = v1.N_HEADS, v1.N_KV_HEADS, v1.GROUP


def _rand(seed, *shape, std=1.0):
    return std * np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, K, V, mask=None, scale=None):
    """torch SDPA for one query: q [64, d], K/V [n, 4, d] -> out [64, d] (fp64)."""
    qt = torch.from_numpy(q)[None, :, None, :]                 # [1, 64, 1, d]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]  # [1, 4, n, d]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    am = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


# ----------------------------------------------------------------------------------
# Brute force: 40-digit arithmetic, plain loops, every step written out again
# ----------------------------------------------------------------------------------

def _brute(q, K, V, Ks, Vs, t, scale, top_blocks, window, gsp, gsw):
    mpmath.mp.dps = 40
    d = q.shape[1]
    sc = mpmath.mpf(scale)

    def dot(a, b):
        return mpmath.fsum(mpmath.mpf(a[i]) * mpmath.mpf(b[i]) for i in range(d))

    def attend(h, g, rows, KK, VV):
        s = [sc * dot(q[h], KK[j][g]) for j in rows]
        z = mpmath.fsum(mpmath.exp(x) for x in s)
        p = [mpmath.exp(x) / z for x in s]
        return [mpmath.fsum(p[n] * mpmath.mpf(VV[j][g][i]) for n, j in enumerate(rows)) for i in range(d)], p

    nblk = t // 64 + 1
    full = list(range(t + 1))
    score = [[mpmath.mpf(0)] * nblk for _ in range(G)]
    for h in range(H):
        g = h // GS
        _, p = attend(h, g, full, K, V)
        for j in full:
            score[g][j // 64] += p[j]
    chosen = []
    for g in range(G):
        rem, ch = list(range(nblk)), []
        for _ in range(min(top_blocks, nblk)):
            best = None
            for b in rem:                      # ascending, strict '>' keeps the smaller index
                if best is None or score[g][b] > score[g][best]:
                    best = b
            ch.append(best)
            rem.remove(best)
        chosen.append(sorted(ch))
    out = np.zeros((H, d))
    for h in range(H):
        g = h // GS
        rows = [j for b in chosen[g] for j in range(64 * b, 64 * b + 64) if j <= t]
        o1, _ = attend(h, g, rows, K, V)
        o2, _ = attend(h, g, [j for j in range(t + 1) if j > t - window], Ks, Vs)
        for i in range(d):
            out[h, i] = float(mpmath.mpf(gsp[h]) * o1[i] + mpmath.mpf(gsw[h]) * o2[i])
    return chosen, [[float(x) for x in row] for row in score], out


@pytest.mark.parametrize("t,top_blocks,window,seed", [(150, 1, 128, 1), (200, 2, 16, 2), (63, 1, 128, 3)])
def test_v1_brute_force(t, top_blocks, window, seed):
    d = 4
    n = t + 1
    q = _rand(seed, H, d, std=1.5)
    K = _rand(seed + 10, n, G, d)
    V = _rand(seed + 20, n, G, d)
    Ks = _rand(seed + 30, n, G, d)
    Vs = _rand(seed + 40, n, G, d)
    gsp = np.random.default_rng(seed + 50).uniform(0, 1, H)
    gsw = np.random.default_rng(seed + 60).uniform(0, 1, H)
    scale = 0.5
    chosen, score, out = _brute(q, K, V, Ks, Vs, t, scale, top_blocks, window, gsp, gsw)
    r = v1.v1_selector_query(q, K, V, t, scale, top_blocks)
    np.testing.assert_allclose(r["scores"], np.array(score), rtol=1e-12, atol=1e-15)
    for g in range(G):
        assert r["sel"][g].tolist() == chosen[g]
        # tau (the block parity band is built on it): the smallest score of the brute-force
        # choice of rank top_blocks; none when every candidate block is kept
        if top_blocks < len(score[g]):
            assert r["tau"][g] == pytest.approx(float(min(score[g][b] for b in chosen[g])), rel=1e-12, abs=0)
        else:
            assert r["tau"][g] is None
    o, _, _ = v1.v1_sparse_query(q, K, V, t, r["sel"], Ks, Vs, gsp, gsw, scale, window)
    np.testing.assert_allclose(o, out, rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------------
# Library routines: torch SDPA with GQA and explicit masks
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("t", [0, 63, 64, 300])
def test_v1_full_attention_is_sdpa_gqa(t):
    d = 16
    q = _rand(4, H, d)
    K = _rand(5, t + 1, G, d)
    V = _rand(6, t + 1, G, d)
    scale = d ** -0.5
    out, lse, p = v1.full_attention_gqa(q, K, V, t, scale)
    np.testing.assert_allclose(out, _sdpa(q, K, V, scale=scale), rtol=1e-12, atol=1e-13)
    # LSE against torch.logsumexp of the GQA logits built with repeat_interleave
    Kr = torch.from_numpy(K).repeat_interleave(GS, dim=1)       # [n, 64, d]
    s = torch.einsum("hd,nhd->hn", torch.from_numpy(q), Kr) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=1e-13)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-13)


def test_v1_block_scores_from_one_hot_values():
    """Attention over one-hot block indicators returns each head's probability mass per
    block; summing the 16 heads of a group gives the block score."""
    t, d = 700, 8
    nb = t // 64 + 1
    q = _rand(7, H, d, std=2.0)
    K = _rand(8, t + 1, G, d)
    onehot = np.zeros((t + 1, G, nb))
    onehot[np.arange(t + 1), :, np.arange(t + 1) // 64] = 1.0
    mass = _sdpa(q, K, onehot, scale=0.3)                    # [64, nb]
    ref = mass.reshape(G, GS, nb).sum(axis=1)
    r = v1.v1_selector_query(q, K, np.zeros((t + 1, G, d)), t, 0.3)
    np.testing.assert_allclose(r["scores"], ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["scores"].sum(axis=1), GS, rtol=1e-13)   # each head sums to 1


def test_v1_swa_branch_is_sdpa_with_window_mask():
    t, d, w = 500, 16, 128
    q = _rand(9, H, d)
    Ks = _rand(10, t + 1, G, d)
    Vs = _rand(11, t + 1, G, d)
    K = _rand(12, t + 1, G, d)
    V = _rand(13, t + 1, G, d)
    mask = np.arange(t + 1) > t - w
    ref = _sdpa(q, Ks, Vs, mask=mask, scale=0.1)
    blocks = [np.array([0, 3]), np.array([1]), np.array([7, 2, -1]), np.array([6, -1])]
    zeros, ones = np.zeros(H), np.ones(H)
    out, o_sp, o_sw = v1.v1_sparse_query(q, K, V, t, blocks, Ks, Vs, zeros, ones, 0.1, w)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o_sw, ref, rtol=1e-12, atol=1e-13)
    # sparse branch of each group: SDPA restricted to that group's blocks
    out1, _, _ = v1.v1_sparse_query(q, K, V, t, blocks, Ks, Vs, ones, zeros, 0.1, w)
    for g, bl in enumerate(blocks):
        bl = bl[bl >= 0]
        m = np.isin(np.arange(t + 1) // 64, bl)
        ref_g = _sdpa(q, K, V, mask=m, scale=0.1)[g * GS:(g + 1) * GS]
        np.testing.assert_allclose(out1[g * GS:(g + 1) * GS], ref_g, rtol=1e-12, atol=1e-13)
    # a linear combination of the two branches
    gsp, gsw = np.linspace(0, 1, H), np.linspace(1, 0.25, H)
    out2, _, _ = v1.v1_sparse_query(q, K, V, t, blocks, Ks, Vs, gsp, gsw, 0.1, w)
    np.testing.assert_allclose(out2, gsp[:, None] * out1 + gsw[:, None] * ref, rtol=1e-12, atol=1e-13)


def test_v1_short_context_sparse_branch_is_full_attention():
    """At most 16 blocks: every block is kept and the sparse branch is exact causal attention."""
    t, d = 64 * 16 - 1, 8
    q = _rand(14, H, d)
    K = _rand(15, t + 1, G, d)
    V = _rand(16, t + 1, G, d)
    r = v1.v1_selector_query(q, K, V, t, 0.35)
    assert all(s.tolist() == list(range(16)) for s in r["sel"]) and all(x is None for x in r["tau"])
    _, o_sp, _ = v1.v1_sparse_query(q, K, V, t, r["sel"], K, V, np.ones(H), np.zeros(H), 0.35)
    np.testing.assert_allclose(o_sp, _sdpa(q, K, V, scale=0.35), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------
# Selection: planted needles, rank definition, ties
# ----------------------------------------------------------------------------------

def test_v1_needle_blocks_selected_per_kv_head():
    t, d = 64 * 40 + 17, 16
    rng = np.random.default_rng(17)
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((t + 1, G, d)) * 0.3
    V = rng.standard_normal((t + 1, G, d))
    planted = {0: 5, 1: 33, 2: 40, 3: 0}           # block 40 is the partial last block
    for g, b in planted.items():
        j = min(64 * b + 11, t)
        qm = q[g * GS:(g + 1) * GS].mean(axis=0)
        K[j, g] = 30.0 * qm / np.linalg.norm(qm) ** 2 * 0.3
    r = v1.v1_selector_query(q, K, V, t, 1.0, top_blocks=3)
    for g, b in planted.items():
        assert b in r["sel"][g].tolist()
        assert int(np.argmax(r["scores"][g])) == b


def test_v1_selection_is_rank_definition_with_ties():
    rng = np.random.default_rng(18)
    scores = rng.integers(0, 6, size=50).astype(np.float64)   # many exact ties
    for k in (1, 5, 16, 49, 50, 60):
        sel, tau = v1.select_blocks(scores, k)
        if k >= 50:
            assert sel.tolist() == list(range(50)) and tau is None
            continue
        # rank of b: blocks strictly better, or equal with a smaller index
        rank = [int(np.sum(scores > scores[b]) + np.sum((scores == scores[b]) & (np.arange(50) < b)))
                for b in range(50)]
        assert sel.tolist() == [b for b in range(50) if rank[b] < k]
        assert tau == float(np.sort(scores)[::-1][k - 1])


def test_v1_group_mapping_is_consecutive_heads():
    """Changing only KV head 2 changes exactly query heads 32..47."""
    t, d = 200, 8
    q = _rand(19, H, d)
    K = _rand(20, t + 1, G, d)
    V = _rand(21, t + 1, G, d)
    a, _, _ = v1.full_attention_gqa(q, K, V, t, 0.4)
    K2, V2 = K.copy(), V.copy()
    K2[:, 2] += 0.5
    V2[:, 2] -= 1.0
    b, _, _ = v1.full_attention_gqa(q, K2, V2, t, 0.4)
    changed = np.abs(a - b).max(axis=1) > 1e-9
    assert changed.tolist() == [32 <= h < 48 for h in range(H)]


def test_v1_empty_sparse_branch_contributes_zero():
    t, d = 300, 8
    q = _rand(22, H, d)
    K = _rand(23, t + 1, G, d)
    V = _rand(24, t + 1, G, d)
    blocks = [np.array([-1])] * G
    out, o_sp, o_sw = v1.v1_sparse_query(q, K, V, t, blocks, K, V, np.ones(H), np.ones(H), 0.2)
    assert np.all(o_sp == 0.0)
    mask = np.arange(t + 1) > t - 128
    np.testing.assert_allclose(out, _sdpa(q, K, V, mask=mask, scale=0.2), rtol=1e-12, atol=1e-13)
