"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against an independent fact: a brute-force
high-precision recomputation written with plain loops (mpmath), a textbook
library routine (torch scaled_dot_product_attention, scipy logsumexp,
numpy argpartition), a closed form or an invariant of the method. Together
they are meant to catch a dropped term, a wrong sign or index, an off-by-one
window, a transposed operand or a wrong tie rule anywhere in the oracle.
"""
import math

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads.configs import BlockSpec, make_block_inputs
from workloads.gen import stored_to_f64

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------------
# P1: brute force in 40-digit arithmetic with plain loops
# ----------------------------------------------------------------------------------

def _brute_block(q, K, V, t, W, k, scale, q_sparse):
    mpmath.mp.dps = 40
    H, d = len(q), len(q[0])
    sc = mpmath.mpf(scale)
    S = [[sc * mpmath.fsum(mpmath.mpf(q[h][i]) * mpmath.mpf(K[j][i]) for i in range(d))
          for j in range(t + 1)] for h in range(H)]
    Z = [mpmath.fsum(mpmath.exp(S[h][j]) for j in range(t + 1)) for h in range(H)]
    P = [[mpmath.exp(S[h][j]) / Z[h] for j in range(t + 1)] for h in range(H)]
    O = [[mpmath.fsum(P[h][j] * mpmath.mpf(V[j][i]) for j in range(t + 1)) for i in range(d)]
         for h in range(H)]
    lse = [mpmath.log(Z[h]) for h in range(H)]
    cands = [j for j in range(t + 1) if j <= t - W]        # everything older than the W most recent
    score = {j: mpmath.fsum(P[h][j] for h in range(H)) for j in cands}
    remaining, chosen = list(cands), []
    for _ in range(min(k, len(cands))):
        best = None
        for j in remaining:                                 # ascending, strict '>' keeps the smaller j on ties
            if best is None or score[j] > score[best]:
                best = j
        chosen.append(best)
        remaining.remove(best)
    recent = [j for j in range(t + 1) if j > t - W]
    A = sorted(set(recent) | set(chosen))
    outs = []
    for qs in q_sparse:
        s2 = [[sc * mpmath.fsum(mpmath.mpf(qs[h][i]) * mpmath.mpf(K[j][i]) for i in range(d)) for j in A]
              for h in range(H)]
        z2 = [mpmath.fsum(mpmath.exp(x) for x in s2[h]) for h in range(H)]
        outs.append([[mpmath.fsum(mpmath.exp(s2[h][a]) / z2[h] * mpmath.mpf(V[A[a]][i]) for a in range(len(A)))
                      for i in range(d)] for h in range(H)])
    return O, lse, score, sorted(chosen), outs


@pytest.mark.parametrize("H,d,n,t,W,k,seed", [
    (4, 8, 24, 23, 4, 8, 0),      # more candidates than k
    (3, 6, 20, 13, 4, 8, 1),      # query not at the end of the cache
    (2, 4, 9, 8, 4, 8, 2),        # fewer candidates than k: all selected
    (2, 4, 6, 2, 4, 8, 3),        # t < W: no candidates at all
    (64, 128, 14, 13, 4, 3, 4),   # the real head count and width
])
def test_p1_brute_force(H, d, n, t, W, k, seed):
    q = _rand(seed, H, d)
    qs = [_rand(seed + 100, H, d)]
    K = _rand(seed + 200, n, d)
    V = _rand(seed + 300, n, d)
    scale = 1.0 / math.sqrt(d)
    r = oracle.block_query(q, qs, K, V, t, W, k, scale)
    O, lse, score, chosen, outs = _brute_block(q.tolist(), K.tolist(), V.tolist(), t, W, k, scale,
                                               [x.tolist() for x in qs])
    np.testing.assert_allclose(r["out"], np.array(O, dtype=float), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["lse"], np.array(lse, dtype=float), rtol=1e-13, atol=1e-13)
    cands = sorted(score)
    np.testing.assert_allclose(r["scores"], np.array([float(score[j]) for j in cands]), rtol=1e-12, atol=1e-15)
    assert r["sel"].tolist() == chosen
    np.testing.assert_allclose(r["sparse"][0][0], np.array(outs[0], dtype=float), rtol=1e-12, atol=1e-13)
    # set optimality: every chosen score >= every unchosen candidate's score
    if chosen and len(chosen) < len(cands):
        unchosen = [j for j in cands if j not in chosen]
        assert min(float(score[j]) for j in chosen) >= max(float(score[j]) for j in unchosen)
    # tau, the k-th largest candidate score (the parity band is built on it): the smallest
    # score of the brute-force choice; none when every candidate (or none) is taken
    if 0 < k < len(cands):
        assert r["tau"] == pytest.approx(min(float(score[j]) for j in chosen), rel=1e-12, abs=0)
    else:
        assert r["tau"] is None


# ----------------------------------------------------------------------------------
# P2: when t+1 <= W + k, sparse attention equals full causal attention
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("t", [0, 1, 127, 128, 600, 1150, 1151])
def test_p2_small_context_sparse_equals_full(t):
    H, d, W, k = 64, 128, 128, 1024
    n = t + 1
    q = _rand(10, H, d)
    qs = _rand(11, H, d)
    K = _rand(12, n, d)
    V = _rand(13, n, d)
    scale = 1.0 / math.sqrt(d)
    r = oracle.selector_query(q, K, V, t, W, k, scale)
    assert r["count"] == max(0, t - W + 1)
    out_sp, lse_sp = oracle.sparse_attention(qs, K, V, t, r["sel"], W, scale)
    out_full, lse_full, _ = oracle.full_attention(qs, K, V, t, scale)
    np.testing.assert_allclose(out_sp, out_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_sp, lse_full, rtol=0, atol=1e-12)


def test_p2_boundary_one_past_budget_drops_exactly_one_row():
    H, d, W, k = 64, 128, 128, 1024
    t = W + k                       # t+1 = 1153 rows: 1025 candidates, one must be dropped
    q = _rand(20, H, d)
    K = _rand(21, t + 1, d)
    V = _rand(22, t + 1, d)
    scale = 1.0 / math.sqrt(d)
    r = oracle.selector_query(q, K, V, t, W, k, scale)
    assert r["count"] == k
    rows = oracle.attended_rows(t, r["sel"], W)
    assert rows.shape[0] == W + k
    dropped = sorted(set(range(t + 1)) - set(rows.tolist()))
    assert len(dropped) == 1 and dropped[0] <= t - W
    # the dropped row has the smallest score of all candidates
    assert r["scores"][dropped[0]] == r["scores"].min()


# ----------------------------------------------------------------------------------
# P3: probability mass
# ----------------------------------------------------------------------------------

def test_p3_probability_mass():
    H, d, W = 64, 128, 128
    t = 3000
    q = _rand(30, H, d)
    K = _rand(31, t + 1, d)
    V = _rand(32, t + 1, d)
    out, lse, p = oracle.full_attention(q, K, V, t, 1 / math.sqrt(d))
    assert abs(p.sum() - H) < 1e-10
    scores = oracle.selection_scores(p, t, W)
    window_mass = p[:, t - W + 1:].sum()
    assert abs(scores.sum() - (H - window_mass)) < 1e-10
    assert scores.shape[0] == t - W + 1


# ----------------------------------------------------------------------------------
# P4: identical heads -> selection equals top-k of the logits (numpy argpartition)
# ----------------------------------------------------------------------------------

def test_p4_identical_heads_select_top_logits():
    H, d, W, k = 64, 128, 128, 1024
    t = 20000
    q1 = _rand(40, 1, d)
    q = np.repeat(q1, H, axis=0)
    K = _rand(41, t + 1, d)
    V = _rand(42, t + 1, d)
    r = oracle.selector_query(q, K, V, t, W, k, 1 / math.sqrt(d))
    cand_logits = (K[: t - W + 1] @ q1[0])
    top = np.sort(np.argpartition(-cand_logits, k - 1)[:k])
    assert r["sel"].tolist() == top.tolist()


# ----------------------------------------------------------------------------------
# P5 / P6: textbook attention from torch (fp64 CPU) and scipy logsumexp
# ----------------------------------------------------------------------------------

def _sdpa(q, K, V, mask, scale):
    qt = torch.from_numpy(q)[None, :, None, :]              # [1, H, 1, d]
    kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1)
    m = torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("t", [0, 5, 300, 2047])
def test_p6_full_attention_is_textbook_causal_attention(t):
    H, d, n = 64, 128, 2048
    q = _rand(50, H, d)
    K = _rand(51, n, d)
    V = _rand(52, n, d)
    scale = 1 / math.sqrt(d)
    out, lse, _ = oracle.full_attention(q, K, V, t, scale)
    mask = np.arange(n) <= t
    np.testing.assert_allclose(out, _sdpa(q, K, V, mask, scale), rtol=0, atol=1e-12)
    ref_lse = scipy.special.logsumexp(scale * np.einsum("hd,nd->hn", q, K[: t + 1]), axis=1)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_p5_k_zero_is_sliding_window_attention():
    H, d, n, W = 64, 128, 1000, 128
    t = 777
    q = _rand(60, H, d)
    qs = _rand(61, H, d)
    K = _rand(62, n, d)
    V = _rand(63, n, d)
    scale = 1 / math.sqrt(d)
    r = oracle.selector_query(q, K, V, t, W, 0, scale)
    assert r["count"] == 0
    out, _ = oracle.sparse_attention(qs, K, V, t, r["sel"], W, scale)
    j = np.arange(n)
    mask = (j <= t) & (j > t - W)                           # exactly W rows ending at t
    assert mask.sum() == W
    np.testing.assert_allclose(out, _sdpa(qs, K, V, mask, scale), rtol=0, atol=1e-12)


def test_p5_k_at_least_candidates_is_full_attention():
    H, d, n, W = 64, 128, 700, 128
    t = 650
    q = _rand(70, H, d)
    qs = _rand(71, H, d)
    K = _rand(72, n, d)
    V = _rand(73, n, d)
    scale = 1 / math.sqrt(d)
    r = oracle.selector_query(q, K, V, t, W, t - W + 1, scale)
    out, _ = oracle.sparse_attention(qs, K, V, t, r["sel"], W, scale)
    mask = np.arange(n) <= t
    np.testing.assert_allclose(out, _sdpa(qs, K, V, mask, scale), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------
# P7: bridging = plain loops (tiny) and torch linear (larger)
# ----------------------------------------------------------------------------------

def test_p7_bridge_brute_force_and_torch_linear():
    Hs = _rand(80, 5, 16)
    wk = [_rand(81, 16, 4), _rand(82, 16, 4)]
    wv = [_rand(83, 16, 4), _rand(84, 16, 4)]
    ks, vs = oracle.bridge_kv(Hs, wk, wv)
    for l in range(2):
        for r in range(5):
            for c in range(4):
                assert abs(ks[l][r, c] - math.fsum(Hs[r, i] * wk[l][i, c] for i in range(16))) < 1e-12
                assert abs(vs[l][r, c] - math.fsum(Hs[r, i] * wv[l][i, c] for i in range(16))) < 1e-12
    Hb = _rand(85, 300, 2048)
    wk = [_rand(86 + l, 2048, 128) * 0.02 for l in range(3)]
    wv = [_rand(90 + l, 2048, 128) * 0.02 for l in range(3)]
    ks, vs = oracle.bridge_kv(Hb, wk, wv)
    for l in range(3):
        ref_k = torch.nn.functional.linear(torch.from_numpy(Hb), torch.from_numpy(wk[l]).T.contiguous()).numpy()
        ref_v = torch.nn.functional.linear(torch.from_numpy(Hb), torch.from_numpy(wv[l]).T.contiguous()).numpy()
        np.testing.assert_allclose(ks[l], ref_k, rtol=0, atol=1e-11)
        np.testing.assert_allclose(vs[l], ref_v, rtol=0, atol=1e-11)


# ----------------------------------------------------------------------------------
# P8: planted needles are selected
# ----------------------------------------------------------------------------------

def test_p8_needles_are_selected():
    spec = BlockSpec("needles", [6000, 9000], [[5990, 5999], [8999]], dtype="bf16", n_sparse=1,
                     needles_per_query=8, seed=7)
    inp = make_block_inputs(spec)
    assert len(inp.needles) == 3 * 8
    K = stored_to_f64(inp.k)
    V = stored_to_f64(inp.v)
    Q = stored_to_f64(inp.q_sel)
    for qi in range(spec.total_q):
        s = int(inp.q_seq[qi])
        a, n = int(inp.kv_start[s]), int(inp.kv_len[s])
        t = int(inp.q_pos[qi])
        r = oracle.selector_query(Q[qi], K[a:a + n], V[a:a + n], t, spec.window, spec.top_k, spec.scale)
        mine = [p for (si, qj, h, p) in inp.needles if qj == qi]
        assert len(mine) == 8
        assert set(mine) <= set(r["sel"].tolist())


# ----------------------------------------------------------------------------------
# P9: permuting candidate rows permutes the selection and leaves outputs unchanged
# ----------------------------------------------------------------------------------

def test_p9_permutation_equivariance():
    H, d, W, k = 64, 128, 128, 1024
    t = 5000
    q = _rand(100, H, d)
    qs = _rand(101, H, d)
    K = _rand(102, t + 1, d)
    V = _rand(103, t + 1, d)
    scale = 1 / math.sqrt(d)
    r = oracle.block_query(q, [qs], K, V, t, W, k, scale)
    nc = t - W + 1
    perm = np.random.default_rng(104).permutation(nc)      # new row i holds old row perm[i]
    K2, V2 = K.copy(), V.copy()
    K2[:nc], V2[:nc] = K[perm], V[perm]
    r2 = oracle.block_query(q, [qs], K2, V2, t, W, k, scale)
    inv = np.empty(nc, dtype=np.int64)
    inv[perm] = np.arange(nc)
    assert sorted(inv[r["sel"]].tolist()) == r2["sel"].tolist()
    np.testing.assert_allclose(r2["out"], r["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r2["sparse"][0][0], r["sparse"][0][0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------
# Ties at the k-th score go to the smaller position
# ----------------------------------------------------------------------------------

def test_ties_prefer_smaller_position():
    H, d, W, k = 64, 128, 4, 3
    t = 20
    q = _rand(110, H, d)
    K = _rand(111, t + 1, d)
    V = _rand(112, t + 1, d)
    # make candidate rows 3, 7, 11, 15 identical and clearly the best: equal scores
    best = q.mean(axis=0)
    best = 6.0 * best / np.linalg.norm(best) * math.sqrt(d)
    for j in (3, 7, 11, 15):
        K[j] = best
    r = oracle.selector_query(q, K, V, t, W, k, 1 / math.sqrt(d))
    s = r["scores"]
    assert s[3] == s[7] == s[11] == s[15]
    assert s[3] > np.delete(s, [3, 7, 11, 15]).max()
    assert r["sel"].tolist() == [3, 7, 11]
    assert r["tau"] == s[3]


# ----------------------------------------------------------------------------------
# FP8 (OCP E4M3) KV cache: the oracle's decoding of the codes
# ----------------------------------------------------------------------------------

def test_e4m3_decode_special_values():
    """Values fixed by the OCP 8-bit floating point specification (E4M3: bias 7, 3
    mantissa bits, subnormals, no infinities, S.1111.111 = NaN), written as closed forms."""
    d = oracle.e4m3_decode
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
             0xB8: -1.0, 0xFE: -448.0}
    got = d(np.array(list(cases), dtype=np.uint8))
    assert got.tolist() == list(cases.values())
    assert np.isnan(d(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    z = d(np.array([0x80], dtype=np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_e4m3_decode_matches_torch_float8():
    """All 256 codes against torch's float8_e4m3fn widening (a library routine)."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_decode_order_and_symmetry():
    """Codes 0x00..0x7E are the 127 non-negative finite values in increasing order, the
    upper half their negatives, and the spacing doubles with each binade."""
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(d[0x80:0xFF], -pos)
    steps = np.diff(pos[8:])                    # normals: step 2^(e-10) inside binade e
    for e in range(1, 15):
        blk = steps[(e - 1) * 8:(e - 1) * 8 + 7]
        assert np.all(blk == 2.0 ** (e - 10))


# ----------------------------------------------------------------------------------
# FP8 (OCP E4M3) KV cache written by KV Bridging: the oracle's encoding
# ----------------------------------------------------------------------------------

def test_e4m3_encode_inverts_decode():
    """Every finite code is the encoding of its own value (also -0.0 -> 0x80)."""
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(oracle.e4m3_encode(vals[fin]), codes[fin])


def test_e4m3_encode_rounds_to_nearest_ties_to_even():
    """Between the values of two adjacent finite codes, a value nearer to one takes that
    code, and the midpoint itself the code with the even mantissa (low bit clear), across
    the subnormals, the binade boundaries and both signs."""
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for base in (0x00, 0x80):
        for c in range(base, base + 0x7E):
            a, b = d[c], d[c + 1]           # codes c, c+1 (values decrease for negatives)
            mid = (a + b) / 2.0
            got = oracle.e4m3_encode(np.array([mid, mid + (a - mid) / 4, mid + (b - mid) / 4]))
            even = c if c % 2 == 0 else c + 1
            assert got.tolist() == [even, c, c + 1], (hex(c), a, b)


def test_e4m3_encode_saturates_and_keeps_nan():
    """Magnitudes above the largest finite value (448) give +-448, infinities too; NaN
    gives 0x7F; values below half the smallest subnormal give a signed zero."""
    x = np.array([448.0, 448.5, 464.0, 480.0, 1e30, np.inf, -449.0, -np.inf, np.nan, 2.0 ** -11, -2.0 ** -11])
    assert oracle.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x00, 0x80]


def test_e4m3_encode_matches_torch_float8():
    """Random float32 values of every binade (including the subnormals), within +-464 where
    torch's float8_e4m3fn conversion (a library routine) neither saturates nor gives NaN."""
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-12.0, np.log2(464.0), 200000)).astype(np.float32)
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x.astype(np.float64)), ref)


def test_bridge_kv_fp8_error_bound():
    """Each code of the FP8 bridging stands for the fp64 projection within half a step of
    the E4M3 grid at that magnitude (relative 2^-4 for normals, 2^-10 absolute for the
    subnormals), times the layer's scale; values beyond 448 * scale saturate."""
    rng = np.random.default_rng(6)
    H = rng.standard_normal((300, 64))
    wk = [rng.standard_normal((64, 16)) * 0.02, rng.standard_normal((64, 16)) * 0.3]
    wv = [rng.standard_normal((64, 16)) * 0.02, rng.standard_normal((64, 16)) * 0.3]
    ks, vs = oracle.bridge_kv(H, wk, wv)
    k_sc, v_sc = [0.004, 0.05], [0.003, 0.0001]     # the last one makes V_1 saturate
    kc, vc = oracle.bridge_kv_fp8(H, wk, wv, k_sc, v_sc)
    for ref, codes, sc in zip(ks + vs, kc + vc, k_sc + v_sc):
        x = ref / sc
        back = oracle.e4m3_decode(codes)
        inside = np.abs(x) <= 448.0
        bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10)
        assert np.all(np.abs(back - x)[inside] <= bound[inside])
        assert np.all(np.abs(back[~inside]) == 448.0) and np.all(np.sign(back[~inside]) == np.sign(x[~inside]))
    assert (np.abs(vs[1] / v_sc[1]) > 448.0).any()


def test_fp8_block_inputs_round_trip():
    """The FP8 workload stores code(x / scale): decoding and rescaling returns x within
    half a step of the format (relative 2^-4 for normals), and planted needle keys
    survive as the largest logits of their head."""
    spec = BlockSpec("fp8", [3000], [[2999]], dtype="fp8", n_sparse=0, needles_per_query=4, seed=31)
    inp = make_block_inputs(spec)
    assert inp.k.dtype == np.uint8 and inp.v.dtype == np.uint8 and inp.q_sel.dtype == np.uint16
    K = oracle.dequantize_kv(inp.k, spec.k_scale)
    assert np.isfinite(K).all() and np.abs(K).max() <= 448 * spec.k_scale
    Q = stored_to_f64(inp.q_sel[0])
    for (_, qi, h, p) in inp.needles:
        s = Q[h] @ K.T * spec.scale
        assert int(np.argmax(s)) == p
