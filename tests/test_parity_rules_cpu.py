"""The comparison rules of tests/parity.py, checked on the CPU against outputs with planted
defects: the rules must accept the oracle's own result (and key swaps inside the tie band)
and reject every defect that a GPU path could plausibly produce. The inputs are small and
seeded; no GPU is used."""
import math

import numpy as np
import pytest

import oracle
from parity import check_attn, check_lse, check_selection, half_ulp_bf16


def _selector(seed=3, t=200, window=16, top_k=24, H=8, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d))
    K = rng.standard_normal((t + 1, d))
    V = rng.standard_normal((t + 1, d))
    r = oracle.selector_query(q, K, V, t, window, top_k, 1.0 / math.sqrt(d))
    nc = oracle.candidate_count(t, window)
    return r, top_k, nc


def _padded(sel, top_k):
    out = np.full(top_k, -1, dtype=np.int64)
    out[: len(sel)] = sel
    return out


def test_selection_accepts_the_oracle_result():
    r, k, nc = _selector()
    assert check_selection(_padded(r["sel"], k), len(r["sel"]), r, k, nc) == 0


@pytest.mark.parametrize("defect", ["swap_out_best", "duplicate", "descending", "short_count", "bad_padding",
                                    "outside_candidates"])
def test_selection_rejects_defects(defect):
    r, k, nc = _selector()
    sel = r["sel"].copy()
    count = len(sel)
    scores = r["scores"]
    unselected = np.setdiff1d(np.arange(nc), sel)
    if defect == "swap_out_best":       # the best key replaced by the worst candidate
        best = sel[np.argmax(scores[sel])]
        worst = unselected[np.argmin(scores[unselected])]
        sel = np.sort(np.append(sel[sel != best], worst))
    elif defect == "duplicate":
        sel[1] = sel[0]
    elif defect == "descending":
        sel = sel[::-1].copy()
    elif defect == "short_count":
        count -= 1
    elif defect == "outside_candidates":  # a window row (>= nc) in place of the last key
        sel[-1] = nc
    gpu = _padded(sel, k)
    if defect == "bad_padding":
        gpu = np.append(gpu, 0)           # an entry past the count that is not -1
    with pytest.raises(AssertionError):
        check_selection(gpu, count, r, k, nc)


def test_selection_accepts_a_swap_inside_the_band_only():
    """Two candidates whose scores differ by less than the band around tau may be swapped;
    the same swap is rejected once their scores are moved apart."""
    r, k, nc = _selector()
    scores = r["scores"].copy()
    sel = r["sel"]
    kth = sel[np.argmin(scores[sel])]                 # holds tau
    out = np.setdiff1d(np.arange(nc), sel)
    nxt = out[np.argmax(scores[out])]                 # the best key left out
    tau = scores[kth]
    for gap, ok in ((1e-7, True), (1e-3, False)):
        s2 = scores.copy()
        s2[nxt] = tau * (1 - gap)
        ref = dict(r, scores=s2, tau=tau)
        swapped = np.sort(np.append(sel[sel != kth], nxt))
        if ok:
            assert check_selection(_padded(swapped, k), k, ref, k, nc) == 1
        else:
            with pytest.raises(AssertionError):
                check_selection(_padded(swapped, k), k, ref, k, nc)


def test_selection_without_tau_needs_the_same_set():
    r, k, nc = _selector(t=30, window=16, top_k=24)   # 15 candidates < k: all taken
    assert r["tau"] is None
    assert check_selection(_padded(r["sel"], k), len(r["sel"]), r, k, nc) == 0
    with pytest.raises(AssertionError):
        check_selection(_padded(r["sel"][:-1], k), len(r["sel"]), r, k, nc)


def _bf16(x):
    """Round to bfloat16 (nearest even) and widen back, as the GPU's output dtype."""
    import torch
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def test_attn_accepts_the_rounded_exact_result():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((64, 128)) * 0.5
    check_attn(_bf16(ref), ref)
    assert np.all(np.abs(_bf16(ref) - ref) <= half_ulp_bf16(ref))


@pytest.mark.parametrize("defect", ["one_element", "uniform_bias", "nan"])
def test_attn_rejects_defects(defect):
    rng = np.random.default_rng(8)
    ref = rng.standard_normal((64, 128)) * 0.5
    gpu = _bf16(ref)
    if defect == "one_element":
        gpu[3, 5] += 0.02
    elif defect == "uniform_bias":
        gpu = gpu + 1.5e-3
    else:
        gpu[0, 0] = np.nan
    with pytest.raises(AssertionError):
        check_attn(gpu, ref)


def test_few_key_rule_takes_errors_beyond_rounding_only():
    """An output of magnitude ~4.3 rounded to bf16 may be 1.6e-2 off: the plain rule rejects
    it, the few-keys rule accepts it; 2e-2 beyond the rounding is rejected by both."""
    ref = np.full((64, 128), 4.3)
    ref[:, ::2] = 4.3 + 2.0 ** -7                      # between two bf16 values near 4.3
    gpu = _bf16(ref)
    assert np.abs(gpu - ref).max() > 1e-2
    with pytest.raises(AssertionError):
        check_attn(gpu, ref)
    check_attn(gpu, ref, few_keys=True)
    gpu[1, 1] += 2e-2
    with pytest.raises(AssertionError):
        check_attn(gpu, ref, few_keys=True)


def test_lse_rule():
    ref = np.linspace(5.0, 12.0, 64)
    check_lse(ref + 5e-4, ref)
    with pytest.raises(AssertionError):
        check_lse(ref + 2e-3, ref)


# ----------------------------------------------------------------------------------
# Bridging rules (bf16 outputs and FP8 E4M3 codes)
# ----------------------------------------------------------------------------------

def _bridge_ref(seed=9, rows=400, d_model=256):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((rows, d_model))
    W = rng.standard_normal((d_model, 128)) * 0.06
    return oracle.bridge_kv(H, [W], [W])[0][0]


def test_bridge_bf16_accepts_the_rounded_result():
    from parity import check_bridge_bf16
    ref = _bridge_ref()
    check_bridge_bf16(_bf16(ref), ref)


@pytest.mark.parametrize("defect", ["two_ulp", "many_one_ulp", "truncated"])
def test_bridge_bf16_rejects_defects(defect):
    from parity import bf16_ulp, check_bridge_bf16
    ref = _bridge_ref()
    g = _bf16(ref)
    if defect == "two_ulp":          # one value two units off
        g[7, 3] += 2 * bf16_ulp(ref[7, 3])
    elif defect == "many_one_ulp":   # 5% of the values one unit off (each within 1 ulp)
        idx = np.random.default_rng(1).random(g.shape) < 0.05
        g[idx] = _bf16(g[idx] + np.sign(ref[idx] - g[idx] + 1e-300) * bf16_ulp(ref[idx]))
    else:                            # rounded toward zero instead of to nearest
        import torch
        f = torch.from_numpy(ref.astype(np.float32)).view(torch.int32) & ~0xFFFF
        g = f.view(torch.float32).numpy().astype(np.float64)
    with pytest.raises(AssertionError):
        check_bridge_bf16(g, ref)


def _fp8_case(seed=11, n=20000, scale=0.01):
    rng = np.random.default_rng(seed)
    val = rng.standard_normal(n) * 0.8
    return val, oracle.e4m3_encode(val / scale), scale


def test_fp8_codes_accept_the_oracle_and_a_midpoint_flip():
    from parity import check_fp8_codes
    val, codes, sc = _fp8_case()
    check_fp8_codes(codes.copy(), val, codes, sc)
    # a value at a rounding midpoint: the other of its two codes is accepted too
    c = oracle.e4m3_encode(np.array([3.0]))[0]               # 3.0 = code of mantissa 4
    lo, hi = oracle.e4m3_decode(np.array([c, c + 1], dtype=np.uint8))
    v = val.copy()
    v[0] = (lo + hi) / 2.0 * sc
    ref = oracle.e4m3_encode(v / sc)
    g = ref.copy()
    g[0] = c if ref[0] == c + 1 else c + 1
    check_fp8_codes(g, v, ref, sc)


@pytest.mark.parametrize("defect", ["two_steps", "one_step_off_midpoint", "too_many"])
def test_fp8_codes_reject_defects(defect):
    from parity import check_fp8_codes
    val, codes, sc = _fp8_case()
    g = codes.copy()
    x = val / sc
    if defect == "two_steps":
        i = int(np.argmax((np.abs(x) > 1.0) & (np.abs(x) < 100.0)))
        g[i] = codes[i] + 2 if (codes[i] & 0x7) < 6 else codes[i] - 2
    elif defect == "one_step_off_midpoint":
        # a value a quarter step from its code: the neighbouring code is wrong
        i = int(np.argmax((np.abs(x) > 1.0) & (np.abs(x) < 100.0)))
        g[i] = codes[i] + 1 if (codes[i] & 0x7) < 7 else codes[i] - 1
        back = oracle.e4m3_decode(codes[i:i + 1])[0]
        step = abs(oracle.e4m3_decode(g[i:i + 1])[0] - back)
        val = val.copy()
        val[i] = (back + np.sign(back) * step / 4.0) * sc
        codes = oracle.e4m3_encode(val / sc)
        assert codes[i] != g[i]
    else:                              # 0.5% of the codes one step off at their midpoints
        val = val.copy()
        for i in range(0, 100):
            c = codes[i]
            nb = c + 1 if (c & 0x7) < 7 else c - 1
            a, b = oracle.e4m3_decode(np.array([c, nb], dtype=np.uint8))
            val[i] = (a + b) / 2.0 * sc
        codes = oracle.e4m3_encode(val / sc)
        g = codes.copy()
        for i in range(0, 100):
            c = codes[i]
            g[i] = c + 1 if (c & 0x7) < 7 else c - 1
            a, b = oracle.e4m3_decode(np.array([c, g[i]], dtype=np.uint8))
            if abs(val[i] / sc - (a + b) / 2.0) > 1e-9:   # not a midpoint pair after all
                g[i] = c - 1 if (c & 0x7) > 0 else c + 1
    with pytest.raises(AssertionError):
        check_fp8_codes(g, val, codes, sc)
