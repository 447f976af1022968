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
