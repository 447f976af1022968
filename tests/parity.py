"""Parity helpers shared by the GPU tests: device upload and the comparison rules.

Comparison rules:
  * index sets: every oracle-selected key whose score exceeds tau*(1+1e-5) must be in
    the GPU set, no key scoring below tau*(1-1e-5) may be in it (tau = the oracle's
    k-th score), the sizes must be equal (min(k, candidates)), and the GPU set must be
    ascending without duplicates. Without a tau (all candidates taken) the sets must
    be equal.
  * attention outputs (full and sparse): max |gpu - fp64| <= 1e-2 and mean <= 1e-3,
    the GPU value taken in its output dtype. With an FP8 K/V cache the mean is taken
    over the error beyond each element's own output rounding, max(0, |gpu - fp64| -
    ulp_bf16(fp64)/2): V's scale makes V's values non-representable in bf16, so even a
    query with a single attended key (out = v_0) carries the bf16 rounding of |v| ~ 1
    (mean ~1.1e-3), which a bf16 cache never has. The max rule is unchanged.
    A query that attends at most FEW_KEYS keys has both its max and its mean taken beyond
    each element's own output rounding: its output mixes two to four unit-scale V rows,
    and their exact mix rounded to bf16 already has a mean error of up to 1.01e-3 over
    64 x 128 values and a max of up to 1.02e-2 (an element of magnitude 4.3, where half a
    bf16 unit is 1.6e-2), so the plain rules would reject the exact result.
  * LSE: |gpu - fp64| <= 1e-3 (fp32 output of a value of magnitude ~10).
  * bridging, bf16 outputs: |gpu - fp64| <= 1 bf16 ulp + 2^-14 everywhere (the absolute
    part covers an fp32 accumulation of d_model products near zero), at most 1% of the
    values differing from the correctly rounded reference, and a mean distance to it of at
    most 1e-4.
  * bridging, FP8 E4M3 outputs: a code may differ from the oracle's code of value/scale
    only by one step, only where the value lies within the GPU's arithmetic error of the
    midpoint between the two codes, and at most 0.1% of the codes may differ.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads.gen import bf16_round, bf16_to_f32, stored_to_f64

REL_BAND = 1e-5
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3
FEW_KEYS = 4      # attended keys up to which the mean is taken beyond output rounding
BRIDGE_ATOL = 2.0 ** -14  # fp32 accumulation of d_model products, for outputs near zero


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_selection(gpu_sel: np.ndarray, gpu_count: int, ref: dict, top_k: int, nc: int, what: str = ""):
    k_eff = min(top_k, nc)
    assert gpu_count == k_eff, f"{what}: count {gpu_count} != {k_eff}"
    sel = np.asarray(gpu_sel[:k_eff], dtype=np.int64)
    assert np.all(np.asarray(gpu_sel[k_eff:]) == -1), f"{what}: padding is not -1"
    if k_eff:
        assert np.all(np.diff(sel) > 0), f"{what}: not strictly ascending"
        assert sel[0] >= 0 and sel[-1] < nc, f"{what}: index outside the candidates"
    tau = ref["tau"]
    if tau is None:
        assert sel.tolist() == ref["sel"].tolist(), f"{what}: selection differs (all candidates expected)"
        return 0
    scores = ref["scores"]
    must = ref["sel"][scores[ref["sel"]] > tau * (1 + REL_BAND)]
    missing = np.setdiff1d(must, sel)
    assert missing.size == 0, f"{what}: {missing.size} clearly-selected keys missing, e.g. {missing[:5]}"
    bad = sel[scores[sel] < tau * (1 - REL_BAND)]
    assert bad.size == 0, f"{what}: {bad.size} clearly-unselected keys chosen, e.g. {bad[:5]}"
    return int(np.setdiff1d(sel, ref["sel"]).size)  # keys swapped inside the tolerance band


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bfloat16 unit in the last place at |x| (the bound of rounding x to bf16)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8.0)


def check_attn(gpu: np.ndarray, ref: np.ndarray, what: str = "", beyond_rounding: bool = False,
               few_keys: bool = False):
    """beyond_rounding: the mean rule over the error beyond output rounding (FP8 K/V);
    few_keys: the max and the mean rules over it (a query attending <= FEW_KEYS keys)."""
    err = np.abs(gpu - ref)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    beyond = np.maximum(0.0, err - half_ulp_bf16(ref))
    mx = beyond if few_keys else err
    assert mx.max() <= MAX_ABS, f"{what}: max abs err {mx.max():.3e}" + (" beyond rounding" if few_keys else "")
    beyond_rounding = beyond_rounding or few_keys
    m = beyond if beyond_rounding else err
    assert m.mean() <= MEAN_ABS, f"{what}: mean abs err {m.mean():.3e}" + (" beyond rounding" if beyond_rounding else "")
    return float(err.max()), float(m.mean())


def check_lse(gpu: np.ndarray, ref: np.ndarray, what: str = ""):
    err = np.abs(gpu - ref)
    assert err.max() <= LSE_ABS, f"{what}: lse max abs err {err.max():.3e}"


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """One bfloat16 unit in the last place at |x|."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 1e-30))) - 7)


def check_bridge_bf16(g: np.ndarray, ref: np.ndarray, what: str = ""):
    """bf16 bridging outputs g (widened) against the fp64 projection ref."""
    err = np.abs(g - ref)
    bad = err > bf16_ulp(ref) + BRIDGE_ATOL
    assert not bad.any(), (f"{what}: {bad.sum()} values beyond tolerance, worst err "
                           f"{err[bad].max():.3e} at |ref| {np.abs(ref[bad]).min():.3e}")
    # against the correctly rounded bf16 value: bf16 output quantisation alone gives a mean
    # |error| of ~1e-3 against fp64 for outputs of this size
    ref_b = bf16_to_f32(bf16_round(ref.astype(np.float32))).astype(np.float64)
    mism = g != ref_b
    assert mism.mean() <= 1e-2, f"{what}: {mism.mean():.2%} differ from the rounded reference"
    assert np.abs(g - ref_b).mean() <= 1e-4, f"{what}: mean distance to the rounded reference"


def check_fp8_codes(g: np.ndarray, val: np.ndarray, codes: np.ndarray, sc: float, what: str = ""):
    """GPU E4M3 codes g against the oracle's codes of val / sc: a code may differ only by
    one step, and only where the exact value lies within the GPU's arithmetic error (fp32
    accumulation as for the bf16 bridging, then one fp32 scaling) of the midpoint between
    the two codes."""
    assert g.dtype == np.uint8
    mism = g != codes
    if mism.any():
        x = val[mism] / sc
        dg, dr = oracle.e4m3_decode(g[mism]), oracle.e4m3_decode(codes[mism])
        eps = np.abs(x) * 2.0 ** -21 + BRIDGE_ATOL / sc
        mid = (dg + dr) / 2.0
        # adjacent codes: no E4M3 value lies strictly between them, so the value
        # nearest to their midpoint is one of the two
        near = oracle.e4m3_decode(oracle.e4m3_encode(mid))
        assert np.all((near == dg) | (near == dr)), f"{what}: codes further apart than one step"
        far = np.abs(x - mid) > eps
        assert not far.any(), (f"{what}: {far.sum()} codes differ away from a rounding midpoint, "
                               f"e.g. x={x[far][:3]}, gpu={dg[far][:3]}, oracle={dr[far][:3]}")
    assert mism.mean() <= 1e-3, f"{what}: {mism.mean():.2%} of the codes differ"


def kv_to_f64(inp, rows: np.ndarray, scale: float) -> np.ndarray:
    """Stored K or V rows as float64: FP8 codes through the oracle's own E4M3 decoding."""
    if rows.dtype == np.uint8:
        return oracle.dequantize_kv(rows, scale)
    return stored_to_f64(rows)


def oracle_query(inp, qi: int):
    """fp64 oracle of query qi's selector, from the stored inputs."""
    s = int(inp.q_seq[qi])
    a = int(inp.kv_start[s])
    t = int(inp.q_pos[qi])
    K = kv_to_f64(inp, inp.k[a:a + t + 1], inp.spec.k_scale)
    V = kv_to_f64(inp, inp.v[a:a + t + 1], inp.spec.v_scale)
    Q = stored_to_f64(inp.q_sel[qi])
    sp = inp.spec
    r = oracle.selector_query(Q, K, V, t, sp.window, sp.top_k, sp.scale)
    r["K"], r["V"], r["t"] = K, V, t
    return r


def oracle_sparse(inp, qi: int, layer: int, sel: np.ndarray, K=None, V=None):
    s = int(inp.q_seq[qi])
    a = int(inp.kv_start[s])
    t = int(inp.q_pos[qi])
    if K is None:
        K = kv_to_f64(inp, inp.k[a:a + t + 1], inp.spec.k_scale)
        V = kv_to_f64(inp, inp.v[a:a + t + 1], inp.spec.v_scale)
    Q = stored_to_f64(inp.q_sp[layer][qi])
    sp = inp.spec
    return oracle.sparse_attention(Q, K, V, t, sel, sp.window, sp.scale)
