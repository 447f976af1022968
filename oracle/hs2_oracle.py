"""Plain fp64 CPU oracle for the HySparse2 attention hot path.

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and
the CPU-baseline leg of the benchmark may import or run this module. The GPU
library never calls it and shares no code with it.

What it computes is the plain definition of each step, in float64, one query at a
time, with numpy matmul / exp / sort as library primitives. Inputs are the stored
values (bfloat16 or float32) widened exactly to float64 by the caller.

Sources (page title and section; the pages are news and commentary about the
HySparse2 paper):
  [arex]     arex-research.com, "Xiaomi MiMo lead Luo Fuli publishes the MiMo-V3 core
             architecture HySparse2" -- sections "Outer KV Bridging, inner KV Reuse"
             and "Numbers computed on three 80B-A3B models".
  [toolnavs] toolnavs.com (German), article on the core architecture of Xiaomi
             MiMo-V3 -- section "Was HySparse2 tut".
  [zgeo]     zgeo.com.cn, "Xiaomi HySparse2 architecture deep dive" -- section
             "Core technical principles".

Readings where the pages are silent (each one is listed with its reason in the
design notes of the repository):
  R1  per-key score = sum over the 64 query heads of the softmax probability of
      that key (the pages only say the full layer selects by its exact attention
      scores); one index set per query, shared by all heads.
  R2  the forced window of the 128 most recent tokens includes the query's own
      position: rows t-127 .. t. Candidates are rows 0 .. t-128.
  R3  softmax scale 1/sqrt(head_dim), passed explicitly; no positional encoding,
      bias, cap or sink: Q and K enter the dot product as given.
  R4  when there are at most k candidates, all of them are selected.
  R5  exact ties at the k-th score go to the smaller position.
  R6  sparse attention is a plain softmax over window U selected rows (no gate,
      no renormalisation against anything else).
  R7  KV Bridging is a plain linear map H @ W (no bias, norm or rotary embedding).
  R8  an FP8 KV cache ([arex] "Numbers computed on three 80B-A3B models" accounts the
      KV cache in FP8; the format is not named) holds OCP FP8 E4M3 codes with one
      scale per tensor: row j stands for scale * decode(codes of row j).
  R9  writing such a cache: the code of a value x is the E4M3 value nearest to
      x / scale, ties to the even mantissa, with magnitudes above 448 saturated to 448
      (the format has no infinities; the pages give no rounding rule).
"""
from __future__ import annotations

import numpy as np


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (R8), in float64.

    The OCP 8-bit floating point specification, E4M3 encoding: bit 7 is the sign, bits
    6..3 the exponent e (bias 7), bits 2..0 the mantissa m. e = 0 encodes the subnormals
    (m/8) * 2^-6; otherwise the value is (1 + m/8) * 2^(e-7). The pattern e = 15, m = 7
    (0x7F, 0xFF) is NaN; there are no infinities, so the largest finite value is
    (1 + 6/8) * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes of float64 values (R9).

    Each magnitude is rounded onto the E4M3 grid of its binade: [2^e, 2^(e+1)) for
    e >= -6 holds the 8 values (1 + m/8) * 2^e, and below 2^-6 the subnormals (m/8) * 2^-6
    share the step 2^-9 of the lowest binade. Halfway cases go to the even m (a value
    that rounds up to 2^(e+1) becomes the first value of the next binade). Magnitudes
    above 448 give 448; NaN gives 0x7F. The sign bit is kept, also for zero.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.where(np.isnan(x), 0.0, np.abs(x))
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))        # max(a, 2^-6) = f * 2^ex, f in [0.5, 1)
    step = np.exp2(ex.astype(np.float64) - 1.0 - 3.0)  # binade 2^(ex-1), 3 mantissa bits
    r = np.minimum(np.round(a / step) * step, 448.0)   # numpy rounds halves to even
    _, er = np.frexp(np.maximum(r, 2.0 ** -6))
    er = er.astype(np.int64) - 1                       # binade of the rounded value
    normal = r >= 2.0 ** -6
    e_field = np.where(normal, er + 7, 0)
    m_field = np.where(normal, r / np.exp2(er.astype(np.float64)) * 8.0 - 8.0, r / 2.0 ** -9)
    code = (e_field << 3) | np.rint(m_field).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def dequantize_kv(codes: np.ndarray, scale: float) -> np.ndarray:
    """Rows of an FP8 KV cache as the values they stand for: scale * decode(codes) (R8)."""
    return float(scale) * e4m3_decode(codes)


def logits(q: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """s[h, j] = scale * <q[h], k_j> for every query head h and given key row j.

    MQA: the single key head is shared by all query heads ([arex] "Numbers
    computed on three 80B-A3B models": 64 query heads share one KV head).
    """
    return scale * (q @ k_rows.T)


def full_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, scale: float):
    """Exact causal attention of one query at position t over rows 0..t.

    [arex] "Outer KV Bridging, inner KV Reuse": the full-attention layer computes
    exact attention, and its exact scores serve as the indexer.
    Returns (out [H, d], lse [H] natural log, p [H, t+1] softmax probabilities).
    """
    s = logits(q, K[: t + 1], scale)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    out = p @ V[: t + 1]
    return out, lse, p


def window_rows(t: int, window: int) -> np.ndarray:
    """Rows always attended: the `window` most recent positions, t included (R2).

    [arex] "Outer KV Bridging, inner KV Reuse"; [toolnavs] "Was HySparse2 tut":
    the 128 most recent tokens are always selected.
    """
    return np.arange(max(0, t - window + 1), t + 1)


def candidate_count(t: int, window: int) -> int:
    """Number of candidate rows outside the window: rows 0 .. t-window."""
    return max(0, t - window + 1)


def selection_scores(p: np.ndarray, t: int, window: int) -> np.ndarray:
    """score_j = sum_h p[h, j] for candidate rows j = 0 .. t-window (R1).

    The probabilities p are normalised over all rows 0..t, window included.
    """
    nc = candidate_count(t, window)
    return p[:, :nc].sum(axis=0)


def select_topk(scores: np.ndarray, top_k: int):
    """The top_k candidates by score, as ascending positions (R4, R5).

    [arex] "Outer KV Bridging, inner KV Reuse": 1,024 global tokens are picked by
    score from outside the window. Returns (positions ascending, tau) where tau is
    the k-th largest score (None when every candidate is taken).
    """
    nc = scores.shape[0]
    if nc <= top_k:
        return np.arange(nc, dtype=np.int64), None
    if top_k == 0:
        return np.zeros(0, dtype=np.int64), None
    order = np.lexsort((np.arange(nc), -scores))  # score descending, then position ascending
    chosen = order[:top_k]
    tau = float(scores[order[top_k - 1]])
    return np.sort(chosen), tau


def attended_rows(t: int, sel: np.ndarray, window: int) -> np.ndarray:
    """Window rows united with the selected rows (entries < 0 are padding)."""
    sel = np.asarray(sel)
    sel = sel[sel >= 0]
    return np.union1d(window_rows(t, window), sel)


def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, sel: np.ndarray,
                     window: int, scale: float):
    """Softmax attention of one query over the window plus the selected rows only (R6).

    [arex] "Outer KV Bridging, inner KV Reuse" and [zgeo] "Core technical principles":
    each sparse layer of a hybrid block reuses the full layer's KV cache and its
    selection indices; the recent window and the global tokens share that cache.
    Returns (out [H, d], lse [H]).
    """
    rows = attended_rows(t, sel, window)
    s = logits(q, K[rows], scale)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ V[rows], lse


def bridge_kv(H: np.ndarray, w_k: list, w_v: list):
    """K_l = H @ W_K^l and V_l = H @ W_V^l for every bridged layer l (R7).

    [arex] "Outer KV Bridging, inner KV Reuse"; [toolnavs] "Was HySparse2 tut":
    each cross-decoder full layer builds its own KV cache from the input hidden
    states of the matching self-decoder full layer, through its own K/V projection;
    one hidden-state source may feed several layers.
    """
    return [H @ w for w in w_k], [H @ w for w in w_v]


def bridge_kv_fp8(H: np.ndarray, w_k: list, w_v: list, k_scales: list, v_scales: list):
    """KV Bridging into FP8 caches (R7, R8, R9): layer l's K cache holds the E4M3 codes
    of (H @ W_K^l) / k_scales[l], its V cache those of (H @ W_V^l) / v_scales[l]."""
    ks, vs = bridge_kv(H, w_k, w_v)
    return ([e4m3_encode(k / float(s)) for k, s in zip(ks, k_scales)],
            [e4m3_encode(v / float(s)) for v, s in zip(vs, v_scales)])


def selector_query(q_sel: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, window: int,
                   top_k: int, scale: float) -> dict:
    """The full-attention selector for one query: output, LSE, scores, selection."""
    out, lse, p = full_attention(q_sel, K, V, t, scale)
    scores = selection_scores(p, t, window)
    sel, tau = select_topk(scores, top_k)
    padded = np.full(top_k, -1, dtype=np.int64)
    padded[: sel.shape[0]] = sel
    return {"out": out, "lse": lse, "scores": scores, "sel": sel, "sel_padded": padded,
            "count": int(sel.shape[0]), "tau": tau}


def block_query(q_sel: np.ndarray, q_sparse: list, K: np.ndarray, V: np.ndarray, t: int,
                window: int, top_k: int, scale: float) -> dict:
    """One hybrid block for one query: selector, then every sparse layer on its index set."""
    r = selector_query(q_sel, K, V, t, window, top_k, scale)
    r["sparse"] = [sparse_attention(q, K, V, t, r["sel"], window, scale) for q in q_sparse]
    return r
