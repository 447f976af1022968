"""Plain fp64 CPU oracle of the first-generation HySparse layout (the comparison variant).

TEST INFRASTRUCTURE. Only the tests, the smoke check of the package entry file and
the CPU-baseline leg of the benchmark may import or run this module. The GPU
library never calls it and shares no code with it.

Sources (page title and section):
  [arex]     arex-research.com, "Xiaomi MiMo lead Luo Fuli publishes the MiMo-V3 core
             architecture HySparse2" -- section "Outer KV Bridging, inner KV Reuse" (the
             predecessor picks 1,024 global tokens as 64-token blocks and adds a separate
             128-token SWA branch fused through a gate; each full layer hands its KV
             cache and top-k block indices to the following sparse layers); section
             "Numbers computed on three 80B-A3B models" (the predecessor uses GQA with
             64 query heads on 4 KV heads); section "Lost points, the 290B check and
             open questions" (the gated SWA branch has its own projections and local
             KV cache).
  [toolnavs] toolnavs.com (German), article on the core architecture of Xiaomi MiMo-V3,
             section "Was HySparse2 tut" (block-level selection of the first generation).

Readings where the pages are silent (each listed with its reason in the design notes):
  V1  GQA 64:4: query head h reads KV head h // 16 (16 consecutive query heads share one
      KV head).
  V2  Blocks are the aligned 64-position spans 64b .. 64b+63 of a sequence. Every block
      holding at least one position <= t is a candidate, the partial block of t included.
  V3  Block score (one index set per query and KV head): the softmax probabilities of the
      full layer, summed over the block's positions <= t and over the 16 query heads of
      that KV head.
  V4  The 16 best blocks are kept (1,024 tokens); all of them when there are at most 16;
      exact ties go to the smaller block index.
  V5  The sparse branch of head h attends to every position <= t of the blocks selected
      for its KV head. The SWA branch attends to positions max(0, t-127) .. t of the
      layer's own K/V (its own projections, a separate local cache), with the same query.
      Each branch is its own softmax; a branch with no attended position (only padding
      entries given) contributes zero.
  V6  Gated fusion: out_h = g_sparse[h] * o_sparse_h + g_swa[h] * o_swa_h with gate
      values given per query and head (how the gate is computed is not on the pages).
  V7  The full layer itself is plain exact causal attention (no SWA branch, no gate).
  Scale, positional encoding and storage widening are as in the HySparse2 oracle (R3).
"""
from __future__ import annotations

import numpy as np

N_HEADS = 64
N_KV_HEADS = 4
GROUP = N_HEADS // N_KV_HEADS   # 16 query heads per KV head
BLOCK = 64                      # tokens per selection block
TOP_BLOCKS = 16                 # 16 x 64 = 1,024 selected tokens
SWA_WINDOW = 128


def kv_head_of(h: int) -> int:
    """KV head read by query head h (V1)."""
    return h // GROUP


def gqa_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, rows_of_group):
    """Softmax attention of the 64 query heads, head h over K[rows, h//16], V[rows, h//16].

    q: [64, d]; K, V: [n_rows, 4, d]; rows_of_group(g) gives the attended rows of KV head g.
    Returns (out [64, d], lse [64], p) where p[h] are the probabilities over head h's rows.
    """
    out = np.zeros((q.shape[0], q.shape[1]))
    lse = np.zeros(q.shape[0])
    probs = []
    for h in range(q.shape[0]):
        g = kv_head_of(h)
        rows = rows_of_group(g)
        if len(rows) == 0:          # empty branch: contributes zero (V5)
            lse[h] = -np.inf
            probs.append(np.zeros(0))
            continue
        s = K[rows, g] @ q[h]
        m = s.max()
        lse[h] = m + np.log(np.exp(s - m).sum())
        p = np.exp(s - lse[h])
        out[h] = p @ V[rows, g]
        probs.append(p)
    return out, lse, probs


def full_attention_gqa(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, scale: float):
    """Exact causal attention of one query at position t over rows 0..t (V7).

    Returns (out [64, d], lse [64] natural log, p [64, t+1] probabilities).
    """
    rows = np.arange(t + 1)
    out, lse, probs = gqa_attention(scale * q, K, V, lambda g: rows)
    return out, lse, np.stack(probs)


def block_count(t: int) -> int:
    """Candidate blocks of a query at position t: every block with a position <= t (V2)."""
    return t // BLOCK + 1


def block_scores(p: np.ndarray, t: int) -> np.ndarray:
    """score[g, b] = sum over heads h of group g and positions j <= t of block b of p[h, j] (V3)."""
    nb = block_count(t)
    per_head = np.zeros((p.shape[0], nb))
    for b in range(nb):
        per_head[:, b] = p[:, b * BLOCK: min(t + 1, (b + 1) * BLOCK)].sum(axis=1)
    return per_head.reshape(N_KV_HEADS, GROUP, nb).sum(axis=1)


def select_blocks(scores: np.ndarray, top_blocks: int):
    """The top_blocks best blocks of one KV head, ascending; ties to the smaller index (V4).

    Returns (blocks ascending, tau) with tau the kept score of rank top_blocks (None when
    every candidate is kept).
    """
    nb = scores.shape[0]
    if nb <= top_blocks:
        return np.arange(nb, dtype=np.int64), None
    order = np.lexsort((np.arange(nb), -scores))  # score descending, then index ascending
    return np.sort(order[:top_blocks]), float(scores[order[top_blocks - 1]])


def v1_selector_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, scale: float,
                      top_blocks: int = TOP_BLOCKS) -> dict:
    """The v1 full-attention layer for one query: exact output, LSE, block scores and the
    block index set of every KV head."""
    out, lse, p = full_attention_gqa(q, K, V, t, scale)
    sc = block_scores(p, t)
    sel, tau = [], []
    for g in range(N_KV_HEADS):
        s_g, tau_g = select_blocks(sc[g], top_blocks)
        sel.append(s_g)
        tau.append(tau_g)
    return {"out": out, "lse": lse, "scores": sc, "sel": sel, "tau": tau}


def sparse_rows(t: int, blocks: np.ndarray) -> np.ndarray:
    """Positions <= t of the given blocks (entries < 0 are padding) (V5)."""
    blocks = np.asarray(blocks)
    blocks = np.unique(blocks[blocks >= 0])
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    rows = (blocks[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    return rows[rows <= t]


def swa_rows(t: int, window: int = SWA_WINDOW) -> np.ndarray:
    """Positions of the SWA branch: the `window` most recent, t included (V5)."""
    return np.arange(max(0, t - window + 1), t + 1)


def v1_sparse_query(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int, blocks: list,
                    K_swa: np.ndarray, V_swa: np.ndarray, gate_sparse: np.ndarray,
                    gate_swa: np.ndarray, scale: float, window: int = SWA_WINDOW):
    """A v1 sparse layer for one query: sparse branch over the selected blocks of the
    shared cache K, V (indexed by position), SWA branch over the layer's own K_swa, V_swa
    (indexed by position), fused by the gates (V5, V6).

    Returns (out [64, d], o_sparse [64, d], o_swa [64, d]).
    """
    rows_sp = [sparse_rows(t, blocks[g]) for g in range(N_KV_HEADS)]
    o_sp, _, _ = gqa_attention(scale * q, K, V, lambda g: rows_sp[g])
    w = swa_rows(t, window)
    o_sw, _, _ = gqa_attention(scale * q, K_swa, V_swa, lambda g: w)
    out = gate_sparse[:, None] * o_sp + gate_swa[:, None] * o_sw
    return out, o_sp, o_sw
