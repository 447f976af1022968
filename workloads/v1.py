"""Workloads of the first-generation HySparse layout (the comparison variant).

Shapes: 64 query heads on 4 KV heads (GQA 64:4), head_dim 128, 64-token selection blocks
with 16 kept per KV head (1,024 tokens), a 128-token sliding-window branch on each sparse
layer's own K/V, one selector layer plus n_sparse sparse layers per hybrid block.

Input recipe (as for the HySparse2 workloads; only the tags differ):
  * Q of the selector and of each sparse layer, K and V of the shared cache, and K and V
    of each sparse layer's window ring: N(0, std^2) drawn in float32 from chunk-seeded
    PCG64 streams, rounded to bfloat16 (RNE). Cache rows are [4 KV heads][128].
  * The window ring of sequence s has `swa_slots` rows; position p lives in slot
    p mod swa_slots (the ring holds the recent positions of every query of s).
  * Gates: uniform on [0, 1) in float32, one per query, head and branch.
  * Needles: needle n of global query i sits in KV head g = n mod 4 for query head
    h = 16 g + (i + n // 4) mod 16; the K row of KV head g at position p is replaced by
    12 * Q_sel[i, h] / |Q_sel[i, h]| (float64 from the stored query, rounded to bf16), so
    head h sees a logit near 12 there and p's block dominates KV head g's block scores.
    Positions are distinct and uniform over 0 .. (smallest query position of the
    sequence) - 128.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .gen import bf16_round, bf16_to_f32, normal_f32, normal_f32_range, rng

N_HEADS = 64
N_KV = 4
GROUP = 16
HEAD_DIM = 128
BLOCK = 64
TOP_BLOCKS = 16
WINDOW = 128
NEEDLE_LOGIT = 12.0
ROW = N_KV * HEAD_DIM   # elements per cache row

_TAG_K, _TAG_V, _TAG_QSEL, _TAG_NEEDLE_POS = 1001, 1002, 1003, 1007
_TAG_QSP, _TAG_KSWA, _TAG_VSWA, _TAG_GSP, _TAG_GSW = 1100, 1200, 1300, 1400, 1500


@dataclass
class V1Spec:
    name: str
    seq_lens: list[int]
    q_positions: list[list[int]]
    n_sparse: int = 7
    needles_per_query: int = 8
    seed: int = 0
    kv_std: float = 1.0
    window: int = WINDOW
    top_blocks: int = TOP_BLOCKS
    swa_slots: int = 0      # 0: window + the spread of one sequence's query positions, rounded up to 64

    @property
    def total_q(self) -> int:
        return sum(len(p) for p in self.q_positions)

    @property
    def total_rows(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)

    @property
    def ring(self) -> int:
        if self.swa_slots:
            return self.swa_slots
        spread = max((max(p) - min(p)) if p else 0 for p in self.q_positions)
        return (self.window + spread + 63) // 64 * 64


@dataclass
class V1Inputs:
    spec: V1Spec
    q_sel: np.ndarray                 # uint16 bf16 [total_q, 64, 128]
    q_sp: list[np.ndarray]            # n_sparse x [total_q, 64, 128]
    k_swa: list[np.ndarray]           # n_sparse x uint16 [num_seqs, ring, 4, 128]
    v_swa: list[np.ndarray]
    gate_sp: list[np.ndarray]         # n_sparse x float32 [total_q, 64]
    gate_swa: list[np.ndarray]
    kv_start: np.ndarray              # int64 [S]
    kv_len: np.ndarray                # int32 [S]
    q_start: np.ndarray               # int32 [S+1]
    q_pos: np.ndarray                 # int32 [total_q]
    q_seq: np.ndarray                 # int32 [total_q]
    needles: list[tuple[int, int, np.ndarray]] = field(default_factory=list)  # (row, kv head, bf16 [128])
    k: np.ndarray | None = None       # uint16 [total_rows, 4, 128] when built whole
    v: np.ndarray | None = None


def kv_rows(inp: V1Inputs, name: str, lo: int, hi: int) -> np.ndarray:
    """Stored rows lo .. hi-1 of the shared cache ("k" or "v"), needles included:
    uint16 bf16 [hi-lo, 4, 128]. Identical to the same rows of the whole tensor."""
    sp = inp.spec
    tag = _TAG_K if name == "k" else _TAG_V
    x = bf16_round(normal_f32_range(sp.seed, tag, lo * ROW, hi * ROW, sp.kv_std)).reshape(hi - lo, N_KV, HEAD_DIM)
    if name == "k":
        for row, g, vec in inp.needles:
            if lo <= row < hi:
                x[row - lo, g] = vec
    return x


def make_v1_inputs(spec: V1Spec, with_kv: bool = True) -> V1Inputs:
    S = len(spec.seq_lens)
    assert len(spec.q_positions) == S
    nq = spec.total_q
    s = spec.seed
    R = spec.ring
    q_sel = bf16_round(normal_f32(s, _TAG_QSEL, nq * N_HEADS * HEAD_DIM)).reshape(nq, N_HEADS, HEAD_DIM)
    q_sp, k_swa, v_swa, g_sp, g_sw = [], [], [], [], []
    for l in range(spec.n_sparse):
        q_sp.append(bf16_round(normal_f32(s, _TAG_QSP + l, nq * N_HEADS * HEAD_DIM)).reshape(nq, N_HEADS, HEAD_DIM))
        k_swa.append(bf16_round(normal_f32(s, _TAG_KSWA + l, S * R * ROW, spec.kv_std)).reshape(S, R, N_KV, HEAD_DIM))
        v_swa.append(bf16_round(normal_f32(s, _TAG_VSWA + l, S * R * ROW, spec.kv_std)).reshape(S, R, N_KV, HEAD_DIM))
        g_sp.append(rng(s, _TAG_GSP + l).random((nq, N_HEADS), dtype=np.float32))
        g_sw.append(rng(s, _TAG_GSW + l).random((nq, N_HEADS), dtype=np.float32))
    kv_len = np.asarray(spec.seq_lens, dtype=np.int32)
    kv_start = np.zeros(S, dtype=np.int64)
    if S > 1:
        kv_start[1:] = np.cumsum(kv_len[:-1].astype(np.int64))
    q_start = np.zeros(S + 1, dtype=np.int32)
    q_start[1:] = np.cumsum([len(p) for p in spec.q_positions])
    q_pos = np.concatenate([np.asarray(p, dtype=np.int32) for p in spec.q_positions]) if nq else np.zeros(0, np.int32)
    q_seq = (np.concatenate([np.full(len(p), i, dtype=np.int32) for i, p in enumerate(spec.q_positions)])
             if nq else np.zeros(0, np.int32))
    inp = V1Inputs(spec, q_sel, q_sp, k_swa, v_swa, g_sp, g_sw, kv_start, kv_len, q_start, q_pos, q_seq)

    g = rng(s, _TAG_NEEDLE_POS)
    qsel32 = bf16_to_f32(q_sel)
    for si in range(S):
        qs = range(int(q_start[si]), int(q_start[si + 1]))
        if not len(qs) or spec.needles_per_query == 0:
            continue
        hi = min(spec.q_positions[si]) - spec.window
        want = len(qs) * spec.needles_per_query
        if hi + 1 < want:
            continue
        pos = g.choice(hi + 1, size=want, replace=False)
        c = 0
        for qi in qs:
            for n in range(spec.needles_per_query):
                kvh = n % N_KV
                h = GROUP * kvh + (qi + n // N_KV) % GROUP
                qv = qsel32[qi, h].astype(np.float64)
                vec = bf16_round((NEEDLE_LOGIT * qv / np.linalg.norm(qv)).astype(np.float32))
                inp.needles.append((int(kv_start[si] + pos[c]), kvh, vec))
                c += 1
    if with_kv:
        inp.k = kv_rows(inp, "k", 0, spec.total_rows)
        inp.v = kv_rows(inp, "v", 0, spec.total_rows)
    return inp


def v1_config(n: int, **over) -> V1Spec:
    """Workload 9: the v1 layout on the decode batch of workload 2 (64 sequences of
    131,072 tokens, one query each, one selector and seven sparse layers). Workload 10:
    a small ragged case (short sequences, partial blocks, t = 0, several queries per
    sequence) the oracle finishes in seconds."""
    if n == 9:
        L = 131072
        spec = V1Spec("decode-64x128k-gqa4-v1", [L] * 64, [[L - 1]] * 64, n_sparse=7, seed=9)
    elif n == 10:
        spec = V1Spec("ragged-small-gqa4-v1", [4096, 1000, 64, 1, 2100],
                      [[4095, 4000, 2047, 1100, 1023, 64, 63], [999, 500], [63, 0], [0], [2099, 2050]],
                      n_sparse=2, needles_per_query=8, seed=10)
    else:
        raise ValueError(n)
    for key, val in over.items():
        setattr(spec, key, val)
    return spec
