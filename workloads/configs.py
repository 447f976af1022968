"""The five workloads of the hot path and a builder for scaled-down variants.

Shapes follow the method's constants: 64 query heads sharing one KV head (MQA),
head_dim 128, a forced window of the 128 most recent tokens plus 1,024 selected
tokens, and 2,048-wide self-decoder hidden states for KV Bridging.

Input recipe (identical for every workload; only sizes, dtype and seed change):
  * Q of the selector layer and of each sparse layer, K and V: N(0, std^2) drawn
    in float32 from chunk-seeded PCG64 streams, rounded to the stored dtype
    (bfloat16 RNE, or kept float32). dtype "fp8": Q in bfloat16, K and V as OCP FP8
    E4M3 codes of value / k_scale and value / v_scale (RNE, saturated at 448).
  * Needles: for needle n of global query i, head h = (needles_per_query*i + n)
    mod 64; the key row at position p is replaced by 12 * Q_sel[i, h] / |Q_sel[i, h]|
    (computed in float64 from the stored query, then rounded to the stored dtype),
    so that head h of query i sees a logit near 12 there. Positions are distinct,
    uniform over the keys that are candidates (outside the window) for every query
    of that sequence. V rows are left as drawn.
  * Bridging: H ~ N(0, 1) bf16 [N, 2048]; W_K^l, W_V^l ~ N(0, 0.02^2) bf16 [2048, 128].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .gen import bf16_round, bf16_to_f32, e4m3_encode, normal_f32, rng

N_HEADS = 64
HEAD_DIM = 128
WINDOW = 128
TOP_K = 1024
D_MODEL = 2048
NEEDLE_LOGIT = 12.0

# tensor tags for the chunk-seeded streams
_TAG_K, _TAG_V, _TAG_QSEL, _TAG_QSP = 1, 2, 3, 100
_TAG_H, _TAG_WK, _TAG_WV = 10, 20, 40
_TAG_NEEDLE_POS, _TAG_LENGTHS = 7, 8


@dataclass
class BlockSpec:
    """One hybrid block workload: a selector layer plus `n_sparse` sparse layers."""

    name: str
    seq_lens: list[int]
    q_positions: list[list[int]]          # per sequence, the positions t of its queries
    dtype: str = "bf16"                   # "bf16", "f32" or "fp8" (FP8 E4M3 K/V, bf16 Q)
    n_sparse: int = 7
    needles_per_query: int = 8
    seed: int = 0
    kv_std: float = 1.0
    window: int = WINDOW
    top_k: int = TOP_K
    n_heads: int = N_HEADS
    head_dim: int = HEAD_DIM
    k_scale: float = 0.05                 # dtype "fp8": value = scale * E4M3 code value
    v_scale: float = 0.03

    @property
    def total_q(self) -> int:
        return sum(len(p) for p in self.q_positions)

    @property
    def total_rows(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclass
class BlockInputs:
    spec: BlockSpec
    q_sel: np.ndarray                      # [total_q, H, d] stored (uint16 bf16 bits or float32)
    q_sp: list[np.ndarray]                 # n_sparse x [total_q, H, d]
    k: np.ndarray                          # [total_rows, d]
    v: np.ndarray                          # [total_rows, d]
    kv_start: np.ndarray                   # int64 [S]
    kv_len: np.ndarray                     # int32 [S]
    q_start: np.ndarray                    # int32 [S+1]
    q_pos: np.ndarray                      # int32 [total_q]
    q_seq: np.ndarray                      # int32 [total_q] sequence of each query
    needles: list[tuple[int, int, int, int]] = field(default_factory=list)  # (seq, query, head, pos)

    @property
    def scale(self) -> float:
        return self.spec.scale


@dataclass
class BridgeInputs:
    h: np.ndarray                          # uint16 bf16 [N, D_MODEL]
    w_k: list[np.ndarray]                  # L x uint16 bf16 [D_MODEL, HEAD_DIM]
    w_v: list[np.ndarray]


def _stored(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype in ("bf16", "fp8") else x


def _stored_kv(x: np.ndarray, spec: "BlockSpec", scale: float) -> np.ndarray:
    return e4m3_encode(x, scale) if spec.dtype == "fp8" else _stored(x, spec.dtype)


def _as_f32(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(x) if x.dtype == np.uint16 else x


def make_block_inputs(spec: BlockSpec) -> BlockInputs:
    H, d = spec.n_heads, spec.head_dim
    S = len(spec.seq_lens)
    assert len(spec.q_positions) == S
    rows = spec.total_rows
    nq = spec.total_q
    s = spec.seed

    k = _stored_kv(normal_f32(s, _TAG_K, rows * d, spec.kv_std), spec, spec.k_scale).reshape(rows, d)
    v = _stored_kv(normal_f32(s, _TAG_V, rows * d, spec.kv_std), spec, spec.v_scale).reshape(rows, d)
    q_sel = _stored(normal_f32(s, _TAG_QSEL, nq * H * d), spec.dtype).reshape(nq, H, d)
    q_sp = [
        _stored(normal_f32(s, _TAG_QSP + l, nq * H * d), spec.dtype).reshape(nq, H, d)
        for l in range(spec.n_sparse)
    ]

    kv_len = np.asarray(spec.seq_lens, dtype=np.int32)
    kv_start = np.zeros(S, dtype=np.int64)
    if S > 1:
        kv_start[1:] = np.cumsum(kv_len[:-1], dtype=np.int64)
    q_start = np.zeros(S + 1, dtype=np.int32)
    q_start[1:] = np.cumsum([len(p) for p in spec.q_positions])
    q_pos = np.concatenate([np.asarray(p, dtype=np.int32) for p in spec.q_positions]) if nq else np.zeros(0, np.int32)
    q_seq = np.concatenate([np.full(len(p), i, dtype=np.int32) for i, p in enumerate(spec.q_positions)]) if nq else np.zeros(0, np.int32)
    for i in range(S):
        assert all(0 <= t < spec.seq_lens[i] for t in spec.q_positions[i]), "query position outside its sequence"

    needles: list[tuple[int, int, int, int]] = []
    g = rng(s, _TAG_NEEDLE_POS)
    qsel32 = _as_f32(q_sel)
    for si in range(S):
        qs = range(int(q_start[si]), int(q_start[si + 1]))
        if not len(qs) or spec.needles_per_query <= 0:
            continue
        hi = min(spec.q_positions[si]) - spec.window  # last position that is a candidate for every query
        want = len(qs) * spec.needles_per_query
        if hi + 1 < want:
            continue
        pos = g.choice(hi + 1, size=want, replace=False)
        c = 0
        for qi in qs:
            for n in range(spec.needles_per_query):
                h = (spec.needles_per_query * qi + n) % H
                qv = qsel32[qi, h].astype(np.float64)
                key = (NEEDLE_LOGIT * qv / np.linalg.norm(qv)).astype(np.float32)
                p = int(pos[c])
                c += 1
                k[kv_start[si] + p] = _stored_kv(key, spec, spec.k_scale)
                needles.append((si, qi, h, p))
    return BlockInputs(spec, q_sel, q_sp, k, v, kv_start, kv_len, q_start, q_pos, q_seq, needles)


def make_bridge_inputs(n_rows: int, n_layers: int = 3, seed: int = 5, d_model: int = D_MODEL,
                       head_dim: int = HEAD_DIM, w_std: float = 0.02) -> BridgeInputs:
    h = bf16_round(normal_f32(seed, _TAG_H, n_rows * d_model)).reshape(n_rows, d_model)
    w_k = [bf16_round(normal_f32(seed, _TAG_WK + l, d_model * head_dim, w_std)).reshape(d_model, head_dim)
           for l in range(n_layers)]
    w_v = [bf16_round(normal_f32(seed, _TAG_WV + l, d_model * head_dim, w_std)).reshape(d_model, head_dim)
           for l in range(n_layers)]
    return BridgeInputs(h, w_k, w_v)


def ragged_lengths(seed: int, n_seqs: int, lo: int, hi: int) -> list[int]:
    """Context lengths log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi)))."""
    g = rng(seed, _TAG_LENGTHS)
    u = g.uniform(math.log(lo), math.log(hi), size=n_seqs)
    return [int(round(math.exp(x))) for x in u]


def block_config(n: int, **over) -> BlockSpec:
    """BlockSpec of workload n (1..6), with optional overrides (for scaled-down variants).

    Workload 6 is workload 2 on an FP8 E4M3 K/V cache (the pages' KV accounting is FP8).
    Workload 7 is a prefill: exact causal attention of every position of a 262,144-token
    sequence (the self-decoder's full-attention layer), followed in the benchmark by the
    KV Bridging of the same number of hidden states."""
    if n == 1:
        spec = BlockSpec("tiny-4096-f32", [4096], [list(range(4080, 4096))], dtype="f32",
                         n_sparse=2, needles_per_query=8, seed=1)
    elif n == 2:
        L = 131072
        spec = BlockSpec("decode-64x128k-bf16", [L] * 64, [[L - 1]] * 64, n_sparse=7,
                         needles_per_query=8, seed=2)
    elif n == 3:
        L = 1048576
        spec = BlockSpec("decode-8x1M-bf16", [L] * 8, [[L - 1]] * 8, n_sparse=7,
                         needles_per_query=8, seed=3)
    elif n == 4:
        L = 262144
        spec = BlockSpec("chunk-4096q-at-256k-bf16", [L], [list(range(258048, 262144))], n_sparse=3,
                         needles_per_query=1, seed=4)
    elif n == 5:
        lens = ragged_lengths(5, 32, 4096, 524288)
        spec = BlockSpec("ragged-decode-32-4k-512k-bf16", lens, [[x - 1] for x in lens], n_sparse=7,
                         needles_per_query=8, seed=5, kv_std=math.sqrt(D_MODEL) * 0.02)
    elif n == 7:
        L = 262144
        spec = BlockSpec("prefill-262144-bf16", [L], [list(range(L))], n_sparse=0, needles_per_query=0, seed=7)
    elif n == 6:
        L = 131072
        spec = BlockSpec("decode-64x128k-fp8kv", [L] * 64, [[L - 1]] * 64, dtype="fp8", n_sparse=7,
                         needles_per_query=8, seed=6)
    else:
        raise ValueError(n)
    for key, val in over.items():
        setattr(spec, key, val)
    return spec


CONFIGS = {
    1: "Tiny block: 1 seq x 4096 ctx, 16 causal queries, fp32, 1 selector + 2 sparse layers",
    2: "Batched decode: 64 seqs x 131072 ctx, 1 query each, bf16, 1 selector + 7 sparse layers",
    3: "Long decode: 8 seqs x 1048576 ctx, 1 query each, bf16, 1 selector + 7 sparse layers",
    4: "Chunked selection: 1 seq x 262144 ctx, 4096 queries at 258048..262143, bf16, 1 selector + 3 sparse",
    5: "KV Bridging N=1048576 x 2048 -> 3 layers' K/V; ragged decode 32 seqs 4k-512k, 1 selector + 7 sparse",
}
