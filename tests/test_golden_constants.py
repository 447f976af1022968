"""The workloads and the oracle use the constants the pages state (tests/golden)."""
import json
import math
import os

import numpy as np

import oracle
from workloads import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "method_constants.json")


def _g():
    with open(GOLDEN) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def test_workload_constants_match_pages():
    g = _g()
    assert configs.WINDOW == g["window"]
    assert configs.TOP_K == g["top_k"]
    assert configs.N_HEADS == g["q_heads"]
    assert configs.D_MODEL == g["d_model"]
    for n in (1, 2, 3, 4):
        s = configs.block_config(n)
        assert (s.window, s.top_k, s.n_heads) == (g["window"], g["top_k"], g["q_heads"])


def test_attended_budget_is_window_plus_topk():
    """At any context, a query attends to at most window + top_k rows (1,152)."""
    g = _g()
    W, k = g["window"], g["top_k"]
    rng = np.random.default_rng(0)
    H, d = g["q_heads"], 128
    for t in (W + k - 1, W + k, W + k + 500):
        q = rng.standard_normal((H, d))
        K = rng.standard_normal((t + 1, d))
        V = rng.standard_normal((t + 1, d))
        r = oracle.selector_query(q, K, V, t, W, k, 1 / math.sqrt(d))
        assert oracle.attended_rows(t, r["sel"], W).shape[0] == min(t + 1, W + k)


def test_pages_accounting_is_self_consistent():
    """The pages' KV-cache figures: 12.09 / 2.69 is the quoted ~4.5x, and
    12.09 / 6.72 matches the 9 : 5 full-attention layer counts."""
    g = _g()
    kv = g["kv_cache_gb_at_1m_fp8"]
    fl = g["full_attention_layers"]
    assert abs(kv["Hybrid SWA"] / kv["HySparse2"] - 4.5) < 0.05
    assert abs(kv["Hybrid SWA"] / kv["HySparse"] - fl["Hybrid SWA"] / fl["HySparse"]) < 0.01
