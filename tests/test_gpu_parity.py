"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases are checked on every output element; the five workloads at full size
are checked element by element on every query of the decode batches (64 x 128k in
bf16 and FP8, 8 x 1M, the 32 ragged sequences) and on 72 queries of the 4,096-query
chunk, plus properties that hold for every query (counts, ordering, planted needles).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_mqa_amd import hs2
from tests.parity import (BRIDGE_ATOL, FEW_KEYS, check_attn, check_bridge_bf16, check_fp8_codes, check_lse,
                          check_selection, from_dev, oracle_query, oracle_sparse, to_dev)
from workloads.configs import BlockSpec, block_config, make_block_inputs, make_bridge_inputs
from workloads.gen import bf16_round, bf16_to_f32, e4m3_encode, stored_to_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_block(inp, selector_only=False):
    """Runs the selector and every sparse layer of a block on the GPU."""
    sp = inp.spec
    dev = "cuda"
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, sp.total_rows, dev)
    k = to_dev(inp.k)
    v = to_dev(inp.v)
    q = to_dev(inp.q_sel)
    fp8 = sp.dtype == "fp8"
    if fp8:
        out, lse, sel, cnt = hs2.full_attn_select_fp8kv(batch, q, k, v, sp.k_scale, sp.v_scale, sp.window, sp.top_k,
                                                        sp.scale)
    else:
        out, lse, sel, cnt = hs2.full_attn_select(batch, q, k, v, sp.window, sp.top_k, sp.scale)
    sparse = []
    if not selector_only:
        for l in range(sp.n_sparse):
            qs = to_dev(inp.q_sp[l])
            if fp8:
                o, _ = hs2.sparse_attn_fp8kv(batch, qs, k, v, sp.k_scale, sp.v_scale, sel, sp.window, sp.top_k,
                                             sp.scale)
            else:
                o, _ = hs2.sparse_attn(batch, qs, k, v, sel, sp.window, sp.top_k, sp.scale)
            sparse.append(from_dev(o))
    torch.cuda.synchronize()
    return {"out": from_dev(out), "lse": from_dev(lse), "sel": sel.cpu().numpy(), "count": cnt.cpu().numpy(),
            "sparse": sparse, "batch": batch, "k": k, "v": v}


def check_queries(inp, g, qis, what):
    sp = inp.spec
    rr = sp.dtype == "fp8"  # FP8 K/V: the mean rule counts the error beyond the bf16 output rounding
    swapped = 0
    for qi in qis:
        r = oracle_query(inp, qi)
        t = r["t"]
        nc = oracle.candidate_count(t, sp.window)
        tag = f"{what} q{qi} t={t}"
        few = t + 1 <= FEW_KEYS   # every layer of such a query attends all t + 1 keys
        check_attn(g["out"][qi], r["out"], tag + " selector out", beyond_rounding=rr, few_keys=few)
        check_lse(g["lse"][qi], r["lse"], tag)
        swapped += check_selection(g["sel"][qi], int(g["count"][qi]), r, sp.top_k, nc, tag)
        for l, o in enumerate(g["sparse"]):
            ref, _ = oracle_sparse(inp, qi, l, g["sel"][qi], r["K"], r["V"])
            check_attn(o[qi], ref, tag + f" sparse layer {l}", beyond_rounding=rr, few_keys=few)
    return swapped


def check_all_queries_properties(inp, g):
    sp = inp.spec
    for qi in range(sp.total_q):
        t = int(inp.q_pos[qi])
        nc = max(0, t - sp.window + 1)
        k_eff = min(sp.top_k, nc)
        assert int(g["count"][qi]) == k_eff
        s = g["sel"][qi][:k_eff]
        assert np.all(np.diff(s) > 0) and (k_eff == 0 or (s[0] >= 0 and s[-1] < nc))
        assert np.all(g["sel"][qi][k_eff:] == -1)
    for (si, qi, h, p) in inp.needles:
        assert p in set(g["sel"][qi].tolist()), f"needle at {p} of query {qi} not selected"
    assert np.isfinite(g["out"]).all()
    for o in g["sparse"]:
        assert np.isfinite(o).all()


# ----------------------------------------------------------------------------------
# small cases: every output checked
# ----------------------------------------------------------------------------------

def test_tiny_block_f32():
    """Workload 1: 1 seq x 4096, 16 queries, fp32, selector + 2 sparse layers."""
    inp = make_block_inputs(block_config(1))
    _say("tiny f32 block")
    g = run_block(inp)
    check_queries(inp, g, range(inp.spec.total_q), "tiny-f32")
    check_all_queries_properties(inp, g)


def test_tiny_block_bf16():
    inp = make_block_inputs(block_config(1, dtype="bf16", seed=11))
    _say("tiny bf16 block")
    g = run_block(inp)
    check_queries(inp, g, range(inp.spec.total_q), "tiny-bf16")
    check_all_queries_properties(inp, g)


def test_tiny_block_fp8():
    """Workload 1's shape with an FP8 E4M3 K/V cache (per-tensor scales 0.05 and 0.03)."""
    inp = make_block_inputs(block_config(1, dtype="fp8", seed=14))
    _say("tiny fp8 block")
    g = run_block(inp)
    check_queries(inp, g, range(inp.spec.total_q), "tiny-fp8")
    check_all_queries_properties(inp, g)


RAGGED = BlockSpec(
    "ragged-small", [700, 1152, 1153, 3000, 9000, 40000],
    [[699, 100, 0], [1151], [1152], [2999, 2000], [8999, 5000, 127, 128, 1151, 1152], [39999]],
    dtype="bf16", n_sparse=2, needles_per_query=2, seed=12)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_ragged_small_contexts(dtype):
    """Several sequences and queries per sequence; t < window, candidates <= k and > k."""
    spec = BlockSpec(**{**RAGGED.__dict__, "dtype": dtype})
    inp = make_block_inputs(spec)
    _say(f"ragged small {dtype}")
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), f"ragged-{dtype}")
    check_all_queries_properties(inp, g)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_few_key_queries(dtype):
    """Decode-shaped selector and sparse layers on queries that attend one to five keys
    (t = 0..4), next to longer ones in the same batch."""
    spec = BlockSpec("few-keys", [2, 3, 4, 5, 6, 50, 2000],
                     [[1], [2, 0], [3, 1], [4, 2], [5, 3, 1], [1, 2, 3, 49], [4, 1999]],
                     dtype=dtype, n_sparse=1, needles_per_query=0, seed=43)
    inp = make_block_inputs(spec)
    _say(f"few-key queries {dtype}")
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), f"few-keys-{dtype}")
    check_all_queries_properties(inp, g)


def test_chunked_ragged_queries():
    """Many queries per sequence (the q-tile kernels): query counts not multiples of the
    tile size, queries with t < window and with at most k candidates in the same tile."""
    spec = BlockSpec("chunked", [3000, 9000, 700],
                     [list(range(2980, 2993)), [8999, 8000, 7000, 5000, 4000, 1200, 1100, 127],
                      [699, 698, 500, 400, 300, 200, 127, 5, 0]],
                     dtype="bf16", n_sparse=1, needles_per_query=1, seed=19)
    inp = make_block_inputs(spec)
    _say("chunked ragged")
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), "chunked")
    check_all_queries_properties(inp, g)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_sparse_layer_many_queries(dtype):
    """A batch of at least two queries per CU (620 here) takes the sparse layer's narrow-slot
    form, one workgroup per query: every query's sparse output against the oracle on the
    GPU's own selection, with t < window, at most k candidates and long slices all present;
    the selector on a sample of them."""
    rng = np.random.default_rng(31)
    seqs = [1500, 5000, 300]
    qpos = [sorted(set([0, 5, 127, 128, 600, 1151, 1152, 1499] + rng.integers(0, 1500, 200).tolist())),
            sorted(set([127, 1200, 4999] + rng.integers(1000, 5000, 300).tolist())),
            sorted(set([0, 1, 200, 299] + rng.integers(0, 300, 130).tolist()))]
    spec = BlockSpec("many-queries", seqs, qpos, dtype=dtype, n_sparse=1, needles_per_query=1, seed=33)
    assert spec.total_q >= 512
    inp = make_block_inputs(spec)
    _say(f"sparse many queries {dtype}: {spec.total_q} queries")
    g = run_block(inp)
    check_all_queries_properties(inp, g)
    rr = dtype == "fp8"
    for qi in range(spec.total_q):
        ref, _ = oracle_sparse(inp, qi, 0, g["sel"][qi])
        few = int(inp.q_pos[qi]) + 1 <= FEW_KEYS
        check_attn(g["sparse"][0][qi], ref, f"many-queries q{qi} sparse", beyond_rounding=rr, few_keys=few)
    check_queries(inp, g, range(0, spec.total_q, 26), f"many-queries-{dtype}")


def test_small_context_sparse_equals_full_on_gpu():
    """When t+1 <= window + top_k, the sparse layer with the selector's own Q reproduces
    the selector's output (the <= 1,152-row invariant)."""
    spec = BlockSpec("inv", [1152, 900, 5000], [[1151, 1000, 64], [899], [1151]], dtype="bf16", n_sparse=0,
                     needles_per_query=0, seed=13)
    inp = make_block_inputs(spec)
    g = run_block(inp, selector_only=True)
    q = to_dev(inp.q_sel)
    o, _ = hs2.sparse_attn(g["batch"], q, g["k"], g["v"], torch.from_numpy(g["sel"]).cuda(), spec.window, spec.top_k,
                           spec.scale)
    o = from_dev(o)
    for qi in range(spec.total_q):
        check_attn(o[qi], g["out"][qi], f"invariant q{qi}")
        r = oracle_query(inp, qi)
        check_attn(o[qi], r["out"], f"invariant-vs-oracle q{qi}")


def test_top_k_zero_and_window_one():
    spec = BlockSpec("k0", [3000, 500], [[2999, 10], [499]], dtype="bf16", n_sparse=1, needles_per_query=0,
                     seed=14, top_k=0, window=1)
    inp = make_block_inputs(spec)
    g = run_block(inp)
    assert np.all(g["count"] == 0)
    for qi in range(spec.total_q):
        r = oracle_query(inp, qi)
        check_attn(g["out"][qi], r["out"], f"k0 q{qi}")
        ref, _ = oracle_sparse(inp, qi, 0, np.zeros(0, dtype=np.int64), r["K"], r["V"])
        check_attn(g["sparse"][0][qi], ref, f"k0 sparse q{qi}")


def test_window_and_k_small():
    spec = BlockSpec("w5k7", [2000, 40], [[1999, 600], [39]], dtype="bf16", n_sparse=1, needles_per_query=1,
                     seed=15, top_k=7, window=5)
    inp = make_block_inputs(spec)
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), "w5k7")
    check_all_queries_properties(inp, g)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_largest_top_k(dtype):
    """top_k at its bound (HS2_MAX_TOP_K = 4096): the selection and the sparse layer's
    4,224-key gather (several sparse splits of up to 2,048 slots)."""
    spec = BlockSpec(f"k4096-{dtype}", [65536, 20000], [[65535, 40000], [19999]], dtype=dtype, n_sparse=1,
                     needles_per_query=8, seed=21, top_k=4096)
    inp = make_block_inputs(spec)
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), f"k4096-{dtype}")
    check_all_queries_properties(inp, g)


def test_largest_window():
    """window at its bound (2^18 = 262,144) over a 300,000-token context: 37,856 and 17,857
    candidates, and a sparse layer of 263,168 keys per query."""
    spec = BlockSpec("w2^18", [300000], [[299999, 280000]], dtype="bf16", n_sparse=1, needles_per_query=4,
                     seed=22, window=1 << 18, top_k=1024)
    inp = make_block_inputs(spec)
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), "w2^18")
    check_all_queries_properties(inp, g)


def test_exact_ties_prefer_smaller_position():
    """Identical key rows give bitwise-equal scores; the k-th place must go to the
    smallest positions among them."""
    spec = BlockSpec("ties", [6000], [[5999]], dtype="bf16", n_sparse=1, needles_per_query=0, seed=16,
                     top_k=16)
    inp = make_block_inputs(spec)
    # 40 identical strong rows at spread positions: only the 16 smallest may be chosen
    qv = bf16_to_f32(inp.q_sel[0]).astype(np.float64).mean(axis=0)
    strong = (8.0 * qv / np.linalg.norm(qv) * math.sqrt(128)).astype(np.float32)
    row = bf16_round(strong)
    pos = np.arange(100, 100 + 40 * 97, 97)
    inp.k[pos] = row
    g = run_block(inp)
    r = oracle_query(inp, 0)
    assert r["sel"].tolist() == pos[:16].tolist()
    assert g["sel"][0].tolist() == pos[:16].tolist()
    ref, _ = oracle_sparse(inp, 0, 0, g["sel"][0], r["K"], r["V"])
    check_attn(g["sparse"][0][0], ref, "ties sparse")


def test_invalid_descriptor_is_not_computed():
    """A query whose position lies outside its sequence is skipped: NaN outputs and
    sel_count -1; the other queries are unaffected."""
    spec = BlockSpec("bad", [3000, 2000], [[2999], [1999]], dtype="bf16", n_sparse=1, needles_per_query=0,
                     seed=17)
    inp = make_block_inputs(spec)
    inp.q_pos[1] = 2500  # beyond kv_len of sequence 1
    g = run_block(inp)
    assert int(g["count"][1]) == -1
    assert np.isnan(g["out"][1]).all()
    assert np.all(g["sel"][1] == -1)
    assert np.isnan(g["sparse"][0][1]).all()
    r = oracle_query(inp, 0)
    check_attn(g["out"][0], r["out"], "valid neighbour")
    check_selection(g["sel"][0], int(g["count"][0]), r, spec.top_k, 3000 - 127, "valid neighbour")


def test_position_beyond_max_kv_len_is_not_computed():
    """max_kv_len sizes the key splits and the score rows: a query at or beyond it (its
    sequence longer than the bound) is skipped like any inconsistent descriptor, nothing
    is written outside the workspace, and the other query is unaffected."""
    spec = BlockSpec("beyond", [3000, 5000], [[2999], [4999]], dtype="bf16", n_sparse=1, needles_per_query=0,
                     seed=19)
    inp = make_block_inputs(spec)
    dev = "cuda"
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, dev)
    batch.max_kv_len = 4000   # below sequence 1's length; its query sits at 4999
    batch.kv_len_host = None  # (a host copy above the bound is rejected on the host)
    k, v, q, qs = to_dev(inp.k), to_dev(inp.v), to_dev(inp.q_sel), to_dev(inp.q_sp[0])
    guard = 1 << 16
    n1 = hs2.full_attn_select_workspace_size(batch, spec.window, spec.top_k)
    n2 = max(1, hs2.sparse_attn_workspace_size(batch, spec.window, spec.top_k))
    ws1 = torch.full((n1 + guard,), 0x5A, dtype=torch.uint8, device=dev)
    ws2 = torch.full((n2 + guard,), 0x5A, dtype=torch.uint8, device=dev)
    out, lse, sel, cnt = hs2.full_attn_select(batch, q, k, v, spec.window, spec.top_k, spec.scale,
                                              workspace=ws1[:n1])
    o, _ = hs2.sparse_attn(batch, qs, k, v, sel, spec.window, spec.top_k, spec.scale, workspace=ws2[:n2])
    torch.cuda.synchronize()
    assert bool((ws1[n1:] == 0x5A).all()) and bool((ws2[n2:] == 0x5A).all())
    g_out, g_sel, g_cnt, g_sp = from_dev(out), sel.cpu().numpy(), cnt.cpu().numpy(), from_dev(o)
    assert int(g_cnt[1]) == -1 and np.all(g_sel[1] == -1)
    assert np.isnan(g_out[1]).all() and np.isnan(g_sp[1]).all()
    r = oracle_query(inp, 0)
    check_attn(g_out[0], r["out"], "query below the bound")
    check_selection(g_sel[0], int(g_cnt[0]), r, spec.top_k, 3000 - 127, "query below the bound")
    ref, _ = oracle_sparse(inp, 0, 0, g_sel[0], r["K"], r["V"])
    check_attn(g_sp[0], ref, "query below the bound, sparse layer")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_host_lengths_below_device_lengths_are_reported(dtype):
    """The decode launches are planned from the host copy of the lengths (kv_len_host).
    A sequence whose device length exceeds its host copy has key splits that were never
    launched: its query is reported as inconsistent (NaN outputs, sel_count -1), also
    with a host length of 0; a host length above the device length only over-covers.
    Nothing is written past the workspaces; the other queries match the oracle."""
    lens = [50000 + 997 * j for j in range(8)]
    spec = BlockSpec("host-lengths", lens, [[n - 1] for n in lens], dtype=dtype, n_sparse=1,
                     needles_per_query=2, seed=41)
    inp = make_block_inputs(spec)
    dev = "cuda"
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, dev)
    host = batch.kv_len_host.copy()
    host[3] = 1000           # far below the device length: most splits of query 3 are missing
    host[5] = 0              # nothing planned: one split is still launched, and it reports
    host[6] = min(batch.max_kv_len, int(host[6]) + 3000)   # above the device length
    batch.kv_len_host = np.ascontiguousarray(host, dtype=np.int32)
    fp8 = dtype == "fp8"
    k, v, q, qs = to_dev(inp.k), to_dev(inp.v), to_dev(inp.q_sel), to_dev(inp.q_sp[0])
    ws_dt = "fp8" if fp8 else torch.bfloat16
    guard = 1 << 16
    n1 = hs2.full_attn_select_workspace_size(batch, spec.window, spec.top_k, ws_dt)
    n2 = max(1, hs2.sparse_attn_workspace_size(batch, spec.window, spec.top_k, ws_dt))
    ws1 = torch.full((n1 + guard,), 0x5A, dtype=torch.uint8, device=dev)
    ws2 = torch.full((n2 + guard,), 0x5A, dtype=torch.uint8, device=dev)
    _say(f"host lengths below device lengths ({dtype})")
    if fp8:
        out, lse, sel, cnt = hs2.full_attn_select_fp8kv(batch, q, k, v, spec.k_scale, spec.v_scale, spec.window,
                                                        spec.top_k, spec.scale, workspace=ws1[:n1])
        o, _ = hs2.sparse_attn_fp8kv(batch, qs, k, v, spec.k_scale, spec.v_scale, sel, spec.window, spec.top_k,
                                     spec.scale, workspace=ws2[:n2])
    else:
        out, lse, sel, cnt = hs2.full_attn_select(batch, q, k, v, spec.window, spec.top_k, spec.scale,
                                                  workspace=ws1[:n1])
        o, _ = hs2.sparse_attn(batch, qs, k, v, sel, spec.window, spec.top_k, spec.scale, workspace=ws2[:n2])
    torch.cuda.synchronize()
    assert bool((ws1[n1:] == 0x5A).all()) and bool((ws2[n2:] == 0x5A).all())
    g_out, g_lse, g_sel, g_cnt, g_sp = from_dev(out), from_dev(lse), sel.cpu().numpy(), cnt.cpu().numpy(), from_dev(o)
    rr = fp8
    for qi in (3, 5):
        assert int(g_cnt[qi]) == -1 and np.all(g_sel[qi] == -1), f"query {qi}: selection not reported"
        assert np.isnan(g_out[qi]).all() and np.isnan(g_lse[qi]).all(), f"query {qi}: outputs not NaN"
        # the sparse layer's own descriptor is consistent: with an all -1 selection it
        # attends the window alone
        ref, _ = oracle_sparse(inp, qi, 0, g_sel[qi])
        check_attn(g_sp[qi], ref, f"host lengths {dtype} q{qi} sparse layer, window only", beyond_rounding=rr)
    for qi in (0, 6, 7):
        r = oracle_query(inp, qi)
        tag = f"host lengths {dtype} q{qi}"
        check_attn(g_out[qi], r["out"], tag, beyond_rounding=rr)
        check_lse(g_lse[qi], r["lse"], tag)
        check_selection(g_sel[qi], int(g_cnt[qi]), r, spec.top_k, oracle.candidate_count(r["t"], spec.window), tag)
        ref, _ = oracle_sparse(inp, qi, 0, g_sel[qi], r["K"], r["V"])
        check_attn(g_sp[qi], ref, tag + " sparse layer", beyond_rounding=rr)


def test_q_start_beyond_total_q_touches_nothing_outside():
    """Q-tile path (many queries per sequence): a q_start that runs past total_q, or that
    starts below 0, makes every query inconsistent (NaN outputs, sel_count -1) and no
    kernel touches a row past the caller's Q, out, LSE, selection or workspace buffers."""
    spec = BlockSpec("qstart", [6000, 9000], [list(range(5988, 6000)), list(range(8992, 9000))], dtype="bf16",
                     n_sparse=0, needles_per_query=0, seed=43)
    inp = make_block_inputs(spec)
    dev = "cuda"
    nq = spec.total_q
    k, v = to_dev(inp.k), to_dev(inp.v)
    extra = 48   # rows of every per-query buffer past total_q, filled with a guard pattern
    q = torch.zeros(nq + extra, 64, 128, dtype=torch.bfloat16, device=dev)
    q[:nq] = to_dev(inp.q_sel)
    for bad in ([0, 12, 40], [-8, 12, 20]):
        batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, dev)
        assert batch.max_q_per_seq >= 8  # the q-tile kernels
        batch.q_start = torch.tensor(bad, dtype=torch.int32, device=dev)
        out = torch.full((nq + extra, 64, 128), 3.0, dtype=torch.bfloat16, device=dev)
        lse = torch.full((nq + extra, 64), 3.0, dtype=torch.float32, device=dev)
        sel = torch.full((nq + extra, spec.top_k), 7, dtype=torch.int32, device=dev)
        cnt = torch.full((nq + extra,), 7, dtype=torch.int32, device=dev)
        n1 = hs2.full_attn_select_workspace_size(batch, spec.window, spec.top_k)
        guard = 1 << 16
        ws = torch.full((n1 + guard,), 0x5A, dtype=torch.uint8, device=dev)
        _say(f"q_start {bad}")
        hs2.full_attn_select(batch, q[:nq], k, v, spec.window, spec.top_k, spec.scale, out=out[:nq], lse=lse[:nq],
                             sel_idx=sel[:nq], sel_count=cnt[:nq], workspace=ws[:n1])
        torch.cuda.synchronize()
        assert bool((ws[n1:] == 0x5A).all()), "workspace guard bytes changed"
        assert bool((out[nq:].float() == 3.0).all()) and bool((lse[nq:] == 3.0).all())
        assert bool((sel[nq:] == 7).all()) and bool((cnt[nq:] == 7).all())
        assert bool(torch.isnan(out[:nq].float()).all()) and bool(torch.isnan(lse[:nq]).all())
        assert bool((cnt[:nq] == -1).all()) and bool((sel[:nq] == -1).all())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_repeat_runs_are_bitwise_identical(dtype):
    inp = make_block_inputs(BlockSpec("det", [20000, 7000], [[19999], [6999, 3000]], dtype=dtype, n_sparse=1,
                                      needles_per_query=4, seed=18))
    a = run_block(inp)
    b = run_block(inp)
    assert np.array_equal(a["sel"], b["sel"])
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["sparse"][0], b["sparse"][0])


def test_sparse_split_merge_and_stage_reuse():
    """100 single-query sequences: each query's 1,152 keys are split over three
    workgroups of 15 tiles (every wave cycles through its LDS stages several times) and
    the split combine merges the partials."""
    lens = [2000 + 37 * j for j in range(100)]
    spec = BlockSpec("split-merge", lens, [[n - 1] for n in lens], dtype="bf16", n_sparse=1, needles_per_query=1,
                     seed=23)
    inp = make_block_inputs(spec)
    _say("sparse split merge")
    g = run_block(inp)
    check_queries(inp, g, range(0, spec.total_q, 7), "split-merge")
    check_all_queries_properties(inp, g)


def test_sparse_workspace_contents_do_not_matter():
    """The sparse call's workspace (the split partials) holds arbitrary bytes on entry
    and is used again and again: every call gives the same output."""
    lens = [3000 + 101 * j for j in range(8)]
    spec = BlockSpec("ws", lens, [[n - 1] for n in lens], dtype="bf16", n_sparse=1, needles_per_query=2, seed=24)
    inp = make_block_inputs(spec)
    g = run_block(inp)
    q = to_dev(inp.q_sp[0])
    sel = torch.from_numpy(g["sel"]).cuda()
    need = hs2.sparse_attn_workspace_size(g["batch"], spec.window, spec.top_k)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for fill in (0xFF, 0x00, 0x01, None, None):
        if fill is not None:
            ws.fill_(fill)
        o, _ = hs2.sparse_attn(g["batch"], q, g["k"], g["v"], sel, spec.window, spec.top_k, spec.scale, workspace=ws)
        outs.append(from_dev(o))
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o, g["sparse"][0])
    for qi in range(spec.total_q):
        r = oracle_query(inp, qi)
        ref, _ = oracle_sparse(inp, qi, 0, g["sel"][qi], r["K"], r["V"])
        check_attn(outs[-1][qi], ref, f"ws q{qi}")


# ----------------------------------------------------------------------------------
# decode-time KV Bridging: new tokens' K/V rows written into the caches
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("n_new,d_model", [(37, 2048), (64, 256), (1, 128)])
def test_bridge_append_rows(n_new, d_model):
    """New tokens' projections into 3 layers' caches at scattered rows (two of them out of
    range, which must be skipped); every other cache row keeps its bytes."""
    bi = make_bridge_inputs(n_new, n_layers=3, seed=28 + n_new, d_model=d_model)
    cache_rows = 3000
    rows = np.random.default_rng(n_new).choice(cache_rows, n_new, replace=False).astype(np.int64)
    if n_new > 8:
        rows[5], rows[6] = cache_rows + 10, -1
    g = torch.Generator().manual_seed(n_new)
    init = [torch.randn(cache_rows, 128, generator=g).to(torch.bfloat16) for _ in range(6)]
    caches = [c.cuda() for c in init]
    hs2.bridge_kv_append(to_dev(bi.h), torch.from_numpy(rows).cuda(), [to_dev(w) for w in bi.w_k],
                         [to_dev(w) for w in bi.w_v], caches[0::2], caches[1::2])
    torch.cuda.synchronize()
    valid = (rows >= 0) & (rows < cache_rows)
    H = stored_to_f64(bi.h)
    ks, vs = oracle.bridge_kv(H, [stored_to_f64(w) for w in bi.w_k], [stored_to_f64(w) for w in bi.w_v])
    for l in range(3):
        for c0, c, ref in ((init[2 * l], caches[2 * l], ks[l]), (init[2 * l + 1], caches[2 * l + 1], vs[l])):
            got = from_dev(c)
            keep = np.ones(cache_rows, bool)
            keep[rows[valid]] = False
            assert np.array_equal(got[keep], c0.float().numpy().astype(np.float64)[keep]), "a row not appended changed"
            g_rows = got[rows[valid]]
            r = ref[valid]
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
            assert np.all(np.abs(g_rows - r) <= ulp + BRIDGE_ATOL), f"layer {l}: appended rows beyond 1 bf16 ulp"


def test_bridge_append_then_select():
    """One decode step: the append writes each sequence's current-token K/V row of layer 0
    (from that token's hidden state), then the selector and a sparse layer read the cache;
    both match the oracle run on a cache holding the oracle's own projections there."""
    spec = BlockSpec("append-step", [3000, 5000, 2200], [[2999], [4999], [2199]], n_sparse=1, needles_per_query=2,
                     seed=29)
    inp = make_block_inputs(spec)
    bi = make_bridge_inputs(3, n_layers=1, seed=30)
    rows = (inp.kv_start + inp.kv_len - 1).astype(np.int64)
    k, v = to_dev(inp.k), to_dev(inp.v)
    hs2.bridge_kv_append(to_dev(bi.h), torch.from_numpy(rows).cuda(), [to_dev(bi.w_k[0])], [to_dev(bi.w_v[0])],
                         [k], [v])
    # the oracle's cache: the generator's rows, with the oracle's own projection at the new rows
    ks, vs = oracle.bridge_kv(stored_to_f64(bi.h), [stored_to_f64(bi.w_k[0])], [stored_to_f64(bi.w_v[0])])
    inp.k[rows] = bf16_round(ks[0].astype(np.float32))
    inp.v[rows] = bf16_round(vs[0].astype(np.float32))
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, "cuda")
    out, lse, sel, cnt = hs2.full_attn_select(batch, to_dev(inp.q_sel), k, v, spec.window, spec.top_k, spec.scale)
    o1, _ = hs2.sparse_attn(batch, to_dev(inp.q_sp[0]), k, v, sel, spec.window, spec.top_k, spec.scale)
    torch.cuda.synchronize()
    g = {"out": from_dev(out), "lse": from_dev(lse), "sel": sel.cpu().numpy(), "count": cnt.cpu().numpy(),
         "sparse": [from_dev(o1)]}
    check_queries(inp, g, range(spec.total_q), "append-step")


@pytest.mark.parametrize("n_new,d_model", [(37, 2048), (64, 256), (1, 128)])
def test_bridge_append_fp8_rows(n_new, d_model):
    """The FP8 append: new tokens' E4M3 codes into 3 layers' FP8 caches at scattered rows
    (two out of range, skipped), a scale per tensor; every other byte of the caches is kept."""
    bi = make_bridge_inputs(n_new, n_layers=3, seed=38 + n_new, d_model=d_model)
    cache_rows = 3000
    rows = np.random.default_rng(n_new + 1).choice(cache_rows, n_new, replace=False).astype(np.int64)
    if n_new > 8:
        rows[5], rows[6] = cache_rows + 10, -1
    init = [np.random.default_rng(100 + i).integers(0, 256, (cache_rows, 128), dtype=np.uint8) for i in range(6)]
    caches = [torch.from_numpy(c).cuda() for c in init]
    k_sc, v_sc = [0.004, 0.01, 0.02], [0.02, 0.003, 0.01]
    hs2.bridge_kv_append_fp8kv(to_dev(bi.h), torch.from_numpy(rows).cuda(), [to_dev(w) for w in bi.w_k],
                               [to_dev(w) for w in bi.w_v], caches[0::2], caches[1::2], k_sc, v_sc)
    torch.cuda.synchronize()
    valid = (rows >= 0) & (rows < cache_rows)
    H = stored_to_f64(bi.h)
    wk, wv = [stored_to_f64(w) for w in bi.w_k], [stored_to_f64(w) for w in bi.w_v]
    ks, vs = oracle.bridge_kv(H, wk, wv)
    kc, vc = oracle.bridge_kv_fp8(H, wk, wv, k_sc, v_sc)
    keep = np.ones(cache_rows, bool)
    keep[rows[valid]] = False
    for l in range(3):
        for c0, c, val, codes, sc, what in ((init[2 * l], caches[2 * l], ks[l], kc[l], k_sc[l], f"K{l}"),
                                            (init[2 * l + 1], caches[2 * l + 1], vs[l], vc[l], v_sc[l], f"V{l}")):
            got = c.cpu().numpy()
            assert np.array_equal(got[keep], c0[keep]), f"{what}: a row not appended changed"
            check_fp8_codes(got[rows[valid]], val[valid], codes[valid], sc, what)


def test_bridge_append_fp8_then_select():
    """One decode step on FP8 caches: the FP8 append writes each sequence's current-token
    row of layer 0, then the FP8 selector and a sparse layer read the caches and match the
    oracle run on the same codes."""
    spec = BlockSpec("append-step-fp8", [3000, 5000, 2200], [[2999], [4999], [2199]], dtype="fp8", n_sparse=1,
                     needles_per_query=2, seed=47)
    inp = make_block_inputs(spec)
    bi = make_bridge_inputs(3, n_layers=1, seed=48)
    rows = (inp.kv_start + inp.kv_len - 1).astype(np.int64)
    k, v = to_dev(inp.k), to_dev(inp.v)
    hs2.bridge_kv_append_fp8kv(to_dev(bi.h), torch.from_numpy(rows).cuda(), [to_dev(bi.w_k[0])],
                               [to_dev(bi.w_v[0])], [k], [v], spec.k_scale, spec.v_scale)
    torch.cuda.synchronize()
    H = stored_to_f64(bi.h)
    ks, vs = oracle.bridge_kv(H, [stored_to_f64(bi.w_k[0])], [stored_to_f64(bi.w_v[0])])
    kc, vc = oracle.bridge_kv_fp8(H, [stored_to_f64(bi.w_k[0])], [stored_to_f64(bi.w_v[0])], [spec.k_scale],
                                  [spec.v_scale])
    gk, gv = k.cpu().numpy(), v.cpu().numpy()
    check_fp8_codes(gk[rows], ks[0], kc[0], spec.k_scale, "K0")
    check_fp8_codes(gv[rows], vs[0], vc[0], spec.v_scale, "V0")
    inp.k[rows], inp.v[rows] = gk[rows], gv[rows]
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, "cuda")
    out, lse, sel, cnt = hs2.full_attn_select_fp8kv(batch, to_dev(inp.q_sel), k, v, spec.k_scale, spec.v_scale,
                                                    spec.window, spec.top_k, spec.scale)
    o1, _ = hs2.sparse_attn_fp8kv(batch, to_dev(inp.q_sp[0]), k, v, spec.k_scale, spec.v_scale, sel, spec.window,
                                  spec.top_k, spec.scale)
    torch.cuda.synchronize()
    g = {"out": from_dev(out), "lse": from_dev(lse), "sel": sel.cpu().numpy(), "count": cnt.cpu().numpy(),
         "sparse": [from_dev(o1)]}
    check_queries(inp, g, range(spec.total_q), "append-step-fp8")


# ----------------------------------------------------------------------------------
# exact causal attention without selection (prefill of the self-decoder's full layer)
# ----------------------------------------------------------------------------------

def _causal_check(spec, qis, what):
    inp = make_block_inputs(spec)
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, "cuda")
    _say(f"causal {what}: {spec.total_q} queries")
    o, lse = hs2.causal_attn(batch, to_dev(inp.q_sel), to_dev(inp.k), to_dev(inp.v), spec.scale)
    torch.cuda.synchronize()
    o, lse = from_dev(o), from_dev(lse)
    for qi in qis:
        s = int(inp.q_seq[qi])
        a, t = int(inp.kv_start[s]), int(inp.q_pos[qi])
        ref, ref_lse, _ = oracle.full_attention(stored_to_f64(inp.q_sel[qi]), stored_to_f64(inp.k[a:a + t + 1]),
                                                stored_to_f64(inp.v[a:a + t + 1]), t, spec.scale)
        check_attn(o[qi], ref, f"causal {what} q{qi} t={t}", few_keys=t + 1 <= FEW_KEYS)
        check_lse(lse[qi], ref_lse, f"causal {what} q{qi} t={t}")
    assert np.isfinite(o).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_prefill_every_position(dtype):
    """Two sequences with every position a query (q-tile kernel writing each query's
    output itself for bf16; one query per workgroup for fp32)."""
    spec = BlockSpec("prefill", [3000, 1500], [list(range(3000)), list(range(1500))], dtype=dtype, n_sparse=0,
                     needles_per_query=0, seed=25)
    _causal_check(spec, list(range(0, 4500, 37)) + [2999, 3000, 4499], f"prefill-{dtype}")


def test_causal_split_keys():
    """Few queries with long contexts: their keys are split over workgroups and merged by
    the split combine, for the q-tile kernel (64 queries of one sequence) and for the
    decode-shaped kernel (3 queries per sequence)."""
    spec = BlockSpec("causal-qtile-split", [100000], [list(range(99936, 100000))], n_sparse=0, needles_per_query=0,
                     seed=26)
    _causal_check(spec, [0, 17, 63], "qtile-split")
    spec = BlockSpec("causal-decode-split", [40000, 30000], [[39999, 20000, 5], [29999, 128, 0]], n_sparse=0,
                     needles_per_query=0, seed=27)
    _causal_check(spec, range(6), "decode-split")


def test_causal_many_sequences():
    """More sequences than one workgroup lists at a time (300 > 256) on the q-tile path:
    sequences with no query, with every position a query and with query counts that are
    not multiples of the tile size; every query against the oracle."""
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 61, 300)]
    qpos = []
    for si, n in enumerate(lens):
        if si % 7 == 3:
            qpos.append([])
        elif si % 5 == 0:
            qpos.append(list(range(n)))
        else:
            m = int(rng.integers(1, min(n, 11) + 1))
            qpos.append(sorted(int(x) for x in rng.choice(n, m, replace=False)))
    assert max(len(p) for p in qpos) >= 8          # at least one sequence takes q-tiles
    spec = BlockSpec("causal-many-seqs", lens, qpos, n_sparse=0, needles_per_query=0, seed=42)
    _causal_check(spec, range(spec.total_q), "many-seqs")


def test_workload7_prefill_262144():
    """Workload 7's attention at full size: every position of a 262,144-token sequence."""
    spec = block_config(7)
    _causal_check(spec, [0, 1, 4095, 131071, 262142, 262143], spec.name)
    torch.cuda.empty_cache()


def _bridge_check(bi, gk, gv, rows):
    H = stored_to_f64(bi.h[rows])
    ks, vs = oracle.bridge_kv(H, [stored_to_f64(w) for w in bi.w_k], [stored_to_f64(w) for w in bi.w_v])
    for l in range(len(bi.w_k)):
        for got, ref in ((gk[l], ks[l]), (gv[l], vs[l])):
            g = from_dev(got[torch.as_tensor(rows, device=got.device)])
            check_bridge_bf16(g, ref, f"bridge layer {l}")


def test_bridge_small_ragged_rows():
    bi = make_bridge_inputs(1000, n_layers=3, seed=21)
    h = to_dev(bi.h)
    gk, gv = hs2.bridge_kv(h, [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v])
    torch.cuda.synchronize()
    _bridge_check(bi, gk, gv, np.arange(1000))


@pytest.mark.parametrize("n_layers", [2, 6])
def test_bridge_layer_counts(n_layers):
    """Both column tilings of the fan-out kernel: 2L = 4 matrices (256-column tiles) and
    2L = 12 (four 384-column tiles, each spanning three output matrices)."""
    bi = make_bridge_inputs(600, n_layers=n_layers, seed=23 + n_layers)
    gk, gv = hs2.bridge_kv(to_dev(bi.h), [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v])
    _say(f"bridge {n_layers} layers")
    _bridge_check(bi, gk, gv, np.arange(600))


def test_bridge_one_layer_and_tiny_rows():
    bi = make_bridge_inputs(37, n_layers=1, seed=22, d_model=256)
    gk, gv = hs2.bridge_kv(to_dev(bi.h), [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v])
    torch.cuda.synchronize()
    _bridge_check(bi, gk, gv, np.arange(37))


def _bridge_fp8_check(bi, gk, gv, rows, k_sc, v_sc):
    """The FP8 bridging of the given rows against the oracle's (bridge_kv_fp8)."""
    H = stored_to_f64(bi.h[rows])
    wk, wv = [stored_to_f64(w) for w in bi.w_k], [stored_to_f64(w) for w in bi.w_v]
    ks, vs = oracle.bridge_kv(H, wk, wv)
    kc, vc = oracle.bridge_kv_fp8(H, wk, wv, k_sc, v_sc)
    idx = torch.as_tensor(rows, device=gk[0].device)
    for l in range(len(wk)):
        check_fp8_codes(gk[l][idx].cpu().numpy(), ks[l], kc[l], k_sc[l], f"K{l}")
        check_fp8_codes(gv[l][idx].cpu().numpy(), vs[l], vc[l], v_sc[l], f"V{l}")


def test_bridge_fp8_small_ragged_rows():
    """3 layers (384-column tiles), 1,000 rows (a ragged last row tile), a different scale
    for every tensor; with the smallest ones 5-14% of the values saturate."""
    bi = make_bridge_inputs(1000, n_layers=3, seed=41)
    k_sc, v_sc = [0.01, 0.02, 0.004], [0.012, 0.003, 0.03]
    gk, gv = hs2.bridge_kv_fp8kv(to_dev(bi.h), [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v], k_sc, v_sc)
    torch.cuda.synchronize()
    assert bool((gk[2] == 0x7E).any()) and bool((gk[2] == 0xFE).any())   # saturated both ways
    _bridge_fp8_check(bi, gk, gv, np.arange(1000), k_sc, v_sc)


@pytest.mark.parametrize("n_layers", [1, 2, 6])
def test_bridge_fp8_layer_counts(n_layers):
    """The 256-column tiles (2L = 2 and 4 matrices) and four 384-column tiles (2L = 12),
    each output matrix with its own scale."""
    bi = make_bridge_inputs(600, n_layers=n_layers, seed=43 + n_layers, d_model=512 if n_layers == 1 else 2048)
    k_sc = [0.008 + 0.001 * l for l in range(n_layers)]
    v_sc = [0.011 - 0.001 * l for l in range(n_layers)]
    gk, gv = hs2.bridge_kv_fp8kv(to_dev(bi.h), [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v], k_sc, v_sc)
    _say(f"fp8 bridge {n_layers} layers")
    _bridge_fp8_check(bi, gk, gv, np.arange(600), k_sc, v_sc)


def test_bridge_fp8_then_fp8_selector():
    """Bridged FP8 caches feed the FP8 selector and a sparse layer: the hidden states of
    10,200 rows (three sequences) are projected into one layer's E4M3 K/V caches on the
    GPU, and the selector and sparse layer on those caches match the oracle run on the
    same codes."""
    seqs = [3000, 5000, 2200]
    spec = BlockSpec("bridged-fp8", seqs, [[2999, 1500], [4999, 300], [2199]], dtype="fp8", n_sparse=1,
                     needles_per_query=0, seed=45, k_scale=0.01, v_scale=0.01)
    inp = make_block_inputs(spec)
    bi = make_bridge_inputs(sum(seqs), n_layers=1, seed=46)
    gk, gv = hs2.bridge_kv_fp8kv(to_dev(bi.h), [to_dev(bi.w_k[0])], [to_dev(bi.w_v[0])], spec.k_scale, spec.v_scale)
    torch.cuda.synchronize()
    inp.k, inp.v = gk[0].cpu().numpy(), gv[0].cpu().numpy()
    _bridge_fp8_check(bi, gk, gv, np.arange(0, sum(seqs), 7), [spec.k_scale], [spec.v_scale])
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q), "bridged-fp8")
    check_all_queries_properties(inp, g)


# ----------------------------------------------------------------------------------
# the workloads at full size: sampled queries + properties of every query
# ----------------------------------------------------------------------------------

def _full(n, sample):
    spec = block_config(n)
    _say(f"workload {n}: generating {spec.name}")
    inp = make_block_inputs(spec)
    _say(f"workload {n}: running")
    g = run_block(inp)
    _say(f"workload {n}: checking")
    check_all_queries_properties(inp, g)
    check_queries(inp, g, sample, spec.name)
    del g
    torch.cuda.empty_cache()


def test_workload2_decode_64x128k():
    _full(2, range(64))


def test_workload3_decode_8x1m():
    _full(3, range(8))


def test_workload6_decode_64x128k_fp8():
    _full(6, range(64))


def test_workload4_chunk_4096_queries():
    # every wave (query index mod 8) of q-tiles spread over the chunk, the first and the
    # last tile included; each query's candidates span several score splits of 32,768 keys
    _full(4, [8 * tile + w for tile in list(range(0, 512, 64)) + [511] for w in range(8)])


def test_workload5_bridge_and_ragged_decode():
    bi = make_bridge_inputs(1048576, n_layers=3, seed=5)
    _say("workload 5: bridging 1M x 2048 -> 3 layers")
    h = to_dev(bi.h)
    gk, gv = hs2.bridge_kv(h, [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v])
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 300), np.random.default_rng(0).choice(1048576, 300, replace=False),
                           np.arange(1048576 - 300, 1048576)])
    _bridge_check(bi, gk, gv, rows)
    del gk, gv
    k_sc, v_sc = [0.01, 0.011, 0.012], [0.009, 0.01, 0.011]
    _say("workload 5: FP8 bridging 1M x 2048 -> 3 layers")
    gk, gv = hs2.bridge_kv_fp8kv(h, [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v], k_sc, v_sc)
    torch.cuda.synchronize()
    _bridge_fp8_check(bi, gk, gv, rows, k_sc, v_sc)
    del h, gk, gv
    torch.cuda.empty_cache()
    _full(5, range(32))


@pytest.mark.parametrize("shape", ["decode", "chunk", "decode-fp8", "many"])
def test_logit_far_above_first_tile_is_recomputed(shape):
    """Keys whose logits for one head lie 150..402 (log2 units) above the other keys, at
    increasing positions over ~16 tiles: a wave whose first tile holds none of them (or
    a smaller one) overflows sums taken against that tile's maximum, and must detect it
    and recompute with its exact maximum. Covers the decode-shaped selector kernel, the
    q-tile selector kernel and the sparse kernel (whose Q equals the selector's, with
    enough queries that its waves take two tiles each; with 520 queries, the narrow-slot
    form, whose workgroup takes the query's 36 tiles in batches)."""
    if shape == "decode":
        spec = BlockSpec("spike-decode", [2000] * 40, [[1999]] * 40, dtype="bf16", n_sparse=1,
                         needles_per_query=0, seed=21)
    elif shape == "decode-fp8":
        # FP8 keys: a K scale large enough for the spike keys (components up to ~90)
        spec = BlockSpec("spike-decode-fp8", [2000] * 40, [[1999]] * 40, dtype="fp8", n_sparse=1,
                         needles_per_query=0, seed=23, k_scale=0.25)
    elif shape == "chunk":
        spec = BlockSpec("spike-chunk", [5000], [list(range(4990, 5000))], dtype="bf16", n_sparse=1,
                         needles_per_query=0, seed=22)
    else:
        spec = BlockSpec("spike-many", [5000], [list(range(4480, 5000))], dtype="bf16", n_sparse=1,
                         needles_per_query=0, seed=24)
    inp = make_block_inputs(spec)
    qi, h = 0, 5
    base = int(inp.kv_start[int(inp.q_seq[qi])])
    qh = stored_to_f64(inp.q_sel[qi][h])
    unit = qh / np.linalg.norm(qh)
    c = spec.scale * math.log2(math.e) * np.linalg.norm(qh)  # x = c * alpha for k = alpha * unit
    pos = 1000 + 8 * np.arange(64)
    fp8 = spec.dtype == "fp8"
    for j, pj in enumerate(pos):
        key = ((150.0 + 4.0 * j) / c * unit).astype(np.float32)
        inp.k[base + pj] = e4m3_encode(key, spec.k_scale) if fp8 else bf16_round(key)
    inp.q_sp[0][qi] = inp.q_sel[qi]
    kk = oracle.dequantize_kv(inp.k[base + pos], spec.k_scale) if fp8 else stored_to_f64(inp.k[base + pos])
    xs = spec.scale * math.log2(math.e) * (kk @ qh)
    assert xs.min() > 140.0
    if not fp8:  # FP8 rounding (2^-4 relative) may reorder neighbouring spikes
        assert np.all(np.diff(xs) > 0)
    _say(f"spike {shape}: x in [{xs.min():.1f}, {xs.max():.1f}]")
    g = run_block(inp)
    check_queries(inp, g, range(spec.total_q) if spec.total_q < 64 else [0, 1, 7, 259, 519], f"spike-{shape}")
    assert int(pos[int(np.argmax(xs))]) in set(g["sel"][qi].tolist())


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_step_replays_from_a_hip_graph(dtype):
    """The entry points launch kernels only (no allocation, memset, copy or synchronisation),
    so a caller can capture a decode step (selector + a sparse layer) into a HIP graph.
    Each replay is checked against the eager run, with eager work on the outputs between
    replays."""
    spec = BlockSpec(f"graph-{dtype}", [30000, 9000], [[29999], [8999]], dtype=dtype, n_sparse=1,
                     needles_per_query=2, seed=33)
    inp = make_block_inputs(spec)
    dev = "cuda"
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, dev)
    k, v, q, qs = to_dev(inp.k), to_dev(inp.v), to_dev(inp.q_sel), to_dev(inp.q_sp[0])
    nq = spec.total_q
    out = torch.empty_like(q)
    lse = torch.empty(nq, 64, dtype=torch.float32, device=dev)
    sel = torch.empty(nq, spec.top_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(nq, dtype=torch.int32, device=dev)
    osp = torch.empty_like(qs)
    size_dt = "fp8" if dtype == "fp8" else torch.bfloat16
    ws1 = torch.empty(hs2.full_attn_select_workspace_size(batch, spec.window, spec.top_k, size_dt),
                      dtype=torch.uint8, device=dev)
    ws2 = torch.empty(max(1, hs2.sparse_attn_workspace_size(batch, spec.window, spec.top_k, size_dt)),
                      dtype=torch.uint8, device=dev)

    def step():
        if dtype == "fp8":
            hs2.full_attn_select_fp8kv(batch, q, k, v, spec.k_scale, spec.v_scale, spec.window, spec.top_k,
                                       spec.scale, out=out, lse=lse, sel_idx=sel, sel_count=cnt, workspace=ws1)
            hs2.sparse_attn_fp8kv(batch, qs, k, v, spec.k_scale, spec.v_scale, sel, spec.window, spec.top_k,
                                  spec.scale, out=osp, workspace=ws2)
        else:
            hs2.full_attn_select(batch, q, k, v, spec.window, spec.top_k, spec.scale, out=out, lse=lse,
                                 sel_idx=sel, sel_count=cnt, workspace=ws1)
            hs2.sparse_attn(batch, qs, k, v, sel, spec.window, spec.top_k, spec.scale, out=osp, workspace=ws2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager reference (and warm-up) on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, lse, sel, cnt, osp)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for _ in range(3):
        for x in (out, osp):
            x.fill_(float("nan"))
        lse.fill_(float("nan"))
        sel.fill_(-7)
        cnt.fill_(-7)
        ws1.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (out, lse, sel, cnt, osp)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
