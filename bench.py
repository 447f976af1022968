#!/usr/bin/env python
"""Benchmark of the HySparse2 attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input resident in HBM:
the full-attention selector (exact causal MQA attention, head-summed scores, top-1024
selection) followed by every sparse layer of the hybrid block on the selector's KV and
indices. The default workload is batched decode: 64 sequences x 131,072 cached tokens,
one query each, 1 selector + 7 sparse layers (bf16). `--workload 3/4/5` measures the
other workloads (5 also runs the KV Bridging projection of 1,048,576 hidden states);
`--workload 6` is the default workload on an FP8 E4M3 K/V cache; `--workload 8` is the
default workload with the decode-time KV Bridging of the 64 new tokens into 3 layers'
caches ahead of the selector; `--workload 7` is a
prefill: KV Bridging of 262,144 hidden states, then exact causal attention of every one of
the 262,144 positions (the self-decoder's full-attention layer, no selection).
`--workload 9` is the first-generation HySparse layout (the comparison variant) on the
default decode batch: GQA 64:4 selector with 64-token block selection, then 7 sparse
layers that fuse the selected blocks with a 128-token window branch through gates.

Prints ONE JSON line. Per-kernel durations come from HIP events recorded by the
library around each kernel it launches, on the stream it launches on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-decode tokens/s & HBM GB/s at 128k/1M ctx; select+attn TFLOP/s vs peak"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
QO_BYTES = 2 * 64 * 128 * 2         # one query's Q and O, bf16
QK_PV_FLOPS = 2 * 2 * 64 * 128      # per (query, key): QK^T and PV over 64 heads
SCORE_FLOPS = 2 * 64 * 128          # per candidate: the score pass recomputes QK^T
COUNTERS = os.path.join(ROOT, "profiles", "attn_pass1_decode_64x128k_counters.json")
SELECT_KERNELS = ["attn_pass1", "split_combine", "score_pass2", "topk_filter", "topk_finish"]
SPARSE_KERNELS = ["sparse_attn", "sparse_combine"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5, 6, 7, 8, 9])
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-1m", action="store_true", help="workload 2 only: skip the 1M-context sub-record")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy 3 times (counter calibration) and exit")
    return p.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("attn_decode.h", "attn_common.h", "kernel_common.h", "hs2_internal.h"):
        with open(os.path.join(ROOT, "long_context_mqa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(per_launch_keys: int):
    """HBM bytes of one pass-1 launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except OSError:
        return None
    if c.get("source_digest") != source_digest() or c.get("keys_per_launch") != per_launch_keys:
        return None
    return float(c["hbm_bytes_per_launch"])


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle, unchanged, on a bounded sample of the same workload's queries."""
    import numpy as np

    import oracle
    from workloads.gen import stored_to_f64

    sp = inp.spec
    order = list(range(sp.total_q))
    rng = np.random.default_rng(0)
    rng.shuffle(order)
    done, spent = 0, 0.0
    def kv(rows, scale):
        return oracle.dequantize_kv(rows, scale) if rows.dtype == np.uint8 else stored_to_f64(rows)

    for qi in order:
        s = int(inp.q_seq[qi])
        a, t = int(inp.kv_start[s]), int(inp.q_pos[qi])
        K = kv(inp.k[a:a + t + 1], sp.k_scale)
        V = kv(inp.v[a:a + t + 1], sp.v_scale)
        q = stored_to_f64(inp.q_sel[qi])
        qs = [stored_to_f64(x[qi]) for x in inp.q_sp]
        t0 = time.perf_counter()
        oracle.block_query(q, qs, K, V, t, sp.window, sp.top_k, sp.scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    return {"value": done / spent, "unit": "tokens/s", **host_cores(), "kind": "oracle",
            "sample": f"{done} of {sp.total_q} queries of {sp.name} (selector + {sp.n_sparse} sparse layers "
                      f"each, fp64, {spent:.1f} s)"}


def host_cores() -> dict:
    """Threads the oracle ran on (numpy's BLAS pool: the matrix products are its only
    multi-threaded steps), the host's logical CPUs and the CPU model name."""
    from threadpoolctl import threadpool_info

    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    model = ""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        model = next((l.split(":", 1)[1].strip() for l in out.splitlines() if l.startswith("Model name")), "")
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"cores": int(min(threads, affinity)), "host_cpus": os.cpu_count(), "cpus_in_affinity": affinity,
            "cpu_model": model}


def to_dev(a, device="cuda"):
    """Uploads stored values (bf16 bit patterns as uint16, or float32) to the GPU."""
    import numpy as np
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the library runs on a "
              f"single MI355X; how the path would shard over several GPUs is described, not built)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    if args.calibrate_copy:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30, "launches": 3}))
        return 0

    from long_context_mqa_amd import hs2
    from workloads.configs import block_config, make_bridge_inputs, make_block_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    hs2.load()
    if args.workload == 7:
        return run_prefill(args, hs2, block_config, make_block_inputs, make_bridge_inputs)
    if args.workload == 9:
        return run_v1(args, hs2)
    res = run_decode(args, hs2, args.workload, args.steps, args.warmup, args.cpu_seconds)
    if args.workload == 2 and not args.no_1m:
        # the same step at 1M context (8 sequences x 1,048,576 tokens): a sub-record, not the value
        log("1M context: decode-8x1M-bf16")
        r = run_decode(args, hs2, 3, max(5, min(args.steps, 20)), min(args.warmup, 3), min(args.cpu_seconds, 12.0))
        res["decode_1m"] = {k: r[k] for k in ("value", "unit", "ms_per_step", "steps", "config", "roofline", "block",
                                             "kernels_ms", "sparse_layer", "cpu_baseline")}
    print(json.dumps(res), flush=True)
    return 0


def run_decode(args, hs2, workload: int, steps: int, warmup: int, cpu_seconds: float) -> dict:
    """Decode-shaped and chunked workloads: a step is the selector plus every sparse
    layer (workload 5: after the KV Bridging of 1,048,576 hidden states; workload 8: after
    the decode-time bridging of the batch's new tokens). Returns the JSON record."""
    import numpy as np
    import torch

    from workloads.configs import block_config, make_bridge_inputs, make_block_inputs

    append = workload == 8
    spec = block_config(2 if append else workload)
    log(f"generating {spec.name}")
    inp = make_block_inputs(spec)
    dev = torch.device("cuda:0")
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, dev)
    k, v = to_dev(inp.k), to_dev(inp.v)
    q_sel = to_dev(inp.q_sel)
    q_sp = [to_dev(x) for x in inp.q_sp]
    nq = spec.total_q
    out = torch.empty_like(q_sel)
    lse = torch.empty(nq, 64, dtype=torch.float32, device=dev)
    sel = torch.empty(nq, spec.top_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(nq, dtype=torch.int32, device=dev)
    fp8 = spec.dtype == "fp8"
    ws_dt = "fp8" if fp8 else torch.bfloat16
    kv_row_bytes = 2 * 128 * (1 if fp8 else 2)  # one K row + one V row
    ws_sel = torch.empty(hs2.full_attn_select_workspace_size(batch, spec.window, spec.top_k, ws_dt),
                         dtype=torch.uint8, device=dev)
    ws_sp = torch.empty(max(1, hs2.sparse_attn_workspace_size(batch, spec.window, spec.top_k, ws_dt)),
                        dtype=torch.uint8, device=dev)

    def select_call():
        if fp8:
            hs2.full_attn_select_fp8kv(batch, q_sel, k, v, spec.k_scale, spec.v_scale, spec.window, spec.top_k,
                                       spec.scale, out=out, lse=lse, sel_idx=sel, sel_count=cnt, workspace=ws_sel)
        else:
            hs2.full_attn_select(batch, q_sel, k, v, spec.window, spec.top_k, spec.scale, out=out, lse=lse,
                                 sel_idx=sel, sel_count=cnt, workspace=ws_sel)

    def sparse_call(l):
        if fp8:
            hs2.sparse_attn_fp8kv(batch, q_sp[l], k, v, spec.k_scale, spec.v_scale, sel, spec.window, spec.top_k,
                                  spec.scale, out=outs[l], workspace=ws_sp)
        else:
            hs2.sparse_attn(batch, q_sp[l], k, v, sel, spec.window, spec.top_k, spec.scale, out=outs[l],
                            workspace=ws_sp)
    outs = [torch.empty_like(q_sel) for _ in range(spec.n_sparse)]
    bridge = None
    if workload == 5:
        log("generating bridging inputs (1,048,576 x 2048)")
        bi = make_bridge_inputs(1048576, n_layers=3, seed=5)
        bridge = {"h": to_dev(bi.h), "wk": [to_dev(w) for w in bi.w_k], "wv": [to_dev(w) for w in bi.w_v]}
        bridge["ko"] = [torch.empty(1048576, 128, dtype=torch.bfloat16, device=dev) for _ in range(3)]
        bridge["vo"] = [torch.empty(1048576, 128, dtype=torch.bfloat16, device=dev) for _ in range(3)]
        bridge["ws"] = torch.empty(hs2.bridge_kv_workspace_size(2048, 3), dtype=torch.uint8, device=dev)
        del bi
        # the decode runs on the bridged caches: sequence s takes bridged layer-0 rows
        # (o_s + j) mod 1,048,576 (o_s = the rows of the sequences before it), copied once,
        # untimed, into its packed rows; the planted needle rows are written on top
        hs2.bridge_kv(bridge["h"], bridge["wk"], bridge["wv"], bridge["ko"], bridge["vo"], workspace=bridge["ws"])
        src = torch.from_numpy(np.arange(spec.total_rows, dtype=np.int64) % 1048576).to(dev)
        k.copy_(bridge["ko"][0].index_select(0, src))
        v.copy_(bridge["vo"][0].index_select(0, src))
        nrow = torch.from_numpy(np.asarray([int(inp.kv_start[si]) + p for (si, _, _, p) in inp.needles],
                                           dtype=np.int64)).to(dev)
        k.index_copy_(0, nrow, to_dev(inp.k[nrow.cpu().numpy()]))
        del src, nrow
    if append:
        # decode-time bridging: the 64 new tokens' hidden states into the current-token
        # rows of 3 layers' caches (layer 0's are the block's K and V)
        log("generating the new tokens' hidden states and 3 layers' weights")
        bi = make_bridge_inputs(nq, n_layers=3, seed=8)
        app = {"h": to_dev(bi.h), "wk": [to_dev(w) for w in bi.w_k], "wv": [to_dev(w) for w in bi.w_v],
               "rows": torch.from_numpy((inp.kv_start + inp.kv_len - 1).astype(np.int64)).to(dev)}
        app["kc"] = [k] + [torch.empty_like(k) for _ in range(2)]
        app["vc"] = [v] + [torch.empty_like(v) for _ in range(2)]
        app["ws"] = torch.empty(max(1, hs2.bridge_kv_append_workspace_size(nq, 2048, 3)), dtype=torch.uint8,
                                device=dev)
        del bi
    torch.cuda.synchronize()

    def append_call():
        hs2.bridge_kv_append(app["h"], app["rows"], app["wk"], app["wv"], app["kc"], app["vc"], workspace=app["ws"])

    def new_events(n):
        """2n timing events plus a start marker; all recorded once so the HIP events exist."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n + 1)]
        s = torch.cuda.current_stream()
        for e in evs:
            e.record(s)
        return evs

    def attach(evs):
        if evs is None:
            hs2.set_kernel_events(None)
            return
        evs[-1].record(torch.cuda.current_stream())   # start marker of this call
        hs2.set_kernel_events([e.cuda_event for e in evs[:-1]])

    def step(ev_sel=None, ev_sp=None, ev_br=None, ev_app=None):
        if bridge is not None:
            attach(ev_br)
            hs2.bridge_kv(bridge["h"], bridge["wk"], bridge["wv"], bridge["ko"], bridge["vo"], workspace=bridge["ws"])
        if append:
            attach(ev_app)
            append_call()
        attach(ev_sel)
        select_call()
        for l in range(spec.n_sparse):
            attach(ev_sp[l] if ev_sp else None)
            sparse_call(l)
        hs2.set_kernel_events(None)

    log(f"warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed steps. Only the kernel the roofline is quoted for carries HIP events here
    # (selector pass 1; the bridging GEMM when bridging is part of the step): a pair of
    # events around every kernel would lengthen the step by ~10%.
    roof_events = []
    for _ in range(steps):
        n_ev = 4 if bridge is not None else 2
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for e in evs:
            e.record(torch.cuda.current_stream())
        roof_events.append(evs)
    torch.cuda.synchronize()

    def timed_step(evs):
        if bridge is not None:
            hs2.set_kernel_events([e.cuda_event for e in evs])      # slots: transpose, GEMM
            hs2.bridge_kv(bridge["h"], bridge["wk"], bridge["wv"], bridge["ko"], bridge["vo"], workspace=bridge["ws"])
            hs2.set_kernel_events(None)
        else:
            if append:
                append_call()
            hs2.set_kernel_events([e.cuda_event for e in evs])      # slot 0: pass 1
        select_call()
        hs2.set_kernel_events(None)
        for l in range(spec.n_sparse):
            sparse_call(l)

    log(f"timing {steps} steps")
    t0 = time.perf_counter()
    for s_ in range(steps):
        timed_step(roof_events[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / steps * 1e3
    if bridge is not None:
        roof_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in roof_events]))
    else:
        roof_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in roof_events]))

    # Per-kernel breakdown: an instrumented pass after the timed steps (events around
    # every kernel), not part of the timed figure.
    n_prof = min(steps, 10)
    ev = [(new_events(5), [new_events(2) for _ in range(spec.n_sparse)], new_events(2) if bridge else None,
           new_events(1) if append else None)
          for _ in range(n_prof)]
    torch.cuda.synchronize()
    for s_ in range(n_prof):
        step(*ev[s_])
    torch.cuda.synchronize()

    def mean_ms(calls, j):
        """Mean duration of slot j over the calls that launched it (None if none did)."""
        vals = [c[2 * j].elapsed_time(c[2 * j + 1]) for c in calls if c[-1].elapsed_time(c[2 * j]) >= 0.0]
        return float(np.mean(vals)) if vals else None

    sel_calls = [e[0] for e in ev]
    kern = {name: mean_ms(sel_calls, j) for j, name in enumerate(SELECT_KERNELS)}
    if spec.n_sparse:
        sp_calls = [ev[s_][1][l] for s_ in range(n_prof) for l in range(spec.n_sparse)]
        kern["sparse_attn"] = mean_ms(sp_calls, 0)
        kern["sparse_combine"] = mean_ms(sp_calls, 1)
    if bridge is not None:
        br = [e[2] for e in ev]
        kern["bridge_transpose"] = mean_ms(br, 0)
        kern["bridge_gemm"] = mean_ms(br, 1)
    if append:
        kern["bridge_append"] = mean_ms([e[3] for e in ev], 0)

    # algorithmic work
    keys = int(sum(int(t) + 1 for t in inp.q_pos))
    cands = int(sum(max(0, int(t) - spec.window + 1) for t in inp.q_pos))
    attended = int(sum(min(int(t) + 1, spec.window + spec.top_k) for t in inp.q_pos))
    decode = all(len(p) == 1 for p in spec.q_positions)
    sel_bytes = keys * kv_row_bytes if decode else spec.total_rows * kv_row_bytes
    layer_bytes = attended * kv_row_bytes + nq * QO_BYTES      # one sparse layer: gathered K+V rows, Q and O
    sparse_bytes = spec.n_sparse * layer_bytes
    step_bytes = sel_bytes + sparse_bytes
    flops_attn = keys * QK_PV_FLOPS + spec.n_sparse * attended * QK_PV_FLOPS
    flops_score = cands * SCORE_FLOPS

    # Sparse layer, warm and cold: a whole hs2_sparse_attn call (attention + split combine)
    # between two events, with no event between its kernels. Warm: right after another
    # sparse layer of the same step, whose gathered rows are then in the 256 MB
    # last-level cache (MALL) and the L2s. Cold: after a 512 MiB read-modify-write, which
    # evicts them both. The attention kernel alone, cold, comes from a second set of calls
    # with the library's events around each kernel.
    sparse_rec = None
    if spec.n_sparse:
        flush = torch.zeros(128 << 20, dtype=torch.int32, device=dev)   # 512 MiB
        reps = 10
        pairs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        kev = [new_events(2) for _ in range(reps)]
        torch.cuda.synchronize()
        for r_ in range(reps):
            e = pairs[r_]
            flush.add_(1)
            e[0].record()
            sparse_call(0)
            e[1].record()
            e[2].record()
            sparse_call(1 % spec.n_sparse)
            e[3].record()
        for r_ in range(reps):
            flush.add_(1)
            attach(kev[r_])
            sparse_call(0)
            hs2.set_kernel_events(None)
        torch.cuda.synchronize()
        del flush
        cold_us = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in pairs]))
        warm_us = float(np.median([e[2].elapsed_time(e[3]) * 1e3 for e in pairs]))
        cold_att = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in kev]))
        sparse_rec = {"alg_bytes": layer_bytes, "bound": "hbm", "peak_gbps": HBM_PEAK_GBPS,
                      "warm_us": warm_us, "warm_gbps": layer_bytes / (warm_us * 1e-6) / 1e9,
                      "warm_frac": layer_bytes / (warm_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                      "cold_us": cold_us, "cold_gbps": layer_bytes / (cold_us * 1e-6) / 1e9,
                      "cold_frac": layer_bytes / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                      "cold_attn_kernel_us": cold_att,
                      "warm_kernels_us": {"attn": (kern.get("sparse_attn") or 0.0) * 1e3,
                                          "combine": (kern.get("sparse_combine") or 0.0) * 1e3},
                      "method": "median of 10 calls, each between two events (attention + split combine); cold "
                                "after a 512 MiB read-modify-write that evicts the L2s and the 256 MB MALL, warm "
                                "right after another sparse layer on the same rows; warm_kernels_us from the "
                                "per-kernel events of the instrumented steps"}

    res = {
        "metric": METRIC,
        "value": nq / (elapsed / steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic: seeded N(0,1) Q (bf16), K/V as OCP FP8 E4M3 codes with per-tensor scales, planted "
                 "needle keys" if fp8 else "synthetic: seeded N(0,1) Q/K/V (bf16) with planted needle keys"),
        "config": {"workload": spec.name, "seqs": len(spec.seq_lens), "queries": nq,
                   "ctx": int(max(spec.seq_lens)), "sparse_layers": spec.n_sparse, "window": spec.window,
                   "top_k": spec.top_k, "q_heads": 64, "kv_heads": 1, "head_dim": 128,
                   "parallelism": "single GPU"},
    }
    if workload == 5:
        res["config"]["bridging"] = {"rows": 1048576, "d_model": 2048, "layers": 3}
        res["data"] = ("synthetic: seeded N(0,1) hidden states and Q (bf16), weights N(0, 0.02^2); the decode "
                       "runs on the bridged layer-0 K/V with planted needle keys")
    if append:
        res["config"]["workload"] = "decode-64x128k-bf16+bridging-append"
        res["config"]["bridging_append"] = {"new_tokens": nq, "d_model": 2048, "layers": 3,
                                            "weights_bytes": 3 * 2 * 2048 * 128 * 2}
    if fp8:
        res["config"]["kv_storage"] = {"format": "OCP FP8 E4M3", "k_scale": spec.k_scale, "v_scale": spec.v_scale,
                                       "compute": "codes converted exactly to bf16 for the MFMA"}
    if bridge is not None:
        f = 2 * 1048576 * 2048 * 256 * 3
        ach = f / (roof_ms * 1e-3) / 1e12
        res["roofline"] = {"kernel": "bridge_gemm (KV Bridging, 1,048,576 x 2,048 x 768)", "bound": "mfma",
                           "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / BF16_PEAK_TFLOPS, "traffic": None, "alg_flops_per_launch": f,
                           "avg_launch_ms": roof_ms}
    elif decode:
        a_bytes = keys * kv_row_bytes
        res["roofline"] = {"kernel": "attn_pass1 (selector exact attention, K+V once)", "bound": "hbm",
                           "achieved": a_bytes / (roof_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": a_bytes / (roof_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                           "traffic": counter_traffic(keys) if workload == 2 else None,
                           "alg_bytes_per_launch": a_bytes, "avg_launch_ms": roof_ms}
    else:
        f = keys * QK_PV_FLOPS
        ach = f / (roof_ms * 1e-3) / 1e12
        res["roofline"] = {"kernel": "attn_pass1 (selector exact attention)", "bound": "mfma", "achieved": ach,
                           "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                           "traffic": None, "alg_flops_per_launch": f, "avg_launch_ms": roof_ms}
    res["block"] = {
        "hbm_gbps_alg": step_bytes / (ms_step * 1e-3) / 1e9,
        "hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "tflops_alg": (flops_attn + flops_score) / (ms_step * 1e-3) / 1e12,
        "alg_bytes_per_step": step_bytes,
        "alg_flops_per_step": flops_attn + flops_score,
    }
    res["kernels_ms"] = kern
    res["kernels_ms_source"] = f"HIP events around every kernel over {n_prof} steps after the timed ones"
    res["sparse_layer"] = sparse_rec
    if bridge is not None:
        bf = 2 * 1048576 * 2048 * 256 * 3
        res["bridging"] = {"ms": kern["bridge_gemm"], "tflops": bf / (kern["bridge_gemm"] * 1e-3) / 1e12,
                           "frac_mfma": bf / (kern["bridge_gemm"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        # the same projection written as FP8 E4M3 caches (one scale per tensor), timed after
        # the timed steps with events around its GEMM
        log("timing the FP8-output bridging")
        ko8 = [torch.empty(1048576, 128, dtype=torch.uint8, device=dev) for _ in range(3)]
        vo8 = [torch.empty(1048576, 128, dtype=torch.uint8, device=dev) for _ in range(3)]
        ev8 = [new_events(2) for _ in range(10)]
        for _ in range(3):   # untimed: the clock ramps back up after the steps' lighter kernels
            hs2.bridge_kv_fp8kv(bridge["h"], bridge["wk"], bridge["wv"], 0.01, 0.01, ko8, vo8,
                                workspace=bridge["ws"])
        torch.cuda.synchronize()
        for e in ev8:
            attach(e)
            hs2.bridge_kv_fp8kv(bridge["h"], bridge["wk"], bridge["wv"], 0.01, 0.01, ko8, vo8,
                                workspace=bridge["ws"])
        hs2.set_kernel_events(None)
        torch.cuda.synchronize()
        ms8 = float(np.median([e[2].elapsed_time(e[3]) for e in ev8]))
        res["bridging_fp8"] = {"ms": ms8, "tflops": bf / (ms8 * 1e-3) / 1e12,
                               "frac_mfma": bf / (ms8 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                               "output": "OCP FP8 E4M3 codes, k_scale = v_scale = 0.01 for every layer",
                               "method": "median GEMM time of 10 calls after 3 untimed ones, HIP events "
                                         "around the kernel"}
        del ko8, vo8
    res["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a sample (cpu baseline)")
        res["cpu_baseline"] = cpu_baseline(inp, cpu_seconds)
    return res


def run_prefill(args, hs2, block_config, make_block_inputs, make_bridge_inputs) -> int:
    """Workload 7: a step is the KV Bridging of N hidden states (3 layers) followed by the
    exact causal attention of all N positions of one sequence (no selection)."""
    import numpy as np
    import torch

    spec = block_config(7)
    n = spec.total_rows
    log(f"generating {spec.name}")
    inp = make_block_inputs(spec)
    dev = torch.device("cuda:0")
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, n, dev)
    k, v, q = to_dev(inp.k), to_dev(inp.v), to_dev(inp.q_sel)
    # what the oracle's timing needs: the caches and the query rows of an even grid of positions
    grid = np.linspace(0, n - 1, 4096).astype(np.int64)
    np.random.default_rng(0).shuffle(grid)
    cpu_in = (inp.k, inp.v, grid, inp.q_sel[grid].copy())
    del inp
    out = torch.empty_like(q)
    lse = torch.empty(n, 64, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, hs2.causal_attn_workspace_size(batch)), dtype=torch.uint8, device=dev)
    log(f"generating bridging inputs ({n} x 2048)")
    bi = make_bridge_inputs(n, n_layers=3, seed=7)
    h = to_dev(bi.h)
    wk, wv = [to_dev(w) for w in bi.w_k], [to_dev(w) for w in bi.w_v]
    ko = [torch.empty(n, 128, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    vo = [torch.empty(n, 128, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    bws = torch.empty(hs2.bridge_kv_workspace_size(2048, 3), dtype=torch.uint8, device=dev)
    del bi
    torch.cuda.synchronize()

    def new_events(m):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(m)]
        for e in evs:
            e.record(torch.cuda.current_stream())
        return evs

    def step(ev_att=None, ev_br=None):
        hs2.set_kernel_events([e.cuda_event for e in ev_br] if ev_br else None)   # slots: transpose, GEMM
        hs2.bridge_kv(h, wk, wv, ko, vo, workspace=bws)
        hs2.set_kernel_events([e.cuda_event for e in ev_att] if ev_att else None)  # slot 0: attention
        hs2.causal_attn(batch, q, k, v, spec.scale, out=out, lse=lse, workspace=ws)
        hs2.set_kernel_events(None)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(new_events(2), new_events(4)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(*evs[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    att_ms = float(np.mean([e[0][0].elapsed_time(e[0][1]) for e in evs]))
    gemm_ms = float(np.mean([e[1][2].elapsed_time(e[1][3]) for e in evs]))
    pairs = n * (n + 1) // 2
    f_att = pairs * QK_PV_FLOPS
    f_br = 2 * n * 2048 * 256 * 3
    ach = f_att / (att_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": n / (elapsed / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V and hidden states (bf16), weights N(0, 0.02^2)",
        "config": {"workload": spec.name, "tokens": n, "queries": n, "q_heads": 64, "kv_heads": 1, "head_dim": 128,
                   "bridging": {"rows": n, "d_model": 2048, "layers": 3}, "parallelism": "single GPU"},
        "roofline": {"kernel": "attn_chunk (causal attention of every position, no selection)", "bound": "mfma",
                     "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                     "traffic": None, "alg_flops_per_launch": f_att, "avg_launch_ms": att_ms},
        "kernels_ms": {"causal_attn_pass1": att_ms, "bridge_gemm": gemm_ms},
        "kernels_ms_source": "HIP events around the two kernels inside the timed steps",
        "bridging": {"ms": gemm_ms, "tflops": f_br / (gemm_ms * 1e-3) / 1e12,
                     "frac_mfma": f_br / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a sample (cpu baseline)")
        res["cpu_baseline"] = cpu_baseline_prefill(spec, *cpu_in, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline_prefill(spec, k_stored, v_stored, grid, q_rows, budget_s: float):
    """The fp64 oracle, unchanged, on evenly spaced positions of the prefill: the bridging
    of the position's hidden state into 3 layers' K/V, then its exact causal attention.
    Positions are visited in a shuffled order of an even grid over [0, n) (`grid`, with
    their query rows `q_rows`), so the mean cost of the visited ones is that of the whole
    prefill."""
    import oracle
    from workloads.configs import make_bridge_inputs
    from workloads.gen import stored_to_f64

    n = spec.total_rows
    K, V = stored_to_f64(k_stored), stored_to_f64(v_stored)
    bi = make_bridge_inputs(64, n_layers=3, seed=7)
    wk = [stored_to_f64(w) for w in bi.w_k]
    wv = [stored_to_f64(w) for w in bi.w_v]
    h = stored_to_f64(bi.h)
    done, spent = 0, 0.0
    for t, qrow in zip(grid, q_rows):
        q = stored_to_f64(qrow)
        t0 = time.perf_counter()
        oracle.bridge_kv(h[done % 64:done % 64 + 1], wk, wv)
        oracle.full_attention(q, K, V, int(t), spec.scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    return {"value": done / spent, "unit": "tokens/s", **host_cores(), "kind": "oracle",
            "sample": f"{done} of {n} positions of {spec.name}, evenly spaced (bridging of one hidden state into "
                      f"3 layers' K/V + exact causal attention of the position, fp64, {spent:.1f} s)"}


def cpu_baseline_v1(inp, budget_s: float):
    """The fp64 first-generation oracle, unchanged, on a bounded sample of the queries."""
    import numpy as np

    from oracle import hysparse_v1 as ov1
    from workloads.gen import stored_to_f64
    from workloads.v1 import kv_rows

    sp = inp.spec
    order = list(range(sp.total_q))
    np.random.default_rng(0).shuffle(order)
    done, spent = 0, 0.0
    for qi in order:
        s = int(inp.q_seq[qi])
        a, t = int(inp.kv_start[s]), int(inp.q_pos[qi])
        K = stored_to_f64(kv_rows(inp, "k", a, a + t + 1))
        V = stored_to_f64(kv_rows(inp, "v", a, a + t + 1))
        R = inp.k_swa[0].shape[1]
        swa = []
        for l in range(sp.n_sparse):
            Ks = np.zeros((t + 1, 4, 128))
            Vs = np.zeros((t + 1, 4, 128))
            for p_ in range(max(0, t - sp.window + 1), t + 1):
                Ks[p_] = stored_to_f64(inp.k_swa[l][s, p_ % R])
                Vs[p_] = stored_to_f64(inp.v_swa[l][s, p_ % R])
            swa.append((Ks, Vs))
        q = stored_to_f64(inp.q_sel[qi])
        qs = [stored_to_f64(x[qi]) for x in inp.q_sp]
        t0 = time.perf_counter()
        r = ov1.v1_selector_query(q, K, V, t, sp.scale, sp.top_blocks)
        for l in range(sp.n_sparse):
            ov1.v1_sparse_query(qs[l], K, V, t, r["sel"], swa[l][0], swa[l][1], inp.gate_sp[l][qi].astype(np.float64),
                                inp.gate_swa[l][qi].astype(np.float64), sp.scale, sp.window)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    return {"value": done / spent, "unit": "tokens/s", **host_cores(), "kind": "oracle",
            "sample": f"{done} of {sp.total_q} queries of {sp.name} (selector + {sp.n_sparse} sparse layers "
                      f"each, fp64, {spent:.1f} s)"}


def run_v1(args, hs2) -> int:
    """Workload 9: the first-generation layout on the decode batch of workload 2. A step is
    the GQA selector (exact attention plus block selection) and 7 gated sparse layers."""
    import numpy as np
    import torch

    from workloads.v1 import kv_rows, make_v1_inputs, v1_config

    spec = v1_config(9)
    log(f"generating {spec.name}")
    inp = make_v1_inputs(spec, with_kv=False)
    dev = torch.device("cuda:0")
    rows = spec.total_rows
    k = torch.empty(rows, 4, 128, dtype=torch.bfloat16, device=dev)
    v = torch.empty(rows, 4, 128, dtype=torch.bfloat16, device=dev)
    for si in range(len(spec.seq_lens)):   # one sequence at a time: no whole host copy
        a, n = int(inp.kv_start[si]), int(inp.kv_len[si])
        k[a:a + n] = to_dev(kv_rows(inp, "k", a, a + n))
        v[a:a + n] = to_dev(kv_rows(inp, "v", a, a + n))
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, rows, dev)
    q_sel = to_dev(inp.q_sel)
    q_sp = [to_dev(x) for x in inp.q_sp]
    k_swa = [to_dev(x) for x in inp.k_swa]
    v_swa = [to_dev(x) for x in inp.v_swa]
    g_sp = [to_dev(x) for x in inp.gate_sp]
    g_sw = [to_dev(x) for x in inp.gate_swa]
    nq = spec.total_q
    out = torch.empty_like(q_sel)
    lse = torch.empty(nq, 64, dtype=torch.float32, device=dev)
    bi = torch.empty(nq, 4, spec.top_blocks, dtype=torch.int32, device=dev)
    bc = torch.empty(nq, 4, dtype=torch.int32, device=dev)
    ws_sel = torch.empty(hs2.v1_full_attn_select_workspace_size(batch, spec.top_blocks), dtype=torch.uint8, device=dev)
    ws_sp = torch.empty(hs2.v1_sparse_attn_workspace_size(batch, spec.top_blocks), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(q_sel) for _ in range(spec.n_sparse)]
    torch.cuda.synchronize()

    def new_events(m):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(m)]
        for e in evs:
            e.record(torch.cuda.current_stream())
        return evs

    def step(ev_sel=None, ev_sp=None):
        hs2.set_kernel_events([e.cuda_event for e in ev_sel] if ev_sel else None)
        hs2.v1_full_attn_select(batch, q_sel, k, v, spec.top_blocks, spec.scale, out=out, lse=lse, blk_idx=bi,
                                blk_count=bc, workspace=ws_sel)
        for l in range(spec.n_sparse):
            hs2.set_kernel_events([e.cuda_event for e in ev_sp[l]] if ev_sp else None)
            hs2.v1_sparse_attn(batch, q_sp[l], k, v, bi, k_swa[l], v_swa[l], g_sp[l], g_sw[l], spec.window,
                               spec.scale, out=outs[l], workspace=ws_sp)
        hs2.set_kernel_events(None)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [new_events(2) for _ in range(args.steps)]   # selector attention pass only
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    att_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    # one instrumented step after the timed ones: every kernel of the step
    ev_all = new_events(4)
    ev_l = [new_events(4) for _ in range(spec.n_sparse)]
    torch.cuda.synchronize()
    step(ev_all, ev_l)
    torch.cuda.synchronize()
    kms = {"v1_attn_pass": ev_all[0].elapsed_time(ev_all[1]), "v1_combine_select": ev_all[2].elapsed_time(ev_all[3]),
           "v1_sparse_attn": float(np.mean([e[0].elapsed_time(e[1]) for e in ev_l])),
           "v1_gate_combine": float(np.mean([e[2].elapsed_time(e[3]) for e in ev_l]))}
    keys = int(np.sum(inp.q_pos.astype(np.int64) + 1))
    alg = keys * 4 * 128 * 2 * 2 + nq * 64 * 128 * 2       # K and V of every key (4 KV heads), plus Q
    ach = alg / (att_ms * 1e-3) / 1e9
    sp_keys = nq * 4 * (spec.top_blocks * 64 + spec.window)
    sp_bytes = sp_keys * 2 * 128 * 2 + nq * 64 * 128 * 2
    res = {
        "metric": METRIC,
        "value": nq / (elapsed / args.steps),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V and window K/V (bf16), uniform [0,1) gates, 8 needles per query",
        "config": {"workload": spec.name, "seqs": len(spec.seq_lens), "ctx": spec.seq_lens[0], "queries": nq,
                   "q_heads": 64, "kv_heads": 4, "head_dim": 128, "block": 64, "top_blocks": spec.top_blocks,
                   "window": spec.window, "layers": {"selector": 1, "sparse": spec.n_sparse},
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "v1_attn_pass (GQA selector attention with block LSEs)", "bound": "hbm",
                     "achieved": ach, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                     "traffic": None, "alg_bytes_per_launch": alg, "avg_launch_ms": att_ms},
        "kernels_ms": kms,
        "kernels_ms_source": "roofline kernel: HIP events inside the timed steps; others: one instrumented step",
        "sparse_layer": {"alg_bytes": sp_bytes, "us": kms["v1_sparse_attn"] * 1e3,
                         "gbps": sp_bytes / (kms["v1_sparse_attn"] * 1e-3) / 1e9},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_v1(inp, args.cpu_seconds),
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
