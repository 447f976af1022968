"""C ABI checks that need no GPU: the library loads, exports what include/hs2.h
declares, and rejects bad arguments on the host before enqueueing anything.

Every call here fails a host-side check, so no HIP call is made; the pointers
passed are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from long_context_mqa_amd import hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs2.h")
FAKE = 0x10000  # a non-null, 256-byte aligned address that is never dereferenced


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hs2.LIB_PATH):
        from long_context_mqa_amd import build
        build.build()
    return hs2.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(hs2.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_version(lib):
    assert lib.hs2_version() == 10000


def _batch(total_q=1, max_kv_len=4096, rows=4096, num_seqs=1):
    return hs2.hs2_seqs(num_seqs, FAKE, FAKE, FAKE, FAKE, total_q, max_kv_len, rows, 1)


def _select(lib, b, n_heads=64, head_dim=128, window=128, top_k=1024, scale=0.088, ws=None, ws_bytes=None,
            dt=hs2.HS2_BF16, q=FAKE, out=FAKE * 2, sel=FAKE * 3):
    if ws_bytes is None:
        ws_bytes = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b), n_heads, head_dim, window, top_k, dt)
    return lib.hs2_full_attn_select(ctypes.byref(b), q, FAKE, FAKE, n_heads, head_dim, window, top_k, scale, out,
                                    None, sel, None, FAKE if ws is None else ws, ws_bytes, dt, None)


def test_select_rejects_bad_arguments(lib):
    b = _batch()
    assert _select(lib, b, n_heads=32) == hs2.HS2_ERR_UNSUPPORTED
    assert b"n_heads=64" in lib.hs2_last_error()
    assert _select(lib, b, head_dim=64) == hs2.HS2_ERR_UNSUPPORTED
    assert _select(lib, b, dt=7) == hs2.HS2_ERR_UNSUPPORTED
    assert _select(lib, b, window=0) == hs2.HS2_ERR_INVALID_ARG
    assert _select(lib, b, top_k=-1) == hs2.HS2_ERR_INVALID_ARG
    assert _select(lib, b, top_k=hs2.MAX_TOP_K + 1) == hs2.HS2_ERR_INVALID_ARG
    assert _select(lib, b, scale=0.0) == hs2.HS2_ERR_INVALID_ARG
    assert _select(lib, b, scale=float("nan")) == hs2.HS2_ERR_INVALID_ARG
    assert _select(lib, b, q=FAKE + 8) == hs2.HS2_ERR_INVALID_ARG        # misaligned
    assert _select(lib, b, out=FAKE) == hs2.HS2_ERR_INVALID_ARG          # aliases k
    assert _select(lib, b, sel=None) == hs2.HS2_ERR_INVALID_ARG
    assert _select(lib, b, ws_bytes=16) == hs2.HS2_ERR_WORKSPACE
    assert b"workspace" in lib.hs2_last_error()
    assert _select(lib, b, ws=FAKE + 64, ws_bytes=1 << 40) == hs2.HS2_ERR_WORKSPACE  # misaligned
    assert lib.hs2_full_attn_select(None, FAKE, FAKE, FAKE, 64, 128, 128, 1024, 0.1, FAKE, None, FAKE, None,
                                    FAKE, 1 << 30, 0, None) == hs2.HS2_ERR_INVALID_ARG
    bad = hs2.hs2_seqs(0, FAKE, FAKE, FAKE, FAKE, 1, 10, 10, 1)
    assert _select(lib, bad) == hs2.HS2_ERR_INVALID_ARG
    bad = hs2.hs2_seqs(1, None, FAKE, FAKE, FAKE, 1, 10, 10, 1)
    assert _select(lib, bad) == hs2.HS2_ERR_INVALID_ARG


def test_host_lengths_beyond_max_kv_len_are_rejected(lib):
    """The split planner sizes its work items from kv_len_host; a value above the
    max_kv_len bound (or negative) is an invalid argument, for selection and sparse calls."""
    import numpy as np
    for lens in ([4096, 4097], [-1, 100]):
        kh = np.asarray(lens, dtype=np.int32)
        b = hs2.hs2_seqs(2, FAKE, FAKE, FAKE, FAKE, 2, 4096, 8193, 1, kh.ctypes.data)
        assert _select(lib, b, ws_bytes=1 << 40) == hs2.HS2_ERR_INVALID_ARG
        assert b"kv_len_host" in lib.hs2_last_error()
        assert lib.hs2_sparse_attn(ctypes.byref(b), FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 64, 128, 128, 1024, 0.088,
                                   FAKE * 5, None, FAKE * 6, 1 << 40, hs2.HS2_BF16, None) == hs2.HS2_ERR_INVALID_ARG
        assert b"kv_len_host" in lib.hs2_last_error()
    kh = np.asarray([4096, 17], dtype=np.int32)  # within the bound: accepted by the host checks
    b = hs2.hs2_seqs(2, FAKE, FAKE, FAKE, FAKE, 2, 4096, 8193, 1, kh.ctypes.data)
    assert _select(lib, b, ws_bytes=16) == hs2.HS2_ERR_WORKSPACE  # fails later, at the workspace size


def test_sparse_rejects_bad_arguments(lib):
    b = _batch()
    ws = lib.hs2_sparse_attn_workspace_size(ctypes.byref(b), 64, 128, 128, 1024, 0)
    assert ws > 0  # one query is split over several workgroups
    call = lambda **kw: lib.hs2_sparse_attn(ctypes.byref(b), FAKE, FAKE, FAKE, kw.get("sel", FAKE * 3), 64,
                                            kw.get("hd", 128), 128, kw.get("k", 1024), 0.088, FAKE * 2, None,
                                            FAKE, kw.get("ws", ws), 0, None)
    assert call(hd=96) == hs2.HS2_ERR_UNSUPPORTED
    assert call(sel=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(ws=ws - 1) == hs2.HS2_ERR_WORKSPACE


def test_bridge_rejects_bad_arguments(lib):
    P = ctypes.c_void_p * 3
    w = P(FAKE, FAKE, FAKE)
    o = P(FAKE * 2, FAKE * 3, FAKE * 4)
    ws = lib.hs2_bridge_kv_workspace_size(2048, 3, 128)
    assert ws == 2 * 3 * 128 * 2048 * 2
    ok_args = dict(h=FAKE * 5, n=1000, d=2048, L=3, hd=128, ws=ws, dt=0)

    def call(**kw):
        a = {**ok_args, **kw}
        return lib.hs2_bridge_kv(a["h"], a["n"], a["d"], a["L"], w, w, o, o, a["hd"], FAKE * 8, a["ws"], a["dt"],
                                 None)
    assert call(dt=1) == hs2.HS2_ERR_UNSUPPORTED
    assert call(hd=64) == hs2.HS2_ERR_UNSUPPORTED
    assert call(d=2000) == hs2.HS2_ERR_UNSUPPORTED
    assert call(L=9) == hs2.HS2_ERR_UNSUPPORTED
    assert call(n=-1) == hs2.HS2_ERR_INVALID_ARG
    assert call(h=FAKE * 5 + 2) == hs2.HS2_ERR_INVALID_ARG
    assert call(ws=ws - 2) == hs2.HS2_ERR_WORKSPACE


def test_fp8_bridge_rejects_bad_arguments(lib):
    """The FP8-output bridging checks everything hs2_bridge_kv checks, plus its scales."""
    P = ctypes.c_void_p * 3
    F = ctypes.c_float * 3
    w = P(FAKE, FAKE, FAKE)
    o = P(FAKE * 2, FAKE * 3, FAKE * 4)
    ws = lib.hs2_bridge_kv_workspace_size(2048, 3, 128)
    good = F(0.05, 0.05, 0.05)

    def call(ks=good, vs=good, ws_bytes=ws, hd=128, n=1000):
        return lib.hs2_bridge_kv_fp8kv(FAKE * 5, n, 2048, 3, w, w, o, o, ks, vs, hd, FAKE * 8, ws_bytes, None)
    assert call(ks=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(vs=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(ks=F(0.05, 0.0, 0.05)) == hs2.HS2_ERR_INVALID_ARG
    assert call(vs=F(0.05, 0.05, -1.0)) == hs2.HS2_ERR_INVALID_ARG
    assert call(ks=F(0.05, float("inf"), 0.05)) == hs2.HS2_ERR_INVALID_ARG
    assert call(ks=F(0.05, float("nan"), 0.05)) == hs2.HS2_ERR_INVALID_ARG
    assert call(vs=F(1e-45, 0.05, 0.05)) == hs2.HS2_ERR_INVALID_ARG   # reciprocal overflows
    assert call(hd=64) == hs2.HS2_ERR_UNSUPPORTED
    assert call(n=-1) == hs2.HS2_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 2) == hs2.HS2_ERR_WORKSPACE


def test_fp8_append_rejects_bad_arguments(lib):
    """The FP8 append checks everything hs2_bridge_kv_append checks, plus its scales."""
    P = ctypes.c_void_p * 2
    F = ctypes.c_float * 2
    w = P(FAKE, FAKE)
    c = P(FAKE * 2, FAKE * 3)
    ws = lib.hs2_bridge_kv_append_workspace_size(64, 2048, 2, 128)
    good = F(0.05, 0.05)

    def call(ks=good, vs=good, n_new=64, ws_bytes=ws, hd=128):
        return lib.hs2_bridge_kv_append_fp8kv(FAKE * 5, n_new, FAKE * 6, 3000, 2048, 2, w, w, c, c, ks, vs, hd,
                                              FAKE * 8, ws_bytes, None)
    assert call(ks=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(vs=F(0.05, 0.0)) == hs2.HS2_ERR_INVALID_ARG
    assert call(ks=F(float("inf"), 0.05)) == hs2.HS2_ERR_INVALID_ARG
    assert call(n_new=-1) == hs2.HS2_ERR_INVALID_ARG
    assert call(hd=64) == hs2.HS2_ERR_UNSUPPORTED
    assert call(ws_bytes=ws - 1) == hs2.HS2_ERR_WORKSPACE


def test_workspace_sizes_grow_with_the_batch(lib):
    small = _batch(total_q=4, max_kv_len=8192, rows=8192 * 4, num_seqs=4)
    big = _batch(total_q=64, max_kv_len=131072, rows=131072 * 64, num_seqs=64)
    s = lib.hs2_full_attn_select_workspace_size(ctypes.byref(small), 64, 128, 128, 1024, 0)
    g = lib.hs2_full_attn_select_workspace_size(ctypes.byref(big), 64, 128, 128, 1024, 0)
    assert 0 < s < g
    # scores of every candidate of every query fit
    assert g >= 64 * (131072 - 127) * 4
    assert lib.hs2_full_attn_select_workspace_size(None, 64, 128, 128, 1024, 0) == 0


def test_sparse_workspace_of_many_query_batches_is_empty(lib):
    """bf16 / FP8 sparse layers of at least two queries per CU (512) take one workgroup per
    query with no split partials: no workspace; below that the keys are split and the
    partials need one."""
    for dt in (hs2.HS2_BF16, hs2.HS2_FP8_E4M3):
        few = _batch(total_q=511, max_kv_len=8192, rows=8192, num_seqs=1)
        many = _batch(total_q=512, max_kv_len=8192, rows=8192, num_seqs=1)
        assert lib.hs2_sparse_attn_workspace_size(ctypes.byref(few), 64, 128, 128, 1024, dt) > 0
        assert lib.hs2_sparse_attn_workspace_size(ctypes.byref(many), 64, 128, 128, 1024, dt) == 0


def test_workspace_sizes_follow_host_lengths(lib):
    """Ragged single-query batches with a host copy of the lengths are planned from those
    lengths: the selector's workspace (per-split partials) differs from the equal-length
    plan, and both sizes are positive and 256-byte multiples."""
    import numpy as np
    lens = np.array([4096, 6000, 300000, 510000, 9000, 120000] * 5, dtype=np.int32)
    b0 = hs2.hs2_seqs(len(lens), FAKE, FAKE, FAKE, FAKE, len(lens), int(lens.max()), int(lens.sum()), 1)
    b1 = hs2.hs2_seqs(len(lens), FAKE, FAKE, FAKE, FAKE, len(lens), int(lens.max()), int(lens.sum()), 1,
                      lens.ctypes.data)
    s0 = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b0), 64, 128, 128, 1024, hs2.HS2_BF16)
    s1 = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b1), 64, 128, 128, 1024, hs2.HS2_BF16)
    assert s0 > 0 and s1 > 0 and s0 % 256 == 0 and s1 % 256 == 0
    assert s0 != s1


def test_fp8kv_rejects_bad_arguments(lib):
    b = _batch()
    ws = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b), 64, 128, 128, 1024, hs2.HS2_FP8_E4M3)
    assert ws > 0

    def sel(ks=0.05, vs=0.03, hd=128, w=ws):
        return lib.hs2_full_attn_select_fp8kv(ctypes.byref(b), FAKE, FAKE, FAKE, ks, vs, 64, hd, 128, 1024, 0.088,
                                              FAKE * 2, None, FAKE * 3, None, FAKE, w, None)
    assert sel(ks=0.0) == hs2.HS2_ERR_INVALID_ARG
    assert sel(vs=float("inf")) == hs2.HS2_ERR_INVALID_ARG
    assert b"k_scale" in lib.hs2_last_error()
    assert sel(hd=64) == hs2.HS2_ERR_UNSUPPORTED
    assert sel(w=ws - 1) == hs2.HS2_ERR_WORKSPACE
    # the bf16 entry points do not take FP8 K/V (they have no scales)
    assert _select(lib, b, dt=hs2.HS2_FP8_E4M3, ws_bytes=ws) == hs2.HS2_ERR_UNSUPPORTED
    assert b"fp8kv" in lib.hs2_last_error()
    sws = lib.hs2_sparse_attn_workspace_size(ctypes.byref(b), 64, 128, 128, 1024, hs2.HS2_FP8_E4M3)
    assert lib.hs2_sparse_attn_fp8kv(ctypes.byref(b), FAKE, FAKE, FAKE, -1.0, 0.03, FAKE * 3, 64, 128, 128, 1024,
                                     0.088, FAKE * 2, None, FAKE, sws, None) == hs2.HS2_ERR_INVALID_ARG
    assert lib.hs2_sparse_attn(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE * 3, 64, 128, 128, 1024, 0.088, FAKE * 2,
                               None, FAKE, sws, hs2.HS2_FP8_E4M3, None) == hs2.HS2_ERR_UNSUPPORTED


def test_causal_rejects_bad_arguments(lib):
    b = _batch(total_q=4096, max_kv_len=4096, rows=4096)
    b.max_q_per_seq = 4096
    ws = lib.hs2_causal_attn_workspace_size(ctypes.byref(b), 64, 128, hs2.HS2_BF16)
    call = lambda **kw: lib.hs2_causal_attn(ctypes.byref(b), FAKE, FAKE, FAKE, 64, kw.get("hd", 128),
                                            kw.get("scale", 0.088), FAKE * 2, None, FAKE, kw.get("ws", ws),
                                            kw.get("dt", hs2.HS2_BF16), None)
    assert call(hd=256) == hs2.HS2_ERR_UNSUPPORTED
    assert call(scale=-1.0) == hs2.HS2_ERR_INVALID_ARG
    assert call(dt=hs2.HS2_FP8_E4M3) == hs2.HS2_ERR_UNSUPPORTED
    if ws > 0:
        assert call(ws=ws - 1) == hs2.HS2_ERR_WORKSPACE
    # one sequence of 4,096 queries: q-tiles whose keys are not split need no partials,
    # so the prefill workspace is only the q-tile list, far below the selector's
    s_sel = lib.hs2_full_attn_select_workspace_size(ctypes.byref(b), 64, 128, 128, 1024, hs2.HS2_BF16)
    assert ws < 64 * 1024 < s_sel


def test_bridge_append_rejects_bad_arguments(lib):
    P = ctypes.c_void_p * 3
    w = P(FAKE, FAKE, FAKE)
    c = P(FAKE * 2, FAKE * 3, FAKE * 4)
    ws = lib.hs2_bridge_kv_append_workspace_size(64, 2048, 3, 128)
    assert ws == 2048 // 128 * 64 * 6 * 128 * 4
    ok_args = dict(h=FAKE * 5, n=64, rows=FAKE * 6, cr=1 << 20, d=2048, L=3, hd=128, ws=ws, dt=0)

    def call(**kw):
        a = {**ok_args, **kw}
        return lib.hs2_bridge_kv_append(a["h"], a["n"], a["rows"], a["cr"], a["d"], a["L"], w, w, c, c, a["hd"],
                                        FAKE * 8, a["ws"], a["dt"], None)
    assert call(dt=1) == hs2.HS2_ERR_UNSUPPORTED
    assert call(d=2000) == hs2.HS2_ERR_UNSUPPORTED       # not a multiple of 128
    assert call(hd=64) == hs2.HS2_ERR_UNSUPPORTED
    assert call(n=-1) == hs2.HS2_ERR_INVALID_ARG
    assert call(n=70000) == hs2.HS2_ERR_INVALID_ARG
    assert call(rows=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(rows=FAKE * 6 + 4) == hs2.HS2_ERR_INVALID_ARG  # misaligned
    assert call(cr=-5) == hs2.HS2_ERR_INVALID_ARG
    assert call(ws=ws - 4) == hs2.HS2_ERR_WORKSPACE


def test_v1_select_rejects_bad_arguments(lib):
    b = _batch(total_q=4, max_kv_len=8192, rows=8192)
    ws = lib.hs2_v1_full_attn_select_workspace_size(ctypes.byref(b), 64, 4, 128, 16, hs2.HS2_BF16)
    ok_args = dict(nh=64, nkv=4, hd=128, tb=16, scale=0.088, bi=FAKE * 3, ws=ws, dt=hs2.HS2_BF16)

    def call(**kw):
        a = {**ok_args, **kw}
        return lib.hs2_v1_full_attn_select(ctypes.byref(b), FAKE, FAKE, FAKE, a["nh"], a["nkv"], a["hd"], a["tb"],
                                           a["scale"], FAKE * 2, None, a["bi"], None, FAKE, a["ws"], a["dt"], None)
    assert call(nkv=1) == hs2.HS2_ERR_UNSUPPORTED
    assert b"n_kv_heads=4" in lib.hs2_last_error()
    assert call(nh=32) == hs2.HS2_ERR_UNSUPPORTED
    assert call(dt=hs2.HS2_F32) == hs2.HS2_ERR_UNSUPPORTED
    assert call(tb=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(tb=65) == hs2.HS2_ERR_INVALID_ARG
    assert call(scale=0.0) == hs2.HS2_ERR_INVALID_ARG
    assert call(bi=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(bi=FAKE * 3 + 2) == hs2.HS2_ERR_INVALID_ARG
    assert call(ws=ws - 1) == hs2.HS2_ERR_WORKSPACE
    big = _batch(total_q=1, max_kv_len=(1 << 21) + 1, rows=(1 << 21) + 1)
    assert lib.hs2_v1_full_attn_select(ctypes.byref(big), FAKE, FAKE, FAKE, 64, 4, 128, 16, 0.088, FAKE * 2, None,
                                       FAKE * 3, None, FAKE, 1 << 40, hs2.HS2_BF16, None) == hs2.HS2_ERR_UNSUPPORTED
    # the workspace holds the partials and the block LSE table, growing with the context
    b2 = _batch(total_q=4, max_kv_len=4 * 8192, rows=4 * 8192)
    assert lib.hs2_v1_full_attn_select_workspace_size(ctypes.byref(b2), 64, 4, 128, 16, hs2.HS2_BF16) > ws > 0


def test_v1_sparse_rejects_bad_arguments(lib):
    b = _batch(total_q=4, max_kv_len=8192, rows=8192)
    ws = lib.hs2_v1_sparse_attn_workspace_size(ctypes.byref(b), 64, 4, 128, 16, hs2.HS2_BF16)
    assert ws == 4 * 4 * (16 // 2 + 1) * (64 + 16 * 128) * 4
    ok_args = dict(bi=FAKE * 3, tb=16, ks=FAKE * 4, vs=FAKE * 5, R=128, W=128, gs=FAKE * 6, gw=FAKE * 7, nkv=4,
                   ws=ws, dt=hs2.HS2_BF16)

    def call(**kw):
        a = {**ok_args, **kw}
        return lib.hs2_v1_sparse_attn(ctypes.byref(b), FAKE, FAKE, FAKE, a["bi"], a["tb"], a["ks"], a["vs"], a["R"],
                                      a["W"], a["gs"], a["gw"], 64, a["nkv"], 128, 0.088, FAKE * 2, FAKE, a["ws"],
                                      a["dt"], None)
    assert call(nkv=8) == hs2.HS2_ERR_UNSUPPORTED
    assert call(dt=hs2.HS2_FP8_E4M3) == hs2.HS2_ERR_UNSUPPORTED
    assert call(R=64) == hs2.HS2_ERR_INVALID_ARG          # ring shorter than the window
    assert b"swa_slots" in lib.hs2_last_error()
    assert call(W=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(ks=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(gw=None) == hs2.HS2_ERR_INVALID_ARG
    assert call(gs=FAKE * 6 + 2) == hs2.HS2_ERR_INVALID_ARG
    assert call(vs=FAKE * 5 + 8) == hs2.HS2_ERR_INVALID_ARG
    assert call(tb=0) == hs2.HS2_ERR_INVALID_ARG
    assert call(ws=ws - 1) == hs2.HS2_ERR_WORKSPACE


def test_header_is_plain_c99_and_a_c_program_links(lib, tmp_path):
    """include/hs2.h compiles as strict C99 (no C++ or compiler extensions needed) and a
    C program links against libhs2.so and calls it (host-only calls: no GPU needed)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "t.c"
    src.write_text(
        '#include <stdio.h>\n#include "hs2.h"\n'
        "int main(void) {\n"
        "  hs2_seqs b = {0};\n"
        "  if (hs2_version() != HS2_VERSION) return 1;\n"
        "  if (hs2_full_attn_select(&b, 0, 0, 0, 64, 128, 128, 1024, 0.1f, 0, 0, 0, 0, 0, 0, HS2_BF16, 0)\n"
        "      != HS2_ERR_INVALID_ARG) return 2;\n"
        '  printf("%s\\n", hs2_last_error());\n'
        "  return 0;\n}\n")
    exe = tmp_path / "t"
    lib_dir = os.path.dirname(hs2.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-L", lib_dir, "-lhs2", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "num_seqs" in r.stdout


def test_noalloc_rejects_a_batch_beyond_its_scratch(lib):
    """hs2_sparse_attn_noalloc refuses, on the host, a batch whose workspace exceeds the
    fixed scratch array (a wide window splits every query's keys over many workgroups),
    and takes only bf16 or fp32 K/V."""
    b = _batch(total_q=100, max_kv_len=300000, rows=30000000, num_seqs=100)
    window, top_k = 1 << 18, 4096
    need = lib.hs2_sparse_attn_workspace_size(ctypes.byref(b), 64, 128, window, top_k, hs2.HS2_BF16)
    assert need > hs2.NOALLOC_SCRATCH_BYTES
    st = lib.hs2_sparse_attn_noalloc(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE * 3, 64, 128, window, top_k, 0.088,
                                     FAKE * 2, None, hs2.HS2_BF16, None)
    assert st == hs2.HS2_ERR_WORKSPACE
    assert b"scratch" in lib.hs2_last_error()
    st = lib.hs2_sparse_attn_noalloc(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE * 3, 64, 128, 128, 1024, 0.088,
                                     FAKE * 2, None, hs2.HS2_FP8_E4M3, None)
    assert st == hs2.HS2_ERR_UNSUPPORTED
    st = lib.hs2_sparse_attn_noalloc(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE * 3, 32, 128, 128, 1024, 0.088,
                                     FAKE * 2, None, hs2.HS2_BF16, None)
    assert st == hs2.HS2_ERR_UNSUPPORTED
