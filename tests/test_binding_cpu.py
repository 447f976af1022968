"""The Python binding rejects tensors that the library would address with another element
type, row length or row count than the entry point assumes (the C ABI takes plain pointers
and cannot see buffer sizes). Every check raises before anything reaches the device, so
these run without a GPU."""
import numpy as np
import pytest
import torch

from long_context_mqa_amd import hs2


def _batch(rows=600, q_pos=(599, 300)):
    return hs2.Batch.from_host([0, 0][:len(q_pos)], [rows] * len(q_pos), list(range(len(q_pos) + 1)),
                               list(q_pos), rows, device="cpu")


def _qkv(nq=2, rows=600, kv_dtype=torch.bfloat16, q_dtype=torch.bfloat16):
    q = torch.zeros(nq, 64, 128, dtype=q_dtype)
    k = torch.zeros(rows, 128, dtype=kv_dtype)
    v = torch.zeros(rows, 128, dtype=kv_dtype)
    return q, k, v


def test_fp8_codes_given_to_the_bf16_selector_are_rejected():
    """FP8 codes are 128-byte rows: the bf16 kernels would read 256-byte rows past the end."""
    b = _batch()
    q, k, v = _qkv(kv_dtype=torch.uint8)
    with pytest.raises(TypeError, match="k: dtype torch.uint8"):
        hs2.full_attn_select(b, q, k, v)
    with pytest.raises(TypeError, match="k: dtype torch.uint8"):
        hs2.sparse_attn(b, q, k, v, torch.zeros(2, 1024, dtype=torch.int32))
    with pytest.raises(TypeError, match="k: dtype torch.uint8"):
        hs2.causal_attn(b, q, k, v)


def test_kv_dtype_must_match_q():
    b = _batch()
    q, k, v = _qkv(kv_dtype=torch.float32)
    with pytest.raises(TypeError, match="k: dtype torch.float32"):
        hs2.full_attn_select(b, q, k, v)
    q, k, v = _qkv(q_dtype=torch.float32)
    with pytest.raises(TypeError, match="k: dtype torch.bfloat16"):
        hs2.full_attn_select(b, q, k, v)


def test_bf16_cache_given_to_the_fp8_entry_points_is_rejected():
    b = _batch()
    q, k, v = _qkv()
    with pytest.raises(TypeError, match="FP8 K/V"):
        hs2.full_attn_select_fp8kv(b, q, k, v, 1.0, 1.0)
    with pytest.raises(TypeError, match="FP8 K/V"):
        hs2.sparse_attn_fp8kv(b, q, k, v, 1.0, 1.0, torch.zeros(2, 1024, dtype=torch.int32))


def test_kv_rows_shape_and_layout():
    b = _batch(rows=600)
    q, k, v = _qkv(rows=599)
    with pytest.raises(ValueError, match="k: 599 rows, the batch addresses 600"):
        hs2.full_attn_select(b, q, k, v)
    q, k, v = _qkv(rows=600)
    with pytest.raises(ValueError, match=r"v: shape \(600, 64\)"):
        hs2.full_attn_select(b, q, k, v[:, :64])
    vt = torch.zeros(128, 600, dtype=torch.bfloat16).t()
    with pytest.raises(ValueError, match="v must be contiguous"):
        hs2.full_attn_select(b, q, k, vt)
    with pytest.raises(ValueError, match=r"q: shape \(2, 32, 128\)"):
        hs2.full_attn_select(b, q[:, :32].contiguous(), k, v)


def test_q_and_outputs_cover_every_query():
    b = _batch()
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="q: 1 rows, the batch addresses 2"):
        hs2.full_attn_select(b, q[:1], k, v)
    with pytest.raises(TypeError, match="out: dtype torch.float32"):
        hs2.full_attn_select(b, q, k, v, out=torch.zeros(2, 64, 128))
    with pytest.raises(ValueError, match="lse: 1 rows"):
        hs2.full_attn_select(b, q, k, v, lse=torch.zeros(1, 64))
    with pytest.raises(ValueError, match=r"sel_idx: shape \(2, 512\)"):
        hs2.full_attn_select(b, q, k, v, sel_idx=torch.zeros(2, 512, dtype=torch.int32))
    with pytest.raises(ValueError, match=r"sel_idx: shape \(2, 512\)"):
        hs2.sparse_attn(b, q, k, v, torch.zeros(2, 512, dtype=torch.int32), top_k=1024)


def test_bridging_operands():
    h = torch.zeros(100, 256, dtype=torch.bfloat16)
    w = [torch.zeros(256, 128, dtype=torch.bfloat16)]
    with pytest.raises(TypeError, match="w_k: dtype torch.float32"):
        hs2.bridge_kv(h, [torch.zeros(256, 128)], w)
    with pytest.raises(ValueError, match="w_v: 255 rows"):
        hs2.bridge_kv(h, w, [torch.zeros(255, 128, dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="k_out: 99 rows"):
        hs2.bridge_kv(h, w, w, k_out=[torch.zeros(99, 128, dtype=torch.bfloat16)],
                      v_out=[torch.zeros(100, 128, dtype=torch.bfloat16)])
    rows = torch.zeros(4, dtype=torch.int64)
    cache = [torch.zeros(50, 128, dtype=torch.bfloat16)]
    with pytest.raises(ValueError, match=r"w_k: shape \(256, 64\)"):
        hs2.bridge_kv_append(h[:4], rows, [torch.zeros(256, 64, dtype=torch.bfloat16)], w, cache, cache)


def test_v1_cache_layout():
    b = _batch()
    q = torch.zeros(2, 64, 128, dtype=torch.bfloat16)
    k = torch.zeros(600, 128, dtype=torch.bfloat16)      # an MQA cache, not [rows, 4, 128]
    with pytest.raises(ValueError, match=r"k: shape \(600, 128\), expected \[rows, 4, 128\]"):
        hs2.v1_full_attn_select(b, q, k, k)


def test_fp8_bridging_outputs_are_byte_caches():
    h = torch.zeros(100, 256, dtype=torch.bfloat16)
    w = [torch.zeros(256, 128, dtype=torch.bfloat16)]
    with pytest.raises(TypeError, match="k_out: dtype torch.bfloat16"):
        hs2.bridge_kv_fp8kv(h, w, w, 0.05, 0.05, k_out=[torch.zeros(100, 128, dtype=torch.bfloat16)],
                            v_out=[torch.zeros(100, 128, dtype=torch.uint8)])
    with pytest.raises(ValueError, match="one entry per layer"):
        hs2.bridge_kv_fp8kv(h, w, w, [0.05, 0.05], 0.05)
