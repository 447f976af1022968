"""hs2_sparse_attn_noalloc: the sparse layer with its split partials in the library's
fixed per-GPU scratch array, called through the C ABI, against hs2_sparse_attn with a
caller workspace on the same inputs (the same kernels and split plan: the outputs must be
bitwise equal). Two calls in a row, the second on a smaller batch; bf16 and fp32."""
import numpy as np
import pytest
import torch

from long_context_mqa_amd import hs2
from tests.parity import check_attn, from_dev, oracle_query, oracle_sparse, to_dev
from workloads.configs import BlockSpec, make_block_inputs

pytestmark = pytest.mark.gpu


def _layer(spec, inp, check_oracle_q=()):
    dev = "cuda"
    batch = hs2.Batch.from_host(inp.kv_start, inp.kv_len, inp.q_start, inp.q_pos, spec.total_rows, dev)
    k, v, q, qs = to_dev(inp.k), to_dev(inp.v), to_dev(inp.q_sel), to_dev(inp.q_sp[0])
    _, _, sel, _ = hs2.full_attn_select(batch, q, k, v, spec.window, spec.top_k, spec.scale)
    need = hs2.sparse_attn_workspace_size(batch, spec.window, spec.top_k, q.dtype)
    assert 0 < need <= hs2.NOALLOC_SCRATCH_BYTES   # several splits per query: the scratch is used
    ref, ref_lse = hs2.sparse_attn(batch, qs, k, v, sel, spec.window, spec.top_k, spec.scale,
                                   lse=torch.empty(spec.total_q, 64, device=dev))
    got, got_lse = hs2.sparse_attn_noalloc(batch, qs, k, v, sel, spec.window, spec.top_k, spec.scale,
                                           lse=torch.empty(spec.total_q, 64, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32))
    assert torch.equal(got_lse.view(torch.int32), ref_lse.view(torch.int32))
    g, s = from_dev(got), sel.cpu().numpy()
    for qi in check_oracle_q:
        r = oracle_query(inp, qi)
        o, _ = oracle_sparse(inp, qi, 0, s[qi], r["K"], r["V"])
        check_attn(g[qi], o, f"noalloc q{qi}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice(dtype):
    big = [20000 + 311 * j for j in range(48)]
    spec_a = BlockSpec("noalloc-a", big, [[n - 1] for n in big], dtype=dtype, n_sparse=1, needles_per_query=2, seed=51)
    small = [4000, 2500, 9000]
    spec_b = BlockSpec("noalloc-b", small, [[n - 1] for n in small], dtype=dtype, n_sparse=1, needles_per_query=2,
                       seed=52)
    print(f"noalloc {dtype}: 48 queries, then 3", flush=True)
    _layer(spec_a, make_block_inputs(spec_a), check_oracle_q=(0, 47))
    _layer(spec_b, make_block_inputs(spec_b), check_oracle_q=(0, 1, 2))
