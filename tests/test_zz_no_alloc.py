"""The entry point that allocates nothing: paged_decode_attention_balanced_static
(the balanced schedule on the library's static device scratch) against
paged_decode_attention_balanced with a caller workspace, through the C ABI,
on two calls in a row, the second with a smaller input, and both against
the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import paged_attention as ref
from paged_kv_gqa_cache_amd import abi, workloads
from tests.gpu_util import gpu_pool, inputs
from tests.helpers import oracle_pool

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _both(w):
    pool = gpu_pool(w)
    k, v, sc = pool
    q, tables, lens = inputs(w)
    ws = abi.balanced_workspace(q, k, tables)
    ws.fill_(0xFF)   # NaN bit patterns: a slot read before it is written shows up
    want = abi.paged_decode_attention_balanced(q, k, v, tables, lens, w.scale, sc, ws, window=w.spec.window)
    got = abi.paged_decode_attention_balanced_static(q, k, v, tables, lens, w.scale, sc, window=w.spec.window)
    torch.cuda.synchronize()
    return want, got


def _oracle(w):
    k, v, sc = oracle_pool(w)
    return ref.decode_attention(w.q, w.spec.q_dtype, k, v, w.spec.kv_dtype, w.block_tables, w.context_lens,
                                w.scale, sc, window=w.spec.window)


def test_static_scratch_matches_the_workspace_entry_on_two_calls():
    print("case: static scratch, 24-sequence then 5-sequence layer", flush=True)
    big = workloads.generate("qwen25_7b_prefix", num_seqs=24, lengths=("lognormal", 400, 1.0, 16, 4000))
    small = workloads.generate("qwen25_7b_prefix", num_seqs=5, lengths=("uniform", 1, 300))
    for w in (big, small):
        want, got = _both(w)
        # same kernels and split points; the waves' tile claims (and so the
        # summation order) are settled at run time
        assert float((got - want).abs().max()) <= 1e-5
        g = got.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g))
        assert float(np.max(np.abs(g - _oracle(w)))) <= TOL


def test_static_scratch_rejects_a_problem_past_its_size():
    print("case: static scratch size limit", flush=True)
    B, Hq, Hkv, D = 2048, 64, 4, 128      # G = 16: 16 x (2048 x 4 + workers) x 129 x 4 bytes > 32 MiB
    q = torch.zeros(B, Hq, D, dtype=torch.float16, device="cuda")
    k = torch.zeros(4, Hkv, 16 * D, dtype=torch.float16, device="cuda")
    tables = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    with pytest.raises(abi.PkvError) as e:
        abi.paged_decode_attention_balanced_static(q, k, k, tables, lens, 0.125, None)
    assert e.value.code == 1 and "static" in str(e.value)
