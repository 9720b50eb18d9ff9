"""GPU-side plumbing for the parity tests: pool building comes from the
package; this adds one decode step through any of the three entry paths."""
from __future__ import annotations

import torch

from paged_kv_gqa_cache_amd import abi
from paged_kv_gqa_cache_amd.pool import (INT_DT, OUT_DT, POISON, TORCH_DT, empty_pool, gpu_pool,  # noqa: F401
                                         inputs, to_dev, to_raw)


def decode(w, pool, mode="split", partition_size=None, out_dtype=torch.float32, q=None,
           tables=None, lens=None, device="cuda"):
    """Run one decode-attention step on the GPU; returns out (torch, on device).
    mode: single (one pass), split (partial + reduce), fused (split in one
    launch) or balanced (equal tile shares per wave)."""
    k, v, scales = pool
    q0, t0, l0 = inputs(w, device)
    q = q0 if q is None else q
    tables = t0 if tables is None else tables
    lens = l0 if lens is None else lens
    W = w.spec.window
    if mode == "single":
        return abi.paged_decode_attention(q, k, v, tables, lens, w.scale, scales, out_dtype=out_dtype, window=W)
    if mode == "balanced":
        ws = abi.balanced_workspace(q, k, tables)
        ws.fill_(0xFF)   # NaN bit patterns: a slot read before it is written shows up
        return abi.paged_decode_attention_balanced(q, k, v, tables, lens, w.scale, scales, ws,
                                                   out_dtype=out_dtype, window=W)
    P = partition_size or w.spec.partition_size
    if mode == "fused":
        ws = abi.split_workspace(q, k, tables, P)
        return abi.paged_decode_attention_split(q, k, v, tables, lens, w.scale, scales, P, ws,
                                                out_dtype=out_dtype, window=W)
    tmp_out, tmp_lse = abi.alloc_partials(q, tables.shape[1], P)
    abi.paged_decode_attention_partial(q, k, v, tables, lens, w.scale, scales, P, tmp_out, tmp_lse, window=W)
    out = torch.empty(q.shape, dtype=out_dtype, device=device)
    abi.paged_decode_attention_reduce(tmp_out, tmp_lse, lens, P, out, tables.shape[1], window=W)
    return out
