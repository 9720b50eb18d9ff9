"""Device-side setup of a workload: upload its inputs and build the KV pool
through the library's own entry points (kv_cache_write, or
kv_cache_quantize_e4m3 for an E4M3 pool).  Argument marshalling only."""
from __future__ import annotations

import numpy as np
import torch

from paged_kv_gqa_cache_amd import abi

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.uint8}
INT_DT = {"f32": (torch.int32, np.int32), "f16": (torch.int16, np.int16),
          "bf16": (torch.int16, np.int16), "e4m3": (torch.uint8, np.uint8)}
POISON = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}
OUT_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(raw: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """numpy raw storage bits -> device tensor of the storage dtype."""
    tdt, ndt = INT_DT[dtype]
    t = torch.from_numpy(np.ascontiguousarray(raw).view(ndt)).to(device)
    return t if dtype == "e4m3" else t.view(TORCH_DT[dtype])


def to_raw(t: torch.Tensor, dtype: str) -> np.ndarray:
    """device tensor -> numpy raw unsigned bits."""
    tdt, ndt = INT_DT[dtype]
    a = t.view(tdt).cpu().numpy() if dtype != "e4m3" else t.cpu().numpy()
    unsigned = {np.int32: np.uint32, np.int16: np.uint16, np.uint8: np.uint8}[ndt]
    return a.view(unsigned)


def empty_pool(w, device="cuda"):
    s = w.spec
    shape = (w.num_blocks, s.num_kv_heads, 16 * s.head_dim)
    tdt, _ = INT_DT[s.kv_dtype]
    k = torch.empty(shape, dtype=tdt, device=device)
    v = torch.empty(shape, dtype=tdt, device=device)
    poison = POISON[s.kv_dtype]
    if tdt == torch.int32 and poison >= 2 ** 31:
        poison -= 2 ** 32
    k.fill_(poison)
    v.fill_(poison)
    if s.kv_dtype != "e4m3":
        k, v = k.view(TORCH_DT[s.kv_dtype]), v.view(TORCH_DT[s.kv_dtype])
    return k, v


def gpu_pool(w, device="cuda", with_new_tokens=True):
    """The pool as the library builds it: NaN-filled, context written with
    kv_cache_write (or quantised with kv_cache_quantize_e4m3), then the new
    tokens written.  Returns (k_cache, v_cache, kv_scales or None)."""
    s = w.spec
    k, v = empty_pool(w, device)
    scales = None
    if s.kv_dtype == "e4m3":
        scales = torch.ones((2, w.num_blocks, s.num_kv_heads), dtype=torch.float32, device=device)
        ksrc = torch.from_numpy(w.fill_k.view(np.float32)).to(device)
        vsrc = torch.from_numpy(w.fill_v.view(np.float32)).to(device)
        ids = torch.from_numpy(w.fill_blocks.astype(np.int32)).to(device)
        valid = torch.from_numpy(w.fill_valid.astype(np.int32)).to(device)
        abi.kv_cache_quantize_e4m3(ksrc, vsrc, ids, valid, k, v, scales)
    else:
        slots, kt, vt = w.fill_tokens()
        abi.kv_cache_write(to_dev(kt, s.kv_dtype, device), to_dev(vt, s.kv_dtype, device),
                           torch.from_numpy(slots).to(device), k, v)
    if with_new_tokens and w.new_slots is not None:
        abi.kv_cache_write(to_dev(w.new_k, s.kv_dtype, device), to_dev(w.new_v, s.kv_dtype, device),
                           torch.from_numpy(w.new_slots).to(device), k, v)
    return k, v, scales


def inputs(w, device="cuda"):
    s = w.spec
    q = to_dev(w.q, s.q_dtype, device)
    tables = torch.from_numpy(w.block_tables).to(device)
    lens = torch.from_numpy(w.context_lens).to(device)
    return q, tables, lens


