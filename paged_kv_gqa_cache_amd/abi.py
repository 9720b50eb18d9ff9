"""ctypes binding of libpagedkv.so (C ABI in include/pagedkv.h).

Argument marshalling only: torch tensors are used for device memory and
streams; every step of the computation runs in the library's HIP kernels.
The functions carry the C entry points' names.  If the library is missing
the import fails: there is no fallback.

Cache tensors have shape [num_blocks, num_kv_heads, 16 * head_dim] and hold
the tile layout documented in pagedkv.h; e4m3 caches are uint8 (or
torch.float8_e4m3fn) tensors of codes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(_HERE, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_E4M3 = 0, 1, 2, 3
_TORCH_CODE = {
    torch.float32: PKV_F32,
    torch.float16: PKV_F16,
    torch.bfloat16: PKV_BF16,
    torch.uint8: PKV_E4M3,
    torch.float8_e4m3fn: PKV_E4M3,
}
BLOCK_SIZE = 16


class PkvDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "q_dtype", "kv_dtype", "out_dtype", "sliding_window")]


class PkvError(RuntimeError):
    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} failed with status {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m paged_kv_gqa_cache_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.POINTER(PkvDesc)
    sigs = {
        "kv_cache_write": (ctypes.c_int, [P, P, P, I64, P, P, D, P]),
        "kv_cache_quantize_e4m3": (ctypes.c_int, [P, P, P, P, I32, P, P, P, D, P]),
        "kv_cache_copy_blocks": (ctypes.c_int, [P, I32, P, P, P, D, P]),
        "kv_cache_append_e4m3": (ctypes.c_int, [P, P, P, I64, P, P, P, D, P]),
        "paged_decode_attention": (ctypes.c_int, [P, P, P, P, P, F, P, P, D, P]),
        "paged_decode_attention_partial": (ctypes.c_int, [P, P, P, P, P, F, P, I32, P, P, D, P]),
        "paged_decode_attention_reduce": (ctypes.c_int, [P, P, P, I32, P, D, P]),
        "paged_decode_attention_split": (ctypes.c_int, [P, P, P, P, P, F, P, I32, P, I64, P, D, P]),
        "paged_decode_split_workspace_bytes": (ctypes.c_int64, [D, I32]),
        "paged_decode_step": (ctypes.c_int, [P, P, P, P, P, P, P, F, I32, P, I64, P, D, P]),
        "paged_decode_attention_balanced": (ctypes.c_int, [P, P, P, P, P, F, P, P, I64, P, D, P]),
        "paged_decode_balanced_workspace_bytes": (ctypes.c_int64, [D]),
        "paged_decode_attention_balanced_static": (ctypes.c_int, [P, P, P, P, P, F, P, P, D, P]),
        "paged_decode_attention_balanced_partial": (ctypes.c_int, [P, P, P, P, P, F, P, P, I64, P, D, P]),
        "paged_decode_attention_balanced_reduce": (ctypes.c_int, [P, I64, P, D, P]),
        "paged_prefill_attention": (ctypes.c_int, [P, P, P, P, P, P, I32, F, P, I32, P, I64, P, D, P]),
        "paged_prefill_workspace_bytes": (ctypes.c_int64, [D, I32, I32]),
        "paged_decode_num_partitions": (ctypes.c_int64, [D, I32]),
        "paged_decode_workspace_bytes": (ctypes.c_int64, [D, I32]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_version": (ctypes.c_char_p, []),
        "pagedkv_last_error": (ctypes.c_char_p, []),
        "pagedkv_version": (ctypes.c_char_p, []),
        "pkv_read_bandwidth_probe": (ctypes.c_int, [P, I64, P, I32, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()
EXPORTED = ("kv_cache_write", "kv_cache_quantize_e4m3", "kv_cache_append_e4m3", "kv_cache_copy_blocks",
            "paged_decode_attention",
            "paged_decode_attention_partial", "paged_decode_attention_reduce",
            "paged_decode_attention_split", "paged_decode_split_workspace_bytes", "paged_decode_step",
            "paged_decode_attention_balanced", "paged_decode_balanced_workspace_bytes",
            "paged_decode_attention_balanced_static",
            "paged_decode_attention_balanced_partial", "paged_decode_attention_balanced_reduce",
            "paged_prefill_attention", "paged_prefill_workspace_bytes",
            "paged_decode_num_partitions", "paged_decode_workspace_bytes", "pkv_last_error",
            "pkv_version", "pagedkv_last_error", "pagedkv_version", "pkv_read_bandwidth_probe")


def lib():
    return _lib


def version() -> str:
    return _lib.pkv_version().decode()


def last_error() -> str:
    return _lib.pkv_last_error().decode()


def pkv_read_bandwidth_probe(buf: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """Read every byte of device tensor ``buf`` once (measurement aid: the
    GPU's sustained read rate); ``out`` (int32, device) receives one
    XOR-folded word per workgroup."""
    _check("pkv_read_bandwidth_probe", _lib.pkv_read_bandwidth_probe(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(out), out.numel(), _stream(stream)))
    return out


def _check(func: str, status: int) -> None:
    if status != 0:
        raise PkvError(func, status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _code(t: torch.Tensor) -> int:
    try:
        return _TORCH_CODE[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def make_desc(num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
              q_dtype, kv_dtype, out_dtype, sliding_window=0) -> PkvDesc:
    return PkvDesc(num_seqs, num_q_heads, num_kv_heads, head_dim, BLOCK_SIZE, num_blocks,
                   max_blocks_per_seq, q_dtype, kv_dtype, out_dtype, sliding_window)


def _attn_desc(q, k_cache, block_tables, out_dtype_code, window=0) -> PkvDesc:
    B, Hq, D = q.shape
    NB, Hkv = k_cache.shape[0], k_cache.shape[1]
    return make_desc(B, Hq, Hkv, D, NB, block_tables.shape[1], _code(q), _code(k_cache), out_dtype_code,
                     int(window))


# ---------------------------------------------------------------- entries ---

def kv_cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """k, v [T, Hkv, D] -> their slots of k_cache / v_cache (slot_mapping int64 [T])."""
    T, Hkv, D = k.shape
    desc = make_desc(0, Hkv, Hkv, D, k_cache.shape[0], 1, _code(k), _code(k_cache), _code(k))
    _check("kv_cache_write", _lib.kv_cache_write(
        _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache),
        ctypes.byref(desc), _stream(stream)))


def kv_cache_quantize_e4m3(k_src, v_src, block_ids, valid_tokens, k_cache, v_cache, kv_scales,
                           stream=None) -> None:
    """fp32 blocks k_src/v_src [n, 16, Hkv, D] -> e4m3 codes of blocks block_ids, and scales."""
    n, _, Hkv, D = k_src.shape
    desc = make_desc(0, Hkv, Hkv, D, k_cache.shape[0], 1, PKV_F32, PKV_E4M3, PKV_F32)
    _check("kv_cache_quantize_e4m3", _lib.kv_cache_quantize_e4m3(
        _ptr(k_src), _ptr(v_src), _ptr(block_ids), _ptr(valid_tokens), n, _ptr(k_cache),
        _ptr(v_cache), _ptr(kv_scales), ctypes.byref(desc), _stream(stream)))


def kv_cache_append_e4m3(k, v, slot_mapping, k_cache, v_cache, kv_scales, stream=None) -> None:
    """fp32 k, v [T, Hkv, D] quantised on append into their slots of an e4m3 pool."""
    T, Hkv, D = k.shape
    desc = make_desc(0, Hkv, Hkv, D, k_cache.shape[0], 1, PKV_F32, PKV_E4M3, PKV_F32)
    _check("kv_cache_append_e4m3", _lib.kv_cache_append_e4m3(
        _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), _ptr(kv_scales),
        ctypes.byref(desc), _stream(stream)))


def kv_cache_copy_blocks(block_mapping, k_cache, v_cache, kv_scales=None, stream=None) -> None:
    """Copy blocks inside the pool: block_mapping int32 [n, 2] of (src, dst) pairs."""
    n = int(block_mapping.shape[0])
    NB, Hkv = k_cache.shape[0], k_cache.shape[1]
    D = k_cache.shape[2] // BLOCK_SIZE
    code = _code(k_cache)
    desc = make_desc(0, Hkv, Hkv, D, NB, 1, code, code, code)
    _check("kv_cache_copy_blocks", _lib.kv_cache_copy_blocks(
        _ptr(block_mapping), n, _ptr(k_cache), _ptr(v_cache), _ptr(kv_scales), ctypes.byref(desc),
        _stream(stream)))


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                           kv_scales=None, out=None, out_dtype=None, stream=None, window=0):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_attention", _lib.paged_decode_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(kv_scales), _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def num_partitions(max_blocks_per_seq: int, partition_size: int) -> int:
    desc = make_desc(1, 1, 1, 64, 1, max_blocks_per_seq, 0, 0, 0)
    s = _lib.paged_decode_num_partitions(ctypes.byref(desc), partition_size)
    if s < 0:
        raise PkvError("paged_decode_num_partitions", 1, last_error())
    return int(s)


def alloc_partials(q, max_blocks_per_seq: int, partition_size: int):
    """(tmp_out fp32 [B, Hq, S, D], tmp_lse fp32 [B, Hq, S]) on q's device."""
    B, Hq, D = q.shape
    S = num_partitions(max_blocks_per_seq, partition_size)
    return (torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device),
            torch.empty((B, Hq, S), dtype=torch.float32, device=q.device))


def paged_decode_attention_partial(q, k_cache, v_cache, block_tables, context_lens, scale,
                                   kv_scales, partition_size, tmp_out, tmp_lse, stream=None,
                                   window=0) -> None:
    desc = _attn_desc(q, k_cache, block_tables, PKV_F32, window)
    _check("paged_decode_attention_partial", _lib.paged_decode_attention_partial(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(kv_scales), int(partition_size), _ptr(tmp_out), _ptr(tmp_lse),
        ctypes.byref(desc), _stream(stream)))


def paged_decode_attention_reduce(tmp_out, tmp_lse, context_lens, partition_size, out,
                                  max_blocks_per_seq: int, stream=None, window=0) -> None:
    B, Hq, S, D = tmp_out.shape
    desc = make_desc(B, Hq, 1, D, 1, max_blocks_per_seq, PKV_F32, PKV_F32, _code(out), int(window))
    _check("paged_decode_attention_reduce", _lib.paged_decode_attention_reduce(
        _ptr(tmp_out), _ptr(tmp_lse), _ptr(context_lens), int(partition_size), _ptr(out),
        ctypes.byref(desc), _stream(stream)))


def split_workspace(q, k_cache, block_tables, partition_size: int) -> torch.Tensor:
    """A zero-filled workspace for paged_decode_attention_split (reusable across calls)."""
    desc = _attn_desc(q, k_cache, block_tables, PKV_F32)
    n = _lib.paged_decode_split_workspace_bytes(ctypes.byref(desc), int(partition_size))
    if n < 0:
        raise PkvError("paged_decode_split_workspace_bytes", 1, last_error())
    return torch.zeros(int(n), dtype=torch.uint8, device=q.device)


def paged_decode_attention_split(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                                 partition_size, workspace, out=None, out_dtype=None, stream=None,
                                 window=0):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_attention_split", _lib.paged_decode_attention_split(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(kv_scales), int(partition_size), _ptr(workspace), workspace.numel(),
        _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def paged_decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                      workspace, out=None, out_dtype=None, stream=None, window=0):
    """Write each sequence's new token (k_new/v_new [B, Hkv, D]) at position
    context_lens[b] - 1, then attend (the split path), in one launch."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_step", _lib.paged_decode_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), int(partition_size), _ptr(workspace), workspace.numel(),
        _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def balanced_workspace(q, k_cache, block_tables) -> torch.Tensor:
    """A workspace for paged_decode_attention_balanced on q's device."""
    desc = _attn_desc(q, k_cache, block_tables, PKV_F32)
    with torch.cuda.device(q.device):
        n = _lib.paged_decode_balanced_workspace_bytes(ctypes.byref(desc))
    if n < 0:
        raise PkvError("paged_decode_balanced_workspace_bytes", 1, last_error())
    return torch.empty(int(n), dtype=torch.uint8, device=q.device)


def paged_decode_attention_balanced(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                                    workspace, out=None, out_dtype=None, stream=None, window=0):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_attention_balanced", _lib.paged_decode_attention_balanced(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(kv_scales), _ptr(workspace), workspace.numel(),
        _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def paged_decode_attention_balanced_partial(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                                            workspace, out, stream=None, window=0):
    """The first launch of paged_decode_attention_balanced (tiles streamed,
    whole pairs written to ``out``, partials left in ``workspace``)."""
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_attention_balanced_partial", _lib.paged_decode_attention_balanced_partial(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(kv_scales), _ptr(workspace), workspace.numel(),
        _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def paged_decode_attention_balanced_reduce(q, k_cache, block_tables, workspace, out, stream=None, window=0):
    """The second launch of paged_decode_attention_balanced: merges the
    partials the first left in ``workspace`` into ``out`` (q, k_cache and
    block_tables give the shapes and dtypes, as for the first call)."""
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_attention_balanced_reduce", _lib.paged_decode_attention_balanced_reduce(
        _ptr(workspace), workspace.numel(), _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def paged_decode_attention_balanced_static(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                                           out=None, out_dtype=None, stream=None, window=0):
    """paged_decode_attention_balanced with the library's static scratch
    instead of a workspace (no device allocation by the library; ``out`` is
    allocated here only when not given)."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = _attn_desc(q, k_cache, block_tables, _code(out), window)
    _check("paged_decode_attention_balanced_static", _lib.paged_decode_attention_balanced_static(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(kv_scales), _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out


def prefill_workspace(q, k_cache, block_tables, partition_size: int):
    """A workspace for paged_prefill_attention (None for partition_size 0)."""
    if partition_size == 0:
        return None
    desc = make_desc(block_tables.shape[0], q.shape[1], k_cache.shape[1], q.shape[2], k_cache.shape[0],
                     block_tables.shape[1], _code(q), _code(k_cache), PKV_F32)
    n = _lib.paged_prefill_workspace_bytes(ctypes.byref(desc), int(q.shape[0]), int(partition_size))
    if n < 0:
        raise PkvError("paged_prefill_workspace_bytes", 1, last_error())
    return torch.empty(int(n), dtype=torch.uint8, device=q.device)


def paged_prefill_attention(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, kv_scales=None,
                            partition_size=0, workspace=None, out=None, out_dtype=None, stream=None):
    """Causal attention for query rows q [T, Hq, D] packed by query_start [B + 1]."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    if partition_size and workspace is None:
        workspace = prefill_workspace(q, k_cache, block_tables, partition_size)
    desc = make_desc(block_tables.shape[0], q.shape[1], k_cache.shape[1], q.shape[2], k_cache.shape[0],
                     block_tables.shape[1], _code(q), _code(k_cache), _code(out))
    _check("paged_prefill_attention", _lib.paged_prefill_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), _ptr(query_start),
        int(q.shape[0]), float(scale), _ptr(kv_scales), int(partition_size), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _ptr(out), ctypes.byref(desc), _stream(stream)))
    return out
