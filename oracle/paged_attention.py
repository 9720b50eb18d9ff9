"""Paged grouped-query decode attention, written out by its definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Slow on purpose:
per-sequence numpy gathers and float64 arithmetic, no blocking or fusion
beyond what the definition states.

The computation (pages cited by title and section):

* The KV cache is a pool of fixed-size blocks; a per-sequence block table
  maps logical block j of a sequence to a physical block in the pool, and a
  step first writes the new token's K/V at its write position, then reads
  the sequence's blocks ("rvllm - A Small LLM Inference Engine in Rust",
  section "How it's put together"; "rvLLM: High-performance LLM inference in
  Rust", section "CUDA Kernels", rows "Reshape and Cache" and
  "PagedAttention V2").
* Each KV head is shared by a group of query heads ("rvllm - A Small LLM
  Inference Engine in Rust", section "How it's put together"; "LLM Serving
  Kernels", section "Projects", row 04 "GQA/MQA").
* Online softmax ("PagedAttention V2 ... online softmax"; project 04) reaches,
  up to rounding order, the plain softmax(q K^T * scale) V of one query
  against the gathered context; that plain form is what this module computes.
* Sliding-window decode ("rvLLM: High-performance LLM inference in Rust",
  sections "Project Status" and "Changelog", list sliding-window attention;
  "rvLLM: The Inference Engine That Lets TPUs Compete by Writing Less Kernel
  Code", section "The flat-scan trick that makes TPU inference work": Gemma 4
  runs 50 of its 60 layers with it).  The pages do not define the window;
  the plain reading taken here: with a window of W tokens a query attends
  only to the last W positions of its context, [max(0, L - W), L); W = 0
  means the whole context.
* Split-context ("flash-decoding") partials: each partition of the context
  yields its own normalised output and log-sum-exp, and a log-sum-exp
  weighted merge of the partials equals the full softmax.  The pages do not
  describe this step; it is the plain algebra of the softmax over a disjoint
  cover of the context.

Byte layout of the pool (the library's documented format; this module reads
and writes it with its own index arithmetic):

* a K or V cache is ``[num_blocks, num_kv_heads, tile]`` where one tile holds
  the 16 token slots x ``head_dim`` elements of one (block, kv head);
* element size e bytes (4 f32, 2 f16/bf16, 1 e4m3);
* K tile, with x = 16 / e elements per 16-byte chunk: element (t, d) sits at
  ``((d // x) * 16 + t) * x + d % x``;
* V tile, with n = 4 / e: element (t, d) sits at
  ``(((((d // (16 n)) * 4 + t // 4) * 16 + d % 16) * n + (d // 16) % n) * 4 + t % 4``;
* a slot number is ``block * 16 + offset``.
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3

BLOCK_SIZE = 16

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
RAW_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}
# NaN bit patterns used to fill every slot no sequence owns.
POISON = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}


# ---------------------------------------------------------------- values ---

def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of raw storage bits."""
    raw = np.asarray(raw)
    if dtype == "f32":
        return raw.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return raw.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "e4m3":
        return e4m3.decode(raw.astype(np.uint8))
    raise ValueError(dtype)


# ---------------------------------------------------------------- layout ---

def k_tile_index(head_dim: int, dtype: str) -> np.ndarray:
    """int64 [16, D]: element offset of (token slot t, dim d) in a K tile."""
    x = 16 // ELEM_BYTES[dtype]
    t = np.arange(BLOCK_SIZE)[:, None]
    d = np.arange(head_dim)[None, :]
    return ((d // x) * BLOCK_SIZE + t) * x + d % x


def v_tile_index(head_dim: int, dtype: str) -> np.ndarray:
    """int64 [16, D]: element offset of (token slot t, dim d) in a V tile."""
    n = 4 // ELEM_BYTES[dtype]
    t = np.arange(BLOCK_SIZE)[:, None]
    d = np.arange(head_dim)[None, :]
    return (((((d // (16 * n)) * 4 + t // 4) * 16 + d % 16) * n + (d // 16) % n) * 4 + t % 4)


def new_pool(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str):
    """A K and a V cache filled with the dtype's NaN pattern."""
    shape = (num_blocks, num_kv_heads, BLOCK_SIZE * head_dim)
    k = np.full(shape, POISON[dtype], dtype=RAW_DTYPE[dtype])
    v = np.full(shape, POISON[dtype], dtype=RAW_DTYPE[dtype])
    return k, v


# ----------------------------------------------------------------- write ---

def kv_cache_write(k_cache, v_cache, k_raw, v_raw, slot_mapping, dtype: str) -> None:
    """Copy token t's K/V [Hkv, D] bits into its slot; negative slots skip.

    "rvLLM: High-performance LLM inference in Rust", section "CUDA Kernels",
    row "Reshape and Cache"; "rvllm - A Small LLM Inference Engine in Rust",
    section "How it's put together" (write_positions).
    """
    head_dim = k_raw.shape[-1]
    kidx = k_tile_index(head_dim, dtype)
    vidx = v_tile_index(head_dim, dtype)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    blk = slots // BLOCK_SIZE                      # [T] physical block
    off = slots % BLOCK_SIZE                       # [T] slot inside it
    heads = np.arange(k_cache.shape[1])[None, :, None]
    k_cache[blk[:, None, None], heads, kidx[off][:, None, :]] = np.asarray(k_raw)[keep]
    v_cache[blk[:, None, None], heads, vidx[off][:, None, :]] = np.asarray(v_raw)[keep]


def kv_cache_append_e4m3(k_cache, v_cache, kv_scales, k_new, v_new, slot_mapping) -> None:
    """Quantise-on-append of new tokens into an E4M3 pool (``e4m3.append_token``
    per token, kv head, and K or V).

    ``k_new``/``v_new``: float32 [T, Hkv, D]; ``slot_mapping``: [T], negative
    skips.  Tokens are taken in order; the write rule needs at most one token
    per block per call, which the GPU path requires too.
    """
    head_dim = k_cache.shape[-1] // BLOCK_SIZE
    kidx = k_tile_index(head_dim, "e4m3")          # [16, D] tile positions
    vidx = v_tile_index(head_dim, "e4m3")
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = int(slot // BLOCK_SIZE), int(slot % BLOCK_SIZE)
        for h in range(k_cache.shape[1]):
            for which, cache, idx, x in ((0, k_cache, kidx, k_new), (1, v_cache, vidx, v_new)):
                codes, sc = e4m3.append_token(cache[blk, h][idx], kv_scales[which, blk, h], off, x[t, h])
                cache[blk, h][idx] = codes
                kv_scales[which, blk, h] = sc


def kv_cache_write_e4m3_blocks(k_cache, v_cache, kv_scales, k_blocks, v_blocks,
                               block_ids, valid_tokens) -> None:
    """Quantise whole blocks of fp32 K/V to E4M3 and store codes and scales.

    ``k_blocks``/``v_blocks``: float32 [n, 16, Hkv, D] (slot order);
    ``block_ids``: [n] physical block ids; ``valid_tokens``: [n] leading slots
    that hold data.  ``kv_scales`` is float32 [2, num_blocks, Hkv] (0 = K,
    1 = V).  Slots at or past ``valid_tokens`` receive code 0.
    """
    head_dim = k_blocks.shape[-1]
    n, _, hkv, _ = k_blocks.shape
    kidx = k_tile_index(head_dim, "e4m3").ravel()   # (t, d) order
    vidx = v_tile_index(head_dim, "e4m3").ravel()
    ids = np.asarray(block_ids, dtype=np.int64)
    chunk = 2048                                   # bounds the float64 temporaries
    for c0 in range(0, n, chunk):
        sl = slice(c0, min(n, c0 + chunk))
        kc, ks = e4m3.quantize_blocks(k_blocks[sl], valid_tokens[sl])
        vc, vs = e4m3.quantize_blocks(v_blocks[sl], valid_tokens[sl])
        m = kc.shape[0]
        ktile = np.empty((m, hkv, BLOCK_SIZE * head_dim), dtype=np.uint8)
        vtile = np.empty_like(ktile)
        ktile[:, :, kidx] = kc.transpose(0, 2, 1, 3).reshape(m, hkv, -1)
        vtile[:, :, vidx] = vc.transpose(0, 2, 1, 3).reshape(m, hkv, -1)
        k_cache[ids[sl]] = ktile
        v_cache[ids[sl]] = vtile
        kv_scales[0, ids[sl]] = ks
        kv_scales[1, ids[sl]] = vs


def copy_blocks(k_cache, v_cache, block_mapping, kv_scales=None) -> None:
    """Copy whole blocks inside the pool: for each pair (src, dst) of
    ``block_mapping`` [n, 2], block dst's K and V tiles of every kv head, and
    for an E4M3 pool its K and V scales, become bit copies of block src's.
    Every source is read before any destination is written.

    ("rvLLM: High-performance LLM inference in Rust", section "CUDA Kernels",
    row "Block Copy": KV cache block copy for beam search; section
    "Architecture": the block manager's copy-on-write.)
    """
    m = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    src, dst = m[:, 0], m[:, 1]
    k_src, v_src = k_cache[src].copy(), v_cache[src].copy()
    k_cache[dst] = k_src
    v_cache[dst] = v_src
    if kv_scales is not None:
        s_src = kv_scales[:, src].copy()
        kv_scales[:, dst] = s_src


# ---------------------------------------------------------------- gather ---

def window_start(context_len: int, window: int) -> int:
    """First attended position: max(0, L - W) for a window W > 0, else 0."""
    return max(0, int(context_len) - int(window)) if window > 0 else 0


def gather(k_cache, v_cache, kv_dtype: str, table_row, context_len: int,
           kv_head: int, head_dim: int, kv_scales=None, start: int = 0):
    """Dense float64 K and V [L - start, D] of one sequence and one KV head,
    rows for positions start .. L-1.

    Token t lives in physical block table_row[t // 16] at offset t % 16
    ("rvllm - A Small LLM Inference Engine in Rust", section "How it's put
    together": read_blocks + read_num_tokens).  For E4M3 each value is the
    decoded code times its block's K or V scale ("LLM Serving Kernels",
    section "Projects", row 05).
    """
    kidx = k_tile_index(head_dim, kv_dtype)
    vidx = v_tile_index(head_dim, kv_dtype)
    L = int(context_len)
    t = np.arange(int(start), L)
    blk = np.asarray(table_row, dtype=np.int64)[t // BLOCK_SIZE]   # physical block of token t
    off = t % BLOCK_SIZE                                             # its slot in that block
    rows = np.arange(len(t))[:, None]                                # row r of the gathered tiles
    K = to_f64(k_cache[blk, kv_head][rows, kidx[off]], kv_dtype)
    V = to_f64(v_cache[blk, kv_head][rows, vidx[off]], kv_dtype)
    if kv_dtype == "e4m3":
        K = K * kv_scales[0, blk, kv_head].astype(np.float64)[:, None]
        V = V * kv_scales[1, blk, kv_head].astype(np.float64)[:, None]
    return K, V


# ------------------------------------------------------------- attention ---

def softmax_weights(q_vec, K, scale: float) -> np.ndarray:
    """p_t = exp(s_t - max s) / sum_u exp(s_u - max s), s_t = scale * q.K[t]."""
    s = scale * (K @ q_vec)
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def decode_attention(q_raw, q_dtype: str, k_cache, v_cache, kv_dtype: str,
                     block_tables, context_lens, scale: float, kv_scales=None, window: int = 0):
    """float64 [B, Hq, D]: softmax(q K^T * scale) V per sequence and query head,
    over positions [window_start(L, window), L).

    Query head i reads KV head i // G with G = Hq / Hkv (contiguous groups).
    A sequence with context length 0 yields zeros.
    """
    q = to_f64(q_raw, q_dtype)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        lo = window_start(L, window)
        for h in range(Hkv):
            K, V = gather(k_cache, v_cache, kv_dtype, block_tables[b], L, h, D, kv_scales, lo)
            for g in range(G):
                i = h * G + g
                out[b, i] = softmax_weights(q[b, i], K, scale) @ V
    return out


def partition_origin(context_len: int, window: int) -> int:
    """Token where partition 0 starts: the window start rounded down to a
    16-token block (0 without a window)."""
    return window_start(context_len, window) // BLOCK_SIZE * BLOCK_SIZE


def prefill_attention(q_raw, q_dtype: str, k_cache, v_cache, kv_dtype: str, block_tables,
                      context_lens, query_start, scale: float, kv_scales=None):
    """Multi-token step: float64 [T, Hq, D] for the packed query rows.

    Sequence b owns query rows query_start[b] .. query_start[b+1]-1: its
    n_b newest tokens, at positions L_b - n_b .. L_b - 1.  Row j (position
    p = L_b - n_b + j) attends to positions 0 .. p: causal inside the new
    tokens ("rvLLM: High-performance LLM inference in Rust", section "CUDA
    Kernels", row "FlashAttention-2": prefill and decode with causal
    masking).  With n_b = 1 this is decode_attention.
    """
    q = to_f64(q_raw, q_dtype)
    T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    qs = np.asarray(query_start, dtype=np.int64)
    for b in range(len(qs) - 1):
        L = int(context_lens[b])
        n = int(qs[b + 1] - qs[b])
        for h in range(Hkv):
            K, V = gather(k_cache, v_cache, kv_dtype, block_tables[b], L, h, D, kv_scales)
            for j in range(n):
                p = L - n + j
                for g in range(G):
                    i = h * G + g
                    out[qs[b] + j, i] = softmax_weights(q[qs[b] + j, i], K[:p + 1], scale) @ V[:p + 1]
    return out


def num_partitions(context_len: int, partition_size: int, window: int = 0) -> int:
    a = partition_origin(context_len, window)
    return (int(context_len) - a + partition_size - 1) // partition_size


def decode_partials(q_raw, q_dtype: str, k_cache, v_cache, kv_dtype: str,
                    block_tables, context_lens, scale: float, partition_size: int,
                    num_slots: int, kv_scales=None, window: int = 0):
    """Per-partition outputs and log-sum-exps.

    With a = partition_origin(L_b, window) and lo = window_start(L_b, window),
    partition j of sequence b covers tokens [max(lo, a + j P), min(a + (j+1) P, L_b))
    (without a window: [j P, min((j+1) P, L_b))).  For it: o_j = softmax over
    those tokens of the scaled logits, times their V; lse_j = log sum_t exp(s_t)
    over those tokens (natural log).  Partitions at or past
    num_partitions(L_b, P, window) are empty: o = 0 and lse = -inf.

    Returns ``(o float64 [B, Hq, num_slots, D], lse float64 [B, Hq, num_slots])``.
    """
    q = to_f64(q_raw, q_dtype)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, num_slots, D), dtype=np.float64)
    lse = np.full((B, Hq, num_slots), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        w0 = window_start(L, window)
        a = partition_origin(L, window)
        for h in range(Hkv):
            K, V = gather(k_cache, v_cache, kv_dtype, block_tables[b], L, h, D, kv_scales, w0)
            for g in range(G):
                i = h * G + g
                s_all = scale * (K @ q[b, i])          # row r is position w0 + r
                for j in range(num_partitions(L, partition_size, window)):
                    lo = max(w0, a + j * partition_size) - w0
                    hi = min(a + (j + 1) * partition_size, L) - w0
                    s = s_all[lo:hi]
                    m = np.max(s)
                    e = np.exp(s - m)
                    o[b, i, j] = (e / np.sum(e)) @ V[lo:hi]
                    lse[b, i, j] = m + math.log(np.sum(e))
    return o, lse


def merge_partials(o, lse, context_lens, partition_size: int, window: int = 0) -> np.ndarray:
    """LSE-weighted merge: out = sum_j w_j o_j / sum_j w_j, w_j = exp(lse_j - max lse).

    Only partitions j < num_partitions(L_b, P, window) take part; L_b = 0 yields zeros.
    """
    B, Hq, _, D = o.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = num_partitions(context_lens[b], partition_size, window)
        if n == 0:
            continue
        for i in range(Hq):
            l = lse[b, i, :n]
            w = np.exp(l - np.max(l))
            out[b, i] = (w @ o[b, i, :n]) / np.sum(w)
    return out
