"""Seeded synthetic decode-attention workloads.

This module only draws inputs: context lengths, block-id assignment, and
N(0,1) query/key/value values rounded to their storage type.  It holds none
of the attention arithmetic, no cache layout and no FP8 quantisation, so the
HIP library and the CPU oracle can both consume its output without sharing
any of the computation.

Six named workloads, shaped like the models the pages run (SmolLM2-360M in
"rvllm - A Small LLM Inference Engine in Rust"; Qwen2.5-1.5B and Qwen2.5-7B in
"rvLLM: High-performance LLM inference in Rust", sections "Benchmarks" and
the head-to-head tables; a sliding-window layer of the kind Gemma 4 runs in
most of its layers, "rvLLM: The Inference Engine That Lets TPUs Compete by
Writing Less Kernel Code", section "The flat-scan trick"), one attention
layer each:

=================  ====  =======  ===  ======  ================================  ============
name               B     Hq/Hkv   D    dtype   context lengths                   extra
=================  ====  =======  ===  ======  ================================  ============
tiny               4     8/2      64   f32     uniform [1, 300]; pool 128        new-token write
smollm2_360m       16    15/5     64   f16     uniform [64, 2048]
qwen25_1p5b        32    12/2     128  f16     uniform [512, 4096]               new-token write
qwen25_7b_prefix   128   28/4     128  bf16    lognormal(median 1024, sigma 1)   8-seq groups share
                                               clipped to [16, 32768]            32 prefix blocks
qwen25_7b_fp8      64    28/4     128  e4m3    fixed 8192                        q f16
gemma_sliding      64    32/16    128  bf16    uniform [1024, 32768]             window 1024
qwen25_7b_chunk    16    28/4     128  bf16    uniform [512, 4096]               1-256 new
                                                                                 tokens each
=================  ====  =======  ===  ======  ================================  ============

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in this
order): context lengths; a permutation of the pool's block ids, dealt out in
order (per prefix group its shared blocks first, then each sequence's private
blocks); q [B, Hq, D]; K then V for every filled block [n, 16, Hkv, D]; the
new token's K then V [B, Hkv, D] where the workload writes one.  Values are
float32 N(0, 1) rounded to nearest-even into f16/bf16.  Slots no sequence
owns stay unwritten (the caller fills the pool with NaN first).  The pool
holds ceil(1.25 x blocks needed) blocks unless the workload fixes it.
A multi-token workload (chunked prefill, speculative verification) gives
each sequence n_b query tokens, the last n_b positions of its context
(n_b drawn uniformly, at most L_b); q is then [sum n_b, Hq, D] with rows in
sequence order and query_start [B + 1] the offsets.
With a window of W tokens only the blocks holding positions
[max(0, L - W), L) get their own ids and values; every table entry before
them points at one shared block that is never written (it keeps the
caller's NaN fill), so a read outside the window shows up as NaN.
Integer ranges include both ends.  For the FP8 workload K/V stay float32 and
the consumer quantises them per (block, kv head).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16

RAW_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str
    kv_dtype: str
    lengths: tuple                 # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("fixed", L)
    num_blocks: Optional[int] = None
    prefix_group: int = 0          # sequences per prefix-sharing group (0: none)
    prefix_blocks: int = 0         # leading blocks shared inside a group
    new_token_write: bool = False  # the step starts with kv_cache_write of one token per sequence
    partition_size: int = 512      # default split-context partition (tokens)
    window: int = 0                # sliding window in tokens (0: whole context)
    query_tokens: tuple = ()       # multi-token step: ("uniform", lo, hi) new tokens per sequence

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads


SPECS = {
    "tiny": WorkloadSpec("tiny", 1001, 4, 8, 2, 64, "f32", "f32", ("uniform", 1, 300),
                         num_blocks=128, new_token_write=True, partition_size=64),
    "smollm2_360m": WorkloadSpec("smollm2_360m", 1002, 16, 15, 5, 64, "f16", "f16",
                                 ("uniform", 64, 2048), partition_size=256),
    "qwen25_1p5b": WorkloadSpec("qwen25_1p5b", 1003, 32, 12, 2, 128, "f16", "f16",
                                ("uniform", 512, 4096), new_token_write=True, partition_size=768),
    "qwen25_7b_prefix": WorkloadSpec("qwen25_7b_prefix", 1004, 128, 28, 4, 128, "bf16", "bf16",
                                     ("lognormal", 1024, 1.0, 16, 32768), prefix_group=8,
                                     prefix_blocks=32, partition_size=768),
    "qwen25_7b_fp8": WorkloadSpec("qwen25_7b_fp8", 1005, 64, 28, 4, 128, "f16", "e4m3",
                                  ("fixed", 8192), partition_size=1024),
    "gemma_sliding": WorkloadSpec("gemma_sliding", 1006, 64, 32, 16, 128, "bf16", "bf16",
                                  ("uniform", 1024, 32768), partition_size=512, window=1024),
    "qwen25_7b_chunk": WorkloadSpec("qwen25_7b_chunk", 1007, 16, 28, 4, 128, "bf16", "bf16",
                                    ("uniform", 512, 4096), partition_size=512,
                                    query_tokens=("uniform", 1, 256)),
}


@dataclass
class Workload:
    spec: WorkloadSpec
    num_blocks: int
    scale: float                   # fp32-representable softmax scale 1/sqrt(D)
    q: np.ndarray                  # raw bits [B, Hq, D] in q_dtype
    context_lens: np.ndarray       # int32 [B]; includes the token written this step
    block_tables: np.ndarray       # int32 [B, max_blocks_per_seq]; -1 past each sequence's end
    fill_blocks: np.ndarray        # int64 [n] physical blocks holding context before the step
    fill_valid: np.ndarray         # int32 [n] leading slots of each filled block that hold data
    fill_k: np.ndarray             # raw [n, 16, Hkv, D] in ctx_dtype (float32 bits for e4m3 pools)
    fill_v: np.ndarray
    ctx_dtype: str
    new_slots: Optional[np.ndarray] = None   # int64 [B] slot of each sequence's new token
    new_k: Optional[np.ndarray] = None       # raw [B, Hkv, D] in kv_dtype
    new_v: Optional[np.ndarray] = None
    query_start: Optional[np.ndarray] = None # int32 [B + 1] (multi-token workloads)
    meta: dict = field(default_factory=dict)

    # -- views used by both consumers (data plumbing only) -----------------
    def fill_tokens(self):
        """(slots int64 [T], k raw [T, Hkv, D], v raw [T, Hkv, D]) of every filled slot."""
        t = np.arange(BLOCK_SIZE)[None, :]
        valid = t < self.fill_valid[:, None]
        slots = (self.fill_blocks[:, None] * BLOCK_SIZE + t)[valid]
        return slots.astype(np.int64), self.fill_k[valid], self.fill_v[valid]

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> raw storage bits of ``dtype`` (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        bits = x.view(np.uint32).copy()          # finite inputs: no overflow below
        lsb = (bits >> 16) & 1
        bits += np.uint32(0x7FFF)
        bits += lsb
        bits >>= 16
        return bits.astype(np.uint16)
    raise ValueError(f"no rounding to {dtype}")


def _draw_lengths(rng, spec: WorkloadSpec) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "uniform":
        lo, hi = spec.lengths[1], spec.lengths[2]
        return rng.integers(lo, hi, size=spec.num_seqs, endpoint=True).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = spec.lengths[1:]
        z = rng.normal(math.log(median), sigma, size=spec.num_seqs)
        return np.clip(np.round(np.exp(z)), lo, hi).astype(np.int64)
    if kind == "fixed":
        return np.full(spec.num_seqs, spec.lengths[1], dtype=np.int64)
    raise ValueError(kind)


def generate(name: str, **overrides) -> Workload:
    """Draw the named workload; keyword overrides replace spec fields (for
    smaller test variants, e.g. ``num_seqs=4, lengths=("uniform", 1, 200)``)."""
    spec = dataclasses.replace(SPECS[name], **overrides) if overrides else SPECS[name]
    rng = np.random.default_rng(spec.seed)
    B, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")

    L = _draw_lengths(rng, spec)
    nblk = (L + BLOCK_SIZE - 1) // BLOCK_SIZE               # blocks each sequence reads
    ctx_len = L - 1 if spec.new_token_write else L.copy()   # tokens present before the step

    # First block of each sequence's window (0 without a window).
    W = spec.window
    if W and spec.prefix_group:
        raise ValueError("a workload has either a window or prefix sharing")
    jlo = (np.maximum(L - W, 0) // BLOCK_SIZE) if W else np.zeros(B, dtype=np.int64)

    # Which logical blocks are physically shared (prefix groups).
    grp = spec.prefix_group
    shared_per_seq = np.zeros(B, dtype=np.int64)
    groups = []
    if grp:
        for g0 in range(0, B, grp):
            members = list(range(g0, min(g0 + grp, B)))
            for b in members:
                shared_per_seq[b] = min(spec.prefix_blocks, int(nblk[b]))
            groups.append((members, int(max(shared_per_seq[b] for b in members))))
    else:
        groups = [([b], 0) for b in range(B)]

    outside = bool(np.any(jlo > 0))                         # one never-written block
    needed = (sum(n_sh for _, n_sh in groups) + int(np.sum(nblk - shared_per_seq - jlo))
              + int(outside))
    num_blocks = spec.num_blocks if spec.num_blocks is not None else int(math.ceil(1.25 * needed))
    if needed > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {needed}")
    perm = rng.permutation(num_blocks)

    mbps = int(max(1, nblk.max()))
    tables = np.full((B, mbps), -1, dtype=np.int32)
    fill_blocks, fill_valid = [], []
    cursor = 0
    outside_id = -1
    if outside:
        outside_id = int(perm[cursor])
        cursor += 1
    for members, n_shared in groups:
        shared_ids = perm[cursor:cursor + n_shared]
        cursor += n_shared
        for j, blk in enumerate(shared_ids):
            fill_blocks.append(int(blk))
            fill_valid.append(BLOCK_SIZE)     # a shared prefix block is fully written
        for b in members:
            ns = int(shared_per_seq[b])
            tables[b, :ns] = shared_ids[:ns]
            tables[b, ns:ns + int(jlo[b])] = outside_id
            for j in range(ns + int(jlo[b]), int(nblk[b])):
                blk = int(perm[cursor])
                cursor += 1
                tables[b, j] = blk
                valid = int(min(max(ctx_len[b] - j * BLOCK_SIZE, 0), BLOCK_SIZE))
                if valid > 0:
                    fill_blocks.append(blk)
                    fill_valid.append(valid)
    fill_blocks = np.array(fill_blocks, dtype=np.int64)
    fill_valid = np.array(fill_valid, dtype=np.int32)

    query_start = None
    if spec.query_tokens:
        if spec.new_token_write or W:
            raise ValueError("a multi-token workload has no new-token write and no window")
        lo_q, hi_q = spec.query_tokens[1], spec.query_tokens[2]
        nq = np.minimum(rng.integers(lo_q, hi_q, size=B, endpoint=True), L).astype(np.int64)
        query_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
        q = round_to(rng.standard_normal((int(query_start[-1]), Hq, D), dtype=np.float32), spec.q_dtype)
    else:
        q = round_to(rng.standard_normal((B, Hq, D), dtype=np.float32), spec.q_dtype)
    ctx_dtype = "f32" if spec.kv_dtype == "e4m3" else spec.kv_dtype
    n = len(fill_blocks)
    kf = rng.standard_normal((n, BLOCK_SIZE, Hkv, D), dtype=np.float32)
    vf = rng.standard_normal((n, BLOCK_SIZE, Hkv, D), dtype=np.float32)
    invalid = np.arange(BLOCK_SIZE)[None, :] >= fill_valid[:, None]
    kf[invalid] = 0.0
    vf[invalid] = 0.0
    fill_k, fill_v = round_to(kf, ctx_dtype), round_to(vf, ctx_dtype)
    del kf, vf

    new_slots = new_k = new_v = None
    if spec.new_token_write:
        if spec.kv_dtype == "e4m3":
            raise ValueError("the FP8 workload has no new-token write")
        pos = L - 1
        new_slots = (tables[np.arange(B), pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE
                     + pos % BLOCK_SIZE)
        new_k = round_to(rng.standard_normal((B, Hkv, D), dtype=np.float32), spec.kv_dtype)
        new_v = round_to(rng.standard_normal((B, Hkv, D), dtype=np.float32), spec.kv_dtype)

    scale = float(np.float32(1.0 / math.sqrt(D)))
    meta = {"blocks_needed": needed, "outside_block": outside_id}
    return Workload(spec, num_blocks, scale, q, L.astype(np.int32), tables, fill_blocks,
                    fill_valid, fill_k, fill_v, ctx_dtype, new_slots, new_k, new_v,
                    query_start=query_start, meta=meta)


def kv_bytes(w: Workload, unique: bool = True) -> int:
    """Algorithmic K+V bytes one decode step reads.

    logical: every sequence's own context, a shared prefix counted per sequence;
    unique: each distinct (physical block, kv head) tile counted once, by the
    tokens read from it (the most tokens any sequence reads from that block).
    For E4M3 pools each touched (block, kv head) also costs two fp32 scales.
    With a window only positions [max(0, L - W), L) are read.
    """
    e = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}[w.spec.kv_dtype]
    Hkv, D = w.spec.num_kv_heads, w.spec.head_dim
    per_tok = 2 * Hkv * D * e
    per_blk_extra = 2 * 4 * Hkv if w.spec.kv_dtype == "e4m3" else 0
    L = w.context_lens.astype(np.int64)
    W = w.spec.window
    lo = np.maximum(L - W, 0) if W else np.zeros_like(L)
    if not unique:
        nb = (L + BLOCK_SIZE - 1) // BLOCK_SIZE - lo // BLOCK_SIZE
        return int((L - lo).sum() * per_tok + nb.sum() * per_blk_extra)
    used = {}
    for b in range(len(L)):
        for j in range(int(lo[b]) // BLOCK_SIZE, (int(L[b]) + BLOCK_SIZE - 1) // BLOCK_SIZE):
            toks = min(BLOCK_SIZE, int(L[b]) - j * BLOCK_SIZE) - max(0, int(lo[b]) - j * BLOCK_SIZE)
            blk = int(w.block_tables[b, j])
            used[blk] = max(used.get(blk, 0), toks)
    return int(sum(used.values()) * per_tok + len(used) * per_blk_extra)
