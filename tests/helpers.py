"""Shared test plumbing: build the oracle's pool from a workload, and read a
sequence's context straight from the generator's arrays (no tile layout)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import paged_attention as ref

BS = 16


def host_workers() -> int:
    """Threads for the oracle's long full-size runs: the host's cores, at most
    16 (a one-GPU machine's CPU share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_pool(w, workers: int = 1):
    """The pool the oracle attends over: NaN-filled, then every context slot
    written, then (if the workload has one) each sequence's new token.
    Returns (k_cache, v_cache, kv_scales or None).  With workers > 1 an E4M3
    pool's blocks are quantised in that many threads, each on its own
    disjoint set of blocks (the oracle's code unchanged, only run in pieces)."""
    s = w.spec
    k_cache, v_cache = ref.new_pool(w.num_blocks, s.num_kv_heads, s.head_dim, s.kv_dtype)
    kv_scales = None
    if s.kv_dtype == "e4m3":
        kv_scales = np.ones((2, w.num_blocks, s.num_kv_heads), dtype=np.float32)
        kf = w.fill_k.view(np.float32)
        vf = w.fill_v.view(np.float32)
        if workers > 1:
            n = len(w.fill_blocks)
            step = max(1, -(-n // (4 * workers)))

            def piece(i):
                sl = slice(i, min(n, i + step))
                ref.kv_cache_write_e4m3_blocks(k_cache, v_cache, kv_scales, kf[sl], vf[sl],
                                               w.fill_blocks[sl], w.fill_valid[sl])

            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(piece, range(0, n, step)))
        else:
            ref.kv_cache_write_e4m3_blocks(k_cache, v_cache, kv_scales, kf, vf, w.fill_blocks, w.fill_valid)
    else:
        slots, k, v = w.fill_tokens()
        ref.kv_cache_write(k_cache, v_cache, k, v, slots, s.kv_dtype)
    if w.new_slots is not None:
        ref.kv_cache_write(k_cache, v_cache, w.new_k, w.new_v, w.new_slots, s.kv_dtype)
    return k_cache, v_cache, kv_scales


def oracle_pool_unquantised(w):
    """An fp32 pool of an E4M3 workload's K/V before quantisation (the
    generator's float32 values, written with the oracle's slot write):
    what the FP8 path's quantisation error is measured against."""
    s = w.spec
    k_cache, v_cache = ref.new_pool(w.num_blocks, s.num_kv_heads, s.head_dim, "f32")
    slots, k, v = w.fill_tokens()
    ref.kv_cache_write(k_cache, v_cache, k, v, slots, "f32")
    return k_cache, v_cache, None


def logical_kv(w, b, h, start=0, dtype=None):
    """float64 K, V [L_b - start, D] (positions start .. L_b - 1) of sequence b /
    kv head h taken from the generator's per-block arrays and new-token arrays
    (16-bit/f32 workloads; dtype "f32" reads an E4M3 workload's unquantised
    float32 values)."""
    s = w.spec
    kv_dtype = dtype or s.kv_dtype
    where = {int(blk): i for i, blk in enumerate(w.fill_blocks)}
    L = int(w.context_lens[b])
    K = np.empty((L - start, s.head_dim))
    V = np.empty((L - start, s.head_dim))
    for t in range(start, L):
        if w.new_slots is not None and t == L - 1:
            kr, vr = w.new_k[b, h], w.new_v[b, h]
        else:
            i = where[int(w.block_tables[b, t // BS])]
            kr, vr = w.fill_k[i, t % BS, h], w.fill_v[i, t % BS, h]
        K[t - start] = ref.to_f64(kr, kv_dtype)
        V[t - start] = ref.to_f64(vr, kv_dtype)
    return K, V


def small(name, **kw):
    """A reduced variant of a named workload that the oracle runs in well under a second."""
    from paged_kv_gqa_cache_amd import workloads
    return workloads.generate(name, **kw)
