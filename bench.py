"""Benchmark: paged GQA decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one decode-attention step of one layer for the whole batch: the
new-token slot write (for workloads that have one), the split-context
kernel and the LSE merge kernel, all through the C ABI.  The headline runs
the balanced schedule (paged_decode_attention_balanced_partial and _reduce:
equal tile shares per compute unit, split points chosen by load, no
partition size); --path picks another.  Each step
uses the next of several layer pools in turn (distinct HBM buffers, more
bytes than the 256 MB Infinity Cache holds), as consecutive layers of a real
decode step do, so every step reads its K/V from HBM.

Prints ONE JSON line.  ``value`` is the headline workload's K/V-read
throughput: unique K/V bytes per step (each physical (block, kv head) tile
counted once, by the tokens read from it) over the wall time per step.
``roofline`` rates the split kernel alone: the same bytes over its average
duration, measured inside the timed region with HIP events recorded on the
stream the kernel runs on (events created with hipEventDisableSystemFence,
which costs about 1 us per step instead of about 5).  ``cpu_baseline`` is the
float64 oracle on all the host's cores (one worker process per core), on the same batch.  A second workload
(the B=32 Qwen2.5-1.5B-shaped layer with its new-token write) is timed in the
same run and reported as ``b32``.  The other rows of the path (FP8 E4M3
decode, the sliding window, the multi-token step, the E4M3 quantiser and
append, the block copy and the slot write) are measured on their own
workloads in the same run and reported under ``rows``, each against the
roofline that bounds it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HEADLINE = "qwen25_7b_prefix"
SECONDARY = "qwen25_1p5b"

DESCRIPTIONS = {
    "qwen25_7b_prefix": "Qwen2.5-7B-shaped attention layer: 128 seqs, 28 Q / 4 KV heads, head_dim 128, "
                        "bf16 q/K/V, 16-token blocks, lognormal context (median 1024, sigma 1, clip "
                        "[16, 32768]), 8-seq groups share 32 prefix blocks, split-context partitions",
    "qwen25_1p5b": "Qwen2.5-1.5B-shaped attention layer: 32 seqs, 12 Q / 2 KV heads, head_dim 128, "
                   "fp16, 16-token blocks, context uniform [512, 4096], new-token write of 32 tokens",
    "smollm2_360m": "SmolLM2-360M-shaped attention layer: 16 seqs, 15 Q / 5 KV heads, head_dim 64, fp16",
    "qwen25_7b_fp8": "Qwen2.5-7B-shaped attention layer, FP8 E4M3 KV with per-(block, kv head) scales: "
                     "64 seqs, 28 Q / 4 KV heads, head_dim 128, context 8192, q fp16",
    "tiny": "4 seqs, 8 Q / 2 KV heads, head_dim 64, fp32, pool of 128 blocks",
    "gemma_sliding": "sliding-window attention layer: 64 seqs, 32 Q / 16 KV heads, head_dim 128, bf16, "
                     "window 1024 tokens, context uniform [1024, 32768]",
}
DTYPE_NAME = {"f32": "f32", "f16": "f16", "bf16": "bf16", "e4m3": "e4m3"}


class HipEvents:
    """Timing events on a given stream, straight from the HIP runtime."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
            self.ev.append(e)

    def record(self, i: int, stream_handle: int) -> None:
        self.hip.hipEventRecord(self.ev[i], self.ct.c_void_p(stream_handle))

    def elapsed_ms(self, i: int, j: int) -> float:
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return f.value

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def code_only(text: str) -> str:
    """C/C++ source with its comments removed and each line's trailing
    whitespace dropped (string and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).split("\n")]
    return "\n".join(ln for ln in lines if ln)


def source_digest() -> str:
    """Digest of the kernel and launch sources: the code (comments and blank
    lines left out) of every file under csrc/ except abi.hip, the host-side
    ABI layer (argument checks, descriptors), whose changes do not change what
    the kernels execute."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_gqa_cache_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "abi.hip":
            continue
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + code_only(f.read()).encode())
    return h.hexdigest()[:16]


# Kernel whose counters the committed HBM summary must hold, per path.
PATH_KERNEL = {"balanced": "paged_decode_cu_stream", "pair": "paged_decode_persistent",
               "fused": "paged_decode_persistent", "step": "paged_decode_persistent",
               "single": "paged_decode_persistent"}


def counters_traffic(workload: str, digest: str, path: str = "balanced"):
    """HBM bytes per launch of the path's split kernel from the committed
    rocprofv3 counter summary, if it was taken from the current kernel
    sources and for that kernel; else None."""
    fname = os.path.join(ROOT, "profiles", f"paged_decode_{workload}_hbm_counters.txt")
    if not os.path.exists(fname):
        return None
    vals = {}
    for line in open(fname):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != digest or PATH_KERNEL.get(path, "?") not in vals.get("kernel", ""):
        return None
    try:
        return int(float(vals["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


class Runner:
    """Device state for one workload: layer pools, inputs, workspace."""

    def __init__(self, name: str, layers: int, partition_size=None, path: str = "pair", **overrides):
        import torch
        from paged_kv_gqa_cache_amd import abi, workloads
        from paged_kv_gqa_cache_amd.pool import gpu_pool, inputs, to_dev

        self.torch, self.abi = torch, abi
        self.w = w = workloads.generate(name, **overrides)
        self.spec = s = w.spec
        self.P = partition_size or s.partition_size
        base = gpu_pool(w, with_new_tokens=False)
        self.pools = [base] + [tuple(None if t is None else t.clone() for t in base) for _ in range(layers - 1)]
        self.q, self.tables, self.lens = inputs(w)
        self.tmp_out, self.tmp_lse = abi.alloc_partials(self.q, self.tables.shape[1], self.P)
        self.ws = abi.split_workspace(self.q, base[0], self.tables, self.P)
        self.bws = abi.balanced_workspace(self.q, base[0], self.tables) if path == "balanced" else None
        self.path = path
        self.out = torch.empty(self.q.shape, dtype={"f32": torch.float32, "f16": torch.float16,
                                                    "bf16": torch.bfloat16}[s.q_dtype], device="cuda")
        self.new = None
        if w.new_slots is not None:
            self.new = (to_dev(w.new_k, s.kv_dtype), to_dev(w.new_v, s.kv_dtype),
                        torch.from_numpy(w.new_slots).cuda())
        self.unique_bytes = workloads.kv_bytes(w, unique=True)
        self.logical_bytes = workloads.kv_bytes(w, unique=False)
        torch.cuda.synchronize()

    def step(self, i: int, ev=None, e0: int = 0) -> None:
        """One decode step on layer pool i % layers; with ``ev``, events e0 and
        e0 + 1 bracket the dominant kernel (the partial, the fused split, or the fused step)."""
        abi = self.abi
        k, v, sc = self.pools[i % len(self.pools)]
        stream = self.torch.cuda.current_stream().cuda_stream
        if self.new is not None and self.path != "step":
            abi.kv_cache_write(self.new[0], self.new[1], self.new[2], k, v)
        if ev is not None:
            ev.record(e0, stream)
        if self.path == "step":
            abi.paged_decode_step(self.q, self.new[0], self.new[1], k, v, self.tables, self.lens, self.w.scale,
                                  self.P, self.ws, out=self.out, window=self.spec.window)
            if ev is not None:
                ev.record(e0 + 1, stream)
            return
        if self.path == "single":
            abi.paged_decode_attention(self.q, k, v, self.tables, self.lens, self.w.scale, sc, out=self.out,
                                       window=self.spec.window)
            if ev is not None:
                ev.record(e0 + 1, stream)
            return
        if self.path == "balanced":
            abi.paged_decode_attention_balanced_partial(self.q, k, v, self.tables, self.lens, self.w.scale, sc,
                                                        self.bws, self.out, window=self.spec.window)
            if ev is not None:
                ev.record(e0 + 1, stream)
            abi.paged_decode_attention_balanced_reduce(self.q, k, self.tables, self.bws, self.out,
                                                       window=self.spec.window)
        elif self.path == "fused":
            abi.paged_decode_attention_split(self.q, k, v, self.tables, self.lens, self.w.scale, sc,
                                             self.P, self.ws, out=self.out, window=self.spec.window)
            if ev is not None:
                ev.record(e0 + 1, stream)
        else:
            abi.paged_decode_attention_partial(self.q, k, v, self.tables, self.lens, self.w.scale, sc,
                                               self.P, self.tmp_out, self.tmp_lse, window=self.spec.window)
            if ev is not None:
                ev.record(e0 + 1, stream)
            abi.paged_decode_attention_reduce(self.tmp_out, self.tmp_lse, self.lens, self.P, self.out,
                                              self.tables.shape[1], window=self.spec.window)

    # Every EVENT_EVERY-th timed step, from the second on, brackets its
    # dominant kernel with a pair of HIP events: a pair costs ~3-5 us of GPU
    # time, which would otherwise inflate every step of the wall-clock
    # figure, and the first kernel after the synchronisation runs ~15 us long.
    EVENT_EVERY = 4

    def run(self, steps: int, warmup: int):
        """Returns (seconds per step, [dominant-kernel ms of the sampled steps])."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        sampled = list(range(1, steps, self.EVENT_EVERY))
        ev = HipEvents(2 * len(sampled))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if i % self.EVENT_EVERY == 1:
                self.step(warmup + i, ev, 2 * (i // self.EVENT_EVERY))
            else:
                self.step(warmup + i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kernel_ms = [ev.elapsed_ms(2 * j, 2 * j + 1) for j in range(len(sampled))]
        ev.close()
        return wall / steps, kernel_ms

    def run_graph_or_none(self, steps: int, warmup: int):
        """``run_graph``, or (None, the error) if capture fails: the graph
        figure is an extra, never a reason to lose the line."""
        try:
            return self.run_graph(steps, warmup), None
        except Exception as e:   # noqa: BLE001 (reported in the line)
            self.torch.cuda.synchronize()
            return None, f"{type(e).__name__}: {e}"[:200]

    def run_graph(self, steps: int, warmup: int) -> float:
        """Seconds per step with the steps replayed from a HIP graph: one
        captured step per layer pool (same arguments as ``step``), the graph
        replayed until about ``steps`` steps have run.  What a serving loop
        that captures its decode step pays: the kernels without the Python
        binding's per-call host work.  Nothing in a step allocates, clears
        memory or synchronises, so it captures as is."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        n = len(self.pools)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                self.step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // n)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del g
        return wall / (reps * n)


def host_cores() -> int:
    """Cores this process may run on, capped by OMP_NUM_THREADS when set (a
    one-GPU machine exports its CPU share there)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_CPU_STATE = {}


def _oracle_chunk(bounds):
    """One worker's share of a decode step: the oracle over sequences
    [b0, b1) of the workload the parent process set up before forking."""
    from oracle import paged_attention as ref
    w, k, v, sc = _CPU_STATE["w"], _CPU_STATE["k"], _CPU_STATE["v"], _CPU_STATE["sc"]
    b0, b1 = bounds
    s = w.spec
    if w.new_slots is not None:
        ref.kv_cache_write(k, v, w.new_k[b0:b1], w.new_v[b0:b1], w.new_slots[b0:b1], s.kv_dtype)
    ref.decode_attention(w.q[b0:b1], s.q_dtype, k, v, s.kv_dtype, w.block_tables[b0:b1],
                         w.context_lens[b0:b1], w.scale, sc, window=s.window)
    return b1 - b0


def cpu_baseline_child(name: str) -> dict:
    """The float64 oracle on this host's cores, on the full batch: the
    sequences are dealt to one forked worker process per core (each with
    one BLAS thread), and a step is the wall time until every worker has
    finished its sequences (the new-token write included).  Runs in a
    child process of bench.py that never touches the GPU."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from paged_kv_gqa_cache_amd import workloads
    from tests.helpers import oracle_pool

    w = workloads.generate(name)
    k, v, sc = oracle_pool(w)
    _CPU_STATE.update(w=w, k=k, v=v, sc=sc)
    cores = host_cores()
    B = w.spec.num_seqs
    # One task per sequence, longest first, handed to whichever worker is
    # free, so the workers' loads are even (the oracle's cost is linear in
    # the context).
    order = np.argsort(-w.context_lens.astype(np.int64), kind="stable")
    chunks = [(int(b), int(b) + 1) for b in order]
    times = []
    with threadpool_limits(1), mp.get_context("fork").Pool(cores) as pool:
        pool.map(_oracle_chunk, chunks[:cores])   # workers started and warm
        t_all = time.perf_counter()
        while len(times) < 3 or (time.perf_counter() - t_all < 15.0 and len(times) < 1000):
            t = time.perf_counter()
            done = sum(pool.map(_oracle_chunk, chunks, chunksize=1))
            times.append(time.perf_counter() - t)
            assert done == B
    t = float(np.median(times))
    return {"value": round(workloads.kv_bytes(w, unique=True) / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "us_per_step": round(t * 1e6, 1), "seqs_layers_per_s": round(B / t, 1),
            "sample": f"the full {B}-sequence batch of the headline workload, one decode step per sample "
                      f"(gather + softmax + PV in float64 numpy), sequences dealt to {cores} forked worker "
                      f"processes with one BLAS thread each; {len(times)} steps (~{sum(times):.0f} s), "
                      f"median {t * 1e3:.0f} ms per step"}


def cpu_baseline(name: str) -> dict:
    """Runs cpu_baseline_child in a fresh child process (this process has
    the GPU open; the child only uses the host) and returns its record."""
    import subprocess
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--workload", name],
                         capture_output=True, text=True, cwd=ROOT, timeout=600)
    if res.returncode != 0:
        raise RuntimeError(f"cpu baseline child failed ({res.returncode}): {res.stderr[-2000:]}")
    return json.loads(res.stdout.strip().splitlines()[-1])


def time_calls(fn, n: int, warmup: int = 3) -> float:
    """Average milliseconds per call of ``fn`` (which launches on the current
    stream), from HIP events on that stream around n back-to-back calls."""
    import torch
    for _ in range(warmup):
        fn()
    ev = HipEvents(2)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    ev.record(0, stream)
    for _ in range(n):
        fn()
    ev.record(1, stream)
    torch.cuda.synchronize()
    ms = ev.elapsed_ms(0, 1) / n
    ev.close()
    return ms


def hbm_row(bytes_per_call: int, ms: float, what: str) -> dict:
    gbps = bytes_per_call / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 2), "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes": bytes_per_call, "bytes_are": what}


def torch_materialising(r, steps: int) -> dict:
    """The headline decode step in plain PyTorch on the GPU, for context (the
    comparison "LLM Serving Kernels", section "Verified NVIDIA L4 release",
    makes against a materialising PyTorch reference): every sequence's K/V
    is gathered out of the paged pool into dense, zero-padded fp32 tensors
    (the tile layout undone by an index), then matmul, masked softmax,
    matmul.  Layer pools rotate as in the timed steps.  Not part of the path."""
    import torch
    s = r.spec
    B, Hq, Hkv, D = s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim
    G = Hq // Hkv
    e = {"f32": 4, "f16": 2, "bf16": 2}[s.kv_dtype]
    x, nn = 16 // e, 4 // e
    t = torch.arange(16).view(16, 1)
    d = torch.arange(D).view(1, D)
    # tile position of (token slot t, dim d), as the cache layout defines it
    pk = (((d // x) * 16 + t) * x + d % x).reshape(-1).cuda()
    pv = (((((d // (16 * nn)) * 4 + t // 4) * 16 + d % 16) * nn + (d // 16) % nn) * 4 + t % 4).reshape(-1).cuda()
    mbps = r.tables.shape[1]
    T = mbps * 16
    idx = r.tables.long().clamp(min=0)
    keep = torch.arange(T, device="cuda")[None, :] < r.lens.long()[:, None]
    q = r.q.float().view(B, Hkv, G, D)

    def step(i):
        k, v, _ = r.pools[i % len(r.pools)]
        K = k[idx][..., pk].view(B, mbps, Hkv, 16, D).permute(0, 2, 1, 3, 4).reshape(B, Hkv, T, D).float()
        V = v[idx][..., pv].view(B, mbps, Hkv, 16, D).permute(0, 2, 1, 3, 4).reshape(B, Hkv, T, D).float()
        V = V.masked_fill(~keep[:, None, :, None], 0.0)   # slots past the context hold no data
        S = torch.matmul(q, K.transpose(-1, -2).contiguous()) * r.w.scale
        S = S.masked_fill(~keep[:, None, None, :], float("-inf"))
        return torch.matmul(torch.softmax(S, dim=-1), V.contiguous()).reshape(B, Hq, D)

    # agreement with the path on one layer (outside the timing)
    k, v, sc = r.pools[0]
    from paged_kv_gqa_cache_amd import abi
    ours = abi.paged_decode_attention(r.q, k, v, r.tables, r.lens, r.w.scale, sc, out_dtype=torch.float32)
    diff = float((step(0) - ours).abs().max())
    it = [0]

    def call():
        step(it[0])
        it[0] += 1

    ms = time_calls(call, steps, warmup=2)
    return {"us": round(ms * 1e3, 1), "max_abs_diff_vs_path": diff,
            "what": "plain PyTorch on the GPU: gather to dense zero-padded fp32 K/V, matmul, masked softmax, "
                    "matmul (context for the materialising-reference comparison; not part of the path)"}


def unquantised_reference(w, seq_chunk: int = 16):
    """float64 [B, Hq, D] attention of an E4M3 workload over its K/V before
    quantisation (the generator's float32 values), computed in plain
    PyTorch float64 on the GPU: each sequence's blocks gathered to dense K/V
    from the generator's per-block arrays, then softmax(q K^T * scale) V
    with the same fp16 q.  The reference for the FP8 row's mean absolute
    error (quantisation error, not a parity gate); not part of the path."""
    import numpy as np
    import torch
    s = w.spec
    B, Hq, Hkv, D = s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim
    G = Hq // Hkv
    L = w.context_lens.astype(np.int64)
    nb = (L + 15) // 16
    where = np.full(w.num_blocks, -1, np.int64)
    where[w.fill_blocks] = np.arange(len(w.fill_blocks))
    kf = torch.from_numpy(w.fill_k.view(np.float32)).cuda()   # [n, 16, Hkv, D]
    vf = torch.from_numpy(w.fill_v.view(np.float32)).cuda()
    q = torch.from_numpy(w.q.view(np.float16)).cuda().double().view(B, Hkv, G, D)
    out = torch.empty((B, Hq, D), dtype=torch.float64, device="cuda")
    for b0 in range(0, B, seq_chunk):
        b1 = min(B, b0 + seq_chunk)
        m = int(nb[b0:b1].max())
        idx = np.zeros((b1 - b0, m), np.int64)
        for i, b in enumerate(range(b0, b1)):
            idx[i, :nb[b]] = where[w.block_tables[b, :nb[b]]]
        ix = torch.from_numpy(idx).cuda()
        K = kf[ix].double().permute(0, 3, 1, 2, 4).reshape(b1 - b0, Hkv, m * 16, D)
        V = vf[ix].double().permute(0, 3, 1, 2, 4).reshape(b1 - b0, Hkv, m * 16, D).contiguous()
        keep = torch.arange(m * 16, device="cuda")[None, :] < torch.from_numpy(L[b0:b1]).cuda()[:, None]
        S = torch.matmul(q[b0:b1], K.transpose(-1, -2).contiguous()) * w.scale
        S = S.masked_fill(~keep[:, None, None, :], float("-inf"))
        out[b0:b1] = torch.matmul(torch.softmax(S, dim=-1), V).reshape(b1 - b0, Hq, D)
    return out


ROW_NAMES = ("tiny_layer", "smollm2_layer", "headline_other_seeds", "single_pass", "fp8_e4m3_decode", "e4m3_bulk_quantise", "e4m3_append", "sliding_window",
             "chunked_prefill", "spec_verify_4", "copy_blocks", "kv_slot_write")


def measure_rows(args, only=None) -> dict:
    """The other rows of the path, each on its own workload, through the C ABI.
    Attention rows rotate layer pools like the headline (cold K/V); the cache
    maintenance rows are timed back to back (warm), as labelled.  ``only``
    limits the run to the named rows."""
    import numpy as np
    import torch
    from paged_kv_gqa_cache_amd import abi, workloads
    from paged_kv_gqa_cache_amd.pool import gpu_pool, to_dev

    rows = {}
    steps, warm = max(10, args.steps // 2), max(3, args.warmup // 2)
    want = (lambda k: True) if not only else (lambda k: k in only)

    # The two small layers (tiny: 4 fp32 sequences with their new-token
    # write; SmolLM2-360M-shaped: 16 fp16 sequences): launch-bound, reported
    # for the us/step and sequences x layers/s figures.  Each runs as one
    # launch: the tiny layer through the fused decode step (write + split
    # attention), the SmolLM2 layer through the split mode with its
    # in-kernel merge (measured: 14.6 us/step against 22-23 for the
    # partial + reduce pair and 17.7 for the single pass).
    for key, name, path in (("tiny_layer", "tiny", "step"), ("smollm2_layer", "smollm2_360m", "fused")):
        if not want(key):
            continue
        r = Runner(name, args.layers, None, path)
        t, part = r.run(steps, warm)
        ms = sum(part) / len(part)
        row = hbm_row(r.unique_bytes, ms, "unique K/V bytes read per step")
        row.update({"workload": f"{name}: {DESCRIPTIONS[name]}", "path": path, "partition_size": r.P,
                    "us_per_step": round(t * 1e6, 2), "step_GBps": round(r.unique_bytes / t / 1e9, 1),
                    "seqs_layers_per_s": round(r.spec.num_seqs / t, 1)})
        # The same steps replayed from a captured graph: launch-bound layers
        # are paced by the host's per-call work, which a serving loop that
        # captures its decode step does not pay.
        tg, gerr = r.run_graph_or_none(steps, warm)
        row.update({"graph_us_per_step": None if tg is None else round(tg * 1e6, 2),
                    "graph_seqs_layers_per_s": None if tg is None else round(r.spec.num_seqs / tg, 1)})
        if gerr:
            row["graph_error"] = gerr
        rows[key] = row
        del r
        torch.cuda.empty_cache()

    # The headline configuration drawn with two other seeds (other context
    # lengths, prefix groups and block ids; same distributions), on the
    # balanced schedule and on the fixed-partition pair at the headline's
    # partition size, so a schedule tuned to one draw would show.
    if want("headline_other_seeds"):
        seeds = {}
        for seed in (2004, 3004):
            per = {}
            for path in ("balanced", "pair"):
                r = Runner(HEADLINE, args.layers, None, path, seed=seed)
                t, part = r.run(steps, warm)
                ms = sum(part) / len(part)
                row = hbm_row(r.unique_bytes, ms, "unique K/V bytes read per step")
                row.update({"us_per_step": round(t * 1e6, 2),
                            "partition_size": None if path == "balanced" else r.P})
                per[path] = row
                del r
                torch.cuda.empty_cache()
            seeds[str(seed)] = per
        rows["headline_other_seeds"] = {"workload": f"{HEADLINE} with seed 2004 and 3004: {DESCRIPTIONS[HEADLINE]}",
                                        "seeds": seeds}

    # The headline layer through the single-pass entry point (no workspace,
    # one work item per sequence and kv head: the longest context bounds it).
    if want("single_pass"):
        r = Runner(HEADLINE, args.layers, None, "pair")
        it = [0]

        def single():
            k, v, sc = r.pools[it[0] % len(r.pools)]
            it[0] += 1
            abi.paged_decode_attention(r.q, k, v, r.tables, r.lens, r.w.scale, sc, out=r.out, window=r.spec.window)

        ms = time_calls(single, steps)
        rows["single_pass"] = hbm_row(r.unique_bytes, ms, "unique K/V bytes read per step")
        rows["single_pass"]["workload"] = f"{HEADLINE}: {DESCRIPTIONS[HEADLINE]}; paged_decode_attention (one pass)"
        del r
        torch.cuda.empty_cache()

    # FP8 E4M3 decode (per-(block, kv head) scales) and the sliding window:
    # balanced schedule, kernel time = the tile-stream kernel (the events
    # bracket it; the merge runs after them, and us_per_step holds both).
    # Each on its fastest path (measured: FP8 balanced 94 us, single pass 96,
    # pair P = 2048 97; sliding window single pass 88 us, balanced 94, pair
    # 106-112).  The window's items are equal (1024 positions each), so one
    # pass per (sequence, kv head) is balanced without a merge kernel.
    for key, name, P, path in (("fp8_e4m3_decode", "qwen25_7b_fp8", 512, "balanced"),
                               ("sliding_window", "gemma_sliding", None, "single")):
        extra = ("e4m3_bulk_quantise", "e4m3_append") if name == "qwen25_7b_fp8" else ()
        if not any(want(k) for k in (key,) + extra):
            continue
        r = Runner(name, args.layers, P, path)
        if want(key):
            t, part = r.run(steps, warm)
            ms = sum(part) / len(part)
            row = hbm_row(r.unique_bytes, ms, "unique K/V (+ E4M3 scales) bytes read per step")
            row.update({"workload": f"{name}: {DESCRIPTIONS[name]}", "path": path,
                        "us_per_step": round(t * 1e6, 2), "step_GBps": round(r.unique_bytes / t / 1e9, 1)})
            if name == "qwen25_7b_fp8":
                # Quantisation error of the FP8 path: its fp32 output against
                # attention over the unquantised fp32 K/V (same fp16 q).
                k, v, sc = r.pools[0]
                ours = abi.paged_decode_attention_balanced(r.q, k, v, r.tables, r.lens, r.w.scale, sc, r.bws,
                                                           out_dtype=torch.float32).double()
                d = (ours - unquantised_reference(r.w)).abs()
                row.update({"mae_vs_fp32": float(d.mean()), "max_abs_vs_fp32": float(d.max()),
                            "mae_is": "mean over all B x Hq x D outputs of |FP8 path (fp32 out) - attention over "
                                      "the unquantised fp32 K/V with the same fp16 q (float64)|"})
            rows[key] = row
        if name == "qwen25_7b_fp8":
            # Bulk quantiser on the same layer: fp32 blocks in, codes + scales out.
            w, sp = r.w, r.spec
            ksrc = torch.from_numpy(w.fill_k.view(np.float32)).cuda()
            vsrc = torch.from_numpy(w.fill_v.view(np.float32)).cuda()
            ids = torch.from_numpy(w.fill_blocks.astype(np.int32)).cuda()
            valid = torch.from_numpy(w.fill_valid.astype(np.int32)).cuda()
            k, v, sc = r.pools[0]
            nblk = int(ids.numel())
            if want("e4m3_bulk_quantise"):
                ms = time_calls(lambda: abi.kv_cache_quantize_e4m3(ksrc, vsrc, ids, valid, k, v, sc), 10)
                moved = (2 * (ksrc.numel() * 4 + nblk * 16 * sp.num_kv_heads * sp.head_dim)
                         + 2 * nblk * sp.num_kv_heads * 4)
                rows["e4m3_bulk_quantise"] = hbm_row(moved, ms, "fp32 K/V read + E4M3 codes and scales written")
                rows["e4m3_bulk_quantise"]["workload"] = (f"{nblk} blocks x {sp.num_kv_heads} kv heads x 16 tokens "
                                                          f"x {sp.head_dim}, K and V")
            # Append of one token per sequence into its last block (scale growth + re-encode).
            T = sp.num_seqs
            rng = np.random.default_rng(7)
            blocks = rng.permutation(w.num_blocks)[:T]
            slots = torch.tensor(blocks * 16 + 9, dtype=torch.int64, device="cuda")
            kn = torch.from_numpy(rng.standard_normal((T, sp.num_kv_heads, sp.head_dim), dtype=np.float32) * 4).cuda()
            vn = torch.from_numpy(rng.standard_normal((T, sp.num_kv_heads, sp.head_dim), dtype=np.float32) * 4).cuda()
            if want("e4m3_append"):
                ms = time_calls(lambda: abi.kv_cache_append_e4m3(kn, vn, slots, k, v, sc), 50)
                rows["e4m3_append"] = {"us": round(ms * 1e3, 2), "bound": "latency",
                                       "workload": f"{T} tokens (one per sequence) into distinct blocks at offset "
                                                   f"9, {sp.num_kv_heads} kv heads x {sp.head_dim}; every block "
                                                   "re-read and re-encoded when its scale grows"}
        del r
        torch.cuda.empty_cache()

    # Multi-token step: chunked prefill (1-256 new tokens per sequence) and
    # speculative verification (4 tokens per sequence).
    for key, kw, P in (("chunked_prefill", {}, 0),
                       ("spec_verify_4", dict(num_seqs=64, query_tokens=("uniform", 4, 4)), 0)):
        if not want(key):
            continue
        w = workloads.generate("qwen25_7b_chunk", **kw)
        sp = w.spec
        base = gpu_pool(w)
        pools = [base] + [tuple(None if x is None else x.clone() for x in base) for _ in range(args.layers - 1)]
        q = to_dev(w.q, sp.q_dtype)
        tables = torch.from_numpy(w.block_tables).cuda()
        lens = torch.from_numpy(w.context_lens).cuda()
        qs = torch.from_numpy(w.query_start).cuda()
        out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        ws = abi.prefill_workspace(q, base[0], tables, P)
        it = [0]

        def call():
            k, v, sc = pools[it[0] % len(pools)]
            it[0] += 1
            abi.paged_prefill_attention(q, k, v, tables, lens, qs, w.scale, sc, P, ws, out=out)

        ms = time_calls(call, steps)
        n = np.diff(w.query_start).astype(np.int64)
        L = w.context_lens.astype(np.int64)
        attended = int(sum(((L[b] - n[b]) + np.arange(n[b]) + 1).sum() for b in range(len(L))))
        flops = attended * sp.num_q_heads * 4 * sp.head_dim
        kvb = workloads.kv_bytes(w, unique=True)
        tf = flops / (ms * 1e-3) / 1e12
        desc = (f"qwen25_7b_chunk: {len(L)} seqs, 28 Q / 4 KV heads, head_dim 128, bf16, context uniform "
                f"[512, 4096], {int(n.sum())} new query rows ({int(n.min())}-{int(n.max())} per sequence), "
                f"causal within the new tokens, " + (f"P = {P}" if P else "one pass"))
        if key == "chunked_prefill":
            rows[key] = {"us": round(ms * 1e3, 2), "bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0,
                         "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4),
                         "flops": flops, "flops_are": "4 * head_dim per (query row, query head, attended position)",
                         "kv_GBps": round(kvb / (ms * 1e-3) / 1e9, 1), "workload": desc}
        else:
            row = hbm_row(kvb, ms, "unique K/V bytes read per step")
            row.update({"TFLOPs": round(tf, 1), "workload": desc})
            rows[key] = row
        del pools, base
        torch.cuda.empty_cache()

    # Block copy (copy-on-write / beam fork): 4096 (source, destination)
    # pairs of bf16 blocks, 4 kv heads x head_dim 128, four disjoint pair
    # sets in turn.
    if want("copy_blocks"):
        NB, Hkv, D, npairs = 40960, 4, 128, 4096
        kc = torch.zeros((NB, Hkv, 16 * D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        rng = np.random.default_rng(11)
        perm = rng.permutation(NB)
        maps = [torch.tensor(np.stack([perm[i * 2 * npairs:i * 2 * npairs + npairs],
                                       perm[i * 2 * npairs + npairs:(i + 1) * 2 * npairs]], 1).astype(np.int32),
                             device="cuda") for i in range(4)]
        it = [0]

        def copy_call():
            abi.kv_cache_copy_blocks(maps[it[0] % 4], kc, vc)
            it[0] += 1

        ms = time_calls(copy_call, 20)
        moved = 2 * 2 * npairs * Hkv * 16 * D * 2
        rows["copy_blocks"] = hbm_row(moved, ms, "K and V blocks read + written")
        rows["copy_blocks"]["workload"] = f"{npairs} block pairs of {Hkv} kv heads x 16 tokens x {D} bf16, K and V"
        del kc, vc, maps

    # New-token slot write of the B=32 layer (32 tokens, 2 kv heads, f16).
    if want("kv_slot_write"):
        w = workloads.generate(SECONDARY)
        k, v, _ = gpu_pool(w, with_new_tokens=False)
        nk, nv = to_dev(w.new_k, w.spec.kv_dtype), to_dev(w.new_v, w.spec.kv_dtype)
        slots = torch.from_numpy(w.new_slots).cuda()
        ms = time_calls(lambda: abi.kv_cache_write(nk, nv, slots, k, v), 50)
        rows["kv_slot_write"] = {"us": round(ms * 1e3, 2), "bound": "latency",
                                 "workload": f"{SECONDARY}: 32 new tokens x 2 kv heads x 128, f16"}
    return rows


def read_ceiling(gib: int = 4, calls: int = 10) -> dict:
    """Read bandwidth this GPU sustains: pkv_read_bandwidth_probe (16-byte
    non-temporal loads, four in flight per thread) over a fresh buffer,
    timed with HIP events; the practical ceiling beside the published peak."""
    import torch
    from paged_kv_gqa_cache_amd import abi
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(4096, dtype=torch.int32, device="cuda")

    def call():
        abi.pkv_read_bandwidth_probe(buf, out)

    ms = time_calls(call, calls, warmup=2)
    del buf, out
    torch.cuda.empty_cache()
    return {"GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "calls": calls,
            "what": "pkv_read_bandwidth_probe: one read of a 4 GiB buffer, 16-byte non-temporal loads, "
                    "4 in flight per thread, 2 workgroups of 256 per CU; HIP events around 10 back-to-back calls"}


def latency_stats(ms_samples) -> dict:
    """Median, p20, p80 and minimum of the sampled kernel durations (us)."""
    import numpy as np
    a = np.asarray(ms_samples, dtype=np.float64) * 1e3
    return {"median": round(float(np.median(a)), 2), "p20": round(float(np.percentile(a, 20)), 2),
            "p80": round(float(np.percentile(a, 80)), 2), "min": round(float(a.min()), 2), "samples": int(a.size)}


def environment() -> dict:
    """What the run measured on: GPU, architecture, compute units, versions."""
    import torch
    props = torch.cuda.get_device_properties(0)
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""), "compute_units": props.multi_processor_count,
            "torch": torch.__version__, "hip": torch.version.hip}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--layers", type=int, default=4, help="layer pools rotated through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read probe (the measured read ceiling, context for the roofline)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-torch-reference", action="store_true",
                    help="skip timing the materialising PyTorch reference of the headline step")
    ap.add_argument("--only", default=None,
                    help="profiling aid: run only these comma-separated rows (" + ", ".join(ROW_NAMES) +
                         ") and print {\"rows\": ...}; no headline line")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other rows of the path (FP8, window, multi-token, quantise, append, copy, write)")
    ap.add_argument("--path", choices=["pair", "fused", "balanced", "step", "single"], default="balanced",
                    help="balanced: equal tile shares per compute unit + merge (default); pair: fixed "
                         "partitions + reduce; fused: the one-launch split with in-kernel merge; step: fused "
                         "with the new-token write; single: one pass")
    ap.add_argument("--secondary-path", choices=["pair", "fused", "balanced", "step"], default="step",
                    help="path for the B=32 line (its fastest: the fused step, write and attention in one launch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 256 MiB device to device (reference kernel for HBM counters)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.cpu_baseline_child:   # host only: never touches the GPU
        print(json.dumps(cpu_baseline_child(args.workload)), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_gqa_cache_amd import abi

    torch.cuda.set_device(0)
    digest = source_digest()
    if args.only:
        only = [x for x in args.only.split(",") if x]
        bad = [x for x in only if x not in ROW_NAMES]
        if bad:
            print(f"unknown rows {bad}; rows are {list(ROW_NAMES)}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"rows": measure_rows(args, only), "kernel_source_digest": digest}), flush=True)
        return
    if args.copy_calibration:
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
        del a

    r = Runner(args.workload, args.layers, args.partition_size, args.path)
    t_step, part_ms = r.run(args.steps, args.warmup)
    part_avg = sum(part_ms) / len(part_ms)
    t_graph, graph_err = r.run_graph_or_none(args.steps, args.warmup)   # the same steps replayed from a captured graph
    value = r.unique_bytes / t_step / 1e9
    achieved = r.unique_bytes / (part_avg * 1e-3) / 1e9
    s = r.spec

    b32 = None
    if not args.no_secondary and args.workload != SECONDARY:
        r2 = Runner(SECONDARY, args.layers, None, args.secondary_path)
        t2, p2 = r2.run(args.steps, args.warmup)
        k2 = sum(p2) / len(p2)
        t2g, _ = r2.run_graph_or_none(args.steps, args.warmup)
        b32 = {"workload": f"{SECONDARY}: {DESCRIPTIONS[SECONDARY]}", "path": args.secondary_path,
               "partition_size": None if args.secondary_path == "balanced" else r2.P,
               "us_per_step": round(t2 * 1e6, 2),
               "graph_us_per_step": None if t2g is None else round(t2g * 1e6, 2),
               "dominant_kernel_us": round(k2 * 1e3, 2),
               "kv_GBps": round(r2.unique_bytes / t2 / 1e9, 1),
               "seqs_layers_per_s": round(r2.spec.num_seqs / t2, 1),
               "roofline": {"bound": "hbm", "achieved": round(r2.unique_bytes / (k2 * 1e-3) / 1e9, 1),
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(r2.unique_bytes / (k2 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                            "bytes": r2.unique_bytes,
                            "bytes_are": "unique K/V bytes read per step (the 32 new tokens' writes excluded)",
                            "kernel": {"pair": "paged_decode_persistent, split partial mode",
                                       "fused": "paged_decode_persistent, split mode with in-kernel merge",
                                       "balanced": "paged_decode_cu_stream (per-compute-unit tile shares)",
                                       "step": "paged_decode_persistent, split mode with the new-token write "
                                               "and in-kernel merge"}[args.secondary_path]}}
        del r2

    torch_ref = None
    if not args.no_torch_reference:
        torch_ref = torch_materialising(r, 10)
        torch_ref["path_us_per_step"] = round(t_step * 1e6, 2)
        torch_ref["path_speedup"] = round(torch_ref["us"] / (t_step * 1e6), 1)

    rows = None
    if not args.no_rows and args.workload == HEADLINE:
        rows = measure_rows(args)

    line = {
        "metric": "paged GQA decode attn: KV-read HBM GB/s (% of peak) + us/step at B=32/128",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[s.kv_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, seeded context lengths and block tables)",
        "config": {
            "workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}",
            "num_seqs": s.num_seqs, "num_q_heads": s.num_q_heads, "num_kv_heads": s.num_kv_heads,
            "head_dim": s.head_dim, "block_size": 16,
            "partition_size": None if args.path == "balanced" else r.P,
            "layer_pools": args.layers, "mean_context": round(float(r.w.context_lens.mean()), 1),
            "kv_bytes_unique": r.unique_bytes, "kv_bytes_logical": r.logical_bytes,
        },
        "us_per_step": round(t_step * 1e6, 2),
        "graph_us_per_step": None if t_graph is None else round(t_graph * 1e6, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 1),
        "seqs_layers_per_s": round(s.num_seqs / t_step, 1),
        "logical_GBps": round(r.logical_bytes / t_step / 1e9, 1),
        "path": args.path,
        "dominant_kernel_us": round(part_avg * 1e3, 2),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": counters_traffic(args.workload, digest, args.path),
            "kernel": {"pair": "paged_decode_persistent, split partial mode",
                       "fused": "paged_decode_persistent, split mode with in-kernel merge",
                       "balanced": "paged_decode_cu_stream (per-compute-unit tile shares)",
                       "step": "paged_decode_persistent, split mode with the new-token write and in-kernel merge",
                       "single": "paged_decode_persistent, single-pass mode"}[args.path],
        },
        "b32": b32,
        "rows": rows,
        "torch_materialising": torch_ref,
        "kernel_source_digest": digest,
        "library": abi.version(),
    }
    line["dominant_kernel_us_stats"] = latency_stats(part_ms)
    line["environment"] = environment()
    if not args.no_read_ceiling:
        ceiling = read_ceiling()
        ceiling["kernel_frac_of_it"] = round(achieved / ceiling["GBps"], 4)
        line["read_ceiling"] = ceiling
    if graph_err:
        line["graph_error"] = graph_err
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
