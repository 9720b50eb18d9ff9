"""A seeded sweep over random small configurations, each against the float64
oracle at the 2e-3 gate: every decode path (one pass, partial + reduce, the
one-launch split, the balanced schedule; with a new token, the one-launch
step, which must also equal the write followed by the split bit for bit)
and the multi-token step.  Cache dtype, group size, head dim, kv heads,
batch size, length mix, sliding window, prefix sharing and partition size
are drawn per case, so combinations the hand-picked cases leave out are
checked as well."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_gqa_cache_amd import workloads
from tests.gpu_util import decode, gpu_pool
from tests.test_gpu_parity import (TOL, MODES, _announce, _prefill_gpu, _prefill_oracle, _same_bits, _step_pair,
                                   max_err, oracle_out)

pytestmark = pytest.mark.gpu

CASES = 32
BASE = "smollm2_360m"   # no new-token write, window or prefix of its own: every field is drawn


def _draw(i: int, multi_token: bool = False) -> dict:
    rng = np.random.default_rng(7100 + i)
    kv = str(rng.choice(["f32", "f16", "bf16", "e4m3"]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 5, 7, 8, 12, 16]))
    hi = int(rng.choice([16, 90, 600, 2500]))
    spec = dict(seed=7100 + i, num_seqs=int(rng.integers(1, 13)), num_q_heads=g * hkv, num_kv_heads=hkv,
                head_dim=int(rng.choice([64, 128])), kv_dtype=kv, q_dtype="f16" if kv == "e4m3" else kv,
                lengths=("uniform", 1, hi) if rng.random() < 0.6 else ("lognormal", max(2, hi // 5), 1.0, 1, hi),
                partition_size=int(rng.choice([16, 64, 256, 1024])), num_blocks=None)
    extra = rng.random()
    if extra < 0.25 and not multi_token:
        spec["window"] = int(rng.choice([1, 17, 100, 400]))
    elif extra < 0.45:
        spec.update(prefix_group=int(rng.integers(2, 5)), prefix_blocks=int(rng.integers(1, 8)))
    elif extra < 0.65 and kv != "e4m3" and not multi_token:
        spec["new_token_write"] = True
    if multi_token:
        spec["query_tokens"] = ("uniform", 1, int(rng.choice([1, 3, 16, 40])))
    return spec


@pytest.mark.parametrize("i", range(CASES))
def test_sweep_decode_paths(i):
    spec = _draw(i)
    _announce("sweep decode", i, spec)
    w = workloads.generate(BASE, **spec)
    want = oracle_out(w)
    pool = gpu_pool(w)
    for mode in MODES:
        assert max_err(decode(w, pool, mode), want) <= TOL, mode
    if w.spec.new_token_write:
        (out_a, ka, va), (out_b, kb, vb) = _step_pair(w, w.spec.partition_size, window=w.spec.window)
        assert torch.equal(out_a, out_b) and _same_bits(ka, kb) and _same_bits(va, vb)   # the pools hold NaN
        assert max_err(out_b, want) <= TOL


@pytest.mark.parametrize("i", range(CASES))
def test_sweep_multi_token(i):
    spec = _draw(i, multi_token=True)
    P = (0, 64, 256)[i % 3]
    _announce("sweep multi-token", i, spec, P)
    w = workloads.generate(BASE, **spec)
    assert max_err(_prefill_gpu(w, gpu_pool(w), P), _prefill_oracle(w)) <= TOL
