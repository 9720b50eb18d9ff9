"""GPU parity: the HIP library against the float64 oracle, element by element,
on the same seeded inputs.  Gate: max |GPU - oracle| <= 2e-3 on an fp32
output (FP8: against the oracle run on the same dequantised values); integer
and byte work (slot write, E4M3 codes and scales) bit-exact."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import paged_attention as ref
from paged_kv_gqa_cache_amd import workloads
from tests.gpu_util import OUT_DT, decode, gpu_pool, inputs, to_dev, to_raw
from tests.helpers import oracle_pool

pytestmark = pytest.mark.gpu

TOL = 2e-3

# Reduced variants: several blocks per sequence, ragged last blocks, sizes the
# oracle finishes in about a second.
REDUCED = {
    "tiny": dict(),
    "smollm2_360m": dict(num_seqs=5, lengths=("uniform", 1, 700)),
    "qwen25_1p5b": dict(num_seqs=4, lengths=("uniform", 1, 900)),
    "qwen25_7b_prefix": dict(num_seqs=16, lengths=("lognormal", 300, 1.0, 16, 3000)),
    "qwen25_7b_fp8": dict(num_seqs=3, lengths=("uniform", 1, 700)),
    "gemma_sliding": dict(num_seqs=6, lengths=("uniform", 1, 900), window=200),
}
NAMES = list(REDUCED)


def oracle_out(w, pool=None):
    k, v, sc = pool if pool is not None else oracle_pool(w)
    return ref.decode_attention(w.q, w.spec.q_dtype, k, v, w.spec.kv_dtype, w.block_tables,
                                w.context_lens, w.scale, sc, window=w.spec.window)


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - want))) if want.size else 0.0


def _announce(*what):
    print("case:", *what, flush=True)


MODES = ["single", "split", "fused", "balanced"]


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("mode", MODES)
def test_decode_matches_oracle(name, mode):
    _announce(name, mode)
    w = workloads.generate(name, **REDUCED[name])
    want = oracle_out(w)
    got = decode(w, gpu_pool(w), mode)
    assert max_err(got, want) <= TOL


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(num_q_heads=4, num_kv_heads=4, num_seqs=3)),                 # G = 1 (MHA)
    ("tiny", dict(num_q_heads=16, num_kv_heads=1, num_seqs=3)),                # G = 16 (MQA)
    ("smollm2_360m", dict(num_seqs=3, head_dim=128, lengths=("uniform", 1, 300))),
    ("qwen25_7b_prefix", dict(num_seqs=9, head_dim=64, lengths=("uniform", 1, 600))),
    ("qwen25_7b_fp8", dict(num_seqs=3, head_dim=64, lengths=("uniform", 1, 500))),
    ("qwen25_1p5b", dict(num_seqs=2, lengths=("uniform", 1, 16))),             # one block or less
])
@pytest.mark.parametrize("mode", MODES)
def test_decode_shape_variants(name, kw, mode):
    _announce(name, kw, mode)
    w = workloads.generate(name, **kw)
    assert max_err(decode(w, gpu_pool(w), mode, partition_size=64), oracle_out(w)) <= TOL


@pytest.mark.parametrize("mode", MODES)
def test_longest_context(mode):
    """Two sequences at the 32768-token clip of the lognormal workload:
    2048 blocks each, many 64-block id chunks per wave."""
    _announce("longest", mode)
    w = workloads.generate("qwen25_7b_prefix", num_seqs=2, lengths=("fixed", 32768), prefix_group=0)
    assert max_err(decode(w, gpu_pool(w), mode), oracle_out(w)) <= TOL


@pytest.mark.parametrize("name", ["tiny", "qwen25_1p5b", "smollm2_360m", "qwen25_7b_prefix"])
def test_kv_cache_write_is_bit_exact(name):
    _announce("write", name)
    w = workloads.generate(name, **REDUCED[name])
    k_o, v_o, _ = oracle_pool(w)
    k_g, v_g, _ = gpu_pool(w)
    torch.cuda.synchronize()
    assert np.array_equal(to_raw(k_g, w.spec.kv_dtype), k_o)
    assert np.array_equal(to_raw(v_g, w.spec.kv_dtype), v_o)


@pytest.mark.parametrize("kw", [dict(num_seqs=3, lengths=("uniform", 1, 700)),
                                dict(num_seqs=2, lengths=("uniform", 1, 300), head_dim=64),
                                # 3 kv heads, 137 blocks: 822 tiles leave two idle waves in the last workgroup
                                dict(num_seqs=4, lengths=("uniform", 1, 900), num_q_heads=6, num_kv_heads=3)])
def test_quantize_e4m3_is_bit_exact(kw):
    _announce("quantize", kw)
    w = workloads.generate("qwen25_7b_fp8", **kw)
    k_o, v_o, s_o = oracle_pool(w)
    k_g, v_g, s_g = gpu_pool(w)
    torch.cuda.synchronize()
    assert np.array_equal(to_raw(k_g, "e4m3"), k_o)
    assert np.array_equal(to_raw(v_g, "e4m3"), v_o)
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


def test_quantize_e4m3_rounding_boundaries():
    """Every E4M3 value, every midpoint between neighbouring values and the
    fp32 numbers on either side of it, both signs, signed zeros and
    subnormal quotients.  Each (block, kv head) tile holds a 448, so its
    scale is exactly 1 and the quotients are the crafted values themselves:
    the codes then test the encoder's rounding (ties to even) alone."""
    from oracle import e4m3
    from paged_kv_gqa_cache_amd import abi
    _announce("quantize rounding boundaries")
    pos = np.array([e4m3.decode_value(c) for c in range(0x7F)], dtype=np.float64)   # 0 .. 448
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)                          # exact in fp32
    vals = np.concatenate([pos.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(0)),
                           np.float32([2.0 ** -149, 2.0 ** -126, 2.0 ** -10, 3 * 2.0 ** -11, 0.0])])
    vals = np.concatenate([vals, -vals])
    n, hkv, d, nb = 6, 2, 128, 9
    xk = np.resize(vals, n * 16 * hkv * d).astype(np.float32).reshape(n, 16, hkv, d)
    xv = np.resize(vals[::-1], n * 16 * hkv * d).astype(np.float32).reshape(n, 16, hkv, d)
    xk[:, 0, :, 0] = 448.0
    xv[:, 0, :, 5] = -448.0
    ids = np.array([5, 0, 3, 8, 1, 2], dtype=np.int32)
    valid = np.array([16, 16, 16, 16, 16, 11], dtype=np.int32)
    k_o, v_o = ref.new_pool(nb, hkv, d, "e4m3")
    s_o = np.ones((2, nb, hkv), dtype=np.float32)
    ref.kv_cache_write_e4m3_blocks(k_o, v_o, s_o, xk, xv, ids, valid)
    assert np.all(s_o[:, ids] == 1.0)
    k = torch.full((nb, hkv, 16 * d), 0x7F, dtype=torch.uint8, device="cuda")
    v = torch.full_like(k, 0x7F)
    sc = torch.ones((2, nb, hkv), dtype=torch.float32, device="cuda")
    abi.kv_cache_quantize_e4m3(torch.from_numpy(xk).cuda(), torch.from_numpy(xv).cuda(),
                               torch.from_numpy(ids).cuda(), torch.from_numpy(valid).cuda(), k, v, sc)
    torch.cuda.synchronize()
    assert np.array_equal(k.cpu().numpy(), k_o)
    assert np.array_equal(v.cpu().numpy(), v_o)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


@pytest.mark.parametrize("hkv,d", [(4, 128), (3, 64)])
def test_quantize_e4m3_valid_token_edge_cases(hkv, d):
    """valid_tokens of 0, negative, 1, 15, 16 and above 16: the read window
    of each (block, kv head) tile ends at its last valid row, so an empty
    block reads nothing (codes 0, scale 1) and counts past 16 read all 16."""
    from paged_kv_gqa_cache_amd import abi
    _announce("quantize valid edges", hkv, d)
    rng = np.random.default_rng(23)
    valid = np.array([0, -3, 1, 15, 16, 40, 7, 0], dtype=np.int32)
    n, nb = len(valid), 11
    xk = rng.standard_normal((n, 16, hkv, d)).astype(np.float32) * 3
    xv = rng.standard_normal((n, 16, hkv, d)).astype(np.float32)
    ids = np.array([10, 0, 4, 2, 9, 5, 1, 7], dtype=np.int32)
    k_o, v_o = ref.new_pool(nb, hkv, d, "e4m3")
    s_o = np.full((2, nb, hkv), 5.0, dtype=np.float32)
    ref.kv_cache_write_e4m3_blocks(k_o, v_o, s_o, xk, xv, ids, valid)
    k = torch.full((nb, hkv, 16 * d), 0x7F, dtype=torch.uint8, device="cuda")
    v = torch.full_like(k, 0x7F)
    sc = torch.full((2, nb, hkv), 5.0, dtype=torch.float32, device="cuda")
    abi.kv_cache_quantize_e4m3(torch.from_numpy(xk).cuda(), torch.from_numpy(xv).cuda(),
                               torch.from_numpy(ids).cuda(), torch.from_numpy(valid).cuda(), k, v, sc)
    torch.cuda.synchronize()
    assert np.all(s_o[:, ids[valid <= 0]] == 1.0) and np.all(k_o[ids[valid <= 0]] == 0)
    assert np.array_equal(k.cpu().numpy(), k_o)
    assert np.array_equal(v.cpu().numpy(), v_o)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


def test_fp8_attention_on_oracle_codes():
    """The FP8 kernel fed the oracle's own codes and scales (uploaded)."""
    _announce("fp8 oracle codes")
    w = workloads.generate("qwen25_7b_fp8", num_seqs=3, lengths=("uniform", 100, 700))
    k_o, v_o, s_o = oracle_pool(w)
    pool = (to_dev(k_o, "e4m3"), to_dev(v_o, "e4m3"), torch.from_numpy(s_o).cuda())
    want = oracle_out(w, (k_o, v_o, s_o))
    for mode in ("single", "split", "balanced"):
        assert max_err(decode(w, pool, mode), want) <= TOL


@pytest.mark.parametrize("P", [16, 64, 256, 2048])
def test_partials_match_oracle_partials(P):
    _announce("partials", P)
    w = workloads.generate("qwen25_7b_prefix", num_seqs=6, lengths=("uniform", 1, 2500))
    k, v, sc = oracle_pool(w)
    from paged_kv_gqa_cache_amd import abi
    pool = gpu_pool(w)
    q, tables, lens = inputs(w)
    tmp_out, tmp_lse = abi.alloc_partials(q, tables.shape[1], P)
    tmp_out.fill_(float("nan"))
    tmp_lse.fill_(float("nan"))
    abi.paged_decode_attention_partial(q, pool[0], pool[1], tables, lens, w.scale, None, P, tmp_out, tmp_lse)
    S = tmp_out.shape[2]
    o_ref, lse_ref = ref.decode_partials(w.q, "bf16", k, v, "bf16", w.block_tables, w.context_lens,
                                         w.scale, P, S)
    o_g, lse_g = tmp_out.cpu().numpy(), tmp_lse.cpu().numpy()
    for b, L in enumerate(w.context_lens):
        n = ref.num_partitions(L, P)
        assert np.max(np.abs(o_g[b, :, :n] - o_ref[b, :, :n])) <= TOL
        assert np.max(np.abs(lse_g[b, :, :n] - lse_ref[b, :, :n])) <= TOL
        assert np.all(np.isnan(o_g[b, :, n:])) and np.all(np.isnan(lse_g[b, :, n:])), "wrote past its partitions"
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    abi.paged_decode_attention_reduce(tmp_out, tmp_lse, lens, P, out, tables.shape[1])
    assert max_err(out, ref.merge_partials(o_ref, lse_ref, w.context_lens, P)) <= TOL


@pytest.mark.parametrize("mode", ["split", "fused"])
def test_partition_sizes_agree(mode):
    _announce("partition sweep", mode)
    w = workloads.generate("qwen25_1p5b", num_seqs=4, lengths=("uniform", 1, 3000))
    want = oracle_out(w)
    pool = gpu_pool(w)
    for P in (16, 64, 512, 2048, 16 * w.max_blocks_per_seq):
        assert max_err(decode(w, pool, mode, partition_size=P), want) <= TOL, P


@pytest.mark.parametrize("P", [16, 64, 512])
def test_fused_split_equals_pair_bitwise_on_every_run(P):
    """The in-kernel merge reads partials written by other workgroups of the
    same launch; a stale or early read would change bits.  Many runs on a
    batch with many multi-partition sequences must all equal the two-kernel
    result exactly."""
    _announce("fused vs pair", P)
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate("qwen25_7b_prefix", num_seqs=40, lengths=("uniform", 1, 4000))
    k, v, _ = gpu_pool(w)
    q, tables, lens = inputs(w)
    ref_out = decode(w, (k, v, None), "split", partition_size=P)
    ws = abi.split_workspace(q, k, tables, P)
    outs = [abi.paged_decode_attention_split(q, k, v, tables, lens, w.scale, None, P, ws) for _ in range(25)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref_out), f"run {i} differs"


def test_fused_split_reuses_its_workspace():
    """Back-to-back calls on one workspace give the same bits, and leave the
    counter words zero; a smaller batch after a larger one works too."""
    _announce("fused workspace reuse")
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate("qwen25_7b_prefix", num_seqs=24, lengths=("uniform", 1, 3000))
    k, v, _ = gpu_pool(w)
    q, tables, lens = inputs(w)
    P = 256
    ws = abi.split_workspace(q, k, tables, P)
    outs = [abi.paged_decode_attention_split(q, k, v, tables, lens, w.scale, None, P, ws) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    assert max_err(outs[0], oracle_out(w)) <= TOL
    counters = ws[: 24 * w.spec.num_kv_heads * 4].view(torch.int32)
    assert torch.all(counters == 0)
    small_out = abi.paged_decode_attention_split(q[:5].contiguous(), k, v, tables[:5].contiguous(),
                                                 lens[:5].contiguous(), w.scale, None, P, ws)
    assert torch.equal(small_out, outs[0][:5])


@pytest.mark.parametrize("name", ["qwen25_1p5b", "qwen25_7b_prefix", "qwen25_7b_fp8"])
@pytest.mark.parametrize("mode", MODES)
def test_out_in_query_dtype_is_fp32_out_rounded(name, mode):
    _announce("out dtype", name, mode)
    w = workloads.generate(name, **REDUCED[name])
    pool = gpu_pool(w)
    odt = OUT_DT[w.spec.q_dtype]
    o32 = decode(w, pool, mode, out_dtype=torch.float32)
    o16 = decode(w, pool, mode, out_dtype=odt)
    rounded = o32.to(odt)
    # within one unit in the last place of the 16-bit type
    # (f16 values below 2^-14 are subnormal: their spacing is 2^-24)
    ulp = (rounded.float().abs() * (2.0 ** -10 if odt == torch.float16 else 2.0 ** -7)).clamp_min(
        2.0 ** -24 if odt == torch.float16 else 1e-30)
    if mode == "balanced":
        # Two calls of the balanced schedule may sum in different orders
        # (waves claim tiles at run time): the 16-bit output is its own
        # call's fp32 result rounded to nearest, so it lies within half an
        # ulp of that, and the two calls' fp32 results differ by an fp32
        # summation-order error (absolute: ~1e-7 on these unit-scale
        # values, also where the output itself is near zero).
        assert torch.all((o16.float() - o32).abs() <= 0.5 * ulp + 2e-6)
    else:
        assert torch.all((o16.float() - rounded.float()).abs() <= ulp)


@pytest.mark.parametrize("name", ["tiny", "qwen25_1p5b"])
@pytest.mark.parametrize("mode", MODES)
def test_context_len_one_returns_the_new_v(name, mode):
    _announce("L=1", name, mode)
    w = workloads.generate(name, num_seqs=5, lengths=("fixed", 1))
    got = decode(w, gpu_pool(w), mode).cpu().numpy()
    s = w.spec
    v = ref.to_f64(w.new_v, s.kv_dtype)
    for b in range(s.num_seqs):
        for i in range(s.num_q_heads):
            assert np.array_equal(got[b, i].astype(np.float64), v[b, i // s.group_size])


def test_block_relabelling_is_bitwise_invariant():
    _announce("relabel")
    w = workloads.generate("qwen25_7b_prefix", num_seqs=12, lengths=("uniform", 1, 800))
    k, v, _ = gpu_pool(w)
    base = decode(w, (k, v, None), "split")
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.num_blocks)).cuda()
    k2, v2 = torch.empty_like(k), torch.empty_like(v)
    k2[perm], v2[perm] = k, v
    t = torch.from_numpy(w.block_tables).cuda().long()
    t2 = torch.where(t >= 0, perm[t.clamp_min(0)], t).int()
    out = decode(w, (k2, v2, None), "split", tables=t2)
    assert torch.equal(out, base)


def test_equal_queries_in_a_group_are_bitwise_equal():
    _announce("gqa equal")
    w = workloads.generate("qwen25_7b_prefix", num_seqs=6, lengths=("uniform", 1, 800))
    q, _, _ = inputs(w)
    G = w.spec.group_size
    q = q.view(q.shape[0], -1, G, q.shape[2])[:, :, :1].expand(-1, -1, G, -1).reshape(q.shape).contiguous()
    out = decode(w, gpu_pool(w), "split", q=q)
    o = out.view(out.shape[0], -1, G, out.shape[2])
    assert torch.equal(o, o[:, :, :1].expand_as(o))


@pytest.mark.parametrize("mode", MODES)
def test_empty_context_gives_zeros(mode):
    _announce("empty", mode)
    w = workloads.generate("qwen25_1p5b", num_seqs=4, lengths=("uniform", 20, 200))
    lens = torch.from_numpy(w.context_lens).cuda()
    lens[2] = 0
    got = decode(w, gpu_pool(w), mode, lens=lens)
    want = ref.decode_attention(w.q, "f16", *oracle_pool(w)[:2], "f16", w.block_tables,
                                lens.cpu().numpy(), w.scale)
    assert torch.all(got[2] == 0)
    assert max_err(got, want) <= TOL


# --------------------------------------------------------- sliding window ---

@pytest.mark.parametrize("W", [1, 16, 17, 100, 512])
@pytest.mark.parametrize("mode", MODES)
def test_sliding_window_matches_oracle(W, mode):
    """Windows shorter than, equal to a block, unaligned, and spanning
    partitions; blocks before each window hold NaN, so a read outside it
    would show."""
    _announce("window", W, mode)
    w = workloads.generate("gemma_sliding", num_seqs=5, lengths=("uniform", 1, 1500), window=W,
                           num_q_heads=16, num_kv_heads=4)
    assert max_err(decode(w, gpu_pool(w), mode, partition_size=64), oracle_out(w)) <= TOL


def test_sliding_window_partials_match_oracle_partials():
    _announce("window partials")
    from paged_kv_gqa_cache_amd import abi
    W, P = 300, 128
    w = workloads.generate("gemma_sliding", num_seqs=6, lengths=("uniform", 1, 1200), window=W)
    k, v, _ = oracle_pool(w)
    pool = gpu_pool(w)
    q, tables, lens = inputs(w)
    tmp_out, tmp_lse = abi.alloc_partials(q, tables.shape[1], P)
    tmp_out.fill_(float("nan"))
    tmp_lse.fill_(float("nan"))
    abi.paged_decode_attention_partial(q, pool[0], pool[1], tables, lens, w.scale, None, P, tmp_out, tmp_lse,
                                       window=W)
    S = tmp_out.shape[2]
    o_ref, lse_ref = ref.decode_partials(w.q, "bf16", k, v, "bf16", w.block_tables, w.context_lens,
                                         w.scale, P, S, window=W)
    o_g, lse_g = tmp_out.cpu().numpy(), tmp_lse.cpu().numpy()
    for b, L in enumerate(w.context_lens):
        n = ref.num_partitions(L, P, W)
        assert np.max(np.abs(o_g[b, :, :n] - o_ref[b, :, :n])) <= TOL
        assert np.max(np.abs(lse_g[b, :, :n] - lse_ref[b, :, :n])) <= TOL
        assert np.all(np.isnan(o_g[b, :, n:])) and np.all(np.isnan(lse_g[b, :, n:])), "wrote past its partitions"
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    abi.paged_decode_attention_reduce(tmp_out, tmp_lse, lens, P, out, tables.shape[1], window=W)
    assert max_err(out, ref.merge_partials(o_ref, lse_ref, w.context_lens, P, W)) <= TOL


def test_window_wider_than_every_context_equals_no_window_bitwise():
    _announce("window wide")
    w = workloads.generate("qwen25_1p5b", num_seqs=4, lengths=("uniform", 1, 600))
    pool = gpu_pool(w)
    base = decode(w, pool, "split")
    from paged_kv_gqa_cache_amd import abi
    q, tables, lens = inputs(w)
    P = w.spec.partition_size
    tmp_out, tmp_lse = abi.alloc_partials(q, tables.shape[1], P)
    abi.paged_decode_attention_partial(q, pool[0], pool[1], tables, lens, w.scale, None, P, tmp_out, tmp_lse,
                                       window=100000)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    abi.paged_decode_attention_reduce(tmp_out, tmp_lse, lens, P, out, tables.shape[1], window=100000)
    assert torch.equal(out, base)


# ------------------------------------------------------- balanced schedule ---

@pytest.mark.parametrize("lengths", [("uniform", 1, 40), ("lognormal", 200, 1.5, 1, 6000)])
def test_balanced_with_many_sequences(lengths):
    """Up to the 2048-sequence limit: many items per worker (short contexts)
    or items cut between several workers (long ones), every output row
    against the oracle."""
    _announce("balanced many", lengths)
    w = workloads.generate("smollm2_360m", num_seqs=2048 if lengths[0] == "uniform" else 300,
                           lengths=lengths)
    assert max_err(decode(w, gpu_pool(w), "balanced"), oracle_out(w)) <= TOL


@pytest.mark.parametrize("name", ["tiny", "smollm2_360m", "qwen25_7b_prefix", "qwen25_7b_fp8"])
def test_balanced_partial_then_reduce_is_the_one_call(name):
    """The two launches of the balanced schedule called apart (as the
    benchmark times the first) give the one-call result: within fp32
    summation-order differences of it, and within the oracle's tolerance."""
    _announce("balanced partial + reduce", name)
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate(name, **REDUCED.get(name, {}))
    pool = gpu_pool(w)
    k, v, sc = pool
    q, tables, lens = inputs(w)
    ws = abi.balanced_workspace(q, k, tables)
    one = abi.paged_decode_attention_balanced(q, k, v, tables, lens, w.scale, sc, ws)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    abi.paged_decode_attention_balanced_partial(q, k, v, tables, lens, w.scale, sc, ws, out)
    abi.paged_decode_attention_balanced_reduce(q, k, tables, ws, out)
    torch.cuda.synchronize()
    assert float((out - one).abs().max()) <= 1e-5
    assert max_err(out, oracle_out(w)) <= TOL


def test_balanced_runs_agree_and_reuse_their_workspace():
    """Ten calls on one workspace: each within the oracle's tolerance, and
    all within fp32 summation-order differences of each other (the waves of
    a compute unit claim tiles at run time, so the order is not fixed)."""
    _announce("balanced reuse")
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate("qwen25_7b_prefix", num_seqs=40, lengths=("lognormal", 600, 1.0, 1, 5000))
    k, v, _ = gpu_pool(w)
    q, tables, lens = inputs(w)
    ws = abi.balanced_workspace(q, k, tables)
    outs = [abi.paged_decode_attention_balanced(q, k, v, tables, lens, w.scale, None, ws) for _ in range(10)]
    torch.cuda.synchronize()
    want = oracle_out(w)
    for i, o in enumerate(outs):
        assert float((o - outs[0]).abs().max()) <= 1e-5, f"run {i} differs"
        assert max_err(o, want) <= TOL
    # a smaller batch on the same workspace
    small = abi.paged_decode_attention_balanced(q[:7].contiguous(), k, v, tables[:7].contiguous(),
                                                lens[:7].contiguous(), w.scale, None, ws)
    sub = workloads.generate("qwen25_7b_prefix", num_seqs=40, lengths=("lognormal", 600, 1.0, 1, 5000))
    sub.q, sub.block_tables, sub.context_lens = sub.q[:7], sub.block_tables[:7], sub.context_lens[:7]
    assert max_err(small, oracle_out(sub)) <= TOL


@pytest.mark.parametrize("mode", ["single", "split", "fused"])
def test_more_sequences_than_the_persistent_tables_hold(mode):
    """2100 sequences (past the 2048 the persistent kernel's LDS tables hold):
    the one-workgroup-per-item kernel runs, and every row matches."""
    _announce("many sequences", mode)
    w = workloads.generate("smollm2_360m", num_seqs=2100, lengths=("uniform", 1, 60))
    assert max_err(decode(w, gpu_pool(w), mode, partition_size=32), oracle_out(w)) <= TOL


def test_decode_step_with_more_sequences_than_the_persistent_tables_hold():
    _announce("decode step many sequences")
    w = workloads.generate("qwen25_1p5b", num_seqs=2100, lengths=("uniform", 1, 60))
    (oa, ka, va), (ob, kb, vb) = _step_pair(w, 32)
    assert _same_bits(ka, kb) and _same_bits(va, vb) and torch.equal(oa, ob)
    assert max_err(ob, oracle_out(w)) <= TOL


def test_balanced_rejects_too_many_sequences():
    from paged_kv_gqa_cache_amd import abi
    q = torch.zeros(2049, 4, 64, dtype=torch.float16, device="cuda")
    k = torch.zeros(4, 1, 16 * 64, dtype=torch.float16, device="cuda")
    tables = torch.zeros(2049, 1, dtype=torch.int32, device="cuda")
    lens = torch.ones(2049, dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(abi.PkvError) as e:
        abi.paged_decode_attention_balanced(q, k, k, tables, lens, 0.125, None, ws)
    assert e.value.code == 2


# ------------------------------------------------------- full-size configs ---

FULL_SIZE = ["tiny", "smollm2_360m", "qwen25_1p5b", "qwen25_7b_prefix", "qwen25_7b_fp8", "gemma_sliding"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL_SIZE)
def test_full_size_every_sequence(name):
    """Each workload at its full size: every sequence, query head and dim of
    every decode mode (the split pair at the workload's benchmarked partition
    size, the one-launch split, the balanced schedule and the single pass)
    against the oracle on the whole batch."""
    _announce("full", name)
    from tests.helpers import host_workers
    w = workloads.generate(name)
    want = oracle_out(w, oracle_pool(w, workers=host_workers()))
    pool = gpu_pool(w)
    for mode in MODES:
        _announce("full", name, mode)
        assert max_err(decode(w, pool, mode), want) <= TOL, mode


# ------------------------------------------------------------ block copy ---

@pytest.mark.parametrize("name", ["tiny", "qwen25_7b_prefix", "qwen25_7b_fp8", "smollm2_360m"])
def test_copy_blocks_is_bit_exact(name):
    """Pairs from used blocks into free ones (and one pair naming a block past
    the pool, which is skipped): every byte of the pool, and the E4M3 scales,
    equal the oracle's copy."""
    _announce("copy blocks", name)
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate(name, **REDUCED[name]) if name != "tiny" else workloads.generate(name)
    k_o, v_o, s_o = oracle_pool(w)
    k_g, v_g, s_g = gpu_pool(w)
    used = sorted(set(int(x) for x in w.fill_blocks))
    free = [i for i in range(w.num_blocks) if i not in set(used)]
    n = min(len(used), len(free), 7)
    pairs = [(used[i], free[i]) for i in range(n)]
    ref.copy_blocks(k_o, v_o, pairs, s_o)
    mapping = torch.tensor(pairs + [(used[0], w.num_blocks + 3)], dtype=torch.int32, device="cuda")
    abi.kv_cache_copy_blocks(mapping, k_g, v_g, s_g)
    torch.cuda.synchronize()
    kv = w.spec.kv_dtype
    assert np.array_equal(to_raw(k_g, kv), k_o) and np.array_equal(to_raw(v_g, kv), v_o)
    if s_o is not None:
        assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


def test_forked_beam_after_copy_and_write_matches_oracle():
    """Copy-on-write fork on the GPU: each sequence's partly filled last block
    is copied for a second beam, each beam gets a different next token, and
    both beams decode as the oracle says."""
    _announce("beam fork")
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate("qwen25_1p5b", num_seqs=4, lengths=("uniform", 20, 300))
    k_o, v_o, _ = oracle_pool(w)
    k_g, v_g, _ = gpu_pool(w)
    B = w.spec.num_seqs
    used = set(int(x) for x in w.block_tables.ravel() if x >= 0)
    free = [i for i in range(w.num_blocks) if i not in used][:B]
    L = w.context_lens.astype(np.int64)
    last = w.block_tables[np.arange(B), (L - 1) // 16].astype(np.int64)
    # Fork only where the new token lands in the same block as the last one.
    pairs = [(int(last[b]), free[b]) for b in range(B)]
    ref.copy_blocks(k_o, v_o, pairs)
    abi.kv_cache_copy_blocks(torch.tensor(pairs, dtype=torch.int32, device="cuda"), k_g, v_g)
    tables = np.concatenate([w.block_tables, w.block_tables], axis=0)
    for b in range(B):
        tables[B + b, (L[b] - 1) // 16] = free[b]
    # the next token of every beam: position L, slot in the beam's own block (a new block if L % 16 == 0)
    rng = np.random.default_rng(11)
    Hkv, D = w.spec.num_kv_heads, w.spec.head_dim
    extra = [i for i in range(w.num_blocks) if i not in used and i not in free]
    slots = []
    for r in range(2 * B):
        b = r % B
        pos = int(L[b])
        if pos % 16 == 0:
            blk = extra.pop(0)
            tables_row_len = tables.shape[1]
            if pos // 16 >= tables_row_len:
                tables = np.concatenate([tables, np.full((2 * B, 1), -1, np.int32)], axis=1)
            tables[r, pos // 16] = blk
        else:
            blk = int(tables[r, pos // 16])
        slots.append(blk * 16 + pos % 16)
    slots = np.array(slots, np.int64)
    nk = workloads.round_to(rng.standard_normal((2 * B, Hkv, D), dtype=np.float32), "f16")
    nv = workloads.round_to(rng.standard_normal((2 * B, Hkv, D), dtype=np.float32), "f16")
    ref.kv_cache_write(k_o, v_o, nk, nv, slots, "f16")
    abi.kv_cache_write(to_dev(nk, "f16"), to_dev(nv, "f16"), torch.from_numpy(slots).cuda(), k_g, v_g)
    lens = np.concatenate([L + 1, L + 1]).astype(np.int32)
    q = np.concatenate([w.q, w.q], axis=0)
    want = ref.decode_attention(q, "f16", k_o, v_o, "f16", tables, lens, w.scale)
    got = abi.paged_decode_attention(to_dev(q, "f16"), k_g, v_g, torch.from_numpy(tables).cuda(),
                                     torch.from_numpy(lens).cuda(), w.scale)
    assert max_err(got, want) <= TOL
    assert not np.allclose(want[:B], want[B:])   # the beams did diverge


# --------------------------------------------------- E4M3 quantise-on-append ---

def _append_case(seed, mag):
    """The FP8 pool plus one new token per sequence at position L (scaled by
    ``mag`` so some (block, head) scales must grow); sequences whose next
    token would open a block get one from the free list."""
    w = workloads.generate("qwen25_7b_fp8", num_seqs=5, lengths=("uniform", 1, 300))
    B, Hkv, D = 5, w.spec.num_kv_heads, w.spec.head_dim
    L = w.context_lens.astype(np.int64)
    used = set(int(x) for x in w.block_tables.ravel() if x >= 0)
    free = [i for i in range(w.num_blocks) if i not in used]
    tables = np.concatenate([w.block_tables, np.full((B, 1), -1, np.int32)], axis=1)
    slots = []
    for b in range(B):
        j = int(L[b]) // 16
        if tables[b, j] < 0:
            tables[b, j] = free.pop(0)
        slots.append(int(tables[b, j]) * 16 + int(L[b]) % 16)
    rng = np.random.default_rng(seed)
    kn = (rng.standard_normal((B, Hkv, D), dtype=np.float32) * np.float32(mag)).astype(np.float32)
    vn = (rng.standard_normal((B, Hkv, D), dtype=np.float32) * np.float32(mag)).astype(np.float32)
    return w, tables, np.array(slots, np.int64), kn, vn


@pytest.mark.parametrize("seed,mag", [(1, 1.0), (2, 4.0), (3, 0.25)])
def test_append_e4m3_is_bit_exact(seed, mag):
    _announce("append e4m3", seed, mag)
    from paged_kv_gqa_cache_amd import abi
    w, tables, slots, kn, vn = _append_case(seed, mag)
    k_o, v_o, s_o = oracle_pool(w)
    k_g, v_g, s_g = gpu_pool(w)
    ref.kv_cache_append_e4m3(k_o, v_o, s_o, kn, vn, slots)
    abi.kv_cache_append_e4m3(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                             torch.from_numpy(slots).cuda(), k_g, v_g, s_g)
    torch.cuda.synchronize()
    assert np.array_equal(to_raw(k_g, "e4m3"), k_o) and np.array_equal(to_raw(v_g, "e4m3"), v_o)
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    # and attention over the appended tokens agrees with the oracle
    lens = (w.context_lens + 1).astype(np.int32)
    want = ref.decode_attention(w.q, "f16", k_o, v_o, "e4m3", tables, lens, w.scale, s_o)
    got = abi.paged_decode_attention(to_dev(w.q, "f16"), k_g, v_g, torch.from_numpy(tables).cuda(),
                                     torch.from_numpy(lens).cuda(), w.scale, s_g)
    assert max_err(got, want) <= TOL


def test_append_e4m3_fills_a_block_token_by_token():
    """Sixteen appends into fresh blocks, magnitudes rising so the scale grows
    and earlier codes are re-encoded again and again; bit-exact each step."""
    _announce("append e4m3 fill")
    from paged_kv_gqa_cache_amd import abi
    Hkv, D, NB = 4, 128, 8
    k_o = np.full((NB, Hkv, 16 * D), 0x7F, np.uint8)
    v_o = k_o.copy()
    s_o = np.ones((2, NB, Hkv), np.float32)
    k_g, v_g = torch.from_numpy(k_o.copy()).cuda(), torch.from_numpy(v_o.copy()).cuda()
    s_g = torch.from_numpy(s_o.copy()).cuda()
    rng = np.random.default_rng(7)
    blocks = np.array([5, 2, 7], np.int64)
    for t in range(16):
        growth = np.float32(1.0 + 0.4 * t)
        kn = (rng.standard_normal((3, Hkv, D), dtype=np.float32) * growth).astype(np.float32)
        vn = (rng.standard_normal((3, Hkv, D), dtype=np.float32) * growth).astype(np.float32)
        slots = blocks * 16 + t
        ref.kv_cache_append_e4m3(k_o, v_o, s_o, kn, vn, slots)
        abi.kv_cache_append_e4m3(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                                 torch.from_numpy(slots).cuda(), k_g, v_g, s_g)
        torch.cuda.synchronize()
        assert np.array_equal(k_g.cpu().numpy(), k_o) and np.array_equal(v_g.cpu().numpy(), v_o), t
        assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), t


@pytest.mark.parametrize("lead_zeros", [1, 5])
def test_append_e4m3_after_zero_tokens_matches_oracle_and_bulk_scale(lead_zeros):
    """A block whose first tokens are all zero (scale 1, codes 0) and whose
    later tokens are not: bit-exact against the oracle after every append,
    and at the end the scale equals the bulk quantiser's fp32(amax / 448)
    over the same tokens (a later token below 448 must not be stuck at 1)."""
    _announce("append e4m3 after zeros", lead_zeros)
    from oracle import e4m3
    from paged_kv_gqa_cache_amd import abi
    Hkv, D, NB, n = 2, 128, 6, 12
    k_o = np.full((NB, Hkv, 16 * D), 0x7F, np.uint8)
    v_o = k_o.copy()
    s_o = np.ones((2, NB, Hkv), np.float32)
    k_g, v_g = torch.from_numpy(k_o.copy()).cuda(), torch.from_numpy(v_o.copy()).cuda()
    s_g = torch.from_numpy(s_o.copy()).cuda()
    rng = np.random.default_rng(lead_zeros)
    blocks = np.array([4, 1], np.int64)
    xs_k = (rng.standard_normal((n, 2, Hkv, D), dtype=np.float32) * np.float32(0.3)).astype(np.float32)
    xs_v = (rng.standard_normal((n, 2, Hkv, D), dtype=np.float32) * np.float32(0.3)).astype(np.float32)
    xs_k[:lead_zeros] = 0
    xs_v[:lead_zeros] = 0
    xs_k[:lead_zeros, :, 1, :3] = np.float32(-0.0)   # signed zeros still count as zero
    for t in range(n):
        slots = blocks * 16 + t
        ref.kv_cache_append_e4m3(k_o, v_o, s_o, xs_k[t], xs_v[t], slots)
        abi.kv_cache_append_e4m3(torch.from_numpy(xs_k[t]).cuda(), torch.from_numpy(xs_v[t]).cuda(),
                                 torch.from_numpy(slots).cuda(), k_g, v_g, s_g)
        torch.cuda.synchronize()
        assert np.array_equal(k_g.cpu().numpy(), k_o) and np.array_equal(v_g.cpu().numpy(), v_o), t
        assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), t
    for i, blk in enumerate(blocks):
        for which, xs in ((0, xs_k), (1, xs_v)):
            blk_vals = np.zeros((1, 16, Hkv, D), np.float32)
            blk_vals[0, :n] = xs[:, i]
            _, bulk = e4m3.quantize_blocks(blk_vals, np.array([n]))
            assert np.array_equal(s_g.cpu().numpy()[which, blk].view(np.uint32), bulk[0].view(np.uint32))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("spread", ["large_v", "mixed"])
def test_e4m3_decode_with_large_and_mixed_scales(mode, spread):
    """E4M3 pools whose V scales are far from the N(0,1) workloads': V values
    up to ~1000 (scales above 1, where P times the scale would leave f16's
    range without the running power of two), and per-block magnitudes
    spread over 10^-3 .. 10^3 in K and V (scales growing and shrinking
    along a sequence)."""
    _announce("e4m3 scales", spread, mode)
    w = workloads.generate("qwen25_7b_fp8", num_seqs=4, lengths=("uniform", 1, 700))
    kf = w.fill_k.view(np.float32).copy()
    vf = w.fill_v.view(np.float32).copy()
    if spread == "large_v":
        vf *= np.float32(250)
    else:
        rng = np.random.default_rng(5)
        fk = (10.0 ** rng.uniform(-3, 3, size=len(kf))).astype(np.float32)
        fv = (10.0 ** rng.uniform(-3, 3, size=len(vf))).astype(np.float32)
        kf *= np.float32(0.01) * fk[:, None, None, None]   # logits stay O(1..10)
        vf *= fv[:, None, None, None]
    w.fill_k, w.fill_v = kf.view(np.uint32), vf.view(np.uint32)
    pool_o = oracle_pool(w)
    want = oracle_out(w, pool_o)
    k_g, v_g, s_g = gpu_pool(w)
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), pool_o[2].view(np.uint32))
    got = decode(w, (k_g, v_g, s_g), mode, partition_size=64)
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    assert float(np.max(np.abs(g - want))) <= TOL


def test_fp8_path_error_against_unquantised_kv():
    """The FP8 row's quality figure: the GPU E4M3 path's mean absolute error
    against attention over the unquantised fp32 K/V.  The bench computes that
    reference in PyTorch float64 on the GPU; it must equal the oracle's
    (an f32 pool of the same values) to rounding, and the GPU path's error
    must sit within the quantisation-error model the oracle is pinned to."""
    _announce("fp8 mae")
    import math

    import bench
    from tests.helpers import oracle_pool_unquantised
    w = workloads.generate("qwen25_7b_fp8", num_seqs=4, lengths=("fixed", 512))
    k, v, _ = oracle_pool_unquantised(w)
    want32 = ref.decode_attention(w.q, "f16", k, v, "f32", w.block_tables, w.context_lens, w.scale)
    got_ref = bench.unquantised_reference(w).cpu().numpy()
    assert float(np.max(np.abs(got_ref - want32))) <= 1e-9
    got = decode(w, gpu_pool(w), "balanced").cpu().numpy().astype(np.float64)
    mae = float(np.mean(np.abs(got - want32)))
    model = 0.06 / math.sqrt(512)
    assert model / 5 < mae < 3 * model, mae


# ------------------------------------------------- multi-token (causal) step ---

def _prefill_oracle(w, pool=None):
    k, v, sc = pool if pool is not None else oracle_pool(w)
    return ref.prefill_attention(w.q, w.spec.q_dtype, k, v, w.spec.kv_dtype, w.block_tables, w.context_lens,
                                 w.query_start, w.scale, sc)


def _prefill_gpu(w, pool, P, out_dtype=torch.float32):
    from paged_kv_gqa_cache_amd import abi
    k, v, sc = pool
    q = to_dev(w.q, w.spec.q_dtype)
    return abi.paged_prefill_attention(q, k, v, torch.from_numpy(w.block_tables).cuda(),
                                       torch.from_numpy(w.context_lens).cuda(),
                                       torch.from_numpy(w.query_start).cuda(), w.scale, sc, partition_size=P,
                                       out_dtype=out_dtype)


PREFILL_SHAPES = [
    dict(),                                                                  # G = 7: 2 tokens per pack
    dict(num_q_heads=16, num_kv_heads=4, head_dim=64),                      # G = 4: 4 tokens
    dict(num_q_heads=4, num_kv_heads=4),                                    # G = 1: 16 tokens
    dict(num_q_heads=32, num_kv_heads=2),                                   # G = 16: 1 token
    dict(num_q_heads=8, num_kv_heads=4, q_dtype="f16", kv_dtype="f16"),     # G = 2
    dict(q_dtype="f32", kv_dtype="f32", head_dim=64, num_q_heads=12, num_kv_heads=4),
    dict(q_dtype="f16", kv_dtype="e4m3"),
]


@pytest.mark.parametrize("P", [0, 64, 512])
@pytest.mark.parametrize("kw", PREFILL_SHAPES)
def test_prefill_matches_oracle(kw, P):
    _announce("prefill", kw, P)
    w = workloads.generate("qwen25_7b_chunk", num_seqs=5, lengths=("uniform", 1, 700),
                           query_tokens=("uniform", 1, 40), **kw)
    assert max_err(_prefill_gpu(w, gpu_pool(w), P), _prefill_oracle(w)) <= TOL


@pytest.mark.parametrize("rows", [(16, 48), (1, 6)])
@pytest.mark.parametrize("kw", [dict(), dict(num_q_heads=8, num_kv_heads=4, q_dtype="f16", kv_dtype="f16"),
                                dict(num_q_heads=32, num_kv_heads=2), dict(num_q_heads=4, num_kv_heads=4)])
def test_prefill_both_tile_paths(kw, rows):
    """16-bit caches take tiles in pairs (PV on the K = 32 form) when the
    sequences average 16 or more query rows, one at a time otherwise: each
    path against the oracle, with odd and even tile counts per wave."""
    _announce("prefill tile paths", kw, rows)
    w = workloads.generate("qwen25_7b_chunk", num_seqs=7, lengths=("uniform", 48, 600),
                           query_tokens=("uniform", *rows), **kw)
    avg = w.query_start[-1] / len(w.context_lens)
    assert (avg >= 16) == (rows[0] >= 16)
    for P in (0, 64):
        assert max_err(_prefill_gpu(w, gpu_pool(w), P), _prefill_oracle(w)) <= TOL, P


@pytest.mark.parametrize("P", [0, 64])
@pytest.mark.parametrize("kw", [dict(), dict(num_q_heads=32, num_kv_heads=2)])
def test_prefill_partial_pack_groups(kw, P):
    """1-9 new tokens per sequence: a wave carries two packs, so groups whose
    second pack is empty or partly filled (G = 7: 2 tokens per pack; G = 16:
    1) must still match the oracle row by row."""
    _announce("prefill partial groups", kw, P)
    w = workloads.generate("qwen25_7b_chunk", num_seqs=12, lengths=("uniform", 9, 500),
                           query_tokens=("uniform", 1, 9), **kw)
    assert set(np.diff(w.query_start).tolist()) >= {1, 2, 3}
    assert max_err(_prefill_gpu(w, gpu_pool(w), P), _prefill_oracle(w)) <= TOL


def test_prefill_with_one_new_token_is_decode_bitwise():
    _announce("prefill n=1")
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate("qwen25_7b_chunk", num_seqs=6, lengths=("uniform", 1, 900), query_tokens=("uniform", 1, 1))
    pool = gpu_pool(w)
    got = _prefill_gpu(w, pool, 0)
    q, tables, lens = inputs(w)
    dec = abi.paged_decode_attention(q, pool[0], pool[1], tables, lens, w.scale, None)
    assert torch.equal(got, dec)
    assert max_err(got, _prefill_oracle(w)) <= TOL


def test_prefill_whole_context_new_and_16bit_output():
    """Every position new (pure prefill of short prompts), bf16 output equal to
    the fp32 output rounded, within one ulp."""
    _announce("prefill full")
    w = workloads.generate("qwen25_7b_chunk", num_seqs=4, lengths=("uniform", 1, 200),
                           query_tokens=("uniform", 200, 200))
    assert np.array_equal(np.diff(w.query_start), w.context_lens)
    pool = gpu_pool(w)
    o32 = _prefill_gpu(w, pool, 64)
    assert max_err(o32, _prefill_oracle(w)) <= TOL
    o16 = _prefill_gpu(w, pool, 64, torch.bfloat16)
    r = o32.to(torch.bfloat16)
    ulp = (r.float().abs() * 2.0 ** -7).clamp_min(1e-30)
    assert torch.all((o16.float() - r.float()).abs() <= ulp)


@pytest.mark.parametrize("rows", [(24, 40), (2, 6)])
def test_prefill_long_contexts_cross_block_id_chunks(rows):
    """Contexts past 4096 tokens: each wave reads more than 64 blocks, so its
    block ids arrive in several 64-entry chunks and the tile loop restarts
    per chunk (with tile pairs, the runs of masked and unmasked pairs too).
    Both tile paths (16+ rows per sequence: pairs), one pass and
    partitioned."""
    _announce("prefill long contexts", rows)
    w = workloads.generate("qwen25_7b_chunk", num_seqs=3, lengths=("uniform", 5000, 9000),
                           query_tokens=("uniform", *rows))
    assert w.context_lens.max() > 4096
    want = _prefill_oracle(w)
    pool = gpu_pool(w)
    for P in (0, 2048):
        assert max_err(_prefill_gpu(w, pool, P), want) <= TOL, P


def test_prefill_full_size_sampled():
    """The 16-sequence chunked-prefill workload at full size, in one pass (the
    benchmarked configuration) and partitioned, checked on three sequences'
    rows."""
    _announce("prefill full size")
    w = workloads.generate("qwen25_7b_chunk")
    pool = gpu_pool(w)
    runs = [_prefill_gpu(w, pool, P).cpu().numpy() for P in (0, 512)]
    assert all(np.all(np.isfinite(g)) for g in runs)
    pick = [int(np.argmax(np.diff(w.query_start))), int(np.argmin(w.context_lens)), 5]
    for b in pick:
        q0, q1 = int(w.query_start[b]), int(w.query_start[b + 1])
        sub = workloads.Workload(**{**w.__dict__})
        sub.q = w.q[q0:q1]
        sub.block_tables = w.block_tables[b:b + 1]
        sub.context_lens = w.context_lens[b:b + 1]
        sub.query_start = np.array([0, q1 - q0], np.int32)
        used = np.unique(sub.block_tables[sub.block_tables >= 0])
        keep = np.isin(w.fill_blocks, used)
        sub.fill_blocks, sub.fill_valid = w.fill_blocks[keep], w.fill_valid[keep]
        sub.fill_k, sub.fill_v = w.fill_k[keep], w.fill_v[keep]
        want = _prefill_oracle(sub)
        for got in runs:
            assert float(np.max(np.abs(got[q0:q1] - want))) <= TOL, b


# ------------------------------------------------------ fused decode step ---

def _same_bits(a, b):
    """Bitwise equality of two caches (unwritten slots hold NaN, which == would reject)."""
    it = {4: torch.int32, 2: torch.int16, 1: torch.uint8}[a.element_size()]
    return torch.equal(a.view(it), b.view(it))


def _step_pair(w, P, window=0):
    """(out, k, v) of kv_cache_write + paged_decode_attention_split, and of
    paged_decode_step, on two copies of the same pool."""
    from paged_kv_gqa_cache_amd import abi
    s = w.spec
    k0, v0, _ = gpu_pool(w, with_new_tokens=False)
    q, tables, lens = inputs(w)
    nk, nv = to_dev(w.new_k, s.kv_dtype), to_dev(w.new_v, s.kv_dtype)
    slots = torch.from_numpy(w.new_slots).cuda()
    ka, va, kb, vb = k0.clone(), v0.clone(), k0.clone(), v0.clone()
    ws_a = abi.split_workspace(q, ka, tables, P).zero_()
    ws_b = abi.split_workspace(q, kb, tables, P).zero_()
    abi.kv_cache_write(nk, nv, slots, ka, va)
    out_a = abi.paged_decode_attention_split(q, ka, va, tables, lens, w.scale, None, P, ws_a, window=window)
    out_b = abi.paged_decode_step(q, nk, nv, kb, vb, tables, lens, w.scale, P, ws_b, window=window)
    torch.cuda.synchronize()
    return (out_a, ka, va), (out_b, kb, vb)


@pytest.mark.parametrize("name,P", [("tiny", 64), ("qwen25_1p5b", 512), ("qwen25_1p5b", 128), ("tiny", 1024)])
def test_decode_step_equals_write_then_split(name, P):
    """One launch writing the new tokens and attending equals the write
    followed by the split path, bit for bit (cache and output), and the
    oracle within the tolerance."""
    _announce("decode step", name, P)
    w = workloads.generate(name, **REDUCED[name])
    (oa, ka, va), (ob, kb, vb) = _step_pair(w, P)
    assert _same_bits(ka, kb) and _same_bits(va, vb)
    assert torch.equal(oa, ob)
    assert max_err(ob, oracle_out(w)) <= TOL


@pytest.mark.parametrize("name,mode", [("tiny", "step"), ("smollm2_360m", "fused"), ("qwen25_7b_prefix", "balanced")])
def test_steps_replay_from_a_graph(name, mode):
    """Steps captured in a HIP graph (as the bench's graph figures replay
    them): every replay, with eager work and a synchronisation between
    replays, equals the eager call, output and cache, bit for bit for the
    one-launch paths (the step's new-token write lands on the same slot each
    time; the split counters return to zero inside the kernel, so no memory
    clear is recorded) and within 1e-5 for the balanced schedule."""
    _announce("graph replay", name, mode)
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate(name, **REDUCED[name])
    s = w.spec
    P = s.partition_size
    k, v, sc = gpu_pool(w, with_new_tokens=(mode != "step"))
    q, tables, lens = inputs(w)
    ws = abi.split_workspace(q, k, tables, P).zero_()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    if mode == "step":
        nk, nv = to_dev(w.new_k, s.kv_dtype), to_dev(w.new_v, s.kv_dtype)
        call = lambda: abi.paged_decode_step(q, nk, nv, k, v, tables, lens, w.scale, P, ws, out=out)
    elif mode == "fused":
        call = lambda: abi.paged_decode_attention_split(q, k, v, tables, lens, w.scale, sc, P, ws, out=out)
    else:   # the balanced schedule's two launches (its workspace needs no clearing)
        bws = abi.balanced_workspace(q, k, tables)
        call = lambda: abi.paged_decode_attention_balanced(q, k, v, tables, lens, w.scale, sc, bws, out=out)
    call()
    torch.cuda.synchronize()
    want_out, want_k, want_v = out.clone(), k.clone(), v.clone()
    assert max_err(want_out, oracle_out(w)) <= TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if mode == "balanced":   # its waves claim tiles at run time: fp32 sums in varying order
            assert float((out - want_out).abs().max()) <= 1e-5, rep
        else:
            assert torch.equal(out, want_out), rep
        assert _same_bits(k, want_k) and _same_bits(v, want_v), rep
        decode(w, (k, v, sc), "single")   # eager work between replays
        torch.cuda.synchronize()


def test_decode_step_with_window_and_repeated_calls():
    """Sliding window, and the same workspace reused across calls (the split
    counters return to zero): every call equals the two-launch result."""
    _announce("decode step window")
    from paged_kv_gqa_cache_amd import abi
    w = workloads.generate("qwen25_1p5b", num_seqs=6, lengths=("uniform", 1, 900))
    (oa, ka, va), (ob, kb, vb) = _step_pair(w, 128, window=300)
    assert _same_bits(ka, kb) and _same_bits(va, vb) and torch.equal(oa, ob)
    q, tables, lens = inputs(w)
    nk, nv = to_dev(w.new_k, w.spec.kv_dtype), to_dev(w.new_v, w.spec.kv_dtype)
    ws = abi.split_workspace(q, kb, tables, 128).zero_()
    for _ in range(5):
        o = abi.paged_decode_step(q, nk, nv, kb, vb, tables, lens, w.scale, 128, ws, window=300)
        torch.cuda.synchronize()
        assert torch.equal(o, ob)
    assert _same_bits(kb, ka) and _same_bits(vb, va)


def test_decode_step_full_size_at_the_benchmarked_partition():
    """The B=32 Qwen2.5-1.5B-shaped layer at full size through the fused
    step at the partition size the benchmark times: every output row
    against the oracle, and equal, cache and output, to the two-launch
    result."""
    P = workloads.SPECS["qwen25_1p5b"].partition_size
    _announce("decode step full size", P)
    w = workloads.generate("qwen25_1p5b")
    (oa, ka, va), (ob, kb, vb) = _step_pair(w, P)
    assert _same_bits(ka, kb) and _same_bits(va, vb) and torch.equal(oa, ob)
    assert max_err(ob, oracle_out(w)) <= TOL


# -------------------------------------------------- read-bandwidth probe ---

@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20])
def test_read_probe_reads_every_word(nbytes):
    """The measurement probe's per-workgroup XOR words fold to the XOR of
    every 32-bit word of the buffer (each word read exactly once), for a
    single 16-byte chunk, a ragged size and a multi-megabyte buffer."""
    _announce("read probe", nbytes)
    from paged_kv_gqa_cache_amd import abi
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(2048, dtype=torch.int32, device="cuda")
    abi.pkv_read_bandwidth_probe(buf, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
