"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/pagedkv.h declares, and rejects bad arguments with the
documented status before touching the device."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from paged_kv_gqa_cache_amd import abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pagedkv.h")
OK, INVALID, UNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 9, names
    lib = ctypes.CDLL(abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pagedkv.h but not exported"
    assert set(abi.EXPORTED) == set(names)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: with the library absent, importing the binding
    raises (a fresh interpreter, the library path pointed at nothing)."""
    import subprocess
    import sys
    env = dict(os.environ, PAGEDKV_LIB=str(tmp_path / "libpagedkv.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", "import paged_kv_gqa_cache_amd.abi"], cwd=root, env=env,
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "ImportError" in res.stderr and "is not built" in res.stderr


def test_version():
    assert "gfx950" in abi.version()


def desc(**kw):
    base = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64, num_blocks=10,
                max_blocks_per_seq=4, q_dtype=abi.PKV_F16, kv_dtype=abi.PKV_F16, out_dtype=abi.PKV_F32)
    block_size = kw.pop("block_size", None)
    base.update(kw)
    d = abi.make_desc(**base)
    if block_size is not None:
        d.block_size = block_size
    return d


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


def attn(d, scale=0.125, kv_scales=None, ptr=FAKE):
    return abi.lib().paged_decode_attention(ptr, ptr, ptr, ptr, ptr, scale, kv_scales, ptr,
                                            ctypes.byref(d), None)


def partial(d, P, scale=0.125):
    return abi.lib().paged_decode_attention_partial(FAKE, FAKE, FAKE, FAKE, FAKE, scale, None, P,
                                                    FAKE, FAKE, ctypes.byref(d), None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), UNSUPPORTED),
    (dict(head_dim=256), UNSUPPORTED),
    (dict(num_q_heads=34, num_kv_heads=2), UNSUPPORTED),          # G = 17 > 16
    (dict(num_q_heads=9, num_kv_heads=2), INVALID),               # not a multiple
    (dict(block_size=32), INVALID),
    (dict(num_blocks=0), INVALID),
    (dict(max_blocks_per_seq=0), INVALID),
    (dict(num_seqs=-1), INVALID),
    (dict(q_dtype=abi.PKV_BF16), UNSUPPORTED),                    # q bf16 with f16 KV
    (dict(out_dtype=abi.PKV_BF16), UNSUPPORTED),                  # f16 path cannot emit bf16
    (dict(q_dtype=abi.PKV_F32, kv_dtype=abi.PKV_F32, out_dtype=abi.PKV_F16), UNSUPPORTED),
    (dict(q_dtype=abi.PKV_F16, kv_dtype=abi.PKV_E4M3), INVALID),  # e4m3 without kv_scales
    (dict(q_dtype=7), UNSUPPORTED),
])
def test_attention_rejects_bad_descriptors(kw, code):
    assert attn(desc(**kw)) == code
    assert abi.last_error()


def test_attention_rejects_null_pointers_and_bad_scale():
    assert attn(desc(), ptr=None) == INVALID
    assert "null" in abi.last_error()
    assert attn(desc(), scale=math.inf) == INVALID
    assert attn(desc(), scale=math.nan) == INVALID
    scales = ctypes.c_void_p(0x2000)
    assert attn(desc(), kv_scales=scales) == INVALID            # scales for a 16-bit cache


def test_empty_batch_is_a_no_op():
    assert attn(desc(num_seqs=0), ptr=None) == OK
    assert abi.last_error() == ""


@pytest.mark.parametrize("P", [0, -16, 8, 24, 100])
def test_partial_rejects_bad_partition_sizes(P):
    assert partial(desc(), P) == INVALID
    assert "partition_size" in abi.last_error()


def test_reduce_rejects_bad_arguments():
    d = desc(out_dtype=abi.PKV_E4M3)
    assert abi.lib().paged_decode_attention_reduce(FAKE, FAKE, FAKE, 64, FAKE, ctypes.byref(d), None) == UNSUPPORTED
    d = desc()
    assert abi.lib().paged_decode_attention_reduce(FAKE, FAKE, FAKE, 40, FAKE, ctypes.byref(d), None) == INVALID
    assert abi.lib().paged_decode_attention_reduce(None, FAKE, FAKE, 64, FAKE, ctypes.byref(d), None) == INVALID


def test_write_rejects_e4m3_and_bad_sizes():
    d = desc(kv_dtype=abi.PKV_E4M3)
    assert abi.lib().kv_cache_write(FAKE, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(d), None) == UNSUPPORTED
    d = desc()
    assert abi.lib().kv_cache_write(FAKE, FAKE, FAKE, -1, FAKE, FAKE, ctypes.byref(d), None) == INVALID
    assert abi.lib().kv_cache_write(None, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(d), None) == INVALID
    assert abi.lib().kv_cache_write(None, None, None, 0, None, None, ctypes.byref(d), None) == OK


def test_quantize_requires_e4m3_cache():
    d = desc()
    assert abi.lib().kv_cache_quantize_e4m3(FAKE, FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE,
                                            ctypes.byref(d), None) == INVALID
    d = desc(kv_dtype=abi.PKV_E4M3)
    assert abi.lib().kv_cache_quantize_e4m3(FAKE, None, FAKE, FAKE, 3, FAKE, FAKE, FAKE,
                                            ctypes.byref(d), None) == INVALID


def test_partition_count_and_workspace_size():
    d = desc(num_seqs=128, num_q_heads=28, num_kv_heads=4, head_dim=128, max_blocks_per_seq=533)
    assert abi.lib().paged_decode_num_partitions(ctypes.byref(d), 512) == math.ceil(533 * 16 / 512)
    S = math.ceil(533 * 16 / 512)
    assert abi.lib().paged_decode_workspace_bytes(ctypes.byref(d), 512) == 128 * 28 * S * (128 + 1) * 4
    assert abi.lib().paged_decode_num_partitions(ctypes.byref(d), 40) == -1
    assert abi.num_partitions(533, 512) == S


def balanced(d, ws=FAKE, nbytes=1 << 30, ptr=FAKE):
    return abi.lib().paged_decode_attention_balanced(ptr, ptr, ptr, ptr, ptr, 0.125, None, ws, nbytes, ptr,
                                                     ctypes.byref(d), None)


def test_balanced_rejects_before_touching_the_device():
    assert balanced(desc(num_seqs=2049)) == UNSUPPORTED
    assert "2048" in abi.last_error()
    assert abi.lib().paged_decode_balanced_workspace_bytes(ctypes.byref(desc(num_seqs=2049))) == -1
    assert balanced(desc(), ptr=None) == INVALID
    assert balanced(desc(), ws=ctypes.c_void_p(0x1010)) == INVALID     # not 256-byte aligned
    assert "aligned" in abi.last_error()
    assert balanced(desc(max_blocks_per_seq=1 << 20, num_seqs=2048, num_kv_heads=2)) == INVALID
    assert balanced(desc(q_dtype=abi.PKV_BF16)) == UNSUPPORTED
    assert balanced(desc(num_seqs=0), ptr=None) == OK


def test_balanced_partial_and_reduce_reject_before_touching_the_device():
    lib = abi.lib()

    def partial(d, ws=FAKE, nbytes=1 << 30, ptr=FAKE):
        return lib.paged_decode_attention_balanced_partial(ptr, ptr, ptr, ptr, ptr, 0.125, None, ws, nbytes, ptr,
                                                           ctypes.byref(d), None)

    def reduce(d, ws=FAKE, nbytes=1 << 30, out=FAKE):
        return lib.paged_decode_attention_balanced_reduce(ws, nbytes, out, ctypes.byref(d), None)

    assert partial(desc(num_seqs=2049)) == UNSUPPORTED
    assert partial(desc(), ptr=None) == INVALID
    assert partial(desc(), ws=ctypes.c_void_p(0x1010)) == INVALID
    assert partial(desc(), nbytes=16) == INVALID
    assert "smaller" in abi.last_error()
    assert partial(desc(num_seqs=0), ptr=None) == OK
    assert reduce(desc(num_seqs=2049)) == UNSUPPORTED
    assert reduce(desc(), out=None) == INVALID
    assert reduce(desc(), ws=None) == INVALID
    assert reduce(desc(), ws=ctypes.c_void_p(0x1010)) == INVALID
    assert reduce(desc(), nbytes=16) == INVALID
    assert reduce(desc(num_seqs=0), out=None) == OK


def test_copy_blocks_validates_before_touching_the_device():
    lib = abi.lib()
    d = desc()
    assert lib.kv_cache_copy_blocks(None, 0, None, None, None, ctypes.byref(d), None) == OK
    assert lib.kv_cache_copy_blocks(FAKE, -1, FAKE, FAKE, None, ctypes.byref(d), None) == INVALID
    assert lib.kv_cache_copy_blocks(None, 2, FAKE, FAKE, None, ctypes.byref(d), None) == INVALID
    assert lib.kv_cache_copy_blocks(FAKE, 2, FAKE, FAKE, FAKE, ctypes.byref(d), None) == INVALID   # scales, 16-bit
    d8 = desc(kv_dtype=abi.PKV_E4M3)
    assert lib.kv_cache_copy_blocks(FAKE, 2, FAKE, FAKE, None, ctypes.byref(d8), None) == INVALID  # e4m3, no scales
    assert lib.kv_cache_copy_blocks(FAKE, 2, FAKE, FAKE, None, ctypes.byref(desc(kv_dtype=9)), None) == UNSUPPORTED


def test_append_e4m3_validates_before_touching_the_device():
    lib = abi.lib()
    d8 = desc(kv_dtype=abi.PKV_E4M3)
    assert lib.kv_cache_append_e4m3(FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE, ctypes.byref(desc()), None) == INVALID
    assert lib.kv_cache_append_e4m3(FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE, ctypes.byref(d8), None) == INVALID
    assert lib.kv_cache_append_e4m3(FAKE, FAKE, FAKE, 3, FAKE, FAKE, None, ctypes.byref(d8), None) == INVALID
    assert lib.kv_cache_append_e4m3(None, None, None, 0, None, None, None, ctypes.byref(d8), None) == OK


def test_prefill_validates_before_touching_the_device():
    lib = abi.lib()

    def call(d, n=4, P=0, ws=None, ptr=FAKE, nbytes=0):
        return lib.paged_prefill_attention(ptr, ptr, ptr, ptr, ptr, ptr, n, 0.125, None, P, ws, nbytes, ptr,
                                           ctypes.byref(d), None)
    assert call(desc(num_seqs=2049)) == UNSUPPORTED
    assert call(desc(sliding_window=8)) == UNSUPPORTED
    assert call(desc(), P=24) == INVALID
    assert call(desc(), n=-1) == INVALID
    assert call(desc(), ptr=None) == INVALID
    assert call(desc(), P=64) == INVALID                           # partitioned without a workspace
    assert call(desc(), P=64, ws=ctypes.c_void_p(0x1010), nbytes=1 << 30) == INVALID   # misaligned
    assert call(desc(), n=0, ptr=None) == OK
    d = desc(num_seqs=3, num_q_heads=28, num_kv_heads=4, head_dim=128, max_blocks_per_seq=100)
    S = math.ceil(100 * 16 / 512)
    rows = 50 * 28 * S
    assert lib.paged_prefill_workspace_bytes(ctypes.byref(d), 50, 512) == (rows * 4 + 255) // 256 * 256 + rows * 128 * 4
    assert lib.paged_prefill_workspace_bytes(ctypes.byref(d), 50, 0) == 0


def test_decode_step_rejects_e4m3_and_null_rows():
    from paged_kv_gqa_cache_amd.abi import PKV_E4M3, PKV_F16, PKV_F32, make_desc, lib
    import ctypes
    d = make_desc(2, 8, 2, 128, 16, 4, PKV_F16, PKV_E4M3, PKV_F32)
    one = ctypes.c_void_p(256)
    rc = lib().paged_decode_step(one, one, one, one, one, one, one, 1.0, 64, one, 1 << 20, one,
                                 ctypes.byref(d), None)
    assert rc != 0 and "e4m3" in abi.last_error()
    d = make_desc(2, 8, 2, 128, 16, 4, PKV_F16, PKV_F16, PKV_F32)
    rc = lib().paged_decode_step(one, None, one, one, one, one, one, 1.0, 64, one, 1 << 20, one,
                                 ctypes.byref(d), None)
    assert rc != 0 and "null" in abi.last_error()


def test_read_probe_validates_before_launching():
    """The read-bandwidth probe rejects a null pointer, a size that is not a
    positive multiple of 16 and a misaligned source, without launching."""
    from paged_kv_gqa_cache_amd.abi import lib
    buf, out = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    probe = lib().pkv_read_bandwidth_probe
    assert probe(None, 1024, out, 16, None) == INVALID and "null" in abi.last_error()
    assert probe(buf, 1000, out, 16, None) == INVALID and "multiple of 16" in abi.last_error()
    assert probe(buf, 0, out, 16, None) == INVALID
    assert probe(ctypes.c_void_p(4100), 1024, out, 16, None) == INVALID and "aligned" in abi.last_error()
    assert probe(buf, 1024, out, 0, None) == INVALID
