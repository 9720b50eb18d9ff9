"""OCP FP8 E4M3 ("e4m3fn") codec and per-(block, kv-head) quantisation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the pages fix: the KV cache may be stored as E4M3 with a scale per page
and per head, and dequantised inside attention ("rvLLM: High-performance LLM
inference in Rust", section "CUDA Kernels", row "FP8 KV Cache"; "LLM Serving
Kernels", section "Projects", row 05 "E4M3 storage, page scales, fused
dequantization").  The pages do not define the bit format, so this module
follows the OCP 8-bit floating point specification (OFP8, v1.0) for E4M3:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 encodes subnormals  (-1)^s * 2^-6 * m/8;
* exponent field 1..15 encodes normals (-1)^s * 2^(e-7) * (1 + m/8);
* the one pattern with all exponent and mantissa bits set (0x7F / 0xFF) is
  NaN; there are no infinities, so the largest finite magnitude is
  2^8 * 1.75 = 448.

Readings taken where the pages are silent:

* the format is OCP E4M3FN (max 448), not the FNUZ variant (max 240): the
  per-block scale amax/448 only makes sense for a maximum of 448;
* scale = fp32(amax / 448) over the block's valid tokens, one scale for K and
  one for V per (block, kv head); a block whose amax is 0 gets scale 1;
* code = round-to-nearest-even(clamp(fp32(x / scale), -448, 448)), the
  division done in fp32 (the precision the GPU quantiser works in), so a
  code decided by floating point is decided in the same precision on both
  sides.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode_value(code: int) -> float:
    """Value of one E4M3 code from the OCP definition (float64, exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (2.0 ** -6) * (mant / 8.0)
    return sign * (2.0 ** (exp_field - 7)) * (1.0 + mant / 8.0)


# All 256 values, built once from the definition above.
DECODE_TABLE = np.array([decode_value(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64 values."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


# Non-negative finite codes 0x00..0x7E in increasing value order.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE_TABLE[:0x7F]


def encode(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest E4M3 code, ties to the even code.

    Magnitudes above 448 saturate to 448 (the clamp comes before rounding,
    so 464, the midpoint between 448 and the missing 480, maps to 448).
    NaN maps to 0x7F.  Negative values, including those that round to zero,
    keep their sign bit, as an IEEE cast does.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    nan = np.isnan(flat)
    mag = np.minimum(np.abs(np.where(nan, 0.0, flat)), E4M3_MAX)
    # Index of the first representable value >= mag.
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    # Exact hits: searchsorted(left) already lands on the value itself.
    code = np.where(_POS_VALUES[hi] == mag, _POS_CODES[hi], code)
    neg = np.signbit(flat) & ~nan
    out[:] = (code | np.where(neg, 0x80, 0)).astype(np.uint8)
    out[nan] = NAN_CODE
    return out.reshape(x.shape)


def quantize_blocks(x_blocks: np.ndarray, valid_tokens: np.ndarray):
    """Quantise K (or V) blocks to E4M3 with one fp32 scale per (block, head).

    ``x_blocks``: float32 [n, 16, Hkv, D], the 16 token slots of each block in
    slot order; ``valid_tokens``: int [n], how many leading slots of each block
    hold data (the rest are ignored and get code 0).

    Returns ``(codes uint8 [n, 16, Hkv, D], scales float32 [n, Hkv])``.
    Follows "LLM Serving Kernels", section "Projects", row 05 (E4M3 storage
    with page scales) and "rvLLM: High-performance LLM inference in Rust",
    section "CUDA Kernels", row "FP8 KV Cache" (per-head scaling).
    """
    x_blocks = np.asarray(x_blocks, dtype=np.float32)
    n, bs, hkv, d = x_blocks.shape
    valid = np.arange(bs)[None, :] < np.asarray(valid_tokens, dtype=np.int64)[:, None]   # [n, 16]
    vals = np.where(valid[:, :, None, None], x_blocks, np.float32(0))
    amax = np.max(np.abs(vals), axis=(1, 3)).astype(np.float32)                          # [n, Hkv]
    scales = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
    scaled = (x_blocks / scales[:, None, :, None]).astype(np.float32)  # fp32 division, correctly rounded
    codes = encode(np.clip(scaled.astype(np.float64), -E4M3_MAX, E4M3_MAX))
    codes[~valid] = 0
    return codes, scales


def append_token(block_codes: np.ndarray, scale, offset: int, x: np.ndarray):
    """One step of quantise-on-append for one (block, kv head), K or V.

    ``block_codes``: uint8 [16, D], the block's codes in slot order (slots at
    or past ``offset`` are ignored); ``scale``: the block's current fp32 scale
    (ignored when ``offset`` is 0); ``x``: float32 [D], the token going to slot
    ``offset``.  Returns ``(codes, scale)`` after the step.

    The pages fix a scale per page and head but no append policy.  Reading
    taken: the block keeps the bulk quantiser's
    invariant scale = fp32(amax / 448) over its tokens so far, 1 while they
    are all zero.  The token's own s = fp32(amax(|x|) / 448).  When the token
    is the block's first, or every earlier code of the block is a zero
    (0x00 or 0x80: the earlier tokens' amax is 0, since the token that set a
    non-zero scale holds a code of magnitude 448), the token sets the scale
    (1 if s is 0) and the earlier codes stay as they are.  Otherwise a token
    with s above the current scale grows it to s, and the block's earlier
    codes are re-encoded: value = fp32(decode(c) * old scale), code =
    nearest-even E4M3 of clamp(fp32(value / s)).  The token itself is then
    encoded against the (new) scale like the bulk quantiser.  Every rounding
    step is fp32, as on the GPU.
    """
    codes = np.array(block_codes, dtype=np.uint8, copy=True)
    x = np.asarray(x, dtype=np.float32)
    s_tok = np.float32(np.max(np.abs(x))) / np.float32(E4M3_MAX)
    earlier_zero = not np.any(codes[:offset] & 0x7F)   # vacuously true for the first token
    if earlier_zero:
        s = s_tok if s_tok > 0 else np.float32(1)
    else:
        s = np.float32(scale)
        if s_tok > s:
            old = decode(codes[:offset]).astype(np.float32) * s              # fp32 product
            codes[:offset] = encode(np.clip((old / s_tok).astype(np.float32).astype(np.float64),
                                            -E4M3_MAX, E4M3_MAX))
            s = s_tok
    codes[offset] = encode(np.clip((x / s).astype(np.float32).astype(np.float64), -E4M3_MAX, E4M3_MAX))
    return codes, np.float32(s)


def storage_saving(block_size: int, head_dim: int, scale_bytes: int = 4,
                   separate_kv_scales: bool = True) -> float:
    """Fraction of KV bytes saved by E4M3 + fp32 page scales versus fp16.

    Per (block, kv head): fp16 K and V take 2 * bs * D * 2 bytes; E4M3 takes
    2 * bs * D * 1 bytes plus one fp32 scale for K and one for V (or a single
    scale shared by both).
    """
    fp16 = 2 * block_size * head_dim * 2
    n_scales = 2 if separate_kv_scales else 1
    fp8 = 2 * block_size * head_dim * 1 + n_scales * scale_bytes
    return 1.0 - fp8 / fp16
