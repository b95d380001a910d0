"""Oracle for the TurboQuant paged KV cache: plain, slow CPU definitions.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The library in
bit_quantized_paged_turbo_amd/ never imports it and shares no code with it; the two
meet only through the seeded inputs of workloads/.

Sources (the pages):
  [xInfer]  "xInfer: Pure-Rust LLM Inference Without a Python Runtime" (hysenlabs.com)
    - section "What actually sits between the request and the tokens": TurboQuant rotates
      each K/V head vector with a Walsh-Hadamard transform, then quantizes it with a
      per-head absmax scale; the rotation spreads outlier channels across the head
      dimension before the absmax is taken. The cache it produces is 2 to 4 bits wide, so
      a 2-bit width (turbo2, codes -1..1) is read as the same recipe with qmax = 1.
    - section "Getting a server up: the commands in the README": cache types fp8, turbo8,
      turbo4, turbo3; BF16 when none is given. The compression table of the same page puts
      fp8 at 2x against BF16, so an fp8 row is 128 one-byte elements with nothing beside
      them: each bf16 element cast to OCP FP8 E4M3 (round to nearest, ties to even,
      saturating at +-448), with no rotation and no scale.
    - section "TurboQuant is a memory trade, and the README does not price it fully":
      attention dequantizes the cache on every step.
  [infero]  infero landing page, section "Beyond plain text decode", item "Continuous
    batching": decode runs over a paged KV cache.

The pages do not fix the number format. The readings used here (one per function):
  - orthonormal FWHT over 128 in natural (Sylvester) order, no random signs; fp32 stages
    h = 1, 2, ..., 64 of (a+b, a-b), then one fp32 multiply by C = fp32(1/sqrt(128));
  - one fp16 scale per (token, kv_head) row: fp16_rne(min(absmax/qmax, 65504));
  - codes clamp(rint_half_even(x / float(s16)), -qmax, qmax), all zero when s16 == 0;
  - codes packed little-endian, `bits`-wide two's complement fields, 16*bits bytes a row;
  - attention per (sequence, query head) in float64 over the dequantized rows in the
    rotated space, then rotated back with H (H is symmetric and orthonormal);
  - query head j reads kv head j // (Hq // Hkv); all positions < context length attend;
  - fp8: the nearest finite OCP E4M3 value of each bf16 element, ties to the even code,
    magnitudes past 448 saturating to 448, the sign kept (also on zero);
  - chunked prefill: query i of a chunk starting at position P attends to positions 0 .. P + i
    of the cache as stored, the chunk's own rows included.

Every function here is pinned by tests/test_oracle_*.py against something other than
itself (dense Hadamard matrices, closed forms, hand-worked values, brute force,
textbook attention); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
QMAX = {8: 127, 4: 7, 3: 3, 2: 1}
FP8 = 16          # cache-type value of the fp8 (E4M3) cache; 0 is bf16, 2..8 the turbo widths
# fp32 round-to-nearest of 1/sqrt(128); its bit pattern is 0x3DB504F3.
C_F32 = np.float32(1.0 / np.sqrt(np.float64(HEAD_DIM)))
FP16_MAX = np.float32(65504.0)


# --------------------------------------------------------------------------------------
# Hadamard rotation
# --------------------------------------------------------------------------------------
def hadamard_matrix(n: int = HEAD_DIM) -> np.ndarray:
    """Dense orthonormal Walsh-Hadamard matrix in natural (Sylvester) order, float64.

    H[i, k] = (-1)^popcount(i & k) / sqrt(n). This is the plain definition of the rotation
    the xInfer page names ("What actually sits between the request and the tokens").
    """
    i = np.arange(n)[:, None]
    k = np.arange(n)[None, :]
    parity = np.zeros((n, n), dtype=np.int64)
    x = i & k
    while np.any(x):
        parity ^= x & 1
        x = x >> 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(float(n))


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along the last axis.

    Stages h = 1, 2, 4, ..., n/2 in that order; each stage replaces the pair
    (x[i], x[i+h]) for every i with bit h clear by (x[i] + x[i+h], x[i] - x[i+h]).
    Arithmetic is in x's own dtype, one correctly rounded add or subtract per output.
    """
    y = np.array(x, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        blocks = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = blocks[..., 0, :].copy()
        b = blocks[..., 1, :].copy()
        blocks[..., 0, :] = a + b
        blocks[..., 1, :] = a - b
        y = blocks.reshape(y.shape)
        h *= 2
    return y


def rotate_f32(rows: np.ndarray) -> np.ndarray:
    """Orthonormal rotation of fp32 rows as the codec computes it: fp32 FWHT, then x C."""
    rows = np.asarray(rows, dtype=np.float32)
    return fwht(rows) * C_F32


# --------------------------------------------------------------------------------------
# bf16 / fp16 number formats
# --------------------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_saturating(x: np.ndarray) -> np.ndarray:
    """fp32 -> binary16 with round-half-even, saturating at 65504, subnormals kept."""
    return np.minimum(np.asarray(x, dtype=np.float32), FP16_MAX).astype(np.float16)


# --------------------------------------------------------------------------------------
# fp8 cache: OCP FP8 E4M3 elements
# --------------------------------------------------------------------------------------
def fp8_e4m3_value(code) -> np.ndarray:
    """Value of OCP FP8 E4M3 bit patterns, float64 (NaN for S.1111.111).

    Fields: sign (bit 7), exponent E (bits 6..3, bias 7), mantissa M (bits 2..0).
    E = 0: M * 2^-9 (subnormal); otherwise (1 + M/8) * 2^(E-7). E = 15 with M = 7 is NaN;
    there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(x) -> np.ndarray:
    """Round finite values to OCP FP8 E4M3 bit patterns (uint8).

    The result is the finite E4M3 value nearest to |x| (codes 0x00..0x7E, which increase
    with the value), the even code on a tie, with x's sign bit on top (so -0.0 -> 0x80).
    Anything beyond 448 has 448 as its nearest finite value: the cast saturates.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the fp8 cast's contract")
    mags = fp8_e4m3_value(np.arange(0x7F))             # 0 .. 448, strictly increasing
    a = np.abs(x)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)   # first magnitude >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a >= mags[0x7E], 0x7E, np.where(pick_hi, hi, lo))
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def fp8_encode_rows_bf16(bits_u16: np.ndarray) -> np.ndarray:
    """The fp8 cache row of bf16 rows [..., 128]: one E4M3 byte per element, nothing else."""
    return fp8_e4m3_encode(bf16_bits_to_f32(bits_u16))


# --------------------------------------------------------------------------------------
# Quantizer
# --------------------------------------------------------------------------------------
def quantize_rotated(x: np.ndarray, bits: int):
    """Per-row absmax quantization of already-rotated fp32 rows [..., 128].

    Returns (codes int8 [..., 128], scales float16 [...]). Steps, in fp32:
      m = max_d |x[d]|;  s32 = m / qmax;  s16 = fp16(min(s32, 65504));
      c[d] = clamp(rint(x[d] / float32(s16)), -qmax, qmax), or 0 when s16 == 0.
    The xInfer page gives the per-head absmax step; the fp16 scale, half-even rounding and
    quantizing against the stored fp16 scale are this library's reading of it.
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the codec's contract")
    qmax = QMAX[bits]
    m = np.max(np.abs(x), axis=-1)
    s32 = m / np.float32(qmax)
    s16 = f32_to_f16_saturating(s32)
    s = s16.astype(np.float32)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s)
    c = np.rint(x / s_safe[..., None])
    c = np.clip(c, -qmax, qmax)
    c = np.where(zero[..., None], np.float32(0.0), c)
    return c.astype(np.int8), s16


def quantize_rows_bf16(bits_u16: np.ndarray, bits: int):
    """Full codec for bf16 rows [..., 128]: widen, rotate (fp32 FWHT, x C), quantize."""
    return quantize_rotated(rotate_f32(bf16_bits_to_f32(bits_u16)), bits)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack signed codes [..., 128] into [..., 16*bits] bytes.

    Code d is a `bits`-wide two's complement field at bit offset bits*d of the row's
    little-endian bitstream (byte k holds bits 8k .. 8k+7).
    """
    codes = np.asarray(codes, dtype=np.int64)
    lead = codes.shape[:-1]
    n = codes.shape[-1]
    field = codes & ((1 << bits) - 1)                     # two's complement field value
    bitpos = np.arange(n * bits)
    owner = bitpos // bits                                # which code this bit belongs to
    within = bitpos % bits
    bitvals = (field[..., owner] >> within) & 1           # [..., n*bits]
    bitvals = bitvals.reshape(lead + (n * bits // 8, 8))
    weights = (1 << np.arange(8)).astype(np.int64)
    return (bitvals * weights).sum(axis=-1).astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, n: int = HEAD_DIM) -> np.ndarray:
    """Inverse of pack_codes: [..., 16*bits] bytes -> int8 codes [..., n]."""
    packed = np.asarray(packed, dtype=np.uint8)
    lead = packed.shape[:-1]
    bitvals = (packed[..., :, None].astype(np.int64) >> np.arange(8)) & 1
    bitvals = bitvals.reshape(lead + (n, bits))
    field = (bitvals << np.arange(bits)).sum(axis=-1)
    signed = np.where(field >= (1 << (bits - 1)), field - (1 << bits), field)
    return signed.astype(np.int8)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Rotated-space reconstruction s16 * c, float64 (exact: both factors are short)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def row_bytes(bits: int) -> int:
    """Stored bytes of one turbo row: 16*bits code bytes plus a 2-byte fp16 scale."""
    return 16 * bits + 2


# --------------------------------------------------------------------------------------
# Decode attention
# --------------------------------------------------------------------------------------
def _attend(qvec: np.ndarray, keys: np.ndarray, vals: np.ndarray, softmax_scale: float):
    """softmax(scale * keys @ q) @ vals in float64 for one query vector."""
    if keys.shape[0] == 0:
        return np.zeros(vals.shape[-1], dtype=np.float64)
    z = softmax_scale * (keys @ qvec)
    p = np.exp(z - np.max(z))
    return (p @ vals) / np.sum(p)


def decode_attention_turbo(q_bits: np.ndarray, k_codes: np.ndarray, k_scales: np.ndarray,
                           v_codes: np.ndarray, v_scales: np.ndarray,
                           softmax_scale: float) -> np.ndarray:
    """Decode attention of one sequence over a TurboQuant cache, in float64.

    q_bits    bf16 bit patterns [Hq, 128]
    k_codes   int codes [L, Hkv, 128];  k_scales fp16 [L, Hkv]   (same for v)
    Returns   float64 [Hq, 128]

    Per query head j (kv head j // g): q' = H q; k'_t = s_k[t] c_k[t]; v'_t = s_v[t] c_v[t];
    z_t = scale * q'.k'_t; o = sum_t softmax(z)_t v'_t; out = H o. The cache holds
    rotated rows (xInfer page, "What actually sits between the request and the tokens"),
    so the query is rotated by the same H and the result rotated back by H = H^-1.
    """
    H = hadamard_matrix()
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    hq = q.shape[0]
    hkv = k_codes.shape[1]
    g = hq // hkv
    out = np.zeros((hq, HEAD_DIM), dtype=np.float64)
    for kvh in range(hkv):
        keys = dequantize(k_codes[:, kvh, :], k_scales[:, kvh])
        vals = dequantize(v_codes[:, kvh, :], v_scales[:, kvh])
        for j in range(kvh * g, (kvh + 1) * g):
            q_rot = H @ q[j]
            o_rot = _attend(q_rot, keys, vals, softmax_scale)
            out[j] = H @ o_rot
    return out


def decode_attention_bf16(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                          softmax_scale: float) -> np.ndarray:
    """Decode attention of one sequence over an unquantized bf16 cache, in float64.

    q_bits [Hq, 128], k_bits / v_bits [L, Hkv, 128] as bf16 bit patterns. The cache type
    used when none is given (xInfer page, "Getting a server up: the commands in the
    README"): no rotation, no scale.
    """
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    k = bf16_bits_to_f32(k_bits).astype(np.float64)
    v = bf16_bits_to_f32(v_bits).astype(np.float64)
    hq = q.shape[0]
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((hq, HEAD_DIM), dtype=np.float64)
    for j in range(hq):
        kvh = j // g
        out[j] = _attend(q[j], k[:, kvh, :], v[:, kvh, :], softmax_scale)
    return out


def decode_attention_fp8(q_bits: np.ndarray, k_fp8: np.ndarray, v_fp8: np.ndarray,
                         softmax_scale: float) -> np.ndarray:
    """Decode attention of one sequence over an fp8 (E4M3) cache, in float64.

    q_bits bf16 bit patterns [Hq, 128]; k_fp8 / v_fp8 E4M3 bytes [L, Hkv, 128]. The cached
    rows are the elements' E4M3 values, unrotated and unscaled, so this is textbook softmax
    attention over those values.
    """
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    k = fp8_e4m3_value(k_fp8)
    v = fp8_e4m3_value(v_fp8)
    hq = q.shape[0]
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((hq, HEAD_DIM), dtype=np.float64)
    for j in range(hq):
        kvh = j // g
        out[j] = _attend(q[j], k[:, kvh, :], v[:, kvh, :], softmax_scale)
    return out


def decode_sequence(dtype_bits: int, q_bits: np.ndarray, k_bits: np.ndarray,
                    v_bits: np.ndarray, softmax_scale: float):
    """Quantize one sequence's K/V rows (if turbo or fp8) and run decode attention.

    dtype_bits 0 = bf16, FP8 (16) = E4M3, else 8/4/3/2. Returns (out [Hq,128] float64, codec)
    where codec is None for bf16, (k_fp8, v_fp8) for fp8 or (k_codes, k_scales, v_codes,
    v_scales) for turbo types.
    """
    if dtype_bits == 0:
        return decode_attention_bf16(q_bits, k_bits, v_bits, softmax_scale), None
    if dtype_bits == FP8:
        kf, vf = fp8_encode_rows_bf16(k_bits), fp8_encode_rows_bf16(v_bits)
        return decode_attention_fp8(q_bits, kf, vf, softmax_scale), (kf, vf)
    kc, ks = quantize_rows_bf16(k_bits, dtype_bits)
    vc, vs = quantize_rows_bf16(v_bits, dtype_bits)
    out = decode_attention_turbo(q_bits, kc, ks, vc, vs, softmax_scale)
    return out, (kc, ks, vc, vs)


# --------------------------------------------------------------------------------------
# Chunked prefill over the quantized cache
# --------------------------------------------------------------------------------------
def prefill_sequence(dtype_bits: int, q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                     start: int, softmax_scale: float) -> np.ndarray:
    """Attention of a prefill chunk over its sequence's cache, in float64.

    q_bits     bf16 bits [C, Hq, 128]: the chunk's queries, query i at position start + i
    k_bits     bf16 bits [start + C, Hkv, 128] (same for v): every row of the sequence up to the
               chunk's end, the chunk's own rows included (appended before the attention)
    Returns    float64 [C, Hq, 128]

    Query i attends to positions 0 .. start + i (causal, nothing past itself), over the cache as
    stored: quantized (turbo, fp8) or not (bf16) by the same definitions as decode. The infero
    landing page, section "Beyond plain text decode", item "Continuous batching": decodes go
    first and prefill fills what is left of a step, split across steps, so a chunk attends to
    the cached prefix of earlier chunks plus itself.
    """
    c = q_bits.shape[0]
    out = np.zeros((c,) + q_bits.shape[1:], dtype=np.float64)
    if dtype_bits == 0:
        for i in range(c):
            n = start + i + 1
            out[i] = decode_attention_bf16(q_bits[i], k_bits[:n], v_bits[:n], softmax_scale)
        return out
    if dtype_bits == FP8:
        kf, vf = fp8_encode_rows_bf16(k_bits), fp8_encode_rows_bf16(v_bits)
        for i in range(c):
            n = start + i + 1
            out[i] = decode_attention_fp8(q_bits[i], kf[:n], vf[:n], softmax_scale)
        return out
    kc, ks = quantize_rows_bf16(k_bits, dtype_bits)
    vc, vs = quantize_rows_bf16(v_bits, dtype_bits)
    for i in range(c):
        n = start + i + 1
        out[i] = decode_attention_turbo(q_bits[i], kc[:n], ks[:n], vc[:n], vs[:n], softmax_scale)
    return out
