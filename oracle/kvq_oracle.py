"""CPU oracle for quantize-on-write into a paged KV cache, for dequantizing
paged decode attention and for causal chunked-prefill attention over the
cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It is a plain,
slow, deliberately unoptimised statement of what the GPU path computes, and it
shares no code with that path.

Sources (four web pages on KV-cache quantization; cited by title and section):
  [P1] "Use Less Memory: Quantization and Offloading" (int8ai.com)
  [P2] "12 KV Cache Quantization" (learning-materials, Inference Engineering)
  [P3] "Quantized KV caches in production: FP8 vs INT8 vs INT4" (llms.blog)
  [P4] "KV Cache Quantization" glossary entry (inferensys.com)

Arithmetic precision.  The encoding steps (scale, quotient, rounding) are done
in IEEE binary32 with round-to-nearest-even, and the scale is then rounded to
binary16 for storage, exactly as the stored format requires; NumPy float32
operations, ``np.rint`` and ``astype(np.float16)`` provide those roundings.
Attention is computed in float64 over the dequantized values.

Readings taken where the pages leave a step open (each is repeated at its use):
  * the quotient divides by the STORED fp16 scale, so dequantization x_hat =
    code * s reproduces what was divided by;
  * "round" is round-half-to-even; INT8 codes are in [-127, 127] and INT4
    codes in [-7, 7] (the symmetric clip range of [P1] section 2.1);
  * FP8 is the OCP E4M3FN encoding (max 448, no infinities, S.1111.111 = NaN),
    rounded to nearest-even and saturated at +-448.  [P1] section 2.3 prints
    +-240, which is the maximum of the FNUZ variant, not of E4M3FN;
  * the E5M2 variant ([P1] section 2.3 table, +-57344) is the OCP E5M2
    encoding (bias 15, infinities and NaN in exponent field 31), scaled per
    token and head like E4M3FN with q_max 57344, rounded to nearest-even and
    saturated at +-57344;
  * a group whose fp16 scale is 0 (all-zero input, or a scale that underflows
    fp16) stores scale 0 and all codes 0;
  * INT4 packs two codes per byte, the even channel in the low nibble;
  * KIVI-style keys: one fp16 scale and one fp16 zero point (= the group
    minimum) per channel per 32-token group, unsigned codes 0..15; the rows of a
    page wait in a per-sequence fp16 tail until the page's last row arrives;
  * chunked prefill: a sequence's chunk of n queries are its last n
    positions (their keys and values already in the cache), and query i
    attends causally to tokens 0 .. L - n + i.

Parity unpinned: nothing here.  Every function below is pinned by a test in
tests/test_oracle_*.py against the pages' worked example, closed forms,
invariants, brute force or an independent library routine.
"""

from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# Formats
# --------------------------------------------------------------------------

INT8 = "int8"
FP8_E4M3FN = "fp8_e4m3fn"
INT4_G32 = "int4_g32"
INT4_KIVI = "int4_kivi"
FP8_E5M2 = "fp8_e5m2"

SYM_FORMATS = (INT8, FP8_E4M3FN, INT4_G32, FP8_E5M2)
FP8_FORMATS = (FP8_E4M3FN, FP8_E5M2)
K_FORMATS = SYM_FORMATS + (INT4_KIVI,)
V_FORMATS = SYM_FORMATS

# Largest representable magnitude of each symmetric target ([P1] section 2.1
# table: signed INT8 127, signed INT4 7; OCP E4M3FN 448; [P1] section 2.3
# table: E5M2 57344).
QMAX = {INT8: 127.0, INT4_G32: 7.0, FP8_E4M3FN: 448.0, FP8_E5M2: 57344.0}

# Channels per scale group along head_dim ([P2] section 5, "Where the scales
# live": INT4 with group=32).  Per-token-per-head formats have one group = D.
INT4_GROUP = 32

# KIVI keys: tokens per quantization group along the sequence, and the number
# of steps of the unsigned 4-bit range ([P4] asymmetric quantization maps
# [min, max] onto the full integer range 0..15).
KIVI_GROUP = 32
KIVI_LEVELS = 15


def groups_per_row(fmt: str, head_dim: int) -> int:
    """Number of fp16 scales stored per (token, head) for a symmetric format."""
    return head_dim // INT4_GROUP if fmt == INT4_G32 else 1


def code_bytes_per_row(fmt: str, head_dim: int) -> int:
    """Bytes of codes per (token, head): 1 B/element for 8-bit, 0.5 for 4-bit
    ([P1] section 2.1 table, bytes per element)."""
    return head_dim // 2 if fmt in (INT4_G32, INT4_KIVI) else head_dim


# --------------------------------------------------------------------------
# FP8 E4M3FN, written from the OCP 8-bit floating point definition:
# 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
# holds subnormals m * 2^-9; no infinities; S.1111.111 is NaN, so the largest
# finite magnitude is 1.75 * 2^8 = 448.  [P3] "Numerical Formats" gives the
# 1-4-3 split and the 8 levels per power of two.
# --------------------------------------------------------------------------

E4M3FN_MAX_CODE = 0x7E  # 448


def e4m3fn_value(code) -> np.ndarray:
    """Exact float64 value of each E4M3FN byte (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3fn_encode(y) -> np.ndarray:
    """Round float32 values to E4M3FN bytes: nearest, ties to the even code,
    saturating at +-448.  The sign of zero (and of values that round to zero)
    is kept.  NaN and infinite inputs are outside the contract."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)  # exact
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # Subnormal range: the value is m * 2^-9; m = 8 lands on the smallest
    # normal (code 0x08) by continuity of the encoding.
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    frac, exp = np.frexp(a[nrm])  # a = frac * 2^exp, frac in [0.5, 1)
    e = exp.astype(np.int64) - 1  # a = (1 + f) * 2^e
    mant = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)  # 0..8, ties even
    # A mantissa that rounds up to 8 carries into the exponent, which the
    # additive form below does by itself.
    code[nrm] = ((e + 7) << 3) + mant
    code = np.minimum(code, E4M3FN_MAX_CODE)  # saturate: 448 is the largest finite
    code |= np.where(np.signbit(y), 0x80, 0)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# FP8 E5M2, from the OCP 8-bit floating point definition: 1 sign bit, 5
# exponent bits with bias 15, 2 mantissa bits; exponent field 0 holds
# subnormals m * 2^-16; exponent field 31 holds infinities (mantissa 0) and
# NaN, so the largest finite magnitude is 1.75 * 2^15 = 57344 ([P1] section
# 2.3 table: 5 exponent bits, 2 mantissa bits, +-57344; [P3] "Numerical
# Formats": 1-5-2 split, 4 levels per power of two).
# --------------------------------------------------------------------------

E5M2_MAX_CODE = 0x7B  # 57344


def e5m2_value(code) -> np.ndarray:
    """Exact float64 value of each E5M2 byte (+-inf for S.11111.00, NaN for
    the other codes of exponent field 31)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 0x1F
    m = (c & 0x3).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def e5m2_encode(y) -> np.ndarray:
    """Round float32 values to E5M2 bytes: nearest, ties to the even code,
    saturating at +-57344 (never an infinity).  The sign of zero (and of
    values that round to zero) is kept.  NaN and infinite inputs are outside
    the contract."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)  # exact
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -14
    # subnormal range: the value is m * 2^-16; m = 4 is the smallest normal
    # (code 0x04) by continuity of the encoding
    code[sub] = np.rint(a[sub] * 2.0 ** 16).astype(np.int64)
    nrm = ~sub
    frac, exp = np.frexp(a[nrm])  # a = frac * 2^exp, frac in [0.5, 1)
    e = exp.astype(np.int64) - 1  # a = (1 + f) * 2^e
    mant = np.rint((2.0 * frac - 1.0) * 4.0).astype(np.int64)  # 0..4, ties even
    code[nrm] = ((e + 15) << 2) + mant  # a carry into the exponent is the + above
    code = np.minimum(code, E5M2_MAX_CODE)  # saturate at 57344
    code |= np.where(np.signbit(y), 0x80, 0)
    return code.astype(np.uint8)


def fp8_value(code, fmt: str) -> np.ndarray:
    return e4m3fn_value(code) if fmt == FP8_E4M3FN else e5m2_value(code)


def fp8_encode(y, fmt: str) -> np.ndarray:
    return e4m3fn_encode(y) if fmt == FP8_E4M3FN else e5m2_encode(y)


# --------------------------------------------------------------------------
# Symmetric quantization ([P1] section 2.1):
#   s = max|x| / q_max;  x_q = clip(round(x / s), -q_max, q_max);  x_hat = x_q s
# Granularity: per token per head ([P2] section 5 "Where the scales live":
# k_scale (num_blocks, block_size, n_kv_heads) in FP16), or one scale per 32
# channels for INT4 (same section: 4 groups x 2 bytes at head_dim 128).
# --------------------------------------------------------------------------


def quantize_sym(x16: np.ndarray, fmt: str):
    """Quantize fp16 rows (..., D) -- or the fp32 rows of a rotated cache
    (rotate_rows) -- the same way.  Returns (codes, scales):
    codes int8 (INT8/INT4, values in [-q_max, q_max]) or uint8 (FP8 bytes),
    shape (..., D); scales float16 of shape (..., D // group)."""
    assert x16.dtype in (np.float16, np.float32)
    D = x16.shape[-1]
    g = INT4_GROUP if fmt == INT4_G32 else D
    x = x16.astype(np.float32).reshape(x16.shape[:-1] + (D // g, g))
    amax = np.max(np.abs(x), axis=-1)  # exact
    # Two roundings: the fp32 quotient, then fp16 for storage ([P1] section 2.1
    # keeps s in FP32; [P1] Exercise 1 step 2 and [P2] section 5 store it as
    # FP16).  The quotient below divides by the stored value.
    s32 = amax / np.float32(QMAX[fmt])
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    # A scale beyond the fp16 range (possible only for the fp32 rows of a
    # rotated cache, whose entries reach D times the largest fp16 value) is
    # stored as the largest finite fp16 value; the quotients then saturate.
    s16 = np.minimum(s16, np.float16(65504.0))
    return _codes_for_scale(x, s16, fmt).reshape(x16.shape), s16


def _codes_for_scale(x, s16, fmt):
    """Codes of fp32 groups x (..., n_groups, g) for fp16 scales s16 (...,
    n_groups): the IEEE binary32 quotient by the stored scale, then the
    format's rounding with saturation at +-q_max ([P1] section 2.1 clip);
    a zero scale gives zero codes."""
    s = s16.astype(np.float32)
    zero = s == 0
    safe = np.where(zero, np.float32(1.0), s)
    with np.errstate(over="ignore", invalid="ignore"):
        y = x / safe[..., None]  # IEEE binary32 quotient
    if fmt in FP8_FORMATS:
        c = fp8_encode(y, fmt)
        c[np.broadcast_to(zero[..., None], c.shape)] = 0
        return c
    q = QMAX[fmt]
    c = np.clip(np.rint(y), -q, q)  # rint: round half to even
    c[np.broadcast_to(zero[..., None], c.shape)] = 0
    return c.astype(np.int8)


def quantize_sym_static(x16: np.ndarray, fmt: str, s16: np.ndarray):
    """Quantize fp16 rows (..., D) with given (calibrated) fp16 scales s16 of
    shape (...,), one per row, instead of max|x| / q_max: the fixed scaling
    factors computed ahead of deployment of [P3] Implementation Best Practices
    (calibrated scaling factors) and [P4] (static calibration).  Quotients beyond +-q_max saturate.  For
    INT4 group-32 rows the row's scale serves every group.  Returns (codes,
    scales) like quantize_sym, the scales being s16 repeated per group.  Rows
    may be the fp32 rows of a rotated cache."""
    assert x16.dtype in (np.float16, np.float32) and s16.dtype == np.float16
    D = x16.shape[-1]
    g = INT4_GROUP if fmt == INT4_G32 else D
    x = x16.astype(np.float32).reshape(x16.shape[:-1] + (D // g, g))
    sg = np.broadcast_to(s16[..., None], x.shape[:-1]).astype(np.float16)
    return _codes_for_scale(x, sg, fmt).reshape(x16.shape), sg.copy()


def dequant_sym(codes: np.ndarray, scales16: np.ndarray, fmt: str) -> np.ndarray:
    """x_hat = code * s in float64 ([P1] section 2.1, Exercise 1 step 4)."""
    D = codes.shape[-1]
    g = INT4_GROUP if fmt == INT4_G32 else D
    if fmt in FP8_FORMATS:
        v = fp8_value(codes, fmt)
    else:
        v = codes.astype(np.int8).astype(np.float64)
    v = v.reshape(codes.shape[:-1] + (D // g, g))
    return (v * scales16.astype(np.float64)[..., None]).reshape(codes.shape)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte (0.5 B/element, [P1] section 2.1 table): byte j
    holds channel 2j in its low nibble and channel 2j+1 in its high nibble.
    Signed codes are stored as two's-complement nibbles."""
    n = codes.astype(np.int64) & 0xF
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray, signed: bool) -> np.ndarray:
    p = packed.astype(np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out


# --------------------------------------------------------------------------
# KIVI-style keys ([P2] section 5 "K is more sensitive than V": keys are
# quantized channel by channel, values token by token; [P3] "Numerical
# Formats": KIVI's keys are quantized per channel; [P4]: the asymmetric
# scheme stretches the observed [min, max] over the whole integer range).
# One group = 32 consecutive tokens of one head; per channel:
#   s = (max - min) / 15 (fp32, stored fp16),  z = min (stored fp16, exact),
#   code = clip(round((x - z) / s), 0, 15),     x_hat = code * s + z.
# --------------------------------------------------------------------------


def kivi_quantize_group(x16: np.ndarray):
    """x16: float16 (32, D) rows of one head.  Returns (codes uint8 (32, D) in
    0..15, scale float16 (D,), zero float16 (D,))."""
    assert x16.dtype == np.float16 and x16.shape[0] == KIVI_GROUP
    x = x16.astype(np.float32)
    mn = x.min(axis=0)
    mx = x.max(axis=0)
    s32 = (mx - mn) / np.float32(KIVI_LEVELS)  # fl32(fl32(mx - mn) / 15)
    s16 = s32.astype(np.float16)
    z16 = mn.astype(np.float16)  # exact: mn is an fp16 value
    s = s16.astype(np.float32)
    z = z16.astype(np.float32)
    zero = s == 0
    safe = np.where(zero, np.float32(1.0), s)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (x - z) / safe  # fl32(fl32(x - z) / s)
    c = np.clip(np.rint(y), 0, KIVI_LEVELS)
    c[:, zero] = 0
    return c.astype(np.uint8), s16, z16


def kivi_dequant(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    return codes.astype(np.float64) * s16.astype(np.float64) + z16.astype(np.float64)


# --------------------------------------------------------------------------
# Walsh-Hadamard rotation ([P3] "Numerical Formats": QuaRot rotates rows with
# randomized orthogonal Walsh-Hadamard transforms, so an outlier channel's
# energy is shared by every channel before the 4-bit quantizer; "Accuracy, Latency, and
# Serving Economics": rotated INT4 stays close to unquantized quality).
# Reading: the rotation of a head_dim row x is R x with R = H diag(sigma) /
# sqrt(D), H the Sylvester Hadamard matrix (entries +-1) and sigma a vector
# of random signs drawn by the caller ("randomized").  The cache stores the
# unnormalised rotation y = H (sigma * x): each entry of y is a sum of +-x_c,
# computed exactly and rounded once to fp32, and y is quantized like any row
# (its per-row scale absorbs the factor sqrt(D)).  The inverse of a stored
# row is x = sigma * (H y) / D.  Scores need no inverse on the keys side:
# q . x_hat = q' . y_hat with q' = H (sigma * q) / D.
# --------------------------------------------------------------------------


def hadamard(D: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order D (a power of two), int64 +-1:
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    H = np.ones((1, 1), np.int64)
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    assert H.shape[0] == D
    return H


def sign_vector(sign_bits, D: int) -> np.ndarray:
    """sigma (D,) float64 of +-1 from a bit array: bit c (bit c % 32 of word
    c // 32) set means sigma_c = -1."""
    w = np.asarray(sign_bits, dtype=np.uint64)
    c = np.arange(D)
    bit = (w[c // 32] >> (c % 32).astype(np.uint64)) & np.uint64(1)
    return np.where(bit == 1, -1.0, 1.0)


def rotate_rows(x16: np.ndarray, sign_bits) -> np.ndarray:
    """fp16 rows (..., D) -> fp32 rows y = H (sigma * x), each entry rounded
    once to fp32.  The float64 sums are exact: every term is an fp16 value
    (a multiple of 2^-24 below 2^16), so any partial sum of at most 256
    terms needs fewer than 53 significant bits."""
    D = x16.shape[-1]
    x = x16.astype(np.float64) * sign_vector(sign_bits, D)
    y = x @ hadamard(D).T.astype(np.float64)
    return y.astype(np.float32)


def unrotate_rows(y, sign_bits) -> np.ndarray:
    """float64 rows x = sigma * (H y) / D (the inverse of the rotation, since
    H H = D I)."""
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    return (y @ hadamard(D).T.astype(np.float64)) * sign_vector(sign_bits, D) / D


def rotate_query(q16: np.ndarray, sign_bits) -> np.ndarray:
    """float64 q' = H (sigma * q) / D: q . x_hat = q' . y_hat for the stored
    (rotated) rows y_hat of a key."""
    D = q16.shape[-1]
    return (q16.astype(np.float64) * sign_vector(sign_bits, D)) @ hadamard(D).T.astype(np.float64) / D


# --------------------------------------------------------------------------
# Paged cache ([P2] section 5: k_cache (num_blocks, block_size, n_kv_heads,
# head_dim) with k_scale (num_blocks, block_size, n_kv_heads) in FP16; [P4]
# PagedAttention: fixed-size, non-contiguous physical blocks).
# --------------------------------------------------------------------------


class OracleCache:
    """NumPy mirror of the device cache buffers, in the same layouts:
      codes  uint8  (num_blocks, block_size, H, D or D/2)
      scales fp16   (num_blocks, block_size, H, groups)  symmetric formats
             fp16   (num_blocks, H, D)                   KIVI keys
      zeros  fp16   (num_blocks, H, D)                   KIVI keys only
      k_tail, v_tail fp16 (max_seqs, block_size, H, D)   KIVI keys only
    """

    def __init__(self, num_blocks, block_size, n_kv_heads, head_dim, k_fmt, v_fmt, max_seqs=0, rot_k=None,
                 rot_v=None):
        """rot_k / rot_v: sign bits of the keys' / values' rotation (see
        rotate_rows), or None for unrotated rows.  KIVI keys are not
        rotated."""
        assert k_fmt in K_FORMATS and v_fmt in V_FORMATS
        if k_fmt == INT4_KIVI:
            assert block_size == KIVI_GROUP and rot_k is None
        self.rot_k, self.rot_v = rot_k, rot_v
        self.nb, self.bs, self.H, self.D = num_blocks, block_size, n_kv_heads, head_dim
        self.k_fmt, self.v_fmt, self.max_seqs = k_fmt, v_fmt, max_seqs
        nb, bs, H, D = num_blocks, block_size, n_kv_heads, head_dim
        self.k_codes = np.zeros((nb, bs, H, code_bytes_per_row(k_fmt, D)), np.uint8)
        self.v_codes = np.zeros((nb, bs, H, code_bytes_per_row(v_fmt, D)), np.uint8)
        if k_fmt == INT4_KIVI:
            self.k_scales = np.zeros((nb, H, D), np.float16)
            self.k_zeros = np.zeros((nb, H, D), np.float16)
            self.k_tail = np.zeros((max_seqs, bs, H, D), np.float16)
            self.v_tail = np.zeros((max_seqs, bs, H, D), np.float16)
        else:
            self.k_scales = np.zeros((nb, bs, H, groups_per_row(k_fmt, D)), np.float16)
            self.k_zeros = self.k_tail = self.v_tail = None
        self.v_scales = np.zeros((nb, bs, H, groups_per_row(v_fmt, D)), np.float16)

    def buffers(self):
        out = {"k_codes": self.k_codes, "v_codes": self.v_codes,
               "k_scales": self.k_scales, "v_scales": self.v_scales}
        if self.k_fmt == INT4_KIVI:
            out.update(k_zeros=self.k_zeros, k_tail=self.k_tail, v_tail=self.v_tail)
        return out


def _store_sym(codes_buf, scales_buf, fmt, x16_rows, slots, bs, static_s16=None, rot=None):
    """Quantize (n, H, D) rows and scatter them to flat slots (with the given
    per-head scales static_s16 (H,) when present; rotated first when rot
    holds sign bits)."""
    if rot is not None:
        x16_rows = rotate_rows(x16_rows, rot)
    if static_s16 is None:
        codes, s16 = quantize_sym(x16_rows, fmt)
    else:
        rows_s16 = np.broadcast_to(np.asarray(static_s16, np.float16)[None, :], x16_rows.shape[:2])
        codes, s16 = quantize_sym_static(x16_rows, fmt, rows_s16)
    if fmt == INT4_G32:
        stored = pack_int4(codes)
    else:
        stored = codes.view(np.uint8)
    blk, off = slots // bs, slots % bs
    codes_buf[blk, off] = stored
    scales_buf[blk, off] = s16


def write(cache: OracleCache, k16: np.ndarray, v16: np.ndarray, slot_mapping, seq_idx=None):
    """Quantize-on-write of k, v (T, H, D) fp16 into the paged cache.

    Token t goes to flat slot slot_mapping[t] = block * block_size + offset;
    a negative slot means "skip", and so does a slot past the last block
    (num_blocks * block_size or more: there is no page to hold it).
    Symmetric formats quantize each (token, head) row on its own ([P2]
    section 5: per-token, per-head scaling).

    KIVI keys: the rows of one page form one 32-token group.  A page is
    quantized when its last row (offset block_size - 1) is written; its other
    rows come from this call where present, else from the sequence's fp16
    tail (rows written by earlier calls).  Rows of pages not completed by this
    call are stored, K and V in fp16, in the tail of their sequence
    (seq_idx[t]) at their page offset.  Completion reads the tail as it was
    before this call.  V is quantized per token into its page in every case.
    A token whose seq_idx names no tail row (outside [0, max_seqs)) keeps its
    value but its key goes nowhere: it neither completes a page nor enters a
    tail.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    valid = np.nonzero(slot_in_range(cache, slots))[0]
    bs = cache.bs
    _store_sym(cache.v_codes, cache.v_scales, cache.v_fmt, v16[valid], slots[valid], bs, rot=cache.rot_v)
    if cache.k_fmt != INT4_KIVI:
        _store_sym(cache.k_codes, cache.k_scales, cache.k_fmt, k16[valid], slots[valid], bs, rot=cache.rot_k)
        return
    assert seq_idx is not None
    seq_idx = np.asarray(seq_idx, dtype=np.int64)
    pages = {}  # (seq, block) -> {offset: token index}
    for t in valid:
        if not 0 <= seq_idx[t] < cache.max_seqs:
            continue  # no tail row to keep the key in: the key is dropped
        key = (int(seq_idx[t]), int(slots[t] // bs))
        off = int(slots[t] % bs)
        assert off not in pages.setdefault(key, {}), "a slot written twice in one call"
        pages[key][off] = t
    tail_k_before = cache.k_tail.copy()
    for (seq, blk), offs in pages.items():
        if bs - 1 not in offs:
            continue
        rows = np.stack([k16[offs[j]] if j in offs else tail_k_before[seq, j] for j in range(bs)])
        for h in range(cache.H):
            c, s16, z16 = kivi_quantize_group(rows[:, h, :])
            cache.k_codes[blk, :, h, :] = pack_int4(c)
            cache.k_scales[blk, h] = s16
            cache.k_zeros[blk, h] = z16
    for (seq, blk), offs in pages.items():
        if bs - 1 in offs:
            continue
        for off, t in offs.items():
            cache.k_tail[seq, off] = k16[t]
            cache.v_tail[seq, off] = v16[t]


def slot_in_range(cache: OracleCache, slots) -> np.ndarray:
    """Whether each flat slot addresses a row of the cache: 0 <= slot <
    num_blocks * block_size."""
    slots = np.asarray(slots, dtype=np.int64)
    return (slots >= 0) & (slots < cache.nb * cache.bs)


def write_static(cache: OracleCache, k16: np.ndarray, v16: np.ndarray, slot_mapping, k_scale16, v_scale16):
    """Quantize-on-write with calibrated per-KV-head fp16 scales (H,) for K
    and V instead of the per-token amax ([P3] Implementation Best Practices,
    calibrated scaling factors; [P4] static calibration).  Symmetric formats only; every written row
    stores its head's scale in its scale slot, so reading is unchanged."""
    assert cache.k_fmt in SYM_FORMATS and cache.v_fmt in SYM_FORMATS
    slots = np.asarray(slot_mapping, dtype=np.int64)
    valid = np.nonzero(slot_in_range(cache, slots))[0]
    bs = cache.bs
    _store_sym(cache.k_codes, cache.k_scales, cache.k_fmt, k16[valid], slots[valid], bs, k_scale16, rot=cache.rot_k)
    _store_sym(cache.v_codes, cache.v_scales, cache.v_fmt, v16[valid], slots[valid], bs, v_scale16, rot=cache.rot_v)


def _dequant_rows(cache: OracleCache, which: str, blk, off):
    """float64 (n, H, D) rows of K or V at (block, offset) pairs (sym formats)."""
    fmt = cache.k_fmt if which == "k" else cache.v_fmt
    codes_buf = cache.k_codes if which == "k" else cache.v_codes
    scales_buf = cache.k_scales if which == "k" else cache.v_scales
    raw = codes_buf[blk, off]
    if fmt == INT4_G32:
        codes = unpack_int4(raw, signed=True)
    elif fmt in FP8_FORMATS:
        codes = raw
    else:
        codes = raw.view(np.int8)
    rows = dequant_sym(codes, scales_buf[blk, off], fmt)
    rot = cache.rot_k if which == "k" else cache.rot_v
    return rows if rot is None else unrotate_rows(rows, rot)


def token_live(cache: OracleCache, block_table_row, L: int) -> np.ndarray:
    """Which of a sequence's first L tokens take part in attention: those on
    a page whose block id lies in [0, num_blocks).  A page with any other id
    has no storage behind it and contributes nothing.  For KIVI keys the last
    L mod 32 tokens live in the sequence's fp16 tail and always take part."""
    bs = cache.bs
    t = np.arange(L)
    blk = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    live = (blk >= 0) & (blk < cache.nb)
    if cache.k_fmt == INT4_KIVI:
        live[(L // bs) * bs:] = True
    return live


def gather_dequant(cache: OracleCache, block_table_row, L: int, seq: int):
    """Dequantized K_hat, V_hat (L, H, D) float64 of one sequence, gathered
    through its block-table row: token t lives at block
    block_table_row[t // block_size], offset t % block_size.  For KIVI keys
    the last L mod 32 tokens are read from the sequence's fp16 tail.  Tokens
    on a page whose block id is out of range (see token_live) read block 0 in
    its place; the caller leaves them out."""
    bs = cache.bs
    t = np.arange(L)
    blk = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    blk = np.where((blk >= 0) & (blk < cache.nb), blk, 0)
    off = t % bs
    V = _dequant_rows(cache, "v", blk, off)
    if cache.k_fmt != INT4_KIVI:
        K = _dequant_rows(cache, "k", blk, off)
        return K, V
    nfull = (L // bs) * bs
    K = np.empty((L, cache.H, cache.D), np.float64)
    for p in range(nfull // bs):
        b = blk[p * bs]
        codes = unpack_int4(cache.k_codes[b], signed=False)  # (bs, H, D)
        K[p * bs:(p + 1) * bs] = kivi_dequant(codes, cache.k_scales[b][None], cache.k_zeros[b][None])
    K[nfull:] = cache.k_tail[seq, : L - nfull].astype(np.float64)
    V[nfull:] = cache.v_tail[seq, : L - nfull].astype(np.float64)
    return K, V


def dequantized_sequence(k16: np.ndarray, v16: np.ndarray, k_fmt: str, v_fmt: str, block_size: int = 32,
                         rot_k=None, rot_v=None):
    """K_hat, V_hat (L, H, D) float64 of one sequence written whole, without
    paging: what gather_dequant returns for a sequence written in position
    order.  KIVI keys: complete 32-token groups quantized per channel, the
    last L mod 32 tokens (keys and values) kept in fp16.  rot_k / rot_v:
    rotated rows (quantized after rotate_rows, returned unrotated)."""
    L = k16.shape[0]

    def sym(x16, fmt, rot):
        x = x16 if rot is None else rotate_rows(x16, rot)
        codes, s = quantize_sym(x, fmt)
        r = dequant_sym(codes, s, fmt)
        return r if rot is None else unrotate_rows(r, rot)

    V = sym(v16, v_fmt, rot_v)
    if k_fmt != INT4_KIVI:
        return sym(k16, k_fmt, rot_k), V
    assert rot_k is None
    nfull = (L // KIVI_GROUP) * KIVI_GROUP
    K = np.empty(k16.shape, np.float64)
    for p in range(nfull // KIVI_GROUP):
        sl = slice(p * KIVI_GROUP, (p + 1) * KIVI_GROUP)
        for h in range(k16.shape[1]):
            c, sc, z = kivi_quantize_group(k16[sl, h, :])
            K[sl, h, :] = kivi_dequant(c, sc, z)
    K[nfull:] = k16[nfull:].astype(np.float64)
    V[nfull:] = v16[nfull:].astype(np.float64)
    return K, V


def attention_fp64(q, K, V, sm_scale=None, live=None):
    """One decode query per head against L cached tokens, float64:
    o = softmax(q k^T * sm_scale) V  ([P2] section 5 "K is more sensitive than
    V": softmax(q.k^T / sqrt(d)) and sum_i p_i v_i), with grouped-query
    attention: query head hq reads KV head hq // G ([P4] GQA: groups of query
    heads share one key/value head).
    q: (Hq, D); K, V: (L, H, D); live: optional bool (L,), tokens to attend
    (all by default).  Returns (Hq, D); zeros when no token is attended."""
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    if live is not None:
        live = np.asarray(live, dtype=bool)
        K, V = K[live], V[live]
    L, H, _ = K.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out = np.zeros((Hq, D), np.float64)
    if L == 0:
        return out
    G = Hq // H
    for hq in range(Hq):
        h = hq // G
        s = (K[:, h, :] @ q[hq]) * sm_scale
        p = np.exp(s - s.max())
        out[hq] = (p @ V[:, h, :]) / p.sum()
    return out


def decode_attn(cache: OracleCache, q, block_table, ctx_lens, sm_scale=None, seqs=None):
    """Decode attention over the quantized paged cache, float64 (B, Hq, D).
    Sequence b attends to its first ctx_lens[b] tokens, the count taken into
    [0, pages in its block-table row * block_size]; tokens on pages whose
    block id is out of range are left out (token_live).  For KIVI keys, batch
    row b reads tail row b.  `seqs` restricts the work to a subset of batch
    rows (others are left zero)."""
    q = np.asarray(q)
    block_table = np.asarray(block_table)
    B = q.shape[0]
    out = np.zeros(q.shape, np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = min(max(int(ctx_lens[b]), 0), block_table.shape[1] * cache.bs)
        K, V = gather_dequant(cache, block_table[b], L, b)
        out[b] = attention_fp64(q[b], K, V, sm_scale, live=token_live(cache, block_table[b], L))
    return out


# --------------------------------------------------------------------------
# Chunked prefill over the cache ([P1] "What Comes Next": a long prompt is
# processed in scheduled pieces; [P2] "Interaction with prefix caching":
# quantized blocks stay shareable, so a new piece of a prompt attends to a
# prefix already in the cache).
# Reading: the n queries of a sequence's chunk are its last n positions, and
# their keys and values were written into the cache before the call; query i
# of the chunk sits at position p = L - n + i, where L is the sequence's
# context length taken into range as decode_attn takes it, and attends to
# tokens 0..p (causal decoder attention; tokens on pages with an
# out-of-range block id are left out as in decode).  A query at p < 0 (a chunk
# longer than the context) attends to nothing and gets zeros.
# --------------------------------------------------------------------------


def causal_attention_fp64(q, K, V, positions, sm_scale=None, live=None):
    """Queries q (n, Hq, D) at the given positions (n,) against K, V
    (L, H, D), float64: query i attends to the live tokens t <= positions[i]
    (attention_fp64 per query).  Returns (n, Hq, D)."""
    q = np.asarray(q, dtype=np.float64)
    L = K.shape[0]
    out = np.zeros(q.shape, np.float64)
    t = np.arange(L)
    for i, p in enumerate(np.asarray(positions, dtype=np.int64)):
        m = t <= p
        if live is not None:
            m = m & np.asarray(live, dtype=bool)
        out[i] = attention_fp64(q[i], K, V, sm_scale, live=m)
    return out


def prefill_attn(cache: OracleCache, q, q_start, block_table, ctx_lens, sm_scale=None, seqs=None, rows=None):
    """Chunked-prefill attention over the quantized paged cache, float64
    (Tq, Hq, D).  q (Tq, Hq, D) holds the chunks of all sequences one after
    the other: sequence b's queries are rows q_start[b] .. q_start[b+1] - 1.
    `seqs` restricts the work to a subset of sequences and `rows` to a subset
    of query rows (others are left zero).  For KIVI keys, sequence b reads
    tail row b."""
    q = np.asarray(q)
    q_start = np.asarray(q_start, dtype=np.int64)
    block_table = np.asarray(block_table)
    out = np.zeros(q.shape, np.float64)
    want = None if rows is None else set(int(r) for r in rows)
    for b in (range(len(q_start) - 1) if seqs is None else seqs):
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        idx = [r for r in range(r0, r1) if want is None or r in want]
        if not idx:
            continue
        L = min(max(int(ctx_lens[b]), 0), block_table.shape[1] * cache.bs)
        K, V = gather_dequant(cache, block_table[b], L, b)
        live = token_live(cache, block_table[b], L)
        pos = [L - n + (r - r0) for r in idx]
        out[idx] = causal_attention_fp64(q[idx], K, V, pos, sm_scale, live)
    return out


# --------------------------------------------------------------------------
# Offloading whole pages ([P1] section 4 "Pipelining and Latency Overlap":
# quantized blocks move between GPU memory and CPU RAM unchanged; [P1] key
# insight: quantization and offloading compose, the offloaded blocks keep
# their quantized format).
# --------------------------------------------------------------------------


def paged_buffer_names(cache: OracleCache):
    """The buffers that hold one entry per page (the KIVI tails are per
    sequence, not per page)."""
    names = ["k_codes", "v_codes", "k_scales", "v_scales"]
    if cache.k_fmt == INT4_KIVI:
        names.append("k_zeros")
    return names


def copy_blocks(src: OracleCache, dst: OracleCache, src_blocks, dst_blocks):
    """Page dst_blocks[i] of dst becomes page src_blocks[i] of src: every
    paged buffer's entry copied byte for byte, in list order."""
    assert (src.bs, src.H, src.D, src.k_fmt, src.v_fmt) == (dst.bs, dst.H, dst.D, dst.k_fmt, dst.v_fmt)
    for s_id, d_id in zip(np.asarray(src_blocks).ravel(), np.asarray(dst_blocks).ravel()):
        for name in paged_buffer_names(src):
            getattr(dst, name)[int(d_id)] = getattr(src, name)[int(s_id)]


# --------------------------------------------------------------------------
# Closed forms ([P1] Exercise 3 and [P3] "The Mathematics of KV Cache
# Growth": bytes per token = 2 * layers * kv_heads * head_dim * bytes/element;
# [P2] section 5 scale overheads).
# --------------------------------------------------------------------------


def kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_elem):
    return 2 * n_layers * n_kv_heads * head_dim * bytes_per_elem


def stored_bytes_per_token_head(fmt: str, head_dim: int) -> float:
    """Codes + scale metadata per (token, head) as stored by OracleCache.
    KIVI keys amortise one fp16 scale and one fp16 zero per channel over a
    32-token group."""
    if fmt == INT4_KIVI:
        return head_dim / 2 + 2 * 2 * head_dim / KIVI_GROUP
    return code_bytes_per_row(fmt, head_dim) + 2 * groups_per_row(fmt, head_dim)
