"""Pins for the CPU oracle: values printed on the pages, closed forms,
invariants, brute force and an independent library routine.  These run on the
CPU only (no GPU, no HIP library)."""

import math

import numpy as np
import pytest
import torch

import oracle as o
from conftest import read_golden

RNG = np.random.default_rng(1234)

# --------------------------------------------------------------------------
# check_* helpers take the function under test so that tests/test_oracle_
# mutations.py can show that planted mistakes fail them.
# --------------------------------------------------------------------------


def check_worked_example(quantize_sym=o.quantize_sym):
    """'Use Less Memory', Exercise 1: k = [1.20, -0.45, 3.80, -2.10] in FP16,
    per-token symmetric INT8 -> codes [40, -15, 127, -70]."""
    g = read_golden("worked_example_int8.txt")
    x16 = np.array([g["input"]], dtype=np.float16)
    codes, s16 = quantize_sym(x16, o.INT8)
    assert codes[0].tolist() == [int(c) for c in g["codes"]]
    s = float(s16[0, 0])
    # The page computes s from the decimal 3.80; the fp16 input is 3.8008 and
    # the stored scale is fp16.  Within one fp16 ulp of the page's value.
    assert abs(s - g["scale"]) <= 2.0 ** -16
    xhat = codes[0].astype(np.float64) * s
    # The page prints x_hat rounded to 5 decimals from its decimal s; the
    # stored fp16 scale differs from that s by less than 2^-16, so each x_hat
    # may differ by |code| * 2^-16 plus the printing's half unit.
    assert np.all(np.abs(xhat - np.array(g["recon"])) <= np.abs(codes[0]) * 2.0 ** -16 + 5e-6)
    # Errors as the page's table defines them: against the decimal originals.
    orig = np.array(g["input"])
    err = np.abs(xhat - orig)
    assert err.max() <= g["max_abs_err"]
    assert np.all(err <= np.array(g["abs_err"]) + np.abs(codes[0]) * 2.0 ** -16 + 5e-6)
    rel = err / np.abs(orig)
    assert rel.max() <= g["max_rel_err"] + 5e-5


def check_round_half_even(quantize_sym=o.quantize_sym):
    # s16 is exactly 2^-4 (7.9375 / 127); the other elements sit exactly on
    # half-integers of the quotient, so rounding must go to the even code.
    x16 = np.array([[7.9375, 0.15625, 0.21875, -0.15625, -0.21875, 0.03125]], np.float16)
    codes, s16 = quantize_sym(x16, o.INT8)
    assert float(s16[0, 0]) == 0.0625
    assert codes[0].tolist() == [127, 2, 4, -2, -4, 0]


def _bulk_rows(fmt, n=20000, D=128, seed=7):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)).astype(np.float32)
    # mix of magnitudes: outlier channels, tiny rows, exact zeros, large rows
    x[:, :4] *= 20
    x[: n // 8] *= np.float32(1e-3)
    x[n // 8: n // 4] *= np.float32(300)
    x[-5:] = 0
    x16 = x.astype(np.float16)
    return x16


def check_sym_invariants(quantize_sym=o.quantize_sym, dequant=o.dequant_sym, fmts=o.SYM_FORMATS):
    for fmt in fmts:
        x16 = _bulk_rows(fmt)
        codes, s16 = quantize_sym(x16, fmt)
        D = x16.shape[-1]
        g = o.INT4_GROUP if fmt == o.INT4_G32 else D
        x = x16.astype(np.float64).reshape(-1, D // g, g)
        s = s16.astype(np.float64)
        xhat = dequant(codes, s16, fmt).reshape(x.shape)
        q = o.QMAX[fmt]
        normal = s >= 2.0 ** -14  # s16 is a normal fp16 number
        # 1. the largest-magnitude element lands on +-q_max ('Use Less Memory',
        #    Exercise 1 step 3: the absmax element maps to the top code)
        idx = np.argmax(np.abs(x), axis=-1)
        top = np.take_along_axis(xhat, idx[..., None], -1)[..., 0]
        topx = np.take_along_axis(x, idx[..., None], -1)[..., 0]
        ok = normal & (topx != 0)
        assert np.all(np.abs(top[ok] / s[ok]) == q), fmt
        # 2. reconstruction error bound, half a step of the target grid at the
        #    quotient (FP8: 2^(e - m - 1) for a normal quotient in [2^e, 2^(e+1)),
        #    m mantissa bits, and half the subnormal step below 2^emin)
        err = np.abs(x - xhat)
        y = np.abs(x) / np.where(s == 0, 1, s)[..., None]
        if fmt in o.FP8_FORMATS:
            mbits, emin = (3, -6) if fmt == o.FP8_E4M3FN else (2, -14)
            e = np.floor(np.log2(np.maximum(y, 2.0 ** emin)))
            half_step = np.where(y < 2.0 ** emin, 2.0 ** (emin - mbits - 1), 2.0 ** (e - mbits - 1))
            top_half = 2.0 ** (math.floor(math.log2(q)) - mbits - 1)
            bound = s[..., None] * half_step * (1 + 2.0 ** -20)
        else:
            top_half = 0.5
            bound = s[..., None] * (0.5 + 2.0 ** -17)
        bound = np.broadcast_to(bound, x.shape)
        # A quotient beyond q_max plus half a step saturates.  That happens
        # only when s16 rounded well below s32, i.e. in the fp16 subnormal
        # range; a normal s16 keeps every quotient within q_max (1 + 2^-11).
        sat = (s > 0) & (np.max(y, axis=-1) > q + top_half)
        assert not np.any(sat & normal), fmt
        nz = np.broadcast_to(((s > 0) & ~sat)[..., None], x.shape)
        assert np.all(err[nz] <= bound[nz]), fmt
        # 3. codes in range and carrying the sign of x
        vals = xhat / np.where(s == 0, 1, s)[..., None]
        assert np.all(np.abs(vals) <= q), fmt
        assert np.all((vals == 0) | (np.sign(vals) == np.sign(x))), fmt
        # 4. zero rows give scale 0 and code 0
        assert np.all(s[-5:] == 0) and np.all(xhat[-5:] == 0)


def check_fp8_bruteforce(encode=o.e4m3fn_encode):
    # All finite E4M3FN values, magnitude side, by code.
    mags = o.e4m3fn_value(np.arange(0x7F))  # codes 0x00..0x7E
    assert mags[-1] == 448.0
    # Every fp16 bit pattern (finite) taken as a quotient y, plus random fp32.
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    y = h[np.isfinite(h)].astype(np.float32)
    rnd = (np.random.default_rng(5).standard_normal(200000) *
           np.exp2(np.random.default_rng(6).uniform(-14, 10, 200000))).astype(np.float32)
    y = np.concatenate([y, rnd])
    a = np.abs(y).astype(np.float64)
    # nearest finite magnitude, ties to the even code; beyond 448 saturate.
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1)
    cand = d == best[:, None]
    codes = np.arange(0x7F)
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 999).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 999).min(axis=1)
    ties = cand.sum(axis=1) > 1
    expect = np.where(ties, even_pick, any_pick)
    expect = np.where(a > 448, 0x7E, expect) | np.where(np.signbit(y), 0x80, 0)
    got = encode(y)
    assert np.array_equal(got.astype(np.int64), expect.astype(np.int64))


def check_e5m2_bruteforce(encode=o.e5m2_encode):
    # All finite E5M2 magnitudes, by code (0x7C is +inf, 0x7D..0x7F NaN).
    mags = o.e5m2_value(np.arange(0x7C))  # codes 0x00..0x7B
    assert mags[-1] == 57344.0
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    y = h[np.isfinite(h)].astype(np.float32)
    rnd = (np.random.default_rng(8).standard_normal(200000) *
           np.exp2(np.random.default_rng(9).uniform(-20, 18, 200000))).astype(np.float32)
    y = np.concatenate([y, rnd])
    a = np.abs(y).astype(np.float64)
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1)
    cand = d == best[:, None]
    codes = np.arange(0x7C)
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 999).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 999).min(axis=1)
    ties = cand.sum(axis=1) > 1
    expect = np.where(ties, even_pick, any_pick)
    expect = np.where(a > 57344, 0x7B, expect) | np.where(np.signbit(y), 0x80, 0)
    got = encode(y)
    assert np.array_equal(got.astype(np.int64), expect.astype(np.int64))


def check_e5m2_specials(encode=o.e5m2_encode):
    cases = [(57344.0, 0x7B), (61440.0, 0x7B), (65504.0, 0x7B), (1e9, 0x7B), (-1e9, 0xFB),
             (2.0 ** -16, 0x01), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02), (2.0 ** -14, 0x04),
             (1.0, 0x3C), (1.125, 0x3C), (1.375, 0x3E), (-0.0, 0x80), (0.0, 0x00), (-1e-9, 0x80)]
    for y, c in cases:
        assert int(encode(np.array([y], np.float32))[0]) == c, (y, hex(c))


def check_fp8_specials(encode=o.e4m3fn_encode):
    cases = [(448.0, 0x7E), (464.0, 0x7E), (465.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE),
             (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08),
             (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A), (-0.0, 0x80), (0.0, 0x00), (-1e-9, 0x80)]
    for y, c in cases:
        assert int(encode(np.array([y], np.float32))[0]) == c, (y, hex(c))


def check_pack_order(pack=o.pack_int4):
    assert pack(np.array([[1, 2]], np.int8))[0, 0] == 0x21
    assert pack(np.array([[-1, 7]], np.int8))[0, 0] == 0x7F
    assert pack(np.array([[-7, 0]], np.int8))[0, 0] == 0x09


def check_closed_forms(stored=o.stored_bytes_per_token_head, kvb=o.kv_bytes_per_token):
    g = read_golden("closed_forms.txt")
    L, H, D = int(g["llama3_8b_layers"]), int(g["llama3_8b_kv_heads"]), int(g["llama3_8b_head_dim"])
    assert kvb(L, H, D, 2) == g["bytes_per_token_fp16"]
    assert kvb(L, H, D, 1) == g["bytes_per_token_fp8"]
    assert kvb(L, H, D, 0.5) == g["bytes_per_token_int4"]
    assert round(kvb(L, H, D, 2) * 32768 / 1e9, 2) == g["per_seq_gb_fp16_32k"]
    assert round(kvb(L, H, D, 1) * 32768 / 1e9, 2) == g["per_seq_gb_fp8_32k"]
    assert round(kvb(L, H, D, 0.5) * 32768 / 1e9, 2) == g["per_seq_gb_int4_32k"]
    int8 = stored(o.INT8, 128)
    assert int8 == g["int8_d128_data_bytes"] + g["int8_d128_scale_bytes"]
    assert round(100 * (int8 - 128) / 128, 1) == g["int8_d128_overhead_pct"]
    assert stored(o.FP8_E4M3FN, 128) == int8
    i4 = stored(o.INT4_G32, 128)
    assert i4 == g["int4_g32_d128_bytes"]
    assert math.floor(10 * g["fp16_d128_bytes"] / i4) / 10 == g["int4_g32_ratio"]


# --------------------------------------------------------------------------
# Tests
# --------------------------------------------------------------------------


def test_worked_example():
    check_worked_example()


def test_round_half_even():
    check_round_half_even()


def test_sym_invariants():
    check_sym_invariants()


def test_fp8_bruteforce():
    check_fp8_bruteforce()


def test_fp8_specials():
    check_fp8_specials()


def test_e5m2_bruteforce():
    check_e5m2_bruteforce()


def test_e5m2_specials():
    check_e5m2_specials()


def test_e5m2_decode_table():
    vals = o.e5m2_value(np.arange(256))
    fin = np.isfinite(vals)
    assert fin.sum() == 248  # +-inf and six NaN codes in exponent field 31
    assert vals[0x7C] == np.inf and vals[0xFC] == -np.inf and np.isnan(vals[0x7D])
    g = read_golden("closed_forms.txt")
    assert vals[0x7B] == g["e5m2_max"] and vals[0xFB] == -g["e5m2_max"] and vals[0x01] == 2.0 ** -16
    octave = vals[(vals >= 1.0) & (vals < 2.0)]
    assert len(octave) == g["e5m2_levels_per_octave"]
    # E5M2 is the upper byte of an fp16 value: the same bits read as fp16
    as16 = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    assert np.array_equal(as16[fin], vals[fin])
    codes = np.arange(256)[fin]
    assert np.array_equal(o.e5m2_encode(vals[fin].astype(np.float32)), codes.astype(np.uint8))


def test_e5m2_matches_torch_cast():
    # torch's CPU float8_e5m2 cast is an independent RNE implementation; it
    # overflows to infinity from 61440 up instead of saturating, so compare
    # below that.
    rng = np.random.default_rng(12)
    y = (rng.standard_normal(400000) * np.exp2(rng.uniform(-22, 16, 400000))).astype(np.float32)
    y = y[np.abs(y) < 61440]
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) < 61440)]
    y = np.concatenate([y, h])
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(o.e5m2_encode(y), ref)


def test_fp8_decode_table():
    vals = o.e4m3fn_value(np.arange(256))
    fin = np.isfinite(vals)
    assert fin.sum() == 254  # two NaN codes, no infinities
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0 and vals[0x01] == 2.0 ** -9
    # 8 levels per power of two ('Quantized KV caches in production',
    # Numerical Formats)
    g = read_golden("closed_forms.txt")
    octave = vals[(vals >= 1.0) & (vals < 2.0)]
    assert len(octave) == g["e4m3_levels_per_octave"]
    # every finite code round-trips through the encoder
    codes = np.arange(256)[fin]
    assert np.array_equal(o.e4m3fn_encode(vals[fin].astype(np.float32)), codes.astype(np.uint8))


def test_fp8_matches_torch_cast():
    # torch's CPU float8_e4m3fn cast is an independent RNE implementation; it
    # does not saturate (gives NaN) from 464 up, so compare below that.
    rng = np.random.default_rng(11)
    y = (rng.standard_normal(400000) * np.exp2(rng.uniform(-16, 9, 400000))).astype(np.float32)
    y = y[np.abs(y) < 464]
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    h = h[np.isfinite(h) & (np.abs(h) < 464)]
    y = np.concatenate([y, h])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3fn_encode(y), ref)


def test_pack_int4():
    check_pack_order()
    c = np.array(np.meshgrid(np.arange(-7, 8), np.arange(-7, 8))).reshape(2, -1).T.astype(np.int8)
    assert np.array_equal(o.unpack_int4(o.pack_int4(c), signed=True), c)
    u = np.array(np.meshgrid(np.arange(16), np.arange(16))).reshape(2, -1).T.astype(np.uint8)
    assert np.array_equal(o.unpack_int4(o.pack_int4(u), signed=False), u)


def test_closed_forms():
    check_closed_forms()


def test_cache_buffer_sizes_match_closed_forms():
    nb, bs, H, D = 6, 32, 2, 128
    for kf, vf in [(o.INT8, o.INT8), (o.FP8_E4M3FN, o.INT4_G32), (o.INT4_KIVI, o.INT4_G32)]:
        c = o.OracleCache(nb, bs, H, D, kf, vf, max_seqs=1)
        k_bytes = c.k_codes.nbytes + c.k_scales.nbytes + (c.k_zeros.nbytes if c.k_zeros is not None else 0)
        v_bytes = c.v_codes.nbytes + c.v_scales.nbytes
        assert k_bytes / (nb * bs * H) == o.stored_bytes_per_token_head(kf, D)
        assert v_bytes / (nb * bs * H) == o.stored_bytes_per_token_head(vf, D)
    assert o.stored_bytes_per_token_head(o.INT4_KIVI, 128) == 80


def check_kivi_invariants(kivi=o.kivi_quantize_group, deq=o.kivi_dequant):
    rng = np.random.default_rng(3)
    for trial in range(200):
        x = rng.standard_normal((32, 64)).astype(np.float32)
        x[:, :3] *= 20
        x[:4] *= 10
        x[:, 5] += 3  # skewed channel
        x[:, 6] = 0.5  # constant channel -> scale 0
        x16 = x.astype(np.float16)
        c, s16, z16 = kivi(x16)
        xf = x16.astype(np.float64)
        s = s16.astype(np.float64)
        assert c.min() >= 0 and c.max() <= 15
        normal = s >= 2.0 ** -14
        # [P4]: asymmetric quantization maps min and max to the integer range ends
        amin = np.argmin(xf, axis=0)
        amax = np.argmax(xf, axis=0)
        cols = np.arange(64)
        assert np.all(c[amin, cols][normal] == 0)
        assert np.all(c[amax, cols][normal] == 15)
        assert np.all(z16.astype(np.float64) == xf.min(axis=0))
        xh = deq(c, s16, z16)
        err = np.abs(xh - xf)
        assert np.all(err[:, s > 0] <= (s * (0.5 + 2.0 ** -10))[None, s > 0])
        assert np.all(xh[:, 6] == 0.5)


def test_kivi_invariants():
    check_kivi_invariants()


def test_kivi_bruteforce_levels():
    # The code is the nearest of the 16 levels z + c*s to x (checked on the
    # fp32 quotient grid, so an exact tie cannot flip the decision).
    rng = np.random.default_rng(9)
    x16 = (rng.standard_normal((32, 16)) * 3).astype(np.float16)
    c, s16, z16 = o.kivi_quantize_group(x16)
    s, z = s16.astype(np.float64), z16.astype(np.float64)
    levels = z[None, :, None] + np.arange(16)[None, None, :] * s[None, :, None]
    d = np.abs(x16.astype(np.float64)[:, :, None] - levels)
    best = d.min(axis=-1)
    chosen = np.take_along_axis(d, c[..., None].astype(np.int64), -1)[..., 0]
    assert np.all(chosen <= best + s[None, :] * 2.0 ** -18)


# --------------------------------------------------------------------------
# Attention and paging
# --------------------------------------------------------------------------


def _sdpa_fp64(q, K, V, G):
    qt = torch.from_numpy(q)[None, :, None, :]  # (1, Hq, 1, D)
    kt = torch.from_numpy(K.transpose(1, 0, 2).copy())[None]  # (1, H, L, D)
    vt = torch.from_numpy(V.transpose(1, 0, 2).copy())[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, enable_gqa=G > 1)
    return out[0, :, 0, :].numpy()


def check_attention_vs_sdpa(attn=o.attention_fp64):
    rng = np.random.default_rng(21)
    for (Hq, H, D, L) in [(4, 2, 64, 37), (8, 8, 32, 5), (16, 2, 128, 300), (6, 3, 16, 1)]:
        q = rng.standard_normal((Hq, D))
        K = rng.standard_normal((L, H, D)) * 3
        V = rng.standard_normal((L, H, D))
        ref = _sdpa_fp64(q, K, V, Hq // H)
        got = attn(q, K, V)
        assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_vs_sdpa():
    check_attention_vs_sdpa()


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((1, 2, 16))
    V = rng.standard_normal((1, 2, 16))
    q = rng.standard_normal((4, 16))
    out = o.attention_fp64(q, K, V)
    assert np.array_equal(out, V[0][[0, 0, 1, 1]])  # ctx 1 -> v_0 of the head
    K = rng.standard_normal((50, 2, 16))
    V = rng.standard_normal((50, 2, 16))
    out = o.attention_fp64(np.zeros((4, 16)), K, V)
    assert np.allclose(out, V.mean(axis=0)[[0, 0, 1, 1]], atol=1e-14)
    assert np.array_equal(o.attention_fp64(q, K[:0], V[:0]), np.zeros((4, 16)))


def _make_seq_cache(kf, vf, L, bs, H, D, table, seed=0, seqs=1):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((seqs * L, H, D)).astype(np.float16)
    v = rng.standard_normal((seqs * L, H, D)).astype(np.float16)
    nb = int(np.max(table)) + 1
    c = o.OracleCache(nb, bs, H, D, kf, vf, max_seqs=seqs)
    pos = np.tile(np.arange(L), seqs)
    seq = np.repeat(np.arange(seqs), L)
    slots = table[seq, pos // bs].astype(np.int64) * bs + pos % bs
    o.write(c, k, v, slots, seq)
    return c, k, v


@pytest.mark.parametrize("kf,vf", [(o.INT8, o.INT8), (o.FP8_E4M3FN, o.FP8_E4M3FN), (o.FP8_E5M2, o.FP8_E5M2),
                                   (o.INT8, o.INT4_G32), (o.INT4_G32, o.INT4_G32), (o.INT4_G32, o.FP8_E4M3FN),
                                   (o.INT4_KIVI, o.INT4_G32)])
def test_paged_gather_equals_direct_quantization(kf, vf):
    # Writing through a shuffled block table and reading back through it gives
    # exactly the dequantized rows in position order.
    bs, H, D, L = (32 if kf == o.INT4_KIVI else 16), 2, 64, 101
    npages = -(-L // bs)
    table = np.random.default_rng(4).permutation(npages + 3)[:npages][None]
    c, k, v = _make_seq_cache(kf, vf, L, bs, H, D, table)
    K, V = o.gather_dequant(c, table[0], L, 0)
    K2, V2 = o.dequantized_sequence(k, v, kf, vf)
    assert np.array_equal(K, K2) and np.array_equal(V, V2)
    codes, s = o.quantize_sym(v, vf)
    assert np.array_equal(V[: (L // bs) * bs if kf == o.INT4_KIVI else L],
                          o.dequant_sym(codes, s, vf)[: (L // bs) * bs if kf == o.INT4_KIVI else L])
    if kf == o.INT4_KIVI:
        nf = (L // bs) * bs
        for p in range(L // bs):
            for h in range(H):
                cc, ss, zz = o.kivi_quantize_group(k[p * bs:(p + 1) * bs, h])
                assert np.array_equal(K[p * bs:(p + 1) * bs, h], o.kivi_dequant(cc, ss, zz))
        assert np.array_equal(K[nf:], k[nf:].astype(np.float64))
        assert np.array_equal(V[nf:], v[nf:].astype(np.float64))
    else:
        codes, s = o.quantize_sym(k, kf)
        assert np.array_equal(K, o.dequant_sym(codes, s, kf))


def test_block_permutation_invariance():
    bs, H, D, L = 16, 2, 32, 77
    n = -(-L // bs)
    ident = np.arange(n)[None]
    shuf = np.random.default_rng(8).permutation(n + 5)[:n][None]
    q = np.random.default_rng(1).standard_normal((1, 4, D)).astype(np.float16)
    c1, *_ = _make_seq_cache(o.INT8, o.INT4_G32, L, bs, H, D, ident)
    c2, *_ = _make_seq_cache(o.INT8, o.INT4_G32, L, bs, H, D, shuf)
    a = o.decode_attn(c1, q, ident, [L])
    b = o.decode_attn(c2, q, shuf, [L])
    assert np.array_equal(a, b)


def test_negative_slots_are_skipped():
    c = o.OracleCache(4, 16, 2, 32, o.INT8, o.INT8)
    k = np.ones((3, 2, 32), np.float16)
    o.write(c, k, k, np.array([-1, 5, -7]))
    assert np.count_nonzero(c.k_codes) == 2 * 32 and np.all(c.k_codes[0, 5].view(np.int8) == 127)


def test_kivi_incremental_equals_one_shot():
    # A sequence written in one call, or token by token as in decoding, ends
    # in the same cache state (codes, scales, zeros, the valid tail rows).
    bs, H, D, L = 32, 2, 32, 75
    n = -(-L // bs)
    table = np.random.default_rng(12).permutation(n)[None]
    a, k, v = _make_seq_cache(o.INT4_KIVI, o.INT4_G32, L, bs, H, D, table, seed=3)
    b = o.OracleCache(n, bs, H, D, o.INT4_KIVI, o.INT4_G32, max_seqs=1)
    pos = np.arange(L)
    slots = table[0, pos // bs].astype(np.int64) * bs + pos % bs
    # prefill of 40 tokens, then one token per call
    o.write(b, k[:40], v[:40], slots[:40], np.zeros(40, np.int32))
    for t in range(40, L):
        o.write(b, k[t:t + 1], v[t:t + 1], slots[t:t + 1], np.zeros(1, np.int32))
    for name in ("k_codes", "k_scales", "k_zeros", "v_codes", "v_scales"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    m = L % bs
    assert np.array_equal(a.k_tail[0, :m], b.k_tail[0, :m]) and np.array_equal(a.v_tail[0, :m], b.v_tail[0, :m])
    q = np.random.default_rng(0).standard_normal((1, 4, D)).astype(np.float16)
    assert np.array_equal(o.decode_attn(a, q, table, [L]), o.decode_attn(b, q, table, [L]))


def test_quantized_attention_close_to_fp16_attention():
    # Quality statistic sanity: INT8 per-token-head keys/values stay close to
    # unquantized attention ('Use Less Memory', section 2.4: INT8 near-lossless).
    bs, H, D, L = 16, 2, 64, 200
    n = -(-L // bs)
    table = np.arange(n)[None]
    c, k, v = _make_seq_cache(o.INT8, o.INT8, L, bs, H, D, table, seed=5)
    q = np.random.default_rng(6).standard_normal((1, 4, D)).astype(np.float16)
    a = o.decode_attn(c, q, table, [L])[0]
    ref = o.attention_fp64(q[0].astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    assert np.max(np.abs(a - ref)) < 2e-2


# --------------------------------------------------------------------------
# Static (calibrated) scales
# --------------------------------------------------------------------------


def check_static_reduces_to_dynamic(quantize_static=o.quantize_sym_static):
    # With the scale the dynamic path would store, the static path must give
    # the dynamic codes (the dynamic path is pinned above).
    for fmt in o.SYM_FORMATS:
        x16 = _bulk_rows(fmt, n=3000, seed=21)
        codes, s16 = o.quantize_sym(x16, fmt)
        if fmt == o.INT4_G32:
            continue  # one dynamic scale per group, the static path has one per row
        c2, s2 = quantize_static(x16, fmt, s16[..., 0])
        assert np.array_equal(np.asarray(c2).view(np.uint8), np.asarray(codes).view(np.uint8)), fmt
        assert np.array_equal(s2.view(np.uint16), s16.view(np.uint16)), fmt


def check_static_saturation_bruteforce(quantize_static=o.quantize_sym_static):
    # Scales well below max|x| / q_max: every element goes to the nearest
    # level of the format's grid times s, ties to the even code, and
    # quotients beyond the grid saturate at +-q_max.  Integer formats by brute
    # force over the levels; FP8 formats through the pinned encoders.
    rng = np.random.default_rng(31)
    x16 = (rng.standard_normal((400, 64)) * 3).astype(np.float16)
    x16[0, :4] = [0.0, -0.0, 1.5, -2.5]
    for fmt in o.SYM_FORMATS:
        q = o.QMAX[fmt]
        s16 = (np.abs(x16.astype(np.float32)).max(axis=-1) / np.float32(q) * np.float32(0.3)).astype(np.float16)
        s16[0] = np.float16(1.0)  # exact half-way quotients in row 0
        s16[1] = np.float16(0.0)  # a zero scale: all codes 0
        codes, sg = quantize_static(x16, fmt, s16)
        g = o.INT4_GROUP if fmt == o.INT4_G32 else 64
        assert sg.shape == (400, 64 // g) and np.all(sg.view(np.uint16) == s16.view(np.uint16)[:, None])
        s = s16.astype(np.float32)[:, None]
        y = (x16.astype(np.float32) / np.where(s == 0, 1, s)).astype(np.float64)
        if fmt in o.FP8_FORMATS:
            expect = o.fp8_encode(y.astype(np.float32), fmt)
            top = o.E4M3FN_MAX_CODE if fmt == o.FP8_E4M3FN else o.E5M2_MAX_CODE
            big = np.abs(y) > q
            assert np.all((expect[big] & 0x7F) == top)
        else:
            levels = np.arange(-int(q), int(q) + 1)
            d = np.abs(y[..., None] - levels)
            best = d.min(axis=-1, keepdims=True)
            cand = d == best
            even = np.where(cand & (levels % 2 == 0), levels, 999).min(axis=-1)
            anyl = np.where(cand, levels, 999).min(axis=-1)
            expect = np.where(cand.sum(axis=-1) > 1, even, anyl)
        expect = np.asarray(expect).copy()
        expect[1] = 0
        got = np.asarray(codes)
        if fmt in o.FP8_FORMATS:
            assert np.array_equal(got.astype(np.uint8), expect.astype(np.uint8)), fmt
        else:
            assert np.array_equal(got.astype(np.int64), expect.astype(np.int64)), fmt
            assert np.abs(got).max() == q  # saturation reached


def test_static_reduces_to_dynamic():
    check_static_reduces_to_dynamic()


def test_static_saturation_bruteforce():
    check_static_saturation_bruteforce()


def test_static_write_layout():
    # write_static stores each head's scale in every written row's slot and
    # leaves skipped slots alone; reading it back uses the ordinary path.
    rng = np.random.default_rng(41)
    H, D, bs = 2, 64, 16
    k16 = (rng.standard_normal((40, H, D)) * 2).astype(np.float16)
    v16 = (rng.standard_normal((40, H, D))).astype(np.float16)
    slots = rng.permutation(4 * bs)[:40].astype(np.int64)
    slots[5] = -1
    ks = np.array([0.02, 0.05], np.float16)
    vs = np.array([0.5, 0.01], np.float16)
    c = o.OracleCache(4, bs, H, D, o.INT8, o.INT4_G32)
    o.write_static(c, k16, v16, slots, ks, vs)
    blk, off = slots // bs, slots % bs
    m = slots >= 0
    assert np.all(c.k_scales[blk[m], off[m], :, 0].view(np.uint16) == ks.view(np.uint16))
    assert np.all(c.v_scales[blk[m], off[m]].view(np.uint16) == vs.view(np.uint16)[:, None])
    codes, _ = o.quantize_sym_static(k16[m], o.INT8, np.broadcast_to(ks, (m.sum(), H)).astype(np.float16))
    assert np.array_equal(c.k_codes[blk[m], off[m]].view(np.int8), codes)
    skipped = np.setdiff1d(np.arange(4 * bs), slots[m])
    assert np.all(c.k_codes[skipped // bs, skipped % bs] == 0)


def test_static_write_int4_group32_keys():
    # INT4 group-32 keys with calibrated per-head scales: every group slot of
    # a written row holds its head's scale, and the read-back keys obey the
    # symmetric-quantizer bounds: |x - x_hat| <= s/2 where |x|/s <= 7, and
    # x_hat = +-7 s (the sign of x) beyond.
    rng = np.random.default_rng(43)
    H, D, bs, n = 2, 64, 16, 30
    k16 = (rng.standard_normal((n, H, D)) * 0.3).astype(np.float16)
    v16 = rng.standard_normal((n, H, D)).astype(np.float16)
    slots = rng.permutation(3 * bs)[:n].astype(np.int64)
    ks = np.array([0.05, 0.02], np.float16)  # head 1 saturates often
    vs = np.array([0.02, 0.03], np.float16)
    c = o.OracleCache(3, bs, H, D, o.INT4_G32, o.INT8)
    o.write_static(c, k16, v16, slots, ks, vs)
    blk, off = slots // bs, slots % bs
    assert c.k_scales.shape[-1] == D // 32
    assert np.all(c.k_scales[blk, off].view(np.uint16) == ks.view(np.uint16)[None, :, None])
    for i in range(n):
        for h in range(H):
            x = k16[i, h].astype(np.float64)
            s_ = float(ks[h])
            xh = o.dequant_sym(o.unpack_int4(c.k_codes[blk[i], off[i], h], signed=True),
                               c.k_scales[blk[i], off[i], h], o.INT4_G32)
            inside = np.abs(x) / s_ <= 7
            assert np.all(np.abs(x - xh)[inside] <= s_ / 2 * (1 + 2.0 ** -20))
            assert np.array_equal(xh[~inside], 7 * s_ * np.sign(x[~inside]))
    assert (np.abs(k16[:, 1].astype(np.float64)) / float(ks[1]) > 7).any()


# --------------------------------------------------------------------------
# Several sequences in one cache: routing of tokens to pages and tails, and of
# batch rows to block-table rows, context lengths and tails
# --------------------------------------------------------------------------


def _three_sequences(kf, vf, ctx, bs, H=2, D=32, seed=40):
    """fp16 K/V of len(ctx) sequences, a shuffled block table over a pool
    with spare blocks, and per-token slots and sequence indices."""
    rng = np.random.default_rng(seed)
    pages = [-(-L // bs) for L in ctx]
    nb = sum(pages) + 3
    perm = rng.permutation(nb)
    table = np.zeros((len(ctx), max(pages)), np.int64)
    o_ = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[o_:o_ + n]
        o_ += n
    ks = [(rng.standard_normal((L, H, D)) * (1 + b)).astype(np.float16) for b, L in enumerate(ctx)]
    vs = [rng.standard_normal((L, H, D)).astype(np.float16) for L in ctx]
    slots = [table[b, np.arange(L) // bs] * bs + np.arange(L) % bs for b, L in enumerate(ctx)]
    return nb, table, ks, vs, slots


def check_multi_sequence_routing(write=o.write, decode=o.decode_attn):
    # Three sequences written interleaved (a prefill chunk holding part of
    # every sequence, then one token per sequence per call, as decoding does)
    # and decoded in one batch must give, row by row, the attention of each
    # sequence quantized on its own.  KIVI tails of lengths 0, 1 and 31.
    for kf, vf in ((o.INT4_KIVI, o.INT4_G32), (o.INT8, o.INT4_G32), (o.FP8_E4M3FN, o.INT8)):
        bs = 32 if kf == o.INT4_KIVI else 16
        ctx = [64, 33, 95]
        H, D, Hq = 2, 32, 4
        nb, table, ks, vs, slots = _three_sequences(kf, vf, ctx, bs, H, D)
        c = o.OracleCache(nb, bs, H, D, kf, vf, max_seqs=len(ctx))
        pre = [20, 9, 40]
        cat = lambda parts: np.concatenate(parts)  # noqa: E731
        write(c, cat([k[:p] for k, p in zip(ks, pre)]), cat([v[:p] for v, p in zip(vs, pre)]),
              cat([s[:p] for s, p in zip(slots, pre)]), cat([np.full(p, b, np.int32) for b, p in enumerate(pre)]))
        for t in range(min(pre), max(ctx)):
            bb = [b for b in range(len(ctx)) if pre[b] <= t < ctx[b]]
            if bb:
                write(c, np.stack([ks[b][t] for b in bb]), np.stack([vs[b][t] for b in bb]),
                      np.array([slots[b][t] for b in bb]), np.array(bb, np.int32))
        q = np.random.default_rng(41).standard_normal((len(ctx), Hq, D)).astype(np.float16)
        got = decode(c, q, table, ctx)
        for b in range(len(ctx)):
            K, V = o.dequantized_sequence(ks[b], vs[b], kf, vf)
            ref = o.attention_fp64(q[b].astype(np.float64), K, V)
            assert np.max(np.abs(got[b] - ref)) <= 1e-12, (kf, vf, b)


def test_multi_sequence_routing():
    check_multi_sequence_routing()


def test_out_of_range_slots_are_skipped():
    # A slot at or past num_blocks * block_size addresses no row: the write
    # equals the write of the other tokens alone (and raises nothing).
    rng = np.random.default_rng(42)
    k = rng.standard_normal((6, 2, 32)).astype(np.float16)
    slots = np.array([3, 64, 17, 1000, -2, 63])
    a = o.OracleCache(4, 16, 2, 32, o.INT8, o.INT4_G32)
    b = o.OracleCache(4, 16, 2, 32, o.INT8, o.INT4_G32)
    o.write(a, k, k, slots)
    keep = np.array([0, 2, 5])
    o.write(b, k[keep], k[keep], slots[keep])
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert np.array_equal(o.slot_in_range(a, slots), [True, False, True, False, False, True])


def test_kivi_token_without_tail_row_keeps_only_its_value():
    # seq_idx outside [0, max_seqs): the value is written, the key goes
    # nowhere (it can neither wait in a tail nor complete a page).
    rng = np.random.default_rng(43)
    k = rng.standard_normal((32, 2, 32)).astype(np.float16)
    c = o.OracleCache(2, 32, 2, 32, o.INT4_KIVI, o.INT8, max_seqs=1)
    o.write(c, k, k, np.arange(32) + 32, np.full(32, 1, np.int32))
    assert not np.any(c.k_codes) and not np.any(c.k_scales) and not np.any(c.k_tail)
    codes, s = o.quantize_sym(k, o.INT8)
    assert np.array_equal(c.v_codes[1].view(np.int8), codes) and np.array_equal(c.v_scales[1], s)


@pytest.mark.parametrize("kf,vf", [(o.INT8, o.INT8), (o.INT4_KIVI, o.INT4_G32)])
def test_pages_with_out_of_range_block_ids_contribute_nothing(kf, vf):
    # Corrupt some block-table entries (negative, or >= num_blocks): decode
    # equals attention over the tokens of the remaining pages, computed from
    # the sequence quantized on its own; KIVI tail tokens always count.
    bs = 32 if kf == o.INT4_KIVI else 16
    ctx = [150, 97]
    H, D, Hq = 2, 32, 4
    nb, table, ks, vs, slots = _three_sequences(kf, vf, ctx, bs, H, D, seed=44)
    c = o.OracleCache(nb, bs, H, D, kf, vf, max_seqs=len(ctx))
    o.write(c, np.concatenate(ks), np.concatenate(vs), np.concatenate(slots),
            np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(ctx)]))
    bad = table.copy()
    bad[0, 1] = -1
    bad[0, 3] = nb
    bad[1, 0] = nb + 1000
    q = np.random.default_rng(45).standard_normal((len(ctx), Hq, D)).astype(np.float16)
    got = o.decode_attn(c, q, bad, ctx)
    for b, L in enumerate(ctx):
        K, V = o.dequantized_sequence(ks[b], vs[b], kf, vf)
        page = np.arange(L) // bs
        keep = ~np.isin(page, [p for p in range(bad.shape[1]) if not 0 <= bad[b, p] < nb])
        if kf == o.INT4_KIVI:
            keep[(L // bs) * bs:] = True
        ref = o.attention_fp64(q[b].astype(np.float64), K[keep], V[keep])
        assert np.max(np.abs(got[b] - ref)) <= 1e-12, b
    # every page of a sequence out of range: nothing attended, zeros (INT8);
    # for KIVI the tail alone
    allbad = np.full_like(table, -5)
    got = o.decode_attn(c, q, allbad, ctx)
    for b, L in enumerate(ctx):
        if kf == o.INT4_KIVI:
            nf = (L // bs) * bs
            ref = o.attention_fp64(q[b].astype(np.float64), ks[b][nf:].astype(np.float64),
                                   vs[b][nf:].astype(np.float64))
            assert np.max(np.abs(got[b] - ref)) <= 1e-12
        else:
            assert not np.any(got[b])


def test_context_length_is_clamped_to_the_block_table():
    # ctx_lens beyond the tokens a block-table row addresses read that many;
    # a negative ctx_len attends to nothing.
    bs, H, D, L = 16, 2, 32, 64
    nb, table, ks, vs, slots = _three_sequences(o.INT8, o.INT8, [L], bs, H, D, seed=46)
    c = o.OracleCache(nb, bs, H, D, o.INT8, o.INT8, max_seqs=1)
    o.write(c, ks[0], vs[0], slots[0])
    q = np.random.default_rng(47).standard_normal((1, 4, D)).astype(np.float16)
    assert np.array_equal(o.decode_attn(c, q, table, [L + 1000]), o.decode_attn(c, q, table, [L]))
    assert not np.any(o.decode_attn(c, q, table, [-3]))


# --------------------------------------------------------------------------
# Offloaded pages
# --------------------------------------------------------------------------


@pytest.mark.parametrize("kf,vf", [(o.FP8_E4M3FN, o.FP8_E4M3FN), (o.INT4_KIVI, o.INT4_G32)])
def test_offload_round_trip_leaves_attention_unchanged(kf, vf):
    # Pages offloaded to a pool and prefetched back into other blocks, with
    # the block table pointing at the new blocks: every paged byte equal and
    # decode bitwise unchanged (the copy is the identity on page contents).
    bs = 32 if kf == o.INT4_KIVI else 16
    ctx = [150, 97]
    H, D, Hq = 2, 32, 4
    nb, table, ks, vs, slots = _three_sequences(kf, vf, ctx, bs, H, D, seed=50)
    c = o.OracleCache(nb + 8, bs, H, D, kf, vf, max_seqs=2)
    o.write(c, np.concatenate(ks), np.concatenate(vs), np.concatenate(slots),
            np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(ctx)]))
    q = np.random.default_rng(51).standard_normal((2, Hq, D)).astype(np.float16)
    before = o.decode_attn(c, q, table, ctx)
    pool = o.OracleCache(16, bs, H, D, kf, vf, max_seqs=1)
    moved = [int(table[0, 0]), int(table[0, 2]), int(table[1, 1]), int(table[1, 0])]
    o.copy_blocks(c, pool, moved, [3, 4, 5, 9])
    for name in o.paged_buffer_names(c):
        for s_id, d_id in zip(moved, [3, 4, 5, 9]):
            assert np.array_equal(getattr(pool, name)[d_id], getattr(c, name)[s_id])
    new = [nb + 1, nb + 2, nb + 3, nb + 7]  # free blocks of the cache
    o.copy_blocks(pool, c, [3, 4, 5, 9], new)
    t2 = table.copy()
    t2[0, 0], t2[0, 2], t2[1, 1], t2[1, 0] = new
    assert np.array_equal(o.decode_attn(c, q, t2, ctx), before)


# --------------------------------------------------------------------------
# Walsh-Hadamard rotation
# --------------------------------------------------------------------------


def _signs(D, seed):
    rng = np.random.default_rng(seed)
    bits = np.zeros(8, np.uint32)
    for c in np.nonzero(rng.integers(0, 2, D))[0]:
        bits[c // 32] |= np.uint32(1) << np.uint32(c % 32)
    return bits


def check_hadamard(hadamard=o.hadamard):
    import scipy.linalg
    for D in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        H = hadamard(D)
        assert np.array_equal(H, scipy.linalg.hadamard(D))  # the library's Sylvester matrix
        assert np.array_equal(H @ H.T, D * np.eye(D, dtype=np.int64))
    # entry (i, j) is (-1)^popcount(i & j)
    H = hadamard(64)
    i, j = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    pc = np.vectorize(lambda x: bin(int(x)).count("1"))(i & j)
    assert np.array_equal(H, np.where(pc % 2 == 1, -1, 1))


def test_hadamard():
    check_hadamard()


def check_rotation_exact(rotate_rows=o.rotate_rows):
    # y = H (sigma * x) rounded once to fp32, against exact rational
    # arithmetic on the fp16 inputs (spread over the whole fp16 range, so an
    # fp32 running sum would round).
    from fractions import Fraction
    rng = np.random.default_rng(60)
    D = 32
    bits = _signs(D, 61)
    sig = o.sign_vector(bits, D)
    x = (rng.standard_normal((6, D)) * np.exp2(rng.integers(-20, 15, (6, D)))).astype(np.float16)
    x[0, :3] = [65504, -6e-8, 1e-7]
    y = rotate_rows(x, bits)
    assert y.dtype == np.float32
    H = scipy_hadamard(D)
    for r in range(x.shape[0]):
        for i in range(D):
            exact = sum(Fraction(float(x[r, c])) * int(sig[c]) * int(H[i, c]) for c in range(D))
            assert y[r, i] == np.float32(float(exact)), (r, i)


def scipy_hadamard(D):
    import scipy.linalg
    return scipy.linalg.hadamard(D)


def test_rotation_exact():
    check_rotation_exact()


def check_rotation_round_trip(rotate_rows=o.rotate_rows, unrotate_rows=o.unrotate_rows):
    # Rotating back gives the row (the fp32 rounding of y aside), and the
    # quantization error of a rotated INT8/INT4 row, measured after the
    # inverse rotation, obeys the closed form ||x - x_hat||_2 <= sqrt(sum_g
    # n_g (s_g/2)^2) / sqrt(D) (the rotation is orthogonal up to sqrt(D)).
    rng = np.random.default_rng(62)
    for D in (64, 128, 256):
        bits = _signs(D, D)
        x = rng.standard_normal((500, D)).astype(np.float16)
        x[:, :4] *= 20
        back = unrotate_rows(rotate_rows(x, bits), bits)
        assert np.max(np.abs(back - x.astype(np.float64))) <= 1e-4 * np.max(np.abs(x.astype(np.float64)))
        for fmt in (o.INT8, o.INT4_G32):
            y = rotate_rows(x, bits)
            codes, s16 = o.quantize_sym(y, fmt)
            xh = unrotate_rows(o.dequant_sym(codes, s16, fmt), bits)
            g = 32 if fmt == o.INT4_G32 else D
            bound = np.sqrt(np.sum(g * (s16.astype(np.float64) / 2) ** 2, axis=-1)) / np.sqrt(D)
            err = np.sqrt(np.sum((xh - x.astype(np.float64)) ** 2, axis=-1))
            # + the fp32 rounding of y, carried back through the rotation
            assert np.all(err <= bound * (1 + 1e-6) + 1e-5 * np.max(np.abs(x.astype(np.float64)))), fmt


def test_rotation_round_trip():
    check_rotation_round_trip()


def test_rotation_spreads_outlier_channels():
    # The reason for the rotation: rows with a few large channels quantize
    # to INT4 with a much smaller error once rotated (the largest element
    # shrinks relative to the row's norm).
    rng = np.random.default_rng(63)
    D = 128
    bits = _signs(D, 64)
    x = rng.standard_normal((2000, D)).astype(np.float32)
    x[:, [3, 40, 77, 101]] *= 20
    x16 = x.astype(np.float16)
    c, s = o.quantize_sym(x16, o.INT4_G32)
    plain = np.mean((o.dequant_sym(c, s, o.INT4_G32) - x16.astype(np.float64)) ** 2)
    y = o.rotate_rows(x16, bits)
    c, s = o.quantize_sym(y, o.INT4_G32)
    rot = np.mean((o.unrotate_rows(o.dequant_sym(c, s, o.INT4_G32), bits) - x16.astype(np.float64)) ** 2)
    assert rot < 0.5 * plain, (rot, plain)


def check_rotated_cache_attention(rotate_query=o.rotate_query):
    # A cache written with rotated keys and values: decode equals fp64
    # attention over the stored rows brought back with the library Hadamard
    # matrix (x_hat = sigma * (H y_hat) / D), and also equals attention of the
    # rotated query q' = H (sigma * q) / D against the stored keys directly,
    # with the values brought back after the weighted sum.
    for kf, vf in ((o.INT8, o.INT4_G32), (o.FP8_E4M3FN, o.FP8_E5M2)):
        bs, H, D, Hq = 16, 2, 64, 4
        ctx = [70, 33]
        nb, table, ks, vs, slots = _three_sequences(kf, vf, ctx, bs, H, D, seed=65)
        rk, rv = _signs(D, 66), _signs(D, 67)
        c = o.OracleCache(nb, bs, H, D, kf, vf, max_seqs=2, rot_k=rk, rot_v=rv)
        o.write(c, np.concatenate(ks), np.concatenate(vs), np.concatenate(slots))
        q = np.random.default_rng(68).standard_normal((2, Hq, D)).astype(np.float16)
        got = o.decode_attn(c, q, table, ctx)
        Hm = scipy_hadamard(D).astype(np.float64)
        sk, sv = o.sign_vector(rk, D), o.sign_vector(rv, D)
        for b, L in enumerate(ctx):
            t = np.arange(L)
            blk, off = table[b, t // bs], t % bs
            def raw(which):
                fmt = kf if which == "k" else vf
                buf = c.k_codes if which == "k" else c.v_codes
                sc = c.k_scales if which == "k" else c.v_scales
                r = buf[blk, off]
                cd = o.unpack_int4(r, True) if fmt == o.INT4_G32 else (r if fmt in o.FP8_FORMATS else r.view(np.int8))
                return o.dequant_sym(cd, sc[blk, off], fmt)
            Yk, Yv = raw("k"), raw("v")
            K = (Yk @ Hm.T) * sk / D
            V = (Yv @ Hm.T) * sv / D
            ref = o.attention_fp64(q[b].astype(np.float64), K, V)
            assert np.max(np.abs(got[b] - ref)) <= 1e-10
            # rotated-query form: scores against the stored keys, values rotated back at the end
            qr = rotate_query(q[b], rk)
            acc = o.attention_fp64(qr, Yk, Yv)
            ref2 = (acc @ Hm.T) * sv / D
            assert np.max(np.abs(got[b] - ref2)) <= 1e-10


def test_rotated_cache_attention():
    check_rotated_cache_attention()


def test_rotated_scale_saturates_at_the_fp16_maximum():
    # Rotated rows reach D x 65504; a scale beyond the fp16 range is stored
    # as 65504 and the quotients saturate at +-q_max (brute force).
    D = 128
    bits = _signs(D, 70)
    x = np.full((3, D), -65504.0, np.float16)
    x[0] = (65504.0 * o.sign_vector(bits, D)).astype(np.float16)  # sigma * x = 65504: y_0 = 65504 D
    x[1, ::2] = 65504.0
    x[2] = 1.0
    y = o.rotate_rows(x, bits)
    for fmt in (o.INT8, o.INT4_G32):
        codes, s16 = o.quantize_sym(y, fmt)
        assert np.all(np.isfinite(s16))
        g = 32 if fmt == o.INT4_G32 else D
        yy = y.reshape(3, D // g, g).astype(np.float64)
        over = np.max(np.abs(yy), axis=-1) / o.QMAX[fmt] > 65519.0
        assert np.any(over) and np.all(s16[over] == np.float16(65504.0))
        q = o.QMAX[fmt]
        want = np.clip(np.rint(yy / 65504.0), -q, q)
        got = codes.reshape(3, D // g, g).astype(np.float64)
        assert np.array_equal(got[over], want[over])


# --------------------------------------------------------------------------
# Chunked prefill: a chunk of queries at the last positions of each sequence,
# causal over the cached tokens
# --------------------------------------------------------------------------

# (key format, value format, context lengths, chunk lengths): chunks shorter
# than the context (a cached prefix), equal to it (a whole prompt) and longer
# than it (queries at negative positions)
PREFILL_CASES = [
    (o.INT8, o.INT4_G32, [11, 7, 2], [5, 7, 3]),
    (o.FP8_E4M3FN, o.FP8_E5M2, [40, 17], [1, 17]),
    (o.INT4_KIVI, o.INT4_G32, [70, 33, 64], [40, 33, 9]),
]


def _prefill_setup(kf, vf, ctx, qlen, H=2, D=32, Hq=4, seed=80):
    bs = 32 if kf == o.INT4_KIVI else 4
    nb, table, ks, vs, slots = _three_sequences(kf, vf, ctx, bs, H, D, seed=seed)
    c = o.OracleCache(nb, bs, H, D, kf, vf, max_seqs=len(ctx))
    seq = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(ctx)])
    o.write(c, np.concatenate(ks), np.concatenate(vs), np.concatenate(slots), seq)
    q_start = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int64)
    q = (np.random.default_rng(seed + 1).standard_normal((int(q_start[-1]), Hq, D)) * 2).astype(np.float16)
    return c, table, ks, vs, q, q_start


def check_prefill_bruteforce(prefill=o.prefill_attn):
    # Explicit loops over query rows, heads and visible tokens with math.exp,
    # against the dequantized rows of each sequence quantized on its own
    # (KIVI: complete 32-token groups quantized, the last L mod 32 tokens fp16).
    for kf, vf, ctx, qlen in PREFILL_CASES:
        c, table, ks, vs, q, q_start = _prefill_setup(kf, vf, ctx, qlen)
        got = prefill(c, q, q_start, table, ctx)
        Hq, D = q.shape[1], q.shape[2]
        G = Hq // c.H
        for b, (L, n) in enumerate(zip(ctx, qlen)):
            K, V = o.dequantized_sequence(ks[b], vs[b], kf, vf)
            for i in range(n):
                r = int(q_start[b]) + i
                pos = L - n + i
                for hq in range(Hq):
                    h = hq // G
                    if pos < 0:
                        assert not np.any(got[r, hq]), (kf, b, i)
                        continue
                    sc = [sum(float(q[r, hq, d]) * K[t, h, d] for d in range(D)) / math.sqrt(D)
                          for t in range(pos + 1)]
                    mx = max(sc)
                    w = [math.exp(x - mx) for x in sc]
                    ref = [sum(w[t] * V[t, h, d] for t in range(pos + 1)) / sum(w) for d in range(D)]
                    assert np.max(np.abs(got[r, hq] - np.array(ref))) <= 1e-12, (kf, b, i, hq)


def check_prefill_rows_are_decodes(prefill=o.prefill_attn):
    # Symmetric formats: every chunk row equals decode attention of that query
    # with the context cut at its position (ctx = p + 1), and chunks of one
    # query equal decode.
    for kf, vf, ctx, qlen in PREFILL_CASES[:2]:
        c, table, ks, vs, q, q_start = _prefill_setup(kf, vf, ctx, qlen, seed=82)
        got = prefill(c, q, q_start, table, ctx)
        for b, (L, n) in enumerate(zip(ctx, qlen)):
            for i in range(n):
                r, pos = int(q_start[b]) + i, L - n + i
                ref = o.decode_attn(c, q[r][None], table[b:b + 1], [pos + 1])[0]
                assert np.array_equal(got[r], ref), (kf, b, i)
        ones = np.arange(len(ctx) + 1)
        last = q[[int(q_start[b + 1]) - 1 for b in range(len(ctx))]]
        assert np.array_equal(prefill(c, last, ones, table, ctx), o.decode_attn(c, last, table, ctx))


def check_prefill_split_chunks(prefill=o.prefill_attn):
    # A chunk computed in two pieces, the first while the context ended where
    # the second piece starts, equals the chunk in one call.
    for kf, vf, ctx, qlen in PREFILL_CASES[:2]:
        c, table, ks, vs, q, q_start = _prefill_setup(kf, vf, ctx, qlen, seed=84)
        whole = prefill(c, q, q_start, table, ctx)
        for b, (L, n) in enumerate(zip(ctx, qlen)):
            r0 = int(q_start[b])
            for m in range(1, n):
                first = prefill(c, q[r0:r0 + m], [0, m], table[b:b + 1], [L - (n - m)])
                second = prefill(c, q[r0 + m:r0 + n], [0, n - m], table[b:b + 1], [L])
                assert np.array_equal(np.concatenate([first, second]), whole[r0:r0 + n]), (kf, b, m)


def check_prefill_special_cases(prefill=o.prefill_attn):
    # A whole prompt: the query at position 0 returns v_hat_0 of its head; a
    # zero query returns the mean of v_hat over tokens 0..p.
    kf, vf, ctx, qlen = o.INT8, o.INT8, [13], [13]
    c, table, ks, vs, q, q_start = _prefill_setup(kf, vf, ctx, qlen, seed=86)
    K, V = o.dequantized_sequence(ks[0], vs[0], kf, vf)
    G = q.shape[1] // c.H
    got = prefill(c, q, q_start, table, ctx)
    assert np.array_equal(got[0], V[0][np.arange(q.shape[1]) // G])
    got = prefill(c, np.zeros_like(q), q_start, table, ctx)
    for p in range(13):
        assert np.max(np.abs(got[p] - V[:p + 1].mean(axis=0)[np.arange(q.shape[1]) // G])) <= 1e-14


def check_prefill_causality(prefill=o.prefill_attn):
    # Rewriting the key and value of token t changes exactly the rows at
    # positions >= t.
    kf, vf, ctx, qlen = o.INT8, o.INT4_G32, [24], [24]
    c, table, ks, vs, q, q_start = _prefill_setup(kf, vf, ctx, qlen, seed=88)
    before = prefill(c, q, q_start, table, ctx)
    t = 9
    slot = np.array([table[0, t // c.bs] * c.bs + t % c.bs])
    rng = np.random.default_rng(89)
    o.write(c, (rng.standard_normal((1, c.H, c.D)) * 3).astype(np.float16),
            rng.standard_normal((1, c.H, c.D)).astype(np.float16), slot)
    after = prefill(c, q, q_start, table, ctx)
    assert np.array_equal(after[:t], before[:t])
    assert np.all(np.any(after[t:] != before[t:], axis=(1, 2)))


def test_prefill_bruteforce():
    check_prefill_bruteforce()


def test_prefill_rows_are_decodes():
    check_prefill_rows_are_decodes()


def test_prefill_split_chunks():
    check_prefill_split_chunks()


def test_prefill_special_cases():
    check_prefill_special_cases()


def test_prefill_causality():
    check_prefill_causality()


def test_prefill_row_subset():
    kf, vf, ctx, qlen = PREFILL_CASES[0]
    c, table, ks, vs, q, q_start = _prefill_setup(kf, vf, ctx, qlen)
    full = o.prefill_attn(c, q, q_start, table, ctx)
    rows = [0, 4, 6, 13]
    part = o.prefill_attn(c, q, q_start, table, ctx, rows=rows)
    assert np.array_equal(part[rows], full[rows])
    assert not np.any(np.delete(part, rows, axis=0))
