"""Planted mistakes in the oracle must fail its pins.  Each case builds a
deliberately wrong variant of one oracle step (on the CPU) and checks that at
least one pin in test_oracle_pins rejects it."""

import types

import numpy as np
import pytest

import oracle as o
import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _quantize_divide_by_fp32_scale(x16, fmt):
    # Mistake: divide by the unrounded fp32 scale instead of the stored fp16 one.
    D = x16.shape[-1]
    g = o.INT4_GROUP if fmt == o.INT4_G32 else D
    x = x16.astype(np.float32).reshape(x16.shape[:-1] + (D // g, g))
    s32 = np.max(np.abs(x), axis=-1) / np.float32(o.QMAX[fmt])
    s16 = s32.astype(np.float16)
    safe = np.where(s32 == 0, np.float32(1), s32)
    y = x / safe[..., None]
    q = o.QMAX[fmt]
    if fmt == o.FP8_E4M3FN:
        return o.e4m3fn_encode(y).reshape(x16.shape), s16
    return np.clip(np.rint(y), -q, q).astype(np.int8).reshape(x16.shape), s16


def _quantize_round_half_up(x16, fmt):
    # Mistake: round half away from zero.
    x = x16.astype(np.float32)
    s16 = (np.max(np.abs(x), axis=-1, keepdims=True) / np.float32(o.QMAX[fmt])).astype(np.float16)
    y = x / s16.astype(np.float32)
    c = np.sign(y) * np.floor(np.abs(y) + 0.5)
    return np.clip(c, -127, 127).astype(np.int8), s16


def _attention_wrong_gqa(q, K, V, sm_scale=None):
    # Mistake: query head hq reads KV head hq % H instead of hq // G.
    q = np.asarray(q, np.float64)
    Hq, D = q.shape
    H = K.shape[1]
    out = np.zeros((Hq, D))
    for hq in range(Hq):
        h = hq % H
        s = K[:, h, :] @ q[hq] / np.sqrt(D)
        p = np.exp(s - s.max())
        out[hq] = p @ V[:, h, :] / p.sum()
    return out


def test_wrong_qmax_fails(monkeypatch):
    monkeypatch.setitem(o.kvq_oracle.QMAX, o.INT8, 128.0)
    assert _fails(pins.check_worked_example, o.kvq_oracle.quantize_sym)


def test_fp32_scale_divisor_fails():
    assert _fails(pins.check_sym_invariants, _quantize_divide_by_fp32_scale, o.dequant_sym, (o.INT8,))


def test_round_half_up_fails():
    assert _fails(pins.check_round_half_even, _quantize_round_half_up)


def test_no_saturation_fails(monkeypatch):
    monkeypatch.setattr(o.kvq_oracle, "E4M3FN_MAX_CODE", 0x7F)
    assert _fails(pins.check_fp8_specials, o.kvq_oracle.e4m3fn_encode)


def test_wrong_fp8_exponent_bias_fails():
    assert _fails(pins.check_fp8_bruteforce, lambda y: o.e4m3fn_encode(np.asarray(y, np.float32) * 2))


def test_e5m2_no_saturation_fails(monkeypatch):
    # Mistake: let large quotients reach the infinity code.
    monkeypatch.setattr(o.kvq_oracle, "E5M2_MAX_CODE", 0x7C)
    assert _fails(pins.check_e5m2_specials, o.kvq_oracle.e5m2_encode)


def test_e5m2_wrong_exponent_bias_fails():
    assert _fails(pins.check_e5m2_bruteforce, lambda y: o.e5m2_encode(np.asarray(y, np.float32) * 2))


def test_e5m2_mantissa_bits_fail():
    # Mistake: E4M3's mantissa width with E5M2's exponent (encode through the
    # E4M3 rounding grid scaled into E5M2's range).
    def wrong(y):
        y = np.asarray(y, np.float32)
        snapped = o.e4m3fn_value(o.e4m3fn_encode(y / np.float32(2 ** 7))) * 2.0 ** 7
        return o.e5m2_encode(snapped.astype(np.float32))
    assert _fails(pins.check_e5m2_bruteforce, wrong)


def test_e5m2_as_e4m3_in_invariants_fails():
    # Mistake: encode E5M2 rows with the E4M3FN encoder (wrong format table).
    def quantize(x16, fmt):
        codes, s16 = o.quantize_sym(x16, fmt)
        if fmt == o.FP8_E5M2:
            s = s16.astype(np.float32)
            y = x16.astype(np.float32) / np.where(s == 0, 1, s)
            codes = o.e4m3fn_encode(y)
        return codes, s16
    assert _fails(pins.check_sym_invariants, quantize, o.dequant_sym, (o.FP8_E5M2,))


def test_swapped_nibbles_fail():
    assert _fails(pins.check_pack_order, lambda c: o.pack_int4(np.asarray(c)[..., ::-1]))


def test_wrong_group_size_fails(monkeypatch):
    monkeypatch.setattr(o.kvq_oracle, "INT4_GROUP", 64)
    assert _fails(pins.check_closed_forms, o.kvq_oracle.stored_bytes_per_token_head)


def test_wrong_kivi_levels_fail(monkeypatch):
    monkeypatch.setattr(o.kvq_oracle, "KIVI_LEVELS", 16)
    assert _fails(pins.check_kivi_invariants, o.kvq_oracle.kivi_quantize_group)


def test_reversed_kivi_codes_fail():
    def bad(x16):
        c, s, z = o.kivi_quantize_group(x16)
        return (15 - c).astype(np.uint8), s, z
    assert _fails(pins.check_kivi_invariants, bad)


def test_dropped_softmax_scale_fails(monkeypatch):
    monkeypatch.setattr(o.kvq_oracle, "math", types.SimpleNamespace(sqrt=lambda x: 1.0))
    assert _fails(pins.check_attention_vs_sdpa, o.kvq_oracle.attention_fp64)


def test_wrong_gqa_mapping_fails():
    assert _fails(pins.check_attention_vs_sdpa, _attention_wrong_gqa)


@pytest.mark.parametrize("fmt", [o.INT8, o.INT4_G32])
def test_unplanted_oracle_passes(fmt):
    # Control: the real oracle passes the same checks.
    pins.check_sym_invariants(o.quantize_sym, o.dequant_sym, (fmt,))



def test_static_ignoring_given_scale_fails():
    # Mistake: the static path recomputes the per-row amax scale.
    def wrong(x16, fmt, s16):
        codes, s = o.quantize_sym(x16, fmt)
        g = s.shape[-1]
        return codes, np.broadcast_to(s16[..., None], s16.shape + (g,)).astype(np.float16)
    assert _fails(pins.check_static_saturation_bruteforce, wrong)


def test_static_without_saturation_fails():
    # Mistake: no clip at +-q_max for the integer formats.
    def wrong(x16, fmt, s16):
        codes, sg = o.quantize_sym_static(x16, fmt, s16)
        if fmt in (o.INT8, o.INT4_G32):
            s = s16.astype(np.float32)[:, None]
            y = x16.astype(np.float32) / np.where(s == 0, 1, s)
            codes = np.where(s == 0, 0, np.rint(y)).astype(np.int64)
        return codes, sg
    assert _fails(pins.check_static_saturation_bruteforce, wrong)

def _decode_tail_row_0(cache, q, block_table, ctx_lens, sm_scale=None):
    # Mistake: every batch row reads tail row 0.
    out = np.zeros(np.asarray(q).shape)
    for b in range(len(ctx_lens)):
        L = int(ctx_lens[b])
        K, V = o.gather_dequant(cache, block_table[b], L, 0)
        out[b] = o.attention_fp64(q[b], K, V, sm_scale, live=o.token_live(cache, block_table[b], L))
    return out


def _decode_table_row_0(cache, q, block_table, ctx_lens, sm_scale=None):
    # Mistake: every batch row reads the pages of block-table row 0.
    out = np.zeros(np.asarray(q).shape)
    for b in range(len(ctx_lens)):
        L = int(ctx_lens[b])
        K, V = o.gather_dequant(cache, block_table[0], L, b)
        out[b] = o.attention_fp64(q[b], K, V, sm_scale, live=o.token_live(cache, block_table[0], L))
    return out


def _write_ignoring_seq_idx(cache, k16, v16, slot_mapping, seq_idx=None):
    # Mistake: every token's tail row is row 0.
    return o.write(cache, k16, v16, slot_mapping, None if seq_idx is None else np.zeros_like(seq_idx))


def test_routing_mistakes_fail():
    assert _fails(pins.check_multi_sequence_routing, o.write, _decode_tail_row_0)
    assert _fails(pins.check_multi_sequence_routing, o.write, _decode_table_row_0)
    assert _fails(pins.check_multi_sequence_routing, _write_ignoring_seq_idx, o.decode_attn)
    pins.check_multi_sequence_routing()


def test_rotation_mistakes_fail():
    # Walsh-Hadamard rotation: signs dropped, the 1/D of the inverse dropped,
    # the query's signs applied after H instead of before, a non-Sylvester
    # block order.
    def rot_no_signs(x16, bits):
        D = x16.shape[-1]
        return (x16.astype(np.float64) @ o.hadamard(D).T.astype(np.float64)).astype(np.float32)

    def unrot_no_div(y, bits):
        return o.unrotate_rows(y, bits) * y.shape[-1]

    def rotq_signs_after(q16, bits):
        D = q16.shape[-1]
        return (q16.astype(np.float64) @ o.hadamard(D).T.astype(np.float64)) * o.sign_vector(bits, D) / D

    def hadamard_wrong(D):
        H = np.ones((1, 1), np.int64)
        while H.shape[0] < D:
            H = np.block([[H, H], [-H, H]])
        return H

    assert _fails(pins.check_rotation_exact, rot_no_signs)
    assert _fails(pins.check_rotation_round_trip, o.rotate_rows, unrot_no_div)
    assert _fails(pins.check_rotated_cache_attention, rotq_signs_after)
    assert _fails(pins.check_hadamard, hadamard_wrong)


def _causal_strict(q, K, V, positions, sm_scale=None, live=None):
    # Mistake: a query does not see its own position (t < p).
    return o.kvq_oracle._causal_ok(q, K, V, [p - 1 for p in positions], sm_scale, live)


def _causal_none(q, K, V, positions, sm_scale=None, live=None):
    # Mistake: no causal mask inside the chunk.
    return o.kvq_oracle._causal_ok(q, K, V, [K.shape[0] - 1] * len(positions), sm_scale, live)


def _prefill_positions_from_zero(cache, q, q_start, block_table, ctx_lens, sm_scale=None, seqs=None, rows=None):
    # Mistake: chunk row i sits at position i instead of L - n + i.
    q = np.asarray(q)
    out = np.zeros(q.shape)
    for b in range(len(q_start) - 1):
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        L = min(max(int(ctx_lens[b]), 0), np.asarray(block_table).shape[1] * cache.bs)
        K, V = o.gather_dequant(cache, block_table[b], L, b)
        live = o.token_live(cache, block_table[b], L)
        out[r0:r1] = o.causal_attention_fp64(q[r0:r1], K, V, list(range(r1 - r0)), sm_scale, live)
    return out


def _prefill_head_major(cache, q, q_start, block_table, ctx_lens, sm_scale=None, seqs=None, rows=None):
    # Mistake: the query tensor read as (Hq, Tq, D) memory.
    q = np.asarray(q)
    qq = np.ascontiguousarray(q).reshape(q.shape[1], q.shape[0], q.shape[2]).transpose(1, 0, 2)
    return o.prefill_attn(cache, qq, q_start, block_table, ctx_lens, sm_scale, seqs, rows)


def test_prefill_mistakes_fail(monkeypatch):
    checks = (pins.check_prefill_bruteforce, pins.check_prefill_rows_are_decodes, pins.check_prefill_split_chunks,
              pins.check_prefill_special_cases, pins.check_prefill_causality)
    monkeypatch.setattr(o.kvq_oracle, "_causal_ok", o.kvq_oracle.causal_attention_fp64, raising=False)
    for wrong in (_causal_strict, _causal_none):
        with monkeypatch.context() as m:
            m.setattr(o.kvq_oracle, "causal_attention_fp64", wrong)
            failed = [c.__name__ for c in checks if _fails(c)]
            assert failed, wrong.__name__
    for wrong in (_prefill_positions_from_zero, _prefill_head_major):
        assert any(_fails(c, wrong) for c in checks), wrong.__name__
    for c in checks:
        c()
