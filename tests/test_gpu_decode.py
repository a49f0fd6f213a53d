"""GPU parity of kvq_decode_attn against the oracle's float64 attention over
the same dequantized keys and values: max |out - o| <= 2e-3."""

import numpy as np
import pytest
import torch

from kvq_testlib import ATOL, decode_both, decode_error, new_caches, oracle_head_attention, write_both
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"

COMBOS = [("int8", "int8"), ("fp8_e4m3fn", "fp8_e4m3fn"), ("int8", "int4_g32"), ("fp8_e4m3fn", "int4_g32"),
          ("int8", "fp8_e4m3fn"), ("int4_kivi", "int4_g32"), ("int4_kivi", "int8"), ("int4_kivi", "fp8_e4m3fn"),
          ("fp8_e5m2", "fp8_e5m2"), ("fp8_e5m2", "int4_g32"), ("int8", "fp8_e5m2"), ("int4_kivi", "fp8_e5m2"),
          ("int4_g32", "int4_g32"), ("int4_g32", "fp8_e4m3fn"), ("int4_g32", "int8")]
RAGGED = [0, 1, 15, 16, 17, 31, 32, 33, 100, 257]


def _setup(kf, vf, D, ctx, H=2, G=4, bs=None, seed=0, sinks=4, extra=3):
    bs = bs or (32 if kf == "int4_kivi" else 16)
    w = wl.Workload("small", len(ctx), H * G, H, D, bs, kf, vf, ("fixed", 0), 2, sink_tokens=sinks)
    inp = wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=extra)
    dev, orc = new_caches(inp.num_blocks, bs, H, D, kf, vf, len(ctx), DEV, seed=seed + 50)
    write_both(inp, dev, orc, DEV)
    return inp, dev, orc


def test_decode_tiny_int8_config():
    inp = wl.make_inputs(wl.WORKLOADS["tiny_int8"], 1, "cpu")
    w = inp.w
    dev, orc = new_caches(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype, w.batch, DEV)
    write_both(inp, dev, orc, DEV)
    got, ref = decode_both(inp, dev, orc, DEV)
    err, _ = decode_error(got, ref)
    assert err <= ATOL, err


@pytest.mark.parametrize("kf,vf", COMBOS)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_decode_formats_ragged(kf, vf, D):
    inp, dev, orc = _setup(kf, vf, D, RAGGED, seed=D)
    got, ref = decode_both(inp, dev, orc, DEV)
    err, err16 = decode_error(got, ref)
    assert err <= ATOL, (err, err16)
    assert np.all(got[0] == 0)  # ctx 0 -> zeros


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_decode_gqa_group_sizes(G):
    inp, dev, orc = _setup("int8", "int4_g32", 128, [40, 300], H=2, G=G, seed=G)
    got, ref = decode_both(inp, dev, orc, DEV)
    assert decode_error(got, ref)[0] <= ATOL


@pytest.mark.parametrize("H,G", [(8, 4), (4, 4), (8, 8), (8, 2), (8, 1), (6, 2), (4, 16)])
@pytest.mark.parametrize("kf,vf", [("fp8_e4m3fn", "fp8_e4m3fn"), ("int8", "int4_g32"), ("int4_kivi", "int4_g32"),
                                   ("int4_g32", "int4_g32")])
def test_decode_head_groups(H, G, kf, vf):
    # a wave reads HP = 4, 2 or 1 KV heads (the most with HP G <= 16 and
    # H % HP == 0): (token, head) tile rows, head-matched score columns; for
    # KIVI keys a 32-token page spans HP tiles (the page's q * s is reused)
    inp, dev, orc = _setup(kf, vf, 128, [0, 9, 130, 611], H=H, G=G, seed=H * 16 + G)
    for st in (0, 64):
        got, ref = decode_both(inp, dev, orc, DEV, split_tokens=st)
        err, err16 = decode_error(got, ref)
        assert err <= ATOL, (st, err, err16)
        assert np.all(got[0] == 0)


@pytest.mark.parametrize("bs", [8, 32, 64, 128])
def test_decode_block_sizes(bs):
    inp, dev, orc = _setup("fp8_e4m3fn", "int8", 128, [7, 64, 300, 513], bs=bs, seed=bs)
    got, ref = decode_both(inp, dev, orc, DEV)
    assert decode_error(got, ref)[0] <= ATOL


@pytest.mark.parametrize("kf,vf", [("int8", "int8"), ("int4_kivi", "int4_g32")])
def test_decode_split_invariance_and_determinism(kf, vf):
    inp, dev, orc = _setup(kf, vf, 128, [1000, 2047, 65], seed=3)
    outs = []
    # automatic, one tile per share, shares that end inside a sequence, one share per sequence or more
    for st in (0, 32, 96, 256, 1000, 4096):
        got, ref = decode_both(inp, dev, orc, DEV, split_tokens=st)
        assert decode_error(got, ref)[0] <= ATOL, st
        outs.append(got)
    for a in outs[1:]:
        assert np.max(np.abs(a - outs[0])) <= 2 * ATOL
    again, _ = decode_both(inp, dev, orc, DEV, split_tokens=96)
    assert np.array_equal(again, outs[2])  # run-to-run bitwise


@pytest.mark.parametrize("kf,vf", [("int8", "int8"), ("fp8_e4m3fn", "int4_g32"), ("int4_kivi", "int4_g32")])
@pytest.mark.parametrize("split_tokens", [0, 32, 4096])
def test_decode_many_short_sequences(kf, vf, split_tokens):
    # 150 sequences of 0..70 tokens: shares run across many sequence ends
    # (4096 tokens = 128 tiles holds more than 64 sequences, so a wave walks
    # past its first window of sequence bounds), with empty sequences between.
    g = np.random.default_rng(11)
    ctx = [int(x) for x in g.integers(0, 71, size=150)]
    for i in (0, 1, 2, 40, 41, 149):
        ctx[i] = 0
    inp, dev, orc = _setup(kf, vf, 64, ctx, seed=21, extra=5)
    got, ref = decode_both(inp, dev, orc, DEV, split_tokens=split_tokens)
    err, err16 = decode_error(got, ref)
    assert err <= ATOL, (err, err16)
    for i in (0, 1, 2, 40, 41, 149):
        assert np.all(got[i] == 0)


def test_decode_custom_sm_scale():
    inp, dev, orc = _setup("int8", "int8", 64, [50, 120], seed=9)
    got, ref = decode_both(inp, dev, orc, DEV, sm_scale=0.05)
    assert decode_error(got, ref)[0] <= ATOL


def test_decode_kivi_tail_lengths():
    ctx = [32, 33, 63, 64, 65, 95]  # tails 0, 1, 31, 0, 1, 31
    inp, dev, orc = _setup("int4_kivi", "int4_g32", 128, ctx, seed=21)
    got, ref = decode_both(inp, dev, orc, DEV)
    assert decode_error(got, ref)[0] <= ATOL


@pytest.mark.parametrize("name", [n for n in wl.ORDER[1:] if not wl.WORKLOADS[n].base])
def test_decode_full_size_sampled(name):
    """The full workload (write of every token, then one decode step) on the
    GPU; sampled (sequence, KV head) pairs recomputed by the oracle."""
    import quantized_paged_kv_write_amd as kvq
    w = wl.WORKLOADS[name]
    seed = wl.seed_of(w)
    inp = wl.make_inputs(w, seed, DEV)
    cache = kvq.PagedKVCache(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype,
                             max_seqs=w.batch, device=DEV)
    kvq.write(cache, inp.k, inp.v, inp.slot_mapping.to(DEV), inp.seq_idx.to(DEV))
    ctx = torch.tensor(inp.ctx_lens, dtype=torch.int32, device=DEV)
    out = kvq.decode_attn(cache, inp.q, inp.block_table.to(DEV), ctx)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(seed)
    G = w.n_q_heads // w.n_kv_heads
    pairs = {(0, 0), (w.batch - 1, w.n_kv_heads - 1)}
    while len(pairs) < 6:
        pairs.add((int(rng.integers(w.batch)), int(rng.integers(w.n_kv_heads))))
    worst = 0.0
    for b, h in sorted(pairs):
        ref = oracle_head_attention(inp, b, h)
        worst = max(worst, float(np.max(np.abs(got[b, h * G:(h + 1) * G] - ref))))
    assert worst <= ATOL, worst


@pytest.mark.parametrize("kf", ["int8", "fp8_e4m3fn", "fp8_e5m2", "int4_kivi", "int4_g32"])
@pytest.mark.parametrize("qmode", ["sharp_positive", "flat"])
def test_decode_query_scales(kf, qmode):
    """Queries far from N(0,1): all-positive and 8x larger (a sharp softmax,
    and for INT8 keys a bias term 128 sum(q) much larger than the score), or
    100x smaller (a nearly flat softmax over every token)."""
    inp, dev, orc = _setup(kf, "int8", 128, [300, 1000, 33], seed=17)
    q = inp.q.float()
    inp.q = ((q.abs() * 8) if qmode == "sharp_positive" else (q * 0.01)).half()
    got, ref = decode_both(inp, dev, orc, DEV)
    err, err16 = decode_error(got, ref)
    assert err <= ATOL, (err, err16)
