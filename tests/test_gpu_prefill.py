"""GPU parity of kvq_prefill_attn (causal chunked prefill over the quantized
pages) against the oracle's float64 attention, over every query row of every
chunk: |out - o| <= 2e-3, or, for outputs of magnitude 4 or more, the fp16
half-ulp of o plus 1e-3 (kvq_fullsize.tolerance)."""

import numpy as np
import pytest
import torch

import oracle as o
from kvq_testlib import excess, new_caches, sign_bits, to_np16, write_both
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"

COMBOS = [("int8", "int8"), ("fp8_e4m3fn", "fp8_e4m3fn"), ("int8", "int4_g32"), ("fp8_e4m3fn", "int4_g32"),
          ("int4_kivi", "int4_g32"), ("int4_kivi", "int8"), ("int4_kivi", "fp8_e5m2"), ("fp8_e5m2", "fp8_e5m2"),
          ("int8", "fp8_e5m2"), ("int4_g32", "int4_g32"), ("int4_g32", "fp8_e4m3fn")]
# context lengths and chunk lengths: an empty context, one token, chunks
# shorter than, equal to and longer than the context, ragged pages
CTX = [0, 1, 33, 100, 257, 70, 64]
QLEN = [0, 1, 10, 100, 257, 80, 3]


def _setup(kf, vf, D, ctx, qlen, H=2, G=4, bs=None, seed=0, rot_k=None, rot_v=None, garbage=True):
    bs = bs or (32 if kf == "int4_kivi" else 16)
    w = wl.Workload("small", len(ctx), H * G, H, D, bs, kf, vf, ("fixed", 0), 2, sink_tokens=4)
    inp = wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=3)
    dev, orc = new_caches(inp.num_blocks, bs, H, D, kf, vf, len(ctx), DEV, seed=seed + 50, rot_k=rot_k, rot_v=rot_v,
                          garbage=garbage)
    write_both(inp, dev, orc, DEV)
    ch = wl.chunk_queries(w, qlen, seed, "cpu")
    return inp, ch, dev, orc


def _run(inp, ch, dev, orc, sm_scale=0.0, max_q_len=None, out=None):
    import quantized_paged_kv_write_amd as kvq
    ctx = torch.tensor(inp.ctx_lens, dtype=torch.int32)
    got = kvq.prefill_attn(dev, ch.q.to(DEV), ch.q_start.to(DEV), inp.block_table.to(DEV), ctx.to(DEV),
                           ch.max_q_len if max_q_len is None else max_q_len, sm_scale=sm_scale, out=out)
    torch.cuda.synchronize()
    ref = o.prefill_attn(orc, to_np16(ch.q), ch.q_start.numpy(), inp.block_table.numpy(), inp.ctx_lens,
                         sm_scale=None if sm_scale == 0 else sm_scale)
    return got.float().cpu().numpy().astype(np.float64), ref


def _ok(got, ref):
    return excess(got, ref) <= 0.0


@pytest.mark.parametrize("kf,vf", COMBOS)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_prefill_formats_ragged(kf, vf, D):
    inp, ch, dev, orc = _setup(kf, vf, D, CTX, QLEN, seed=D)
    got, ref = _run(inp, ch, dev, orc)
    assert _ok(got, ref)
    # rows at negative positions (the chunk of 80 over a context of 70) are zero
    r0 = int(ch.q_start[5])
    assert np.all(got[r0:r0 + 10] == 0)


@pytest.mark.parametrize("G", [1, 2, 3, 8, 16])
def test_prefill_gqa_group_sizes(G):
    inp, ch, dev, orc = _setup("int8", "int4_g32", 128, [40, 300, 129], [40, 150, 7], H=2, G=G, seed=G)
    got, ref = _run(inp, ch, dev, orc)
    assert _ok(got, ref)


@pytest.mark.parametrize("bs", [8, 16, 32, 64])
def test_prefill_block_sizes(bs):
    inp, ch, dev, orc = _setup("fp8_e4m3fn", "int8", 128, [200, 95], [120, 95], bs=bs, seed=bs)
    got, ref = _run(inp, ch, dev, orc)
    assert _ok(got, ref)


@pytest.mark.parametrize("kf,vf", [("int8", "int4_g32"), ("fp8_e4m3fn", "fp8_e5m2"), ("int4_kivi", "int4_g32"),
                                   ("int8", "int8"), ("int4_g32", "int8")])
def test_prefill_rotated(kf, vf):
    s = sign_bits(128, 5)
    rk = None if kf == "int4_kivi" else s
    inp, ch, dev, orc = _setup(kf, vf, 128, [150, 64, 70], [150, 20, 33], seed=9, rot_k=rk, rot_v=s)
    got, ref = _run(inp, ch, dev, orc)
    assert _ok(got, ref)


def test_prefill_sm_scale_and_repeat():
    inp, ch, dev, orc = _setup("int8", "int8", 64, [90, 33], [60, 33], seed=3)
    got, ref = _run(inp, ch, dev, orc, sm_scale=0.3)
    assert _ok(got, ref)
    again, _ = _run(inp, ch, dev, orc, sm_scale=0.3)
    assert np.array_equal(got, again)


def test_prefill_one_query_equals_decode():
    # chunks of one query are decode steps
    import quantized_paged_kv_write_amd as kvq
    inp, ch, dev, orc = _setup("fp8_e4m3fn", "int4_g32", 128, [300, 17, 64], [1, 1, 1], seed=4)
    got, ref = _run(inp, ch, dev, orc)
    assert _ok(got, ref)
    dec = kvq.decode_attn(dev, ch.q.to(DEV), inp.block_table.to(DEV),
                          torch.tensor(inp.ctx_lens, dtype=torch.int32, device=DEV))
    assert float(np.max(np.abs(dec.float().cpu().numpy() - got))) <= 4e-3


def test_prefill_leaves_rows_outside_chunks():
    # q_start need not cover all of q: rows outside every chunk keep out's contents
    inp, ch, dev, orc = _setup("int8", "int8", 64, [50, 40], [10, 5], seed=6)
    import quantized_paged_kv_write_amd as kvq
    q = torch.cat([ch.q, torch.zeros((4, ch.q.shape[1], 64), dtype=torch.float16)]).to(DEV)
    start = ch.q_start.clone()
    out = torch.full(q.shape, 7.0, dtype=torch.float16, device=DEV)
    kvq.prefill_attn(dev, q, start.to(DEV), inp.block_table.to(DEV),
                     torch.tensor(inp.ctx_lens, dtype=torch.int32, device=DEV), ch.max_q_len, out=out)
    torch.cuda.synchronize()
    assert torch.all(out[-4:] == 7.0)


def _clear():
    import quantized_paged_kv_write_amd as kvq
    torch.cuda.synchronize()
    kvq.get_device_error()


def test_prefill_reports_data_errors():
    import quantized_paged_kv_write_amd as kvq
    E = kvq.DEVERR
    # (zeroed cache: the clamped context reaches rows never written)
    inp, ch, dev, orc = _setup("int8", "int4_g32", 64, [90, 60, 50], [30, 20, 10], seed=12, garbage=False)
    _clear()
    got, ref = _run(inp, ch, dev, orc)
    assert _ok(got, ref) and kvq.get_device_error() == 0
    # a block id out of range on a page the call reads: that page is left out
    bt = inp.block_table.clone()
    bt[1, 1] = inp.num_blocks + 5
    inp2 = type(inp)(**{**inp.__dict__, "block_table": bt})
    got, ref = _run(inp2, ch, dev, orc)
    assert _ok(got, ref)
    assert kvq.get_device_error() == E["block"]
    # a context length past the block table: clamped
    ctx = list(inp.ctx_lens)
    ctx[2] = 10_000
    inp3 = type(inp)(**{**inp.__dict__, "ctx_lens": ctx})
    got, ref = _run(inp3, ch, dev, orc)
    assert _ok(got, ref)
    assert kvq.get_device_error() == E["ctx"]
    # a chunk longer than max_q_len: that sequence is skipped, its rows untouched
    out = torch.full(ch.q.shape, 7.0, dtype=torch.float16, device=DEV)
    got, ref = _run(inp, ch, dev, orc, max_q_len=20, out=out)
    assert kvq.get_device_error() == E["qlen"]
    assert np.all(got[:30] == 7.0)
    assert _ok(got[30:], ref[30:])
