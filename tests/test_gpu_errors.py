"""Out-of-range device ids: the kernels' bounds checks handle them as the
header states (the result equals the oracle's, which skips such slots and
leaves such pages out), and kvq_get_device_error reports them."""

import numpy as np
import pytest
import torch

import oracle as o
import quantized_paged_kv_write_amd as kvq
from kvq_testlib import ATOL, compare_buffers, decode_both, decode_error, new_caches, to_np16, write_both
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
E = kvq.DEVERR


def _clear():
    torch.cuda.synchronize()
    kvq.get_device_error()


def test_clean_calls_report_nothing():
    _clear()
    w = wl.WORKLOADS["tiny_int8"]
    inp = wl.make_inputs(w, 1, "cpu")
    dev, orc = new_caches(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype, w.batch, DEV)
    write_both(inp, dev, orc, DEV)
    decode_both(inp, dev, orc, DEV)
    assert kvq.get_device_error() == 0


@pytest.mark.parametrize("kf,vf", [("int8", "int4_g32"), ("fp8_e4m3fn", "fp8_e5m2"), ("int4_kivi", "int8")])
def test_write_reports_out_of_range_slots(kf, vf):
    _clear()
    D, H = 128, 2
    bs = 32 if kf == "int4_kivi" else 16
    nb = 4
    rng = np.random.default_rng(3)
    n = 40
    k = rng.standard_normal((n, H, D)).astype(np.float16)
    v = rng.standard_normal((n, H, D)).astype(np.float16)
    slots = np.arange(n, dtype=np.int64) + bs  # pages 1.. in order
    slots[5] = nb * bs          # first slot past the cache
    slots[17] = nb * bs + 12345
    slots[30] = -3              # negative: a documented skip, not an error
    seq = np.zeros(n, np.int32)
    # KIVI: the page missing rows takes them from the tail, so start from a
    # zero tail (garbage bytes there could be NaN/Inf, outside the contract)
    dev, orc = new_caches(nb, bs, H, D, kf, vf, 1, DEV, seed=31, garbage=kf != "int4_kivi")
    kvq.write(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV),
              torch.from_numpy(seq).to(DEV))
    o.write(orc, k, v, slots, seq)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    assert kvq.get_device_error() == E["slot"]
    assert kvq.get_device_error() == 0  # the read cleared it


def test_write_static_reports_out_of_range_slots():
    _clear()
    D, H, bs, nb = 64, 2, 16, 3
    rng = np.random.default_rng(4)
    k = rng.standard_normal((8, H, D)).astype(np.float16)
    slots = np.array([0, 1, 2, 48, 3, 4, 100, 5], np.int64)
    sc = np.array([0.01, 0.02], np.float16)
    dev, orc = new_caches(nb, bs, H, D, "int8", "int8", 1, DEV, seed=32)
    kvq.write_static(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(k).to(DEV), torch.from_numpy(slots).to(DEV),
                     torch.from_numpy(sc).to(DEV), torch.from_numpy(sc).to(DEV))
    o.write_static(orc, k, k, slots, sc, sc)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    assert kvq.get_device_error() == E["slot"]


@pytest.mark.parametrize("big", [False, True])
def test_kivi_write_reports_sequence_without_tail_row(big):
    # big: a call of more than 2048 tokens (seal and value pass in one launch,
    # tail rows written by their own kernel)
    _clear()
    D, H, bs = 128, 2, 32
    rng = np.random.default_rng(5)
    n0, n1, n2 = (1000, 1088, 20) if big else (40, 64, 20)
    ctx = [n0, n1, n2]
    k = rng.standard_normal((sum(ctx), H, D)).astype(np.float16)
    v = rng.standard_normal((sum(ctx), H, D)).astype(np.float16)
    b1 = -(-n0 // bs) * bs  # first slot of sequence 1 (its own pages)
    b2 = b1 + -(-n1 // bs) * bs
    slots = np.concatenate([np.arange(n0), b1 + np.arange(n1), b2 + np.arange(n2)]).astype(np.int64)
    seq = np.concatenate([np.zeros(n0), np.full(n1, 1), np.full(n2, 2)]).astype(np.int32)
    seq[n0:n0 + n1] = 7  # sequence 1 names tail row 7 of a 2-row tail: its keys go nowhere
    dev, orc = new_caches(-(-(b2 + n2) // bs), bs, H, D, "int4_kivi", "int4_g32", 2, DEV, seed=33)
    keep_seq2 = seq.copy()
    keep_seq2[n0 + n1:] = 1  # the last sequence uses tail row 1
    kvq.write(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV),
              torch.from_numpy(keep_seq2).to(DEV))
    o.write(orc, k, v, slots, keep_seq2)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    assert kvq.get_device_error() == E["seq"]


def _bad_table_setup(kf, vf, H, G, seed, garbage=True):
    bs = 32 if kf == "int4_kivi" else 16
    ctx = [0, 37, 200, 513]
    w = wl.Workload("small", len(ctx), H * G, H, 128, bs, kf, vf, ("fixed", 0), 2, sink_tokens=4)
    inp = wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=3)
    dev, orc = new_caches(inp.num_blocks, bs, H, 128, kf, vf, len(ctx), DEV, seed=seed + 50, garbage=garbage)
    write_both(inp, dev, orc, DEV)
    return inp, dev, orc


@pytest.mark.parametrize("kf,vf", [("fp8_e4m3fn", "fp8_e4m3fn"), ("int8", "int4_g32"), ("int4_kivi", "int4_g32"),
                                   ("int8", "int8")])
@pytest.mark.parametrize("H,G", [(8, 4), (8, 8), (8, 16)])  # 4, 2 and 1 KV heads per wave
def test_decode_pages_with_out_of_range_block_ids(kf, vf, H, G):
    _clear()
    inp, dev, orc = _bad_table_setup(kf, vf, H, G, seed=H * 16 + G)
    nb = inp.num_blocks
    t = inp.block_table.clone()
    t[1, 0] = -1       # the first page of a short sequence
    t[2, 2] = nb       # one past the pool
    t[2, 5] = -7
    t[3, 1] = nb + 999
    t[3, t.shape[1] - 1] = -1  # the last page of the longest sequence (a KIVI tail page when partial)
    inp.block_table = t
    got, ref = decode_both(inp, dev, orc, DEV)
    err, err16 = decode_error(got, ref)
    assert err <= ATOL, (err, err16)
    assert np.all(got[0] == 0)
    bits = kvq.get_device_error()
    assert bits == E["block"], bits


def test_decode_clamps_and_reports_context_lengths():
    _clear()
    # no garbage in the cache: the clamped context reads unwritten rows
    inp, dev, orc = _bad_table_setup("int8", "int8", 2, 2, seed=77, garbage=False)
    maxtok = inp.block_table.shape[1] * inp.w.block_size
    inp.ctx_lens = [0, 37, maxtok + 50, 513]  # beyond what the block-table row addresses
    got, ref = decode_both(inp, dev, orc, DEV)
    assert decode_error(got, ref)[0] <= ATOL
    assert kvq.get_device_error() == E["ctx"]
    inp.ctx_lens = [-4, 37, 200, 513]
    got, ref = decode_both(inp, dev, orc, DEV)
    assert decode_error(got, ref)[0] <= ATOL and np.all(got[0] == 0)
    assert kvq.get_device_error() == E["ctx"]
