"""Walsh-Hadamard rotated caches (KVQ_ROTATE_K / KVQ_ROTATE_V): codes and
scales of the rotated rows bit-exact against the oracle (the rotation is
exact, then one fp32 rounding), decode within 2e-3 of the oracle's float64
attention over the rows rotated back."""

import numpy as np
import pytest
import torch

import oracle as o
import quantized_paged_kv_write_amd as kvq
from kvq_testlib import ATOL, compare_buffers, decode_both, decode_error, new_caches, sign_bits, to_np16, write_both
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
RAGGED = [0, 1, 15, 16, 17, 33, 100, 257]


def _setup(kf, vf, D, ctx, rk, rv, H=2, G=4, seed=0):
    bs = 32 if kf == "int4_kivi" else 16
    w = wl.Workload("small", len(ctx), H * G, H, D, bs, kf, vf, ("fixed", 0), 4, sink_tokens=4)
    inp = wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=3)
    bits = sign_bits(D, seed + 1000)
    dev, orc = new_caches(inp.num_blocks, bs, H, D, kf, vf, len(ctx), DEV, seed=seed + 50,
                          rot_k=bits if rk else None, rot_v=bits if rv else None)
    write_both(inp, dev, orc, DEV)
    return inp, dev, orc


@pytest.mark.parametrize("kf,vf,rk,rv", [("int8", "int4_g32", True, True), ("fp8_e4m3fn", "fp8_e4m3fn", True, False),
                                         ("fp8_e5m2", "int8", False, True), ("int4_kivi", "int4_g32", False, True),
                                         ("int8", "fp8_e5m2", True, True), ("int4_g32", "int4_g32", True, True)])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotated_write_and_decode(kf, vf, rk, rv, D):
    inp, dev, orc = _setup(kf, vf, D, RAGGED, rk, rv, seed=D + (3 if rk else 0) + (5 if rv else 0))
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    got, ref = decode_both(inp, dev, orc, DEV)
    err, err16 = decode_error(got, ref)
    assert err <= ATOL, (err, err16)
    assert np.all(got[0] == 0)


@pytest.mark.parametrize("H,G", [(8, 4), (8, 8), (8, 16), (4, 2)])
def test_rotated_head_groups_and_splits(H, G):
    inp, dev, orc = _setup("int8", "int4_g32", 128, [0, 9, 130, 611], True, True, H=H, G=G, seed=H * 16 + G)
    for st in (0, 64):
        got, ref = decode_both(inp, dev, orc, DEV, split_tokens=st)
        err, err16 = decode_error(got, ref)
        assert err <= ATOL, (st, err, err16)


def test_rotated_write_static():
    D, H, bs = 128, 4, 16
    ctx = [1, 31, 100]
    w = wl.Workload("small", len(ctx), 8, H, D, bs, "fp8_e4m3fn", "int4_g32", ("fixed", 0), 4)
    inp = wl.make_inputs(w, 9, "cpu", ctx_lens=ctx, extra_blocks=3)
    bits = sign_bits(D, 9)
    dev, orc = new_caches(inp.num_blocks, bs, H, D, "fp8_e4m3fn", "int4_g32", len(ctx), DEV, seed=10, rot_k=bits,
                          rot_v=bits)
    k16, v16 = to_np16(inp.k), to_np16(inp.v)
    ks = np.array([0.05, 0.5, 0.0, 2.0], np.float16)  # rotated rows are larger: some saturate
    vs = np.array([0.3, 0.6, 1.2, 0.9], np.float16)
    kvq.write_static(dev, inp.k.to(DEV), inp.v.to(DEV), inp.slot_mapping.to(DEV), torch.from_numpy(ks).to(DEV),
                     torch.from_numpy(vs).to(DEV))
    o.write_static(orc, k16, v16, inp.slot_mapping.numpy(), ks, vs)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def test_rotated_extreme_rows():
    # rows spanning the whole fp16 range (the exact transform must not round
    # before its single fp32 rounding), zeros and single spikes
    D, H, bs = 128, 2, 16
    rng = np.random.default_rng(5)
    rows = [np.zeros(D), np.full(D, -65504.0), rng.standard_normal(D) * 2.0 ** -20]
    r = rng.standard_normal(D) * np.exp2(rng.integers(-24, 15, D)); rows.append(np.clip(r, -65504, 65504))
    r = np.zeros(D); r[7] = 65504.0; r[8] = 6e-8; rows.append(r)
    r = rng.standard_normal(D); r[::5] = -0.0; rows.append(r)
    rows = np.stack(rows).astype(np.float16)
    k = np.stack([rows, rows[::-1]], axis=1)
    v = k[:, ::-1].copy()
    slots = np.arange(len(rows), dtype=np.int64) + 3
    bits = sign_bits(D, 77)
    for kf, vf in (("int8", "int4_g32"), ("fp8_e4m3fn", "fp8_e5m2")):
        dev, orc = new_caches(2, bs, H, D, kf, vf, 1, DEV, seed=6, rot_k=bits, rot_v=bits)
        kvq.write(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV))
        o.write(orc, k, v, slots)
        torch.cuda.synchronize()
        assert compare_buffers(dev, orc) == {}, (kf, vf)


def test_rotation_improves_per_token_key_quality():
    # The point of the rotation: keys whose outliers sit in the same few channels (x20)
    # quantized per token lose the small channels; rotated first, the
    # outliers spread over all channels.  The error of the decode output
    # against unquantized attention drops (about 2.4x on these inputs in the
    # oracle).
    D, H, G = 128, 2, 4
    ctx = [600, 900]
    errs = {}
    for rk in (False, True):
        inp, dev, orc = _setup("int8", "int8", D, ctx, rk, False, H=H, G=G, seed=31)
        got, _ = decode_both(inp, dev, orc, DEV)
        err = 0.0
        for b, L in enumerate(ctx):
            st = inp.seq_start[b]
            ref = o.attention_fp64(to_np16(inp.q[b]).astype(np.float64), to_np16(inp.k[st:st + L]).astype(np.float64),
                                   to_np16(inp.v[st:st + L]).astype(np.float64))
            err = max(err, float(np.sqrt(np.mean((got[b] - ref) ** 2))))
        errs[rk] = err
    assert errs[True] < 0.6 * errs[False], errs


def test_rotated_values_in_a_large_kivi_call():
    # a call of more than 2048 tokens: the value pass and the seal share one
    # launch and the tail rows (unrotated) follow; rotated values bit-exact
    ctx = [1500, 700, 95]
    inp, dev, orc = _setup("int4_kivi", "int4_g32", 128, ctx, False, True, seed=77)
    assert sum(ctx) > 2048
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    got, ref = decode_both(inp, dev, orc, DEV)
    err, err16 = decode_error(got, ref)
    assert err <= ATOL, (err, err16)
