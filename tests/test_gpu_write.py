"""GPU parity of kvq_write against the CPU oracle: codes, scales, zero points
and fp16 tails must be bit-exact."""

import numpy as np
import pytest
import torch

import oracle as o
from kvq_testlib import compare_buffers, new_caches, to_np16, write_both
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"

COMBOS = [("int8", "int8"), ("fp8_e4m3fn", "fp8_e4m3fn"), ("int8", "int4_g32"), ("fp8_e4m3fn", "int4_g32"),
          ("int8", "fp8_e4m3fn"), ("int4_kivi", "int4_g32"), ("int4_kivi", "int8"), ("int4_kivi", "fp8_e4m3fn"),
          ("fp8_e5m2", "fp8_e5m2"), ("fp8_e5m2", "int4_g32"), ("int8", "fp8_e5m2"), ("int4_kivi", "fp8_e5m2"),
          ("int4_g32", "int4_g32"), ("int4_g32", "fp8_e4m3fn"), ("int4_g32", "int8")]


def _small(kf, vf, D, bs, ctx, H=2, G=2, seed=0, outliers=2, sinks=2):
    w = wl.Workload("small", len(ctx), H * G, H, D, bs, kf, vf, ("fixed", 0), outliers, sink_tokens=sinks)
    return wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=3)


def test_write_tiny_int8_config():
    inp = wl.make_inputs(wl.WORKLOADS["tiny_int8"], 1, "cpu")
    w = inp.w
    dev, orc = new_caches(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype, w.batch, DEV)
    write_both(inp, dev, orc, DEV)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


@pytest.mark.parametrize("kf,vf", COMBOS)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_write_formats(kf, vf, D):
    bs = 32 if kf == "int4_kivi" else 16
    ctx = [1, 31, 32, 33, 95, 130]  # ragged, incl. partial last pages and KIVI tails
    inp = _small(kf, vf, D, bs, ctx, seed=D)
    dev, orc = new_caches(inp.num_blocks, bs, 2, D, kf, vf, len(ctx), DEV, seed=D + 1)
    write_both(inp, dev, orc, DEV)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


@pytest.mark.parametrize("bs", [8, 16, 64, 128])
def test_write_block_sizes(bs):
    inp = _small("fp8_e4m3fn", "int4_g32", 128, bs, [5, 64, 200], seed=bs)
    dev, orc = new_caches(inp.num_blocks, bs, 2, 128, "fp8_e4m3fn", "int4_g32", 3, DEV, seed=bs)
    write_both(inp, dev, orc, DEV)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def _edge_rows(D, rng):
    """Rows that stress the encoders: zeros, -0 (alone and beside nonzero
    values: FP8 keeps the sign of zero), max fp16, subnormals, scales that
    underflow fp16, exact half-way quotients, single spikes."""
    rows = []
    rows.append(np.zeros(D))
    rows.append(-np.zeros(D))
    r = rng.standard_normal(D); r[3] = 65504.0; rows.append(r)
    r = np.full(D, -65504.0); rows.append(r)
    rows.append(rng.standard_normal(D) * 2.0 ** -20)             # fp16 subnormals
    rows.append(rng.integers(-3, 4, D) * 2.0 ** -24)             # smallest subnormals
    rows.append(rng.standard_normal(D) * 1e-6)                   # scale underflows fp16
    r = np.zeros(D); r[0] = 7.9375; r[1:] = rng.integers(-254, 255, D - 1) * 0.03125; rows.append(r)  # ties
    r = np.zeros(D); r[0] = 448.0; r[1:] = rng.standard_normal(D - 1); rows.append(r)
    r = np.zeros(D); r[0] = 57344.0; r[1:] = rng.standard_normal(D - 1) * 1e4; rows.append(r)  # E5M2 max
    r = rng.standard_normal(D) * 2.0; r[0] = 3.5; rows.append(r)  # E5M2 scale at the fp16 normal edge
    r = np.zeros(D); r[5] = -1.0; rows.append(r)                 # one spike
    r = rng.standard_normal(D); r[::7] *= 300; rows.append(r)
    rows.append(np.linspace(-1, 1, D) * 3.5)
    r = rng.standard_normal(D); r[::3] = -0.0; r[1::5] = 0.0; rows.append(r)  # signed zeros, scale != 0
    return np.stack(rows).astype(np.float16)


@pytest.mark.parametrize("kf,vf", [("int8", "int4_g32"), ("fp8_e4m3fn", "int8"), ("int8", "fp8_e4m3fn"),
                                   ("fp8_e5m2", "int8"), ("int8", "fp8_e5m2"), ("int4_g32", "int8")])
def test_write_edge_values(kf, vf):
    D, H, bs = 128, 2, 16
    rng = np.random.default_rng(3)
    rows = _edge_rows(D, rng)
    n = len(rows)
    k = np.stack([rows, rows[::-1]], axis=1)  # (n, H, D)
    v = np.stack([rows[::-1], rows], axis=1)
    nb = (n + bs - 1) // bs + 1
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    dev, orc = new_caches(nb, bs, H, D, kf, vf, 1, DEV, seed=5)
    import quantized_paged_kv_write_amd as kvq
    kvq.write(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV))
    o.write(orc, k, v, slots)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def test_write_edge_values_kivi():
    D, H, bs = 128, 2, 32
    rng = np.random.default_rng(4)
    rows = _edge_rows(D, rng)
    k = np.concatenate([rows] * (64 // len(rows) + 1))[:64]
    k = np.stack([k, k[::-1]], axis=1)
    v = k[:, ::-1].copy()
    slots = np.concatenate([np.arange(32) + 32 * 3, np.arange(32) + 32 * 1]).astype(np.int64)
    seq = np.array([0] * 32 + [1] * 32, np.int32)
    dev, orc = new_caches(5, bs, H, D, "int4_kivi", "int4_g32", 2, DEV, seed=6)
    import quantized_paged_kv_write_amd as kvq
    kvq.write(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV),
              torch.from_numpy(seq).to(DEV))
    o.write(orc, k, v, slots, seq)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def test_write_skips_negative_and_out_of_range_slots():
    D, H, bs, nb = 64, 2, 16, 4
    rng = np.random.default_rng(8)
    k = rng.standard_normal((6, H, D)).astype(np.float16)
    slots = np.array([-1, 3, nb * bs, 17, -5, nb * bs + 100], np.int64)
    dev, orc = new_caches(nb, bs, H, D, "int8", "int8", 1, DEV, seed=7)
    import quantized_paged_kv_write_amd as kvq
    kvq.write(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(k).to(DEV), torch.from_numpy(slots).to(DEV))
    keep = (slots >= 0) & (slots < nb * bs)
    o.write(orc, k[keep], k[keep], slots[keep])
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def test_write_kivi_incremental_decode_steps():
    # Prefill of part of each sequence, then one token per sequence per call
    # (as decode does): pages complete from the tail.
    ctx = [45, 70, 33]
    inp = _small("int4_kivi", "int4_g32", 128, 32, ctx, seed=11)
    dev, orc = new_caches(inp.num_blocks, 32, 2, 128, "int4_kivi", "int4_g32", len(ctx), DEV, seed=12)
    import quantized_paged_kv_write_amd as kvq
    pre = 20
    sel = np.concatenate([np.arange(st, st + min(pre, L)) for st, L in zip(inp.seq_start, ctx)])
    selt = torch.from_numpy(sel)

    def step(idx):
        k, v = inp.k[idx], inp.v[idx]
        s, q = inp.slot_mapping[idx], inp.seq_idx[idx]
        kvq.write(dev, k.to(DEV), v.to(DEV), s.to(DEV), q.to(DEV))
        o.write(orc, to_np16(k), to_np16(v), s.numpy(), q.numpy())

    step(selt)
    for t in range(pre, max(ctx)):
        idx = [st + t for st, L in zip(inp.seq_start, ctx) if t < L]
        step(torch.tensor(idx))
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def test_write_kivi_large_decode_step():
    # A decode step of more than 2048 sequences (one large call, one token
    # per sequence): most tokens stay in their sequence's tail, and the
    # sequences at page offset 31 complete a page whose other rows come from
    # the tail written by the previous (also large) call.
    n, H, D, bs = 2100, 2, 128, 32
    rng = np.random.default_rng(23)
    off = rng.integers(0, 32, n)
    off[:70] = 31
    k = (rng.standard_normal((int(off.sum()) + n, H, D)) * 1.5).astype(np.float16)
    v = rng.standard_normal(k.shape).astype(np.float16)
    seq_first = np.repeat(np.arange(n), off).astype(np.int32)
    slot_first = np.concatenate([32 * i + np.arange(o_) for i, o_ in enumerate(off)]).astype(np.int64)
    seq_step = np.arange(n, dtype=np.int32)
    slot_step = (32 * np.arange(n) + off).astype(np.int64)
    dev, orc = new_caches(n, bs, H, D, "int4_kivi", "int4_g32", n, DEV, seed=24)
    import quantized_paged_kv_write_amd as kvq
    m = len(seq_first)
    assert m > 2048
    for lo, hi, sl, sq in ((0, m, slot_first, seq_first), (m, m + n, slot_step, seq_step)):
        kvq.write(dev, torch.from_numpy(k[lo:hi]).to(DEV), torch.from_numpy(v[lo:hi]).to(DEV),
                  torch.from_numpy(sl).to(DEV), torch.from_numpy(sq).to(DEV))
        o.write(orc, k[lo:hi], v[lo:hi], sl, sq)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


def test_write_kivi_large_calls():
    # Calls of more than 2048 tokens (one seal wave per 32 call tokens):
    # sequences start inside a chunk, pages straddle the two calls (their
    # first rows come from the tail), and short sequences stay in the tail.
    ctx = [3000, 2500, 1700, 45, 7]
    inp = _small("int4_kivi", "int4_g32", 128, 32, ctx, seed=17)
    dev, orc = new_caches(inp.num_blocks, 32, 2, 128, "int4_kivi", "int4_g32", len(ctx), DEV, seed=18)
    import quantized_paged_kv_write_amd as kvq
    cut = [int(0.6 * L) + 5 for L in ctx]
    first = np.concatenate([np.arange(st, st + min(c, L)) for st, L, c in zip(inp.seq_start, ctx, cut)])
    rest = np.concatenate([np.arange(st + min(c, L), st + L) for st, L, c in zip(inp.seq_start, ctx, cut)])
    assert len(first) > 2048 and len(rest) > 2048
    for sel in (first, rest):
        idx = torch.from_numpy(sel)
        k, v = inp.k[idx], inp.v[idx]
        s, q = inp.slot_mapping[idx], inp.seq_idx[idx]
        kvq.write(dev, k.to(DEV), v.to(DEV), s.to(DEV), q.to(DEV))
        o.write(orc, to_np16(k), to_np16(v), s.numpy(), q.numpy())
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}


@pytest.mark.parametrize("kf,vf", [("fp8_e4m3fn", "int4_g32"), ("int4_kivi", "int8")])
def test_write_call_beyond_one_launch(kf, vf):
    # A call of more than 2^24 (token, head) rows runs as launches over
    # consecutive token ranges.  With 6 heads the first range ends inside a
    # 32-token page, so that KIVI page is completed by the second launch from
    # the tail the first wrote.  Every row near the range end, sampled rows
    # elsewhere, the KIVI pages around the range end and the open tail are
    # checked against the oracle.
    import quantized_paged_kv_write_amd as kvq
    H, D = 6, 64
    step = (1 << 24) // H
    T = step + 1017
    assert T * H > (1 << 24) and step % 32 != 0
    bs = 32 if kf == "int4_kivi" else 16
    g = torch.Generator(device=DEV).manual_seed(5)
    k = torch.randn((T, H, D), generator=g, device=DEV, dtype=torch.float16)
    v = torch.randn((T, H, D), generator=g, device=DEV, dtype=torch.float16)
    slots = torch.arange(T, dtype=torch.int64, device=DEV)
    seq = torch.zeros(T, dtype=torch.int32, device=DEV)
    cache = kvq.PagedKVCache((T + bs - 1) // bs, bs, H, D, kf, vf, max_seqs=1, device=DEV)
    kvq.write(cache, k, v, slots, seq)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    toks = np.unique(np.concatenate([np.arange(step - 70, step + 70), rng.integers(0, T, 2000), [0, T - 1]]))
    tt = torch.from_numpy(toks).to(DEV)
    blk, off = tt // bs, tt % bs
    checks = [("v", v, vf)] + ([] if kf == "int4_kivi" else [("k", k, kf)])
    for name, x, fmt in checks:
        codes, s16 = o.quantize_sym(to_np16(x[tt]), fmt)
        stored = o.pack_int4(codes) if fmt == "int4_g32" else codes.view(np.uint8)
        assert np.array_equal(getattr(cache, name + "_codes")[blk, off].cpu().numpy(), stored), name
        assert np.array_equal(getattr(cache, name + "_scales")[blk, off].cpu().numpy().view(np.uint16),
                              s16.view(np.uint16)), name
    if kf != "int4_kivi":
        return
    pages = [step // 32 - 1, step // 32, step // 32 + 1, 0] + list(rng.integers(0, T // 32, 3))
    for pb in pages:
        k16 = to_np16(k[32 * pb:32 * pb + 32])
        for h in range(H):
            c, s16, z16 = o.kivi_quantize_group(k16[:, h])
            assert np.array_equal(cache.k_codes[pb, :, h].cpu().numpy(), o.pack_int4(c)), (pb, h)
            assert np.array_equal(cache.k_scales[pb, h].cpu().numpy().view(np.uint16), s16.view(np.uint16))
            assert np.array_equal(cache.k_zeros[pb, h].cpu().numpy().view(np.uint16), z16.view(np.uint16))
    nt = T % 32
    assert nt > 0
    assert np.array_equal(to_np16(cache.k_tail[0, :nt]), to_np16(k[T - nt:]))
    assert np.array_equal(to_np16(cache.v_tail[0, :nt]), to_np16(v[T - nt:]))


@pytest.mark.parametrize("name", [n for n in wl.ORDER[1:] if not wl.WORKLOADS[n].base])
def test_write_full_size_sampled(name):
    """The full workload written in one call on the GPU; sampled rows (and,
    for KIVI keys, sampled pages) re-quantized by the oracle."""
    w = wl.WORKLOADS[name]
    seed = wl.seed_of(w)
    inp = wl.make_inputs(w, seed, DEV)
    import quantized_paged_kv_write_amd as kvq
    max_seqs = w.batch
    cache = kvq.PagedKVCache(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype,
                             max_seqs=max_seqs, device=DEV)
    kvq.write(cache, inp.k, inp.v, inp.slot_mapping.to(DEV), inp.seq_idx.to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    T = inp.k.shape[0]
    toks = np.unique(np.concatenate([rng.integers(0, T, 3000), [0, T - 1], inp.seq_start]))
    tt = torch.from_numpy(toks)
    slots = inp.slot_mapping[tt]
    blk, off = slots // w.block_size, slots % w.block_size
    v16 = to_np16(inp.v[tt.to(DEV)])
    codes, s16 = o.quantize_sym(v16, w.v_dtype)
    stored = o.pack_int4(codes) if w.v_dtype == "int4_g32" else codes.view(np.uint8)
    assert np.array_equal(cache.v_codes[blk.to(DEV), off.to(DEV)].cpu().numpy(), stored)
    assert np.array_equal(cache.v_scales[blk.to(DEV), off.to(DEV)].cpu().numpy().view(np.uint16),
                          s16.view(np.uint16))
    if w.k_dtype != "int4_kivi":
        k16 = to_np16(inp.k[tt.to(DEV)])
        codes, s16 = o.quantize_sym(k16, w.k_dtype)
        assert np.array_equal(cache.k_codes[blk.to(DEV), off.to(DEV)].cpu().numpy(), codes.view(np.uint8))
        assert np.array_equal(cache.k_scales[blk.to(DEV), off.to(DEV)].cpu().numpy().view(np.uint16),
                              s16.view(np.uint16))
        return
    # KIVI keys: sampled complete pages of sampled sequences
    for b in rng.choice(w.batch, size=min(3, w.batch), replace=False):
        L = inp.ctx_lens[b]
        for p in rng.choice(L // 32, size=min(6, L // 32), replace=False):
            st = inp.seq_start[b] + 32 * p
            k16 = to_np16(inp.k[st:st + 32])
            pb = int(inp.block_table[b, p])
            for h in range(w.n_kv_heads):
                c, s16, z16 = o.kivi_quantize_group(k16[:, h])
                assert np.array_equal(cache.k_codes[pb, :, h].cpu().numpy(), o.pack_int4(c))
                assert np.array_equal(cache.k_scales[pb, h].cpu().numpy().view(np.uint16), s16.view(np.uint16))
                assert np.array_equal(cache.k_zeros[pb, h].cpu().numpy().view(np.uint16), z16.view(np.uint16))


@pytest.mark.parametrize("kf,vf", [("int8", "int8"), ("fp8_e4m3fn", "fp8_e4m3fn"), ("fp8_e5m2", "int4_g32"),
                                   ("int8", "fp8_e5m2"), ("int4_g32", "int4_g32")])
@pytest.mark.parametrize("D", [64, 128])
def test_write_static_scales(kf, vf, D):
    """kvq_write_static: calibrated per-head scales at half the median
    dynamic scale (about half the rows saturate), one key head with scale 0;
    codes and stored scales bit-exact, and decode reads the cache as usual."""
    import quantized_paged_kv_write_amd as kvq
    from kvq_testlib import decode_both, decode_error
    H, bs, ctx = 4, 16, [1, 31, 100]
    inp = _small(kf, vf, D, bs, ctx, H=H, G=2, seed=D + 7)
    k16, v16 = to_np16(inp.k), to_np16(inp.v)

    def scales(x16, fmt, zero_head=None):
        amax = np.abs(x16.astype(np.float32)).max(axis=-1)  # (T, H)
        s = (np.median(amax, axis=0) / o.QMAX[fmt] * 0.5).astype(np.float16)
        if zero_head is not None:
            s[zero_head] = 0
        return s

    ks, vs = scales(k16, kf, zero_head=1), scales(v16, vf)
    dev, orc = new_caches(inp.num_blocks, bs, H, D, kf, vf, len(ctx), DEV, seed=D + 8)
    kvq.write_static(dev, inp.k.to(DEV), inp.v.to(DEV), inp.slot_mapping.to(DEV), torch.from_numpy(ks).to(DEV),
                     torch.from_numpy(vs).to(DEV))
    o.write_static(orc, k16, v16, inp.slot_mapping.numpy(), ks, vs)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    got, ref = decode_both(inp, dev, orc, DEV)
    assert decode_error(got, ref)[0] <= 2e-3


@pytest.mark.parametrize("kf,vf", [("fp8_e4m3fn", "fp8_e5m2"), ("int8", "int4_g32"), ("int4_g32", "fp8_e4m3fn")])
def test_write_static_every_fp16_pattern(kf, vf):
    """With a calibrated scale of 1 every quotient is the fp16 input itself,
    so writing all finite fp16 bit patterns checks the hardware encoders
    (v_cvt_pk_fp8_f32, v_cvt_pk_bf8_f32, the integer rounding and clip)
    against the oracle over their whole fp16 domain, signed zeros and
    saturation included."""
    import quantized_paged_kv_write_amd as kvq
    H, D, bs = 2, 128, 16
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)]
    n = -(-h.size // (H * D)) * H * D
    vals = np.concatenate([h, np.zeros(n - h.size, np.float16)])
    T = n // (H * D)
    k = vals.reshape(T, H, D)
    v = k[::-1].copy()
    nb = -(-T // bs)
    slots = np.arange(T, dtype=np.int64)
    ones = np.ones(H, np.float16)
    dev, orc = new_caches(nb, bs, H, D, kf, vf, 1, DEV, seed=12)
    kvq.write_static(dev, torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV),
                     torch.from_numpy(ones).to(DEV), torch.from_numpy(ones).to(DEV))
    o.write_static(orc, k, v, slots, ones, ones)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
