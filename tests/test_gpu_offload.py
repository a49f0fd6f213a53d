"""kvq_copy_blocks: pages offloaded from the device cache to a pool in pinned
host memory and prefetched back into other device blocks (as a double-
buffered prefetch does) are byte copies of the oracle's copy, and decode over
the block table that points at the prefetched blocks is bitwise unchanged.
Prefetches on a second stream run while decode runs on the first."""

import numpy as np
import pytest
import torch

import oracle as o
import quantized_paged_kv_write_amd as kvq
from kvq_testlib import ATOL, compare_buffers, decode_both, decode_error, new_caches, to_np16, write_both
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(kf, vf, ctx, spare, seed):
    bs = 32 if kf == "int4_kivi" else 16
    w = wl.Workload("small", len(ctx), 16, 4, 128, bs, kf, vf, ("fixed", 0), 2, sink_tokens=4)
    inp = wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=spare)
    dev, orc = new_caches(inp.num_blocks, bs, 4, 128, kf, vf, len(ctx), DEV, seed=seed + 3)
    write_both(inp, dev, orc, DEV)
    return inp, dev, orc


def _host_pool(dev, orc, n):
    pool = kvq.PagedKVCache(n, dev.block_size, dev.n_kv_heads, dev.head_dim, dev.k_dtype, dev.v_dtype, max_seqs=1,
                            device="cpu", pin_memory=True)
    opool = o.OracleCache(n, orc.bs, orc.H, orc.D, orc.k_fmt, orc.v_fmt, max_seqs=1)
    return pool, opool


@pytest.mark.parametrize("engine", ["kernel", "dma", "narrow"])
@pytest.mark.parametrize("kf,vf", [("fp8_e4m3fn", "fp8_e4m3fn"), ("int8", "int4_g32"), ("int4_kivi", "int4_g32"),
                                   ("fp8_e5m2", "int8")])
def test_offload_and_prefetch_round_trip(kf, vf, engine):
    ctx = [300, 77, 1000]
    spare = 40
    inp, dev, orc = _setup(kf, vf, ctx, spare, seed=11)
    got0, ref0 = decode_both(inp, dev, orc, DEV)
    assert decode_error(got0, ref0)[0] <= ATOL
    t = inp.block_table.numpy()
    used = set(int(x) for b, L in enumerate(ctx) for x in t[b, :-(-L // dev.block_size)])
    free = [x for x in range(inp.num_blocks) if x not in used]
    assert len(free) == spare
    # offload: pages 0..5 of sequence 2 and pages 0..1 of sequence 0 (scattered
    # device ids) to host slots 10.., one run of consecutive host slots
    pages = [(2, p) for p in range(6)] + [(0, 0), (0, 1)]
    src = [int(t[b, p]) for b, p in pages]
    host = list(range(10, 10 + len(pages)))
    pool, opool = _host_pool(dev, orc, 32)
    kvq.copy_blocks(dev, pool, src, host, engine=engine)
    o.copy_blocks(orc, opool, src, host)
    torch.cuda.synchronize()
    assert compare_buffers(pool, opool, names=o.paged_buffer_names(opool)) == {}
    # prefetch into spare device blocks: a run of consecutive ids, then
    # scattered ones; the table now points at them
    dst = free[:6] + [free[20], free[13]]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        kvq.copy_blocks(pool, dev, host, dst, engine=engine)
    o.copy_blocks(opool, orc, host, dst)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
    t2 = inp.block_table.clone()
    for (b, p), d in zip(pages, dst):
        t2[b, p] = d
    inp.block_table = t2
    got1, ref1 = decode_both(inp, dev, orc, DEV)
    assert np.array_equal(got1, got0)
    assert np.array_equal(ref1, ref0)


@pytest.mark.parametrize("engine", ["kernel", "dma", "narrow"])
def test_prefetch_overlaps_decode_on_another_stream(engine):
    # Double buffering: while decode t reads staging set t % 2, the prefetch
    # of step t + 1 fills set (t + 1) % 2 on a second stream; decode t + 1
    # waits for it through an event.  Every step's output equals the decode
    # of the original pages.
    ctx = [2000, 1500, 700]
    n_off = 8  # pages per sequence served from the staging sets
    inp, dev, orc = _setup("fp8_e4m3fn", "fp8_e4m3fn", ctx, 2 * 3 * n_off, seed=21)
    t = inp.block_table.numpy()
    bs = dev.block_size
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    q = inp.q.to(DEV)
    base = kvq.decode_attn(dev, q, inp.block_table.to(DEV), ctx_d).clone()
    used = set(int(x) for b, L in enumerate(ctx) for x in t[b, :-(-L // bs)])
    free = [x for x in range(inp.num_blocks) if x not in used]
    pool, _ = _host_pool(dev, orc, 3 * n_off)
    offl = [int(t[b, p]) for b in range(3) for p in range(n_off)]
    kvq.copy_blocks(dev, pool, offl, list(range(3 * n_off)))
    torch.cuda.synchronize()
    sets = [free[:3 * n_off], free[3 * n_off:]]
    tables = []
    for s in sets:
        t2 = inp.block_table.clone()
        for i, d in enumerate(s):
            t2[i // n_off, i % n_off] = d
        tables.append(t2.to(DEV))
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(2)]
    with torch.cuda.stream(side):
        kvq.copy_blocks(pool, dev, list(range(3 * n_off)), sets[0], engine=engine)
        ready[0].record(side)
    outs = []
    for step in range(6):
        cur = step % 2
        main.wait_event(ready[cur])
        if step + 1 < 6:
            side.wait_stream(main)  # the set being refilled is not read by an earlier step still in flight
            with torch.cuda.stream(side):
                kvq.copy_blocks(pool, dev, list(range(3 * n_off)), sets[1 - cur], engine=engine)
                ready[1 - cur].record(side)
        outs.append(kvq.decode_attn(dev, q, tables[cur], ctx_d).clone())
    torch.cuda.synchronize()
    for out in outs:
        assert torch.equal(out, base)


def test_prepared_calls_match_the_plain_calls():
    # DecodeCall / CopyCall marshal their arguments once; results are the
    # same as the plain binding calls.
    ctx = [300, 77]
    inp, dev, orc = _setup("int8", "int4_g32", ctx, 16, seed=31)
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    q, table = inp.q.to(DEV), inp.block_table.to(DEV)
    ref = kvq.decode_attn(dev, q, table, ctx_d)
    out = torch.empty_like(q)
    ws = torch.empty(kvq.decode_workspace_bytes(dev, 2, q.shape[1], table.shape[1]), dtype=torch.uint8, device=DEV)
    call = kvq.DecodeCall(dev, q, table, ctx_d, out, ws)
    out.zero_()
    call()
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    pool, opool = _host_pool(dev, orc, 8)
    src = [int(x) for x in inp.block_table[0, :4]]
    kvq.CopyCall(dev, pool, src, [4, 5, 6, 7])()
    o.copy_blocks(orc, opool, src, [4, 5, 6, 7])
    torch.cuda.synchronize()
    assert compare_buffers(pool, opool, names=o.paged_buffer_names(opool)) == {}


def test_copy_kernel_with_many_scattered_runs():
    # more runs than one launch holds (the kernel takes 160 runs per launch),
    # device to device and back, against the oracle's copy
    ctx = [2000, 1500]
    inp, dev, orc = _setup("int8", "fp8_e4m3fn", ctx, 400, seed=41)
    t = inp.block_table.numpy()
    used = sorted(int(x) for b, L in enumerate(ctx) for x in t[b, :-(-L // dev.block_size)])
    free = [x for x in range(inp.num_blocks) if x not in set(used)]
    rng = np.random.default_rng(3)
    src = [int(x) for x in rng.choice(used, 200, replace=False)]
    dst = [int(x) for x in rng.choice(free, 200, replace=False)]
    kvq.copy_blocks(dev, dev, src, dst, engine="kernel")
    o.copy_blocks(orc, orc, src, dst)
    torch.cuda.synchronize()
    assert compare_buffers(dev, orc) == {}
