"""kvq_decode_attn_noalloc (decode with the library's fixed per-device
workspace) against kvq_decode_attn with a caller workspace: bitwise the same
output for the same partition, within 2e-3 of the oracle, on two calls in a
row (the second smaller, so it runs over what the first left in the fixed
workspace)."""

import numpy as np
import pytest
import torch

import quantized_paged_kv_write_amd as kvq
from kvq_testlib import ATOL, new_caches, to_np16, write_both
from quantized_paged_kv_write_amd import workloads as wl

import oracle as o

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(kf, vf, ctx, H, G, seed):
    bs = 32 if kf == "int4_kivi" else 16
    w = wl.Workload("small", len(ctx), H * G, H, 128, bs, kf, vf, ("fixed", 0), 2, sink_tokens=4)
    inp = wl.make_inputs(w, seed, "cpu", ctx_lens=ctx, extra_blocks=2)
    dev, orc = new_caches(inp.num_blocks, bs, H, 128, kf, vf, len(ctx), DEV, seed=seed + 9)
    write_both(inp, dev, orc, DEV)
    return inp, dev, orc


@pytest.mark.parametrize("kf,vf", [("fp8_e4m3fn", "fp8_e4m3fn"), ("int4_kivi", "int4_g32")])
def test_noalloc_matches_workspace_entry_point(kf, vf):
    big = _case(kf, vf, [3000, 17, 0, 4500, 999], 8, 4, seed=5)
    small = _case(kf, vf, [70, 33], 8, 4, seed=6)
    for (inp, dev, orc), st in ((big, 0), (small, 0), (big, 96)):
        q = inp.q.to(DEV)
        table = inp.block_table.to(DEV)
        ctx = torch.tensor(inp.ctx_lens, dtype=torch.int32, device=DEV)
        ref = kvq.decode_attn(dev, q, table, ctx, split_tokens=st)
        out = torch.full_like(q, float("nan"))
        kvq.decode_attn_noalloc(dev, q, table, ctx, out, split_tokens=st)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        exp = o.decode_attn(orc, to_np16(inp.q), inp.block_table.numpy(), inp.ctx_lens)
        assert np.max(np.abs(out.float().cpu().numpy() - exp)) <= ATOL


def test_noalloc_rejects_a_workspace_beyond_its_array():
    inp, dev, orc = _case("int8", "int8", [64, 64], 2, 2, seed=7)
    q = inp.q.to(DEV)
    ctx = torch.tensor(inp.ctx_lens, dtype=torch.int32, device=DEV)
    # a block table addressing 2^24 tokens per sequence, cut into one-tile
    # shares: far more partial records than the fixed array holds
    table = torch.zeros((2, 1 << 20), dtype=torch.int32, device=DEV)
    table[:, :inp.block_table.shape[1]] = inp.block_table.to(DEV)
    need = kvq.decode_workspace_bytes(dev, 2, q.shape[1], table.shape[1], split_tokens=16)
    assert need > kvq.binding.NOALLOC_WORKSPACE_BYTES
    out = torch.empty_like(q)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_noalloc(dev, q, table, ctx, out, split_tokens=16)
    assert e.value.rc == -4  # KVQ_ERR_WORKSPACE
    # within the limit with the automatic partition
    kvq.decode_attn_noalloc(dev, q, table, ctx, out)
    torch.cuda.synchronize()
    exp = o.decode_attn(orc, to_np16(inp.q), table.cpu().numpy(), inp.ctx_lens)
    assert np.max(np.abs(out.float().cpu().numpy() - exp)) <= ATOL
