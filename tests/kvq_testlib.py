"""Shared helpers for the parity tests: feed the same seeded inputs to the CPU
oracle and to the HIP library, and compare what comes back."""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle as o
from quantized_paged_kv_write_amd import workloads as wl

ATOL = 2e-3  # decode attention: max |out_gpu(fp16) - o(fp64)|
from kvq_fullsize import excess, tolerance  # noqa: E402,F401  (the per-element bar, used for prefill)


def garbage_like(shape, dtype, seed):
    """Seeded random bytes (any bit pattern, including NaN/Inf codes)."""
    g = torch.Generator().manual_seed(seed)
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    raw = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)
    return raw.view(dtype).reshape(shape)


def sign_bits(D, seed):
    """Seeded random signs of a Walsh-Hadamard rotation: 8 uint32 words, bit c
    set = channel c negated (about half the channels)."""
    g = np.random.default_rng(seed)
    words = np.zeros(8, np.uint32)
    for c in np.nonzero(g.integers(0, 2, D))[0]:
        words[c // 32] |= np.uint32(1) << np.uint32(c % 32)
    return words


def new_caches(num_blocks, bs, H, D, kf, vf, max_seqs, device, seed=99, garbage=True, rot_k=None, rot_v=None):
    """(device PagedKVCache, OracleCache) holding identical initial bytes;
    rot_k / rot_v: sign words of a Walsh-Hadamard rotation of keys / values
    (one set of signs serves both, so they must be equal when both given)."""
    from quantized_paged_kv_write_amd import PagedKVCache
    signs = rot_k if rot_k is not None else rot_v
    assert rot_k is None or rot_v is None or np.array_equal(rot_k, rot_v)
    dev = PagedKVCache(num_blocks, bs, H, D, kf, vf, max_seqs=max_seqs, device=device, rotate_k=rot_k is not None,
                       rotate_v=rot_v is not None, rot_signs=None if signs is None else [int(x) for x in signs])
    orc = o.OracleCache(num_blocks, bs, H, D, kf, vf, max_seqs=max(max_seqs, 1), rot_k=rot_k, rot_v=rot_v)
    if garbage:
        for i, (name, t) in enumerate(dev.buffers().items()):
            init = garbage_like(tuple(t.shape), t.dtype, seed + i)
            t.copy_(init.to(t.device))
            getattr(orc, name)[...] = init.numpy().view(getattr(orc, name).dtype)
    return dev, orc


def compare_buffers(dev, orc, names=None):
    """Bitwise equality of every cache buffer; returns {name: mismatches}."""
    bad = {}
    for name, t in dev.buffers().items():
        if names is not None and name not in names:
            continue
        a = t.cpu().numpy()
        b = getattr(orc, name)
        a = a.view(np.uint16) if a.dtype == np.float16 else a
        b = b.view(np.uint16) if b.dtype == np.float16 else b
        if a.shape != b.shape:
            bad[name] = f"shape {a.shape} vs {b.shape}"
            continue
        n = int((a != b).sum())
        if n:
            idx = np.argwhere(a != b)[:5]
            bad[name] = (n, [(tuple(i), int(a[tuple(i)]), int(b[tuple(i)])) for i in idx])
    return bad


def to_np16(t):
    return t.detach().cpu().numpy().astype(np.float16)


def write_both(inp: wl.Inputs, dev, orc, device):
    """Quantize-on-write of all tokens of `inp` on the GPU and in the oracle."""
    import quantized_paged_kv_write_amd as kvq
    kvq.write(dev, inp.k.to(device), inp.v.to(device), inp.slot_mapping.to(device), inp.seq_idx.to(device))
    o.write(orc, to_np16(inp.k), to_np16(inp.v), inp.slot_mapping.numpy(), inp.seq_idx.numpy())


def decode_both(inp: wl.Inputs, dev, orc, device, split_tokens=0, sm_scale=0.0):
    import quantized_paged_kv_write_amd as kvq
    ctx = torch.tensor(inp.ctx_lens, dtype=torch.int32)
    out = kvq.decode_attn(dev, inp.q.to(device), inp.block_table.to(device), ctx.to(device), sm_scale=sm_scale,
                          split_tokens=split_tokens)
    torch.cuda.synchronize()
    ref = o.decode_attn(orc, to_np16(inp.q), inp.block_table.numpy(), inp.ctx_lens,
                        sm_scale=None if sm_scale == 0 else sm_scale)
    return out.float().cpu().numpy().astype(np.float64), ref


def decode_error(got, ref):
    """(max |got - ref|, max |got - fp16(ref)|): the second separates the final
    fp16 rounding from arithmetic error."""
    return float(np.max(np.abs(got - ref))), float(np.max(np.abs(got - ref.astype(np.float16).astype(np.float64))))


def oracle_head_attention(inp: wl.Inputs, b: int, h: int, sm_scale=None):
    """fp64 attention of the G query heads of KV head h of sequence b, from the
    oracle's quantization of that sequence's rows (no paging involved)."""
    w = inp.w
    L = inp.ctx_lens[b]
    st = inp.seq_start[b]
    k16 = to_np16(inp.k[st:st + L, h:h + 1])
    v16 = to_np16(inp.v[st:st + L, h:h + 1])
    K, V = o.dequantized_sequence(k16, v16, w.k_dtype, w.v_dtype)
    G = w.n_q_heads // w.n_kv_heads
    q = to_np16(inp.q[b, h * G:(h + 1) * G]).astype(np.float64)
    return o.attention_fp64(q, K, V, sm_scale)


def algorithmic_decode_bytes(w: wl.Workload, ctx_lens) -> int:
    """Bytes the decode step must move: codes + scale metadata of every cached
    token-head, the used block-table entries, q and out."""
    H, D, bs = w.n_kv_heads, w.head_dim, w.block_size
    per_tok = H * (o.stored_bytes_per_token_head(w.k_dtype, D) + o.stored_bytes_per_token_head(w.v_dtype, D))
    total = 0
    for L in ctx_lens:
        if w.k_dtype == o.INT4_KIVI:
            nf = (L // 32) * 32
            total += nf * per_tok + (L - nf) * H * D * 2 * 2
        else:
            total += L * per_tok
        total += math.ceil(L / bs) * 4
    total += 2 * len(ctx_lens) * w.n_q_heads * D * 2
    return total


def algorithmic_write_bytes(w: wl.Workload, T: int) -> int:
    """Bytes a write of T tokens must move: fp16 K and V in, codes + scale
    metadata out, 8-byte slots in (KIVI adds the 4-byte sequence index)."""
    H, D = w.n_kv_heads, w.head_dim
    per = H * (2 * D * 2 + o.stored_bytes_per_token_head(w.k_dtype, D) + o.stored_bytes_per_token_head(w.v_dtype, D))
    return T * (per + 8 + (4 if w.k_dtype == o.INT4_KIVI else 0))
