"""Seeded synthetic inputs for the quantized paged KV cache.

This module only draws inputs (queries, keys, values, context lengths, block
tables, slot mappings).  It contains none of the quantization or attention
arithmetic, so the GPU path and the CPU oracle can both be fed from it.

Value structure follows the pages' description of real KV tensors:
  * keys have a few outlier channels per head, and the same channels stay
    large across tokens (12 KV Cache Quantization, section 5 on why keys are
    more sensitive than values; KIVI in "Quantized KV caches in production",
    Numerical Formats);
  * the first few tokens of a sequence (attention sinks) carry large keys
    ("Use Less Memory: Quantization and Offloading", section 2.2);
  * values and queries are roughly zero-centred (same page, section 2.1).
Paging follows the PagedAttention description (KV Cache Quantization glossary,
PagedAttention): every sequence owns whole fixed-size blocks, and physical
block ids are a seeded shuffle, so consecutive pages of a sequence are not
adjacent in memory.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    k_dtype: str
    v_dtype: str
    ctx: tuple  # ("fixed", L) or ("uniform", lo, hi)
    k_outlier_channels: int  # per KV head
    outlier_mult: float = 20.0
    sink_tokens: int = 0
    sink_mult: float = 10.0
    n_layers: int = 32  # for the attention-only tokens/s projection
    rotate_k: bool = False  # Walsh-Hadamard rotation of the stored keys / values
    rotate_v: bool = False
    base: str = ""  # draw the inputs of this workload (same seed), if set

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five shapes the measurements are quoted on.
WORKLOADS = {
    # batch 2, 4 q / 2 kv heads, D 64, ctx 256, bs 16, INT8 per token-head.
    "tiny_int8": Workload("tiny_int8", 2, 4, 2, 64, 16, "int8", "int8", ("fixed", 256), 2),
    # Llama-3-8B layer, FP8 E4M3FN per token-head, batch 27 x 32k.
    "llama3_8b_fp8": Workload("llama3_8b_fp8", 27, 32, 8, 128, 16, "fp8_e4m3fn", "fp8_e4m3fn",
                              ("fixed", 32768), 4, sink_tokens=4),
    # Mixed bits: INT8 keys, INT4 group-32 values, ragged ctx in [8192, 32768].
    "llama3_8b_int8k_int4v": Workload("llama3_8b_int8k_int4v", 13, 32, 8, 128, 16, "int8", "int4_g32",
                                      ("uniform", 8192, 32768), 2),
    # Llama-3-70B layer, INT8 per token-head, batch 8 x 64k.
    "llama3_70b_int8": Workload("llama3_70b_int8", 8, 64, 8, 128, 16, "int8", "int8",
                                ("fixed", 65536), 4, n_layers=80),
    # KIVI-style INT4 keys (per channel, 32-token groups) + INT4 g32 values.
    "llama3_8b_kivi_int4": Workload("llama3_8b_kivi_int4", 4, 32, 8, 128, 32, "int4_kivi", "int4_g32",
                                    ("fixed", 131072), 4, sink_tokens=4),
    # The Llama-3-8B FP8 shape with the E5M2 variant for keys and values.
    "llama3_8b_e5m2": Workload("llama3_8b_e5m2", 27, 32, 8, 128, 16, "fp8_e5m2", "fp8_e5m2",
                               ("fixed", 32768), 4, sink_tokens=4),
}
# The Llama-3-70B INT8 layer with Walsh-Hadamard rotated keys and values
# (per-token INT8 keys with channel outliers are where the rotation helps).
WORKLOADS["llama3_70b_int8_rot"] = WORKLOADS["llama3_70b_int8"].with_(name="llama3_70b_int8_rot", rotate_k=True,
                                                                       rotate_v=True, base="llama3_70b_int8")
# The KIVI layer's shape with symmetric INT4 group-32 keys and values, both
# Walsh-Hadamard rotated (the 4-bit alternative to per-channel keys).
WORKLOADS["llama3_8b_int4_rot"] = WORKLOADS["llama3_8b_kivi_int4"].with_(
    name="llama3_8b_int4_rot", block_size=16, k_dtype="int4_g32", rotate_k=True, rotate_v=True,
    base="llama3_8b_kivi_int4")
ORDER = ["tiny_int8", "llama3_8b_fp8", "llama3_8b_int8k_int4v", "llama3_70b_int8", "llama3_8b_kivi_int4",
         "llama3_8b_e5m2", "llama3_70b_int8_rot"]


def seed_of(w: Workload) -> int:
    """Seed of a workload's inputs: its position in ORDER plus one (a variant
    with `base` set uses its base's seed, so both see the same inputs)."""
    return ORDER.index(w.base or w.name) + 1


def rotation_signs(head_dim: int, seed: int) -> list:
    """Random signs of a Walsh-Hadamard rotation drawn from a seeded CPU
    generator: 8 uint32 words, bit c set = channel c negated."""
    g = torch.Generator().manual_seed(seed)
    bits = torch.randint(0, 2, (head_dim,), generator=g)
    words = [0] * 8
    for c in range(head_dim):
        if int(bits[c]):
            words[c // 32] |= 1 << (c % 32)
    return words


def ctx_lengths(w: Workload, seed: int) -> list:
    g = torch.Generator().manual_seed(seed)
    if w.ctx[0] == "fixed":
        return [int(w.ctx[1])] * w.batch
    lo, hi = w.ctx[1], w.ctx[2]
    return [int(x) for x in torch.randint(lo, hi + 1, (w.batch,), generator=g)]


@dataclass
class Inputs:
    w: Workload
    ctx_lens: list  # python ints, one per sequence
    q: torch.Tensor  # (B, Hq, D) fp16
    k: torch.Tensor  # (T, H, D) fp16, tokens of seq 0 first, in position order
    v: torch.Tensor  # (T, H, D) fp16
    seq_start: list  # first token index of each sequence in k/v
    num_blocks: int
    block_table: torch.Tensor  # (B, max_blocks) int32, padded with 0
    slot_mapping: torch.Tensor  # (T,) int64
    seq_idx: torch.Tensor  # (T,) int32
    positions: torch.Tensor  # (T,) int64 position of each token in its sequence
    outlier_channels: torch.Tensor  # (H, n) int64


def make_inputs(w: Workload, seed: int, device="cpu", ctx_lens=None, extra_blocks: int = 0) -> Inputs:
    """Draw one workload.  Structure (ctx lens, outlier channels, block
    permutation) comes from a CPU generator, bulk values from a generator on
    `device`; both are seeded with `seed`.  `extra_blocks` adds unused
    physical blocks to the pool (so block ids do not cover it exactly)."""
    cpu = torch.Generator().manual_seed(seed)
    if ctx_lens is None:
        ctx_lens = ctx_lengths(w, seed)
    ctx_lens = [int(x) for x in ctx_lens]
    B, H, Hq, D, bs = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.block_size
    assert len(ctx_lens) == B
    T = sum(ctx_lens)
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed)

    q = torch.randn((B, Hq, D), generator=gen, device=dev, dtype=torch.float32)
    k = torch.randn((T, H, D), generator=gen, device=dev, dtype=torch.float32)
    v = torch.randn((T, H, D), generator=gen, device=dev, dtype=torch.float32)

    n_out = w.k_outlier_channels
    outl = torch.stack([torch.randperm(D, generator=cpu)[:n_out] for _ in range(H)]) if n_out else \
        torch.zeros((H, 0), dtype=torch.int64)
    if n_out:
        mult = torch.ones((H, D), dtype=torch.float32)
        mult.scatter_(1, outl, w.outlier_mult)
        k *= mult.to(dev)[None]
    seq_start, pos_list = [], []
    s = 0
    for L in ctx_lens:
        seq_start.append(s)
        if w.sink_tokens:
            n = min(w.sink_tokens, L)
            k[s:s + n] *= w.sink_mult
        s += L
    positions = torch.cat([torch.arange(L, dtype=torch.int64) for L in ctx_lens]) if T else \
        torch.zeros(0, dtype=torch.int64)
    seq_idx = torch.cat([torch.full((L,), b, dtype=torch.int32) for b, L in enumerate(ctx_lens)]) if T else \
        torch.zeros(0, dtype=torch.int32)

    pages = [(L + bs - 1) // bs for L in ctx_lens]
    num_blocks = sum(pages) + extra_blocks
    perm = torch.randperm(num_blocks, generator=cpu).to(torch.int32)
    max_blocks = max(max(pages), 1)
    block_table = torch.zeros((B, max_blocks), dtype=torch.int32)
    o = 0
    for b, n in enumerate(pages):
        block_table[b, :n] = perm[o:o + n]
        o += n
    slot_mapping = torch.empty(T, dtype=torch.int64)
    for b, L in enumerate(ctx_lens):
        p = torch.arange(L, dtype=torch.int64)
        st = seq_start[b]
        slot_mapping[st:st + L] = block_table[b].to(torch.int64)[p // bs] * bs + p % bs

    return Inputs(w=w, ctx_lens=ctx_lens, q=q.to(torch.float16), k=k.to(torch.float16), v=v.to(torch.float16),
                  seq_start=seq_start, num_blocks=num_blocks, block_table=block_table,
                  slot_mapping=slot_mapping, seq_idx=seq_idx, positions=positions, outlier_channels=outl)


@dataclass
class Chunks:
    """Queries of a chunked-prefill step: sequence b brings q_lens[b] queries
    (its last q_lens[b] positions), stored one sequence after another."""
    q: torch.Tensor        # (Tq, Hq, D) fp16
    q_start: torch.Tensor  # (B + 1,) int32
    q_lens: list
    max_q_len: int


def chunk_queries(w: Workload, q_lens, seed: int, device="cpu") -> Chunks:
    """Draw the chunk queries of one prefill step: N(0, 1) in fp32 from a
    generator on `device` seeded with `seed` + 7919, rounded to fp16 (the
    value distribution of the decode queries)."""
    q_lens = [int(x) for x in q_lens]
    Tq = sum(q_lens)
    gen = torch.Generator(device=torch.device(device)).manual_seed(seed + 7919)
    q = torch.randn((Tq, w.n_q_heads, w.head_dim), generator=gen, device=device, dtype=torch.float32)
    starts = [0]
    for n in q_lens:
        starts.append(starts[-1] + n)
    return Chunks(q=q.to(torch.float16), q_start=torch.tensor(starts, dtype=torch.int32), q_lens=q_lens,
                  max_q_len=max(q_lens + [0]))
