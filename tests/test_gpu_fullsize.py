"""Full-size parity of the large workloads, in the launch configuration the
benchmark times: a prefill write of every token but the last of each
sequence (one call), a write of the last token of every sequence (one call),
then one decode step with the automatic partition.  Every byte of the cache
(codes, scales, zero points, KIVI tails) is compared with the oracle, and so
is every (sequence, query head) row of the decode output (within 2e-3).
Then one chunked-prefill call over the same cache (a chunk of the last
positions of every sequence) is checked on sampled positions: every query
head of each sampled position, against the oracle's causal attention.

The oracle runs per sequence and slice of KV heads, in a pool of fresh
worker processes (NumPy only; they never touch the GPU)."""

import concurrent.futures as cf
import multiprocessing as mp
import os
import sys
import time

import numpy as np
import pytest
import torch

import quantized_paged_kv_write_amd as kvq
from kvq_testlib import ATOL
from quantized_paged_kv_write_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
WORKERS = max(1, min(8, (os.cpu_count() or 2) - 1))

# name -> (workload, context lengths or None for the workload's own, prefill chunk)
CASES = {
    "llama3_8b_fp8": ("llama3_8b_fp8", None, 512),
    "llama3_8b_int8k_int4v": ("llama3_8b_int8k_int4v", None, 1000),
    "llama3_70b_int8": ("llama3_70b_int8", None, 2048),
    "llama3_8b_kivi_int4": ("llama3_8b_kivi_int4", None, 2048),
    # the KIVI shape with fp16 tails of 31, 1 and 15 tokens (and none)
    "llama3_8b_kivi_int4_tails": ("llama3_8b_kivi_int4", [131072, 131071, 131041, 131055], 2048),
    "llama3_8b_e5m2": ("llama3_8b_e5m2", None, 512),
    # Walsh-Hadamard rotated keys and values
    "llama3_70b_int8_rot": ("llama3_70b_int8_rot", None, 2048),
}
PF_SAMPLES = 24  # sampled positions per sequence


@pytest.fixture(scope="module")
def pool():
    ex = cf.ProcessPoolExecutor(max_workers=WORKERS, mp_context=mp.get_context("spawn"))
    yield ex
    ex.shutdown()


def _run_workload(name):
    wname, ctx, chunk = CASES[name]
    w = wl.WORKLOADS[wname]
    seed = wl.seed_of(w)
    inp = wl.make_inputs(w, seed, DEV, ctx_lens=ctx)
    B = w.batch
    signs = wl.rotation_signs(w.head_dim, seed) if (w.rotate_k or w.rotate_v) else None
    cache = kvq.PagedKVCache(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype,
                             max_seqs=B, device=DEV, rotate_k=w.rotate_k, rotate_v=w.rotate_v, rot_signs=signs)
    last = torch.tensor([inp.seq_start[b] + inp.ctx_lens[b] - 1 for b in range(B)])
    mask = torch.ones(inp.k.shape[0], dtype=torch.bool)
    mask[last] = False
    pre = torch.nonzero(mask)[:, 0]
    slots, seqs = inp.slot_mapping, inp.seq_idx
    kvq.write(cache, inp.k[pre.to(DEV)], inp.v[pre.to(DEV)], slots[pre].to(DEV), seqs[pre].to(DEV))
    kvq.write(cache, inp.k[last.to(DEV)].contiguous(), inp.v[last.to(DEV)].contiguous(), slots[last].to(DEV),
              seqs[last].to(DEV))
    ctx_d = torch.tensor(inp.ctx_lens, dtype=torch.int32, device=DEV)
    out = kvq.decode_attn(cache, inp.q, inp.block_table.to(DEV), ctx_d)
    # chunked prefill over the same cache: the last `chunk` positions of every sequence
    qlen = [min(chunk, L) for L in inp.ctx_lens]
    ch = wl.chunk_queries(w, qlen, seed, DEV)
    pf = kvq.prefill_attn(cache, ch.q, ch.q_start.to(DEV), inp.block_table.to(DEV), ctx_d, ch.max_q_len)
    torch.cuda.synchronize()
    assert kvq.get_device_error() == 0
    return w, inp, cache, out, (ch, pf)


def _pieces(w, inp, cache, out, prefill):
    """Per (sequence, KV-head slice): the host data a worker needs."""
    H, D, bs = w.n_kv_heads, w.head_dim, w.block_size
    G = w.n_q_heads // H
    signs = None
    if w.rotate_k or w.rotate_v:
        signs = np.array(wl.rotation_signs(D, wl.seed_of(w)), np.uint32)
    bufs = cache.buffers()
    k_host = inp.k.cpu().numpy()
    v_host = inp.v.cpu().numpy()
    q_host = inp.q.cpu().numpy()
    out_host = out.cpu().numpy()
    ch, pf = prefill
    pf_q, pf_out = ch.q.cpu().numpy(), pf.cpu().numpy()
    rng = np.random.default_rng(wl.seed_of(w) + 100)
    for b in range(w.batch):
        L = inp.ctx_lens[b]
        st = inp.seq_start[b]
        npg = -(-L // bs)
        blocks = inp.block_table[b, :npg].to(DEV).long()
        # slices of about 2^17 token-heads each
        hs = max(1, min(H, (1 << 17) // max(L, 1)))
        while H % hs:
            hs -= 1
        gathered = {}
        for name, t in bufs.items():
            if name in ("k_tail", "v_tail"):
                gathered[name] = t[b].cpu().numpy()
            else:
                gathered[name] = t[blocks].cpu().numpy()
        n = ch.q_lens[b]
        pick = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.integers(0, n, PF_SAMPLES - 4)]))
        pick = pick[(pick >= 0) & (pick < n)]
        rows = int(ch.q_start[b]) + pick
        for h0 in range(0, H, hs):
            pages = {}
            for name, a in gathered.items():
                if (name in ("k_scales", "k_zeros") and w.k_dtype == "int4_kivi") or name in ("k_tail", "v_tail"):
                    pages[name] = a[:, h0:h0 + hs]  # (pages, H, D) or the tail (bs, H, D)
                else:
                    pages[name] = a[:, :, h0:h0 + hs]  # (pages or 32, bs, H, ...)
            yield {
                "b": b, "h0": h0, "k_fmt": w.k_dtype, "v_fmt": w.v_dtype, "block_size": bs, "head_dim": D,
                "k16": k_host[st:st + L, h0:h0 + hs], "v16": v_host[st:st + L, h0:h0 + hs], "pages": pages,
                "q": q_host[b, h0 * G:(h0 + hs) * G], "out": out_host[b, h0 * G:(h0 + hs) * G],
                "rot_k": signs if w.rotate_k else None, "rot_v": signs if w.rotate_v else None,
                "pf_q": pf_q[rows, h0 * G:(h0 + hs) * G], "pf_out": pf_out[rows, h0 * G:(h0 + hs) * G],
                "pf_pos": L - n + pick,
            }


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_whole_cache_and_every_row(name, pool):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import kvq_fullsize
    t0 = time.time()
    w, inp, cache, out, prefill = _run_workload(name)
    print(f"[fullsize] {name}: GPU write + decode done in {time.time() - t0:.1f} s; oracle in {WORKERS} workers",
          flush=True)
    futs = [pool.submit(kvq_fullsize.check_piece, p) for p in _pieces(w, inp, cache, out, prefill)]
    del cache
    bad, worst, worst16, rows, nbytes = [], 0.0, 0.0, 0, 0
    pf_worst, pf_rows, pf_excess, pf_maxref = 0.0, 0, -1.0, 0.0
    for f in cf.as_completed(futs):
        r = f.result()
        if r["mismatch"]:
            bad.append((r["b"], r["h0"], r["mismatch"]))
        worst = max(worst, r["err"])
        worst16 = max(worst16, r["err16"])
        rows += r["rows"]
        nbytes += r["bytes"]
        pf_worst = max(pf_worst, r["pf_err"])
        pf_excess = max(pf_excess, r["pf_excess"])
        pf_maxref = max(pf_maxref, r["pf_maxref"])
        pf_rows += r["pf_rows"]
    print(f"[fullsize] {name}: {nbytes} cache bytes compared, {rows} output rows, max|err| {worst:.3e} "
          f"(vs fp16-rounded oracle {worst16:.3e}); prefill: {pf_rows} sampled rows, max|err| {pf_worst:.3e}, "
          f"max|o| {pf_maxref:.2f}, max excess over the per-element bar {pf_excess:.3e}; "
          f"{time.time() - t0:.1f} s", flush=True)
    assert not bad, bad[:5]
    assert rows == w.batch * w.n_q_heads
    assert worst <= ATOL, (worst, worst16)
    # prefill rows: 2e-3, or the fp16 half-ulp of |o| + 1e-3 where that is larger (|o| >= 4)
    assert pf_rows > 0 and pf_excess <= 0.0, (pf_worst, pf_excess)
