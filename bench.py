"""Benchmark: quantized paged decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--extra A,B,...|none]
                    [--no-cpu-baseline] [--no-probes]

One step is one decode step of the workload's batch: quantize-on-write of the
new token of every sequence into the paged cache (kvq_write), then decode
attention over the whole cache (kvq_decode_attn).  Two identical caches are
filled before timing by a prefill write of all earlier tokens (the write into
the first is timed on its own for the write bandwidth); consecutive timed steps
alternate between them, so no call reads what the previous one left in the
memory-side cache.  Prints one JSON line.

value = decode KV-read bytes per step / step time (GB/s); the roofline entry
is for the decode kernels (split-K attention + split merge), timed with HIP
events on the stream they run on.  Bytes are algorithmic: what the method has
to move (codes, scale metadata, block-table entries, q and out; for the write
the fp16 K/V read, codes and metadata written, slot indices).  For symmetric
formats the same prefill is also timed through kvq_write_static with
calibrated per-head scales (write_static_GBps).

The headline workload (--workload, default the Llama-3-8B FP8 layer) gives
`value`, the roofline and the CPU baseline; every other large workload
(--extra) is measured the same way afterwards and reported, with the headline
one, under "workloads" (decode call and step GB/s, % of peak, write GB/s, and
the quality statistic: the decode output against float64 attention over the
unquantized fp16 K/V).  "stream_probes" are plain streaming rates of this GPU
with the same 16-byte non-temporal accesses (libkvq_probe.so).

Chunked prefill (--prefill A:n,B:m): over the filled cache of workload A, one
kvq_prefill_attn call whose chunks are the last n positions of every
sequence (their keys and values are already in the cache), timed with HIP
events; reported under that workload's "prefill" entry as algorithmic
TFLOP/s (4 D flops per visible (query head, token) pair: q.k and p v) against
the 2.5 PFLOP/s dense fp16 peak, and chunk tokens per second.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD specification
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, AMD specification
QMAX = {"int8": 127.0, "fp8_e4m3fn": 448.0, "fp8_e5m2": 57344.0, "int4_g32": 7.0}  # symmetric formats
# sources of the decode kernels (their hash tags the committed counter summaries)
DECODE_SRC = [os.path.join(ROOT, "quantized_paged_kv_write_amd", "csrc", f) for f in ("kvq_decode.h", "kvq_decode.hip")]
CAL_ELEMS = 1 << 28  # calibration kernel: negate 1 GiB of fp32 (reads 1 GiB, writes 1 GiB)


def decode_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_profile_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_traffic.json")


def load_traffic(workload: str):
    """HBM bytes per decode call from the committed counter summary, or None
    when there is none or the decode kernels changed since it was taken."""
    path = traffic_profile_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("decode_source_sha256_16") != decode_source_hash():
        return None
    return d["hbm_bytes_per_decode_call"]


def pmc_summary(fetch_csv: str, write_csv: str, workload: str, command: str) -> dict:
    """Reduce two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) to HBM bytes per decode call, calibrated by the counters of the
    elementwise negation of CAL_ELEMS fp32 values that bench.py launches
    (algorithmically 4 CAL_ELEMS bytes read and written)."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        vals = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)
        return vals

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, key):
        ks = [k for k in vals if key in k]
        if not ks:
            raise SystemExit(f"no kernel matching {key!r} in the counter file")
        v = [x for k in ks for x in vals[k]]
        return sum(v) / len(v), len(v)

    cal_bytes = 4.0 * CAL_ELEMS
    cal_f, _ = pick(f, "neg_kernel")
    cal_w, _ = pick(w, "neg_kernel")
    kf, kw = cal_bytes / cal_f, cal_bytes / cal_w
    out = {"workload": workload, "decode_source_sha256_16": decode_source_hash(), "command": command,
           "calibration": {"kernel": "elementwise negation of 2^28 fp32", "bytes_each_way": cal_bytes,
                           "fetch_counter_bytes": cal_f, "write_counter_bytes": cal_w,
                           "fetch_factor": kf, "write_factor": kw}, "kernels": {}}
    total = 0.0
    for key in ("plan_kernel", "decode_split_kernel", "merge_kernel"):
        if not any(key in k for k in f):
            continue
        fb, nf = pick(f, key)
        wb, nw = pick(w, key)
        out["kernels"][key] = {"fetch_bytes": fb * kf, "write_bytes": wb * kw, "launches": nf}
        total += fb * kf + wb * kw
    out["hbm_bytes_per_decode_call"] = total
    return out


def row_bytes(fmt: str, D: int) -> float:
    """Stored bytes per (token, head): codes + fp16 scale metadata."""
    if fmt == "int4_kivi":
        return D / 2 + 2 * 2 * D / 32  # scale + zero per channel per 32-token page
    if fmt == "int4_g32":
        return D / 2 + 2 * D / 32
    return D + 2


def decode_bytes(w, ctx_lens) -> int:
    H, D, bs = w.n_kv_heads, w.head_dim, w.block_size
    per_tok = H * (row_bytes(w.k_dtype, D) + row_bytes(w.v_dtype, D))
    total = 0.0
    for L in ctx_lens:
        if w.k_dtype == "int4_kivi":
            nf = (L // 32) * 32
            total += nf * per_tok + (L - nf) * H * D * 2 * 2  # fp16 tail rows
        else:
            total += L * per_tok
        total += math.ceil(L / bs) * 4  # block-table entries
    total += 2 * len(ctx_lens) * w.n_q_heads * D * 2  # q in, out
    return int(total)


def write_bytes(w, T: int) -> int:
    H, D = w.n_kv_heads, w.head_dim
    per = H * (2 * D * 2 + row_bytes(w.k_dtype, D) + row_bytes(w.v_dtype, D))
    return int(T * (per + 8 + (4 if w.k_dtype == "int4_kivi" else 0)))


def host_info() -> dict:
    """Logical CPUs and CPU model of the host the CPU baseline ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_logical_cpus": os.cpu_count(), "host_cpu_model": model}


def cpu_baseline(w, inp, budget_s: float):
    """The CPU oracle, single-threaded, on whole sequences of the same
    workload until about budget_s seconds of decode work have been timed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as o

    dec_t = wr_t = 0.0
    dec_b = wr_b = 0
    seqs = 0
    with threadpool_limits(limits=1):
        for b in range(w.batch):
            L = inp.ctx_lens[b]
            st = inp.seq_start[b]
            k16 = inp.k[st:st + L].cpu().numpy()
            v16 = inp.v[st:st + L].cpu().numpy()
            npg = -(-L // w.block_size)
            table = np.arange(npg, dtype=np.int64)[None]
            pos = np.arange(L)
            slots = table[0, pos // w.block_size] * w.block_size + pos % w.block_size
            cache = o.OracleCache(npg, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype, max_seqs=1)
            t0 = time.perf_counter()
            o.write(cache, k16, v16, slots, np.zeros(L, np.int32))
            t1 = time.perf_counter()
            o.decode_attn(cache, inp.q[b:b + 1].cpu().numpy(), table, [L])
            t2 = time.perf_counter()
            wr_t += t1 - t0
            dec_t += t2 - t1
            wr_b += write_bytes(w, L)
            dec_b += decode_bytes(w.with_(batch=1), [L])
            seqs += 1
            if dec_t + wr_t >= budget_s:
                break
    res = {
        "value": round(dec_b / dec_t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{seqs} of {w.batch} sequences (ctx {inp.ctx_lens[0]}), decode step over their cache; "
                  f"oracle write of the same sequences {wr_b / wr_t / 1e9:.4f} GB/s",
        "decode_s": round(dec_t, 3), "write_s": round(wr_t, 3),
    }
    res.update(host_info())
    return res


def quality(w, inp, out, sm_scale=None, sample=3):
    """Quality statistic (reported, not gated): the decode output against
    float64 attention over the ORIGINAL fp16 keys and values (no
    quantization), on `sample` sequences (first, middle, last) and all their
    query heads: max |out - ref| and ||out - ref||_2 / ||ref||_2.  Plain
    torch float64 on the GPU."""
    import torch
    B, H, D = w.batch, w.n_kv_heads, w.head_dim
    G = w.n_q_heads // H
    scale = sm_scale if sm_scale else 1.0 / math.sqrt(D)
    bs = sorted({0, B // 2, B - 1})[:sample]
    num = den = 0.0
    mx = 0.0
    for b in bs:
        L = inp.ctx_lens[b]
        st = inp.seq_start[b]
        if L == 0:
            continue
        K = inp.k[st:st + L].double()
        V = inp.v[st:st + L].double()
        for h in range(H):
            qh = inp.q[b, h * G:(h + 1) * G].double()  # (G, D)
            s = torch.matmul(K[:, h, :].contiguous(), qh.t().contiguous()) * scale  # (L, G)
            p = torch.softmax(s, dim=0)
            ref = torch.matmul(p.t().contiguous(), V[:, h, :].contiguous())  # (G, D)
            got = out[b, h * G:(h + 1) * G].double()
            d = got - ref
            mx = max(mx, float(d.abs().max()))
            num += float((d * d).sum())
            den += float((ref * ref).sum())
    return {"max_abs": mx, "rel_l2": math.sqrt(num / den) if den > 0 else 0.0,
            "sample": f"sequences {bs}, all {w.n_q_heads} query heads; reference = float64 attention over the "
                      "unquantized fp16 K/V"}


def stream_probes(dev):
    """Plain HBM streaming rates with the same 16-byte non-temporal loads and
    stores the cache kernels use (libkvq_probe.so): read only, copy, and the
    2:1 read/write mix of the write path.  GB/s of bytes moved."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "quantized_paged_kv_write_amd", "libkvq_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.kvq_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.kvq_probe_stream.restype = ctypes.c_int
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for mode, name, moved in ((0, "read_GBps", nbytes), (1, "copy_GBps", 2 * nbytes),
                              (2, "read2_write1_GBps", nbytes + nbytes // 2)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        run = lambda: L.kvq_probe_stream(mode, ctypes.c_void_p(src.data_ptr()),  # noqa: E731
                                         ctypes.c_void_p(dst.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                         0, sp)
        for _ in range(2):
            if run() != 0:
                return None
        ev[0].record(stream)
        for _ in range(10):
            run()
        ev[1].record(stream)
        torch.cuda.synchronize()
        res[name] = round(moved * 10 / (ev[0].elapsed_time(ev[1]) * 1e6), 1)
    del src, dst
    return res


def prefill_flops(w, ctx_lens, q_lens) -> int:
    """Algorithmic flops of one chunked-prefill call: query i of a chunk of n
    over a context of L sees L - n + i + 1 tokens, each costing q.k and p v
    (2 D flops each) per query head."""
    tot = 0
    for L, n in zip(ctx_lens, q_lens):
        n = min(n, L)
        tot += n * (L - n) + n * (n + 1) // 2
    return 4 * w.head_dim * w.n_q_heads * tot


def prefill_measure(w, inp, cache, chunk, reps, dev="cuda"):
    """One chunked-prefill call over the filled cache (chunks = the last
    `chunk` positions of every sequence), timed over `reps` calls."""
    import torch

    import quantized_paged_kv_write_amd as kvq
    from quantized_paged_kv_write_amd import workloads as wl

    qlen = [min(chunk, L) for L in inp.ctx_lens]
    ch = wl.chunk_queries(w, qlen, wl.seed_of(w), dev)
    q_start = ch.q_start.to(dev)
    table = inp.block_table.to(dev)
    ctx_d = torch.tensor(inp.ctx_lens, dtype=torch.int32, device=dev)
    out = torch.empty_like(ch.q)
    need = kvq.prefill_workspace_bytes(cache, ch.q.shape[0], w.n_q_heads)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    stream = torch.cuda.current_stream()
    for _ in range(2):
        kvq.prefill_attn(cache, ch.q, q_start, table, ctx_d, ch.max_q_len, out=out, workspace=ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        kvq.prefill_attn(cache, ch.q, q_start, table, ctx_d, ch.max_q_len, out=out, workspace=ws)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    times = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    ms = times[len(times) // 2]
    flops = prefill_flops(w, inp.ctx_lens, qlen)
    tf = flops / (ms * 1e9)
    res = {"chunk": chunk, "query_rows": int(ch.q.shape[0]), "flops": flops, "call_ms_median": round(ms, 4),
           "call_ms_min": round(times[0], 4), "TFLOPs": round(tf, 2),
           "pct_mfma_peak_fp16": round(100 * tf / MFMA_PEAK_TFLOPS, 2),
           "chunk_tokens_per_s": round(ch.q.shape[0] / (ms * 1e-3), 1),
           "kernel": "prefill_kernel (one kvq_prefill_attn call)"}
    print(f"[bench] {w.name}: prefill chunk {chunk} x {w.batch}: {ms:.3f} ms = {tf:.1f} TFLOP/s "
          f"({res['pct_mfma_peak_fp16']:.1f}% of the fp16 MFMA peak)", file=sys.stderr, flush=True)
    return res


def measure(w, args, steps, warmup, dev="cuda", want_inputs=False):
    """Fill two identical caches with the workload's prefill, time the
    prefill write, then time `steps` decode steps (write of the new token of
    every sequence + decode over the whole cache).  Returns a result dict (and
    the inputs, for the CPU baseline)."""
    import torch

    import quantized_paged_kv_write_amd as kvq
    from quantized_paged_kv_write_amd import workloads as wl

    seed = wl.seed_of(w)
    print(f"[bench] workload {w.name}: B={w.batch} Hq={w.n_q_heads} H={w.n_kv_heads} D={w.head_dim} "
          f"bs={w.block_size} K={w.k_dtype} V={w.v_dtype}", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, seed, dev)
    ctx = inp.ctx_lens
    B = w.batch
    signs = wl.rotation_signs(w.head_dim, seed) if (w.rotate_k or w.rotate_v) else None
    caches = [kvq.PagedKVCache(inp.num_blocks, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype,
                               max_seqs=B, device=dev, rotate_k=w.rotate_k, rotate_v=w.rotate_v, rot_signs=signs)
              for _ in range(args.caches)]
    cache = caches[0]
    pos = inp.positions
    last = torch.tensor([inp.seq_start[b] + ctx[b] - 1 for b in range(B)])
    pre_mask = torch.ones(pos.numel(), dtype=torch.bool)
    pre_mask[last] = False
    pre_idx = torch.nonzero(pre_mask)[:, 0].to(dev)
    k_pre, v_pre = inp.k[pre_idx], inp.v[pre_idx]
    s_pre = inp.slot_mapping.to(dev)[pre_idx]
    q_pre = inp.seq_idx.to(dev)[pre_idx]
    last_d = last.to(dev)
    k_new, v_new = inp.k[last_d].contiguous(), inp.v[last_d].contiguous()
    s_new = inp.slot_mapping.to(dev)[last_d].contiguous()
    q_new = inp.seq_idx.to(dev)[last_d].contiguous()
    q = inp.q
    table = inp.block_table.to(dev)
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(kvq.decode_workspace_bytes(cache, B, w.n_q_heads, table.shape[1]), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    # ---- prefill write (cache fill), timed for the write bandwidth --------
    for c in caches:
        kvq.write(c, k_pre, v_pre, s_pre, q_pre)
    torch.cuda.synchronize()

    # Settle: after idle time or a different heavy kernel, decode calls run
    # at a varying, slower rate for tens of milliseconds (clock and power
    # management adjusting), so untimed decode calls run for a fixed time
    # before each timed phase.
    def settle():
        t_settle = time.perf_counter() + args.settle
        while time.perf_counter() < t_settle:
            for i in range(8):
                kvq.decode_attn(caches[i % len(caches)], q, table, ctx_d, out=out, workspace=ws)
            torch.cuda.synchronize()

    settle()
    # two untimed writes first: the clocks settle on the write's own load
    for _ in range(2):
        kvq.write(cache, k_pre, v_pre, s_pre, q_pre)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.prefill_reps):
        kvq.write(cache, k_pre, v_pre, s_pre, q_pre)
    ev[1].record(stream)
    torch.cuda.synchronize()
    write_ms = ev[0].elapsed_time(ev[1]) / args.prefill_reps
    wbytes = write_bytes(w, pre_idx.numel())
    print(f"[bench] prefill write of {pre_idx.numel()} tokens: {write_ms:.3f} ms, "
          f"{wbytes / write_ms / 1e6:.1f} GB/s", file=sys.stderr, flush=True)
    # The same prefill with calibrated per-head scales (kvq_write_static, no
    # amax pass): one scale per KV head, max|x| over the prefill / q_max,
    # into the second cache (rewritten dynamically before the decode steps).
    static_ms = None
    if w.k_dtype in QMAX and w.v_dtype in QMAX:
        ks = (k_pre.float().abs().amax(dim=(0, 2)) / QMAX[w.k_dtype]).half().contiguous()
        vs = (v_pre.float().abs().amax(dim=(0, 2)) / QMAX[w.v_dtype]).half().contiguous()
        sc = caches[-1]
        kvq.write_static(sc, k_pre, v_pre, s_pre, ks, vs)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.prefill_reps):
            kvq.write_static(sc, k_pre, v_pre, s_pre, ks, vs)
        ev[1].record(stream)
        torch.cuda.synchronize()
        static_ms = ev[0].elapsed_time(ev[1]) / args.prefill_reps
        kvq.write(sc, k_pre, v_pre, s_pre, q_pre)
        torch.cuda.synchronize()
        print(f"[bench] prefill write with calibrated scales: {static_ms:.3f} ms, "
              f"{wbytes / static_ms / 1e6:.1f} GB/s", file=sys.stderr, flush=True)

    # known-size kernel for calibrating the FETCH_SIZE / WRITE_SIZE counters
    cal = torch.ones(CAL_ELEMS, dtype=torch.float32, device=dev)
    cal = cal.neg()
    torch.cuda.synchronize()
    del cal

    # ---- decode steps -------------------------------------------------------
    # Step i writes the new token of every sequence into cache i % caches and
    # decodes it: consecutive steps read different (identical) caches, so a
    # call never reuses what the previous one left in the 256 MB memory-side
    # cache (the steps' working sets are 0.45-1.8 GB).
    def step(i, evs=None):
        c = caches[i % len(caches)]
        if evs is not None:
            evs[0].record(stream)
        kvq.write(c, k_new, v_new, s_new, q_new)
        if evs is not None:
            evs[1].record(stream)
        kvq.decode_attn(c, q, table, ctx_d, out=out, workspace=ws)
        if evs is not None:
            evs[2].record(stream)

    settle()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    stepw_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    ms_per_step = wall * 1e3 / steps
    dbytes = decode_bytes(w, ctx)
    res = {
        "workload": w.name, "batch": B,
        "ctx_lens": "fixed %d" % ctx[0] if len(set(ctx)) == 1
        else f"ragged {min(ctx)}..{max(ctx)} (mean {sum(ctx) / len(ctx):.0f})",
        "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
        "block_size": w.block_size, "k_format": w.k_dtype, "v_format": w.v_dtype,
        "rotated": {"k": w.rotate_k, "v": w.rotate_v},
        "decode_bytes_per_step": dbytes,
        "ms_per_step": round(ms_per_step, 4),
        "step_GBps": round(dbytes / (ms_per_step * 1e6), 2),
        "decode_call_ms": round(dec_ms, 4),
        "decode_call_GBps": round(dbytes / (dec_ms * 1e6), 2),
        "decode_call_pct_hbm_peak": round(100 * dbytes / (dec_ms * 1e6) / HBM_PEAK_GBPS, 2),
        "decode_step_write_ms": round(stepw_ms, 4),
        "decode_tok_s": round(B / (ms_per_step * 1e-3), 1),
        "decode_tok_s_attention_only_all_layers": round(B / (ms_per_step * 1e-3 * w.n_layers), 1),
        "write_GBps": round(wbytes / (write_ms * 1e6), 2),
        "write_pct_hbm_peak": round(100 * wbytes / (write_ms * 1e6) / HBM_PEAK_GBPS, 2),
        "write_ms": round(write_ms, 4),
        "write_tokens": int(pre_idx.numel()),
        "write_static_GBps": None if static_ms is None else round(wbytes / (static_ms * 1e6), 2),
    }
    res["quality"] = quality(w, inp, out)
    if w.name in args.prefill_chunks:
        res["prefill"] = prefill_measure(w, inp, caches[0], args.prefill_chunks[w.name], args.prefill_calls, dev)
    print(f"[bench] {w.name}: decode call {dec_ms:.4f} ms = {res['decode_call_GBps']:.0f} GB/s "
          f"({res['decode_call_pct_hbm_peak']:.1f}% of peak), quality max|err| {res['quality']['max_abs']:.3e} "
          f"rel L2 {res['quality']['rel_l2']:.3e}", file=sys.stderr, flush=True)
    del caches, cache, ws
    if want_inputs:
        return res, inp
    del inp
    return res, None


def room_split_tokens(w, ctx_lens, reserve_waves):
    """split_tokens for a decode call that leaves `reserve_waves` wave slots
    of the GPU free (for a concurrent narrow copy kernel): the decode's
    balanced partition, with as many shares as the remaining slots hold.  A
    wave reads HP KV heads (the most with HP G <= 16 dividing H) in tiles of
    32 / HP tokens; head dims up to 128 run two waves per SIMD."""
    import torch
    G = w.n_q_heads // w.n_kv_heads
    hp = next(h for h in (4, 2, 1) if w.n_kv_heads % h == 0 and h * G <= 16)
    tt = 32 // hp
    lq = [(L & ~31) if w.k_dtype == "int4_kivi" else L for L in ctx_lens]
    tiles = sum((L + tt - 1) // tt for L in lq)
    groups = w.n_kv_heads // hp
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = (2 if w.head_dim <= 128 else 1) * 4 * cus - reserve_waves
    shares = max(1, waves // groups)
    return -(-tiles // shares) * tt


def offload_measure(args, dev="cuda", engine="kernel"):
    """Offloaded pages with double-buffered prefetch ("Use Less Memory",
    section 4): the headline FP8 layer (27 x 32k) whose first --offload-pages
    pages of every sequence live in a pool in pinned host memory.  Each step
    decodes over the cache with those pages read from staging set t % 2,
    while the prefetch of step t + 1 (kvq_copy_blocks, host -> device, on a
    second stream) fills set (t + 1) % 2.  Reports the copy rate, the decode
    time with and without the concurrent prefetch, the overlapped and the
    serial step time, and whether every step's output equals the decode of
    the pages that never left the device (bitwise).  With the narrow copy
    engine the decode calls leave the copy kernel's wave slots free
    (room_split_tokens), so the two run side by side."""
    import torch

    import quantized_paged_kv_write_amd as kvq
    from quantized_paged_kv_write_amd import workloads as wl

    w = wl.WORKLOADS["llama3_8b_fp8"]
    P = args.offload_pages
    B = w.batch
    n_off = B * P
    inp = wl.make_inputs(w, wl.seed_of(w), dev)
    print(f"[bench] offload: {w.name}, {P} pages of every sequence ({n_off} pages) prefetched per step",
          file=sys.stderr, flush=True)
    # the two staging sets are contiguous runs of blocks after the workload's
    # own, so one prefetch is one DMA copy per buffer (a page is 16 KB of
    # codes; page-by-page copies would go to small blit kernels instead)
    nb0 = inp.num_blocks
    cache = kvq.PagedKVCache(nb0 + 2 * n_off, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype,
                             max_seqs=B, device=dev)
    kvq.write(cache, inp.k, inp.v, inp.slot_mapping.to(dev), inp.seq_idx.to(dev))
    q = inp.q.clone()
    ctx_d = torch.tensor(inp.ctx_lens, dtype=torch.int32, device=dev)
    table = inp.block_table
    del inp
    torch.cuda.empty_cache()
    pool = kvq.PagedKVCache(n_off, w.block_size, w.n_kv_heads, w.head_dim, w.k_dtype, w.v_dtype, device="cpu",
                            pin_memory=True)
    import numpy as np
    offl = np.array([int(table[b, p]) for b in range(B) for p in range(P)], np.int32)
    host_ids = np.arange(n_off, dtype=np.int32)
    kvq.copy_blocks(cache, pool, offl, host_ids)  # offload
    sets = [np.arange(nb0, nb0 + n_off, dtype=np.int32), np.arange(nb0 + n_off, nb0 + 2 * n_off, dtype=np.int32)]
    tables = []
    for st in sets:
        t2 = table.clone()
        for i, d in enumerate(st):
            t2[i // P, i % P] = d
        tables.append(t2.to(dev))
    base_table = table.to(dev)
    out = torch.empty_like(q)
    split = (room_split_tokens(w, [int(v) for v in ctx_d.cpu().tolist()], 4 * kvq.COPY_NARROW_WORKGROUPS)
             if engine == "narrow" else 0)
    ws = torch.empty(kvq.decode_workspace_bytes(cache, B, w.n_q_heads, table.shape[1], split), dtype=torch.uint8,
                     device=dev)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ref = kvq.decode_attn(cache, q, base_table, ctx_d, split_tokens=split).clone()
    torch.cuda.synchronize()
    page_bytes = 2 * w.block_size * w.n_kv_heads * (w.head_dim + 2)  # FP8 K and V codes + scales
    nbytes = n_off * page_bytes
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    reps = args.offload_steps

    # prefetch alone
    kvq.copy_blocks(pool, cache, host_ids, sets[0], engine=engine)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(main)
    for r in range(reps):
        kvq.copy_blocks(pool, cache, host_ids, sets[r % 2], engine=engine)
    e1.record(main)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / reps
    # decode alone (over the staging sets)
    for r in range(3):
        kvq.decode_attn(cache, q, tables[r % 2], ctx_d, split_tokens=split, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0.record(main)
    for r in range(reps):
        kvq.decode_attn(cache, q, tables[r % 2], ctx_d, split_tokens=split, out=out, workspace=ws)
    e1.record(main)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / reps
    equal = bool(torch.equal(out, ref))
    # serial: prefetch, then decode, on one stream
    decs_s = [kvq.DecodeCall(cache, q, tables[i], ctx_d, out, ws, split_tokens=split) for i in range(2)]
    cps_s = [kvq.CopyCall(pool, cache, host_ids, sets[i], engine=engine) for i in range(2)]
    torch.cuda.synchronize()
    e0.record(main)
    for r in range(reps):
        cps_s[r % 2](main)
        decs_s[r % 2](main)
    e1.record(main)
    torch.cuda.synchronize()
    serial_ms = e0.elapsed_time(e1) / reps
    equal = equal and bool(torch.equal(out, ref))
    # overlapped: decode t on the main stream while set (t + 1) % 2 is filled
    # on the side stream; decode t + 1 waits for that prefetch (event), and
    # the prefetch into a set waits for the decode that last read it
    ready = [torch.cuda.Event() for _ in range(2)]
    freed = [torch.cuda.Event() for _ in range(2)]
    dev_ev = [(ev(), ev()) for _ in range(reps)]
    outs = [torch.empty_like(out) for _ in range(reps // 8)]
    t_start, t_end = ev(), ev()

    # arguments marshalled once: the loop only calls into the library and
    # records events, so the host keeps ahead of the GPU
    decs = [kvq.DecodeCall(cache, q, tables[i], ctx_d, out, ws, split_tokens=split) for i in range(2)]
    cps = [kvq.CopyCall(pool, cache, host_ids, sets[i], engine=engine) for i in range(2)]
    torch.cuda.synchronize()

    def pipeline(timed):
        cps[0](side)
        ready[0].record(side)
        if timed:
            t_start.record(main)
        for r in range(reps):
            cur = r % 2
            main.wait_event(ready[cur])
            if r + 1 < reps:
                if r >= 1:
                    side.wait_event(freed[1 - cur])  # decode r - 1 read set 1 - cur
                cps[1 - cur](side)
                ready[1 - cur].record(side)
            if timed:
                dev_ev[r][0].record(main)
            decs[cur](main)
            if timed:
                dev_ev[r][1].record(main)
            freed[cur].record(main)
            if timed and r % 8 == 7:
                outs[r // 8].copy_(out)
        if timed:
            t_end.record(main)

    pipeline(False)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    pipeline(True)
    enqueue_ms = (time.perf_counter() - c0) * 1e3 / reps
    torch.cuda.synchronize()
    overlap_ms = t_start.elapsed_time(t_end) / reps
    dec_conc_ms = sum(a.elapsed_time(b) for a, b in dev_ev[1:]) / max(reps - 1, 1)
    equal = equal and all(bool(torch.equal(x, ref)) for x in outs)
    del cache, pool, ws
    torch.cuda.empty_cache()
    res = {
        "workload": w.name, "copy_engine": engine, "decode_split_tokens": split, "pages_per_step": n_off,
        "bytes_per_step": nbytes,
        "prefetch_ms": round(copy_ms, 4), "prefetch_GBps_h2d": round(nbytes / (copy_ms * 1e6), 2),
        "decode_ms_alone": round(dec_ms, 4), "decode_ms_with_concurrent_prefetch": round(dec_conc_ms, 4),
        "step_ms_serial": round(serial_ms, 4), "step_ms_overlapped": round(overlap_ms, 4),
        "host_enqueue_ms_per_step": round(enqueue_ms, 4),
        "bitwise_equal_to_resident_decode": equal,
        "note": "a step is decode over the whole cache with the prefetched pages read from the staging set; "
                "overlapped = max(prefetch, decode) when hidden, serial = prefetch + decode; step times from "
                "HIP events on the decode stream",
    }
    print(f"[bench] offload ({engine}): prefetch {copy_ms:.3f} ms ({res['prefetch_GBps_h2d']:.1f} GB/s), decode {dec_ms:.3f} ms "
          f"alone / {dec_conc_ms:.3f} ms with prefetch, step serial {serial_ms:.3f} / overlapped {overlap_ms:.3f} ms, "
          f"bitwise equal {equal}", file=sys.stderr, flush=True)
    return res


EXTRA_DEFAULT = "llama3_8b_int8k_int4v,llama3_70b_int8,llama3_8b_kivi_int4,llama3_70b_int8_rot"
PREFILL_DEFAULT = "llama3_70b_int8:2048,llama3_8b_kivi_int4:2048,llama3_8b_fp8:512"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_fp8", help="the headline workload (value, roofline)")
    ap.add_argument("--extra", default=EXTRA_DEFAULT,
                    help="comma-separated workloads measured after the headline one, each reported in "
                         "'workloads' ('none' for none)")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed decode calls after the cache fill, before any timing")
    ap.add_argument("--caches", type=int, default=2, choices=(1, 2),
                    help="identical caches the timed decode steps alternate between, so that no call reads "
                         "data the previous call left in the memory-side cache")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--no-offload", action="store_true")
    ap.add_argument("--offload-pages", type=int, default=10, help="pages of every sequence prefetched per step")
    ap.add_argument("--offload-steps", type=int, default=40)
    ap.add_argument("--prefill", default=PREFILL_DEFAULT,
                    help="workload:chunk pairs measured with one chunked-prefill call each ('none' for none)")
    ap.add_argument("--prefill-calls", type=int, default=5)
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="reduce two rocprofv3 counter CSVs to profiles/decode_<workload>_hbm_traffic.json")
    ap.add_argument("--pmc-command", default="", help="the command that produced the counter CSVs")
    args = ap.parse_args()
    args.prefill_chunks = {} if args.prefill in ("", "none") else \
        {x.split(":")[0]: int(x.split(":")[1]) for x in args.prefill.split(",") if x}
    if args.pmc_summary:
        d = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload, args.pmc_command)
        os.makedirs(os.path.dirname(traffic_profile_path(args.workload)), exist_ok=True)
        with open(traffic_profile_path(args.workload), "w") as f:
            json.dump(d, f, indent=1)
        print(json.dumps(d, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode and write kernels shard "
              "by sequence or KV head with no communication, so run one process per GPU instead.", file=sys.stderr)
        sys.exit(2)

    import torch

    from quantized_paged_kv_write_amd import workloads as wl

    dev = "cuda"
    w = wl.WORKLOADS[args.workload]
    head, inp = measure(w, args, args.steps, args.warmup, dev, want_inputs=not args.no_cpu_baseline)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, args.cpu_budget)
    del inp
    torch.cuda.empty_cache()
    workloads = {w.name: head}
    extras = [] if args.extra in ("", "none") else [x for x in args.extra.split(",") if x and x != w.name]
    for name in extras:
        r, _ = measure(wl.WORKLOADS[name], args, args.extra_steps, args.warmup, dev)
        workloads[name] = r
        torch.cuda.empty_cache()
    offload = None if args.no_offload else {e: offload_measure(args, dev, e) for e in ("narrow", "kernel", "dma")}
    probes = None if args.no_probes else stream_probes(dev)

    ms_per_step = head["ms_per_step"]
    dbytes = head["decode_bytes_per_step"]
    value = dbytes / (ms_per_step * 1e6)
    achieved = dbytes / (head["decode_call_ms"] * 1e6)
    res = {
        "metric": "quantized paged-decode KV-read GB/s (% HBM peak) + decode tok/s; write GB/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle,
        "timed_caches": args.caches,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.k_dtype + "+" + w.v_dtype + " codes, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "ctx_lens": head["ctx_lens"], "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "k_format": w.k_dtype, "v_format": w.v_dtype},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_kernels_ms": head["decode_call_ms"],
        "decode_step_write_ms": head["decode_step_write_ms"],
        "decode_bytes_per_step": dbytes,
        "decode_tok_s": head["decode_tok_s"],
        "decode_tok_s_attention_only_all_layers": head["decode_tok_s_attention_only_all_layers"],
        "write_GBps": head["write_GBps"],
        "write_pct_hbm_peak": head["write_pct_hbm_peak"],
        "write_ms": head["write_ms"],
        "write_tokens": head["write_tokens"],
        "write_static_GBps": head["write_static_GBps"],
        "quality": head["quality"],
        "stream_probes": probes,
        "offload": offload,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(w.name),
                     "kernel": "plan_kernel + decode_split_kernel + merge_kernel (one kvq_decode_attn call)"},
        "workloads": workloads,
        "prefill": {k: v["prefill"] for k, v in workloads.items() if "prefill" in v},
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
