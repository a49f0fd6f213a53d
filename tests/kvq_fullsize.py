"""Oracle side of the full-size parity tests, run in worker processes.

Each piece is one sequence and a slice of its KV heads.  The worker
quantizes that piece's fp16 keys and values with the oracle in the GPU
side's two calls (into an oracle cache whose pages are the sequence's pages
in order), compares every byte of
those pages with the GPU cache's pages of the same sequence, and compares the
GPU decode output of the piece's query heads with the oracle's float64
attention.  Imports only NumPy and the oracle, so it runs in fresh processes
that never touch the GPU."""

from __future__ import annotations

import numpy as np

import oracle as o

ATOL = 2e-3        # max |out_gpu(fp16) - o(fp64)| for outputs below 4 in magnitude
ATOL_ARITH = 1e-3  # beyond the fp16 half-ulp of larger outputs


def tolerance(ref):
    """Per-element bar for an fp16 output against the fp64 reference o:
    2e-3, or, where the fp16 format's own half-ulp at |o| exceeds 1e-3 (|o|
    >= 4), that half-ulp plus 1e-3 -- the same arithmetic budget, since an
    fp16 result cannot be closer to o than the rounding of o allows."""
    a = np.abs(np.asarray(ref, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    half_ulp = 2.0 ** (e - 11)
    return np.maximum(ATOL, half_ulp + ATOL_ARITH)


def excess(got, ref):
    """max(|got - ref| - tolerance(ref)): <= 0 when every element meets its bar."""
    if got.size == 0:
        return -1.0
    return float(np.max(np.abs(got - ref) - tolerance(ref)))


def check_piece(p: dict) -> dict:
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        return _check_piece(p)


def _check_piece(p: dict) -> dict:
    kf, vf, bs, D = p["k_fmt"], p["v_fmt"], p["block_size"], p["head_dim"]
    k16, v16 = p["k16"], p["v16"]  # (L, Hs, D) fp16, positions 0..L-1
    L, Hs = k16.shape[0], k16.shape[1]
    npg = -(-L // bs)
    c = o.OracleCache(max(npg, 1), bs, Hs, D, kf, vf, max_seqs=1, rot_k=p.get("rot_k"), rot_v=p.get("rot_v"))
    pos = np.arange(L)
    seq = np.zeros(L, np.int32)
    # page j of the sequence is oracle block j; the same two calls as the GPU
    # side: every token but the last, then the last (a KIVI page completed by
    # the last token keeps its earlier rows in the tail as well)
    o.write(c, k16[:L - 1], v16[:L - 1], pos[:L - 1], seq[:L - 1])
    o.write(c, k16[L - 1:], v16[L - 1:], pos[L - 1:], seq[L - 1:])
    mism = {}
    for name, got in p["pages"].items():
        ref = getattr(c, name)
        if name in ("k_tail", "v_tail"):
            ref = ref[0]
        else:
            ref = ref[:npg]
        a = got.view(np.uint16) if got.dtype == np.float16 else got
        b = ref.view(np.uint16) if ref.dtype == np.float16 else ref
        if a.shape != b.shape:
            mism[name] = f"shape {a.shape} vs {b.shape}"
        else:
            n = int(np.count_nonzero(a != b))
            if n:
                mism[name] = n
    res = {"b": p["b"], "h0": p["h0"], "mismatch": mism, "bytes": int(sum(x.nbytes for x in p["pages"].values()))}
    if p.get("q") is not None:
        K, V = o.gather_dequant(c, np.arange(npg), L, 0)
        ref = o.attention_fp64(p["q"].astype(np.float64), K, V)
        got = p["out"].astype(np.float64)
        res["err"] = float(np.max(np.abs(got - ref))) if got.size else 0.0
        res["err16"] = float(np.max(np.abs(got - ref.astype(np.float16).astype(np.float64)))) if got.size else 0.0
        res["rows"] = int(got.shape[0])
        if p.get("quality"):
            # unquantized fp16 keys and values: the quality statistic
            ref0 = o.attention_fp64(p["q"].astype(np.float64), k16.astype(np.float64), v16.astype(np.float64))
            res["q_maxabs"] = float(np.max(np.abs(got - ref0)))
            res["q_l2_num"] = float(np.sum((got - ref0) ** 2))
            res["q_l2_den"] = float(np.sum(ref0 ** 2))
    if p.get("pf_q") is not None:
        # sampled rows of a chunked-prefill call over the same pages: causal
        # attention of the query at each sampled position
        K, V = o.gather_dequant(c, np.arange(npg), L, 0)
        ref = o.causal_attention_fp64(p["pf_q"], K, V, p["pf_pos"])
        got = p["pf_out"].astype(np.float64)
        res["pf_err"] = float(np.max(np.abs(got - ref))) if got.size else 0.0
        res["pf_excess"] = excess(got, ref)
        res["pf_maxref"] = float(np.max(np.abs(ref))) if got.size else 0.0
        res["pf_rows"] = int(got.shape[0] * got.shape[1])
    return res
