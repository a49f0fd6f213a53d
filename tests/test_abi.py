"""The C-ABI library loads, exports every function include/kvq.h declares, and
rejects bad arguments on the host before anything is launched.  No compute
call is made here (these tests must pass on a machine without a GPU)."""

import ctypes
import os
import re

import pytest

import quantized_paged_kv_write_amd as kvq
from quantized_paged_kv_write_amd.binding import EXPORTS, KvqCacheStruct

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

OK, INVALID, UNSUPPORTED, SHAPE, WORKSPACE, NO_DEVICE = 0, -1, -2, -3, -4, -5
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(EXPORTS)


def test_library_exports_every_declared_symbol():
    L = kvq.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for rc in (OK, INVALID, UNSUPPORTED, SHAPE, WORKSPACE, NO_DEVICE, -6, 12345):
        assert isinstance(kvq.status_string(rc), str) and kvq.status_string(rc)


def _cache(**kw):
    c = KvqCacheStruct(num_blocks=8, block_size=16, n_kv_heads=2, head_dim=128, k_dtype=1, v_dtype=1, max_seqs=0)
    c.k_codes = c.v_codes = c.k_scales = c.v_scales = FAKE
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _write(c, T=4, seq=None):
    return kvq.lib().kvq_write(ctypes.byref(c), FAKE, FAKE, FAKE, seq, T, None)


def _ws(c, batch=1, hq=4, mb=4, pps=0):
    out = ctypes.c_size_t(0)
    rc = kvq.lib().kvq_decode_workspace_bytes(ctypes.byref(c), batch, hq, mb, pps, ctypes.byref(out))
    return rc, out.value


def test_write_argument_errors():
    L = kvq.lib()
    assert L.kvq_write(None, FAKE, FAKE, FAKE, None, 4, None) == INVALID
    assert _write(_cache(k_dtype=0)) == INVALID
    assert _write(_cache(v_dtype=9)) == INVALID
    assert _write(_cache(v_dtype=4)) == UNSUPPORTED  # KIVI is for keys only
    assert _write(_cache(head_dim=96)) == UNSUPPORTED
    assert _write(_cache(block_size=24)) == UNSUPPORTED
    assert _write(_cache(num_blocks=0)) == INVALID
    assert _write(_cache(k_codes=None)) == INVALID
    assert _write(_cache(k_dtype=4, block_size=16, max_seqs=2)) == SHAPE  # KIVI needs 32-token pages
    assert _write(_cache(k_dtype=4, block_size=32, max_seqs=0)) == SHAPE
    assert _write(_cache(k_dtype=4, block_size=32, max_seqs=2)) == INVALID  # zeros / tails missing
    assert _write(_cache(k_dtype=3), T=0) == OK  # INT4 group-32 keys (no-op call)
    assert _write(_cache(), T=-1) == INVALID
    assert _write(_cache(), T=0) == OK  # no-op
    assert L.kvq_write(ctypes.byref(_cache()), None, FAKE, FAKE, None, 4, None) == INVALID
    kc = _cache(k_dtype=4, block_size=32, max_seqs=2, k_zeros=FAKE, k_tail=FAKE, v_tail=FAKE)
    assert _write(kc, seq=None) == INVALID  # KIVI needs seq_idx
    assert _write(_cache(k_dtype=6)) == INVALID
    assert _write(_cache(k_dtype=5, v_dtype=5), T=0) == OK  # FP8 E5M2 keys and values


def _write_static(c, T=4, ks=FAKE, vs=FAKE):
    return kvq.lib().kvq_write_static(ctypes.byref(c), FAKE, FAKE, FAKE, T, ks, vs, None)


def test_write_static_argument_errors():
    L = kvq.lib()
    assert L.kvq_write_static(None, FAKE, FAKE, FAKE, 4, FAKE, FAKE, None) == INVALID
    assert _write_static(_cache(), ks=None) == INVALID
    assert _write_static(_cache(), vs=None) == INVALID
    kc = _cache(k_dtype=4, block_size=32, max_seqs=2, k_zeros=FAKE, k_tail=FAKE, v_tail=FAKE)
    assert _write_static(kc) == UNSUPPORTED  # KIVI keys take no calibrated scale
    assert _write_static(_cache(k_dtype=3), T=0) == OK  # INT4 group-32 keys take a calibrated scale
    assert _write_static(_cache(v_dtype=9)) == INVALID
    assert _write_static(_cache(), T=-1) == INVALID
    assert _write_static(_cache(k_dtype=2, v_dtype=3), T=0) == OK  # no-op


def test_workspace_query():
    # Layout: plan ints (2 + batch + shares, padded to 256 bytes), then
    # (shares + batch) records of n_q_heads x (D + 2) fp32.
    # Tiles are 32 (token, head) rows of HP heads: here 2 KV heads x 2 query
    # heads each -> HP = 2, 16 tokens per tile.
    # mb 10 x bs 16 = 160 tokens = 10 tiles per sequence, 30 for the call; shares of
    # 64 tokens = 4 tiles -> 8 shares; 13 ints -> 256 bytes; 11 records.
    rc, n = _ws(_cache(), batch=3, hq=4, mb=10, pps=64)
    assert rc == OK and n == 256 + 11 * 4 * 130 * 4
    # KIVI, 1 query head per KV head -> HP 2, 16-token tiles: 8 pages = 16 tiles, one
    # share of 256 tokens; records 1 + 1.
    rc, n = _ws(_cache(k_dtype=4, block_size=32, max_seqs=1, k_zeros=FAKE, k_tail=FAKE, v_tail=FAKE),
                batch=1, hq=2, mb=8, pps=256)
    assert rc == OK and n == 256 + 2 * 2 * 130 * 4
    # automatic: min(ceil(4096 / (H / HP)), ceil(tiles / 4)) shares = min(4096, 500); 504 ints -> 2048 bytes
    rc, n = _ws(_cache(), batch=2, hq=4, mb=1000, pps=0)
    assert rc == OK and n == 2048 + 502 * 4 * 130 * 4
    # a split size rounds up to whole tiles (16 tokens here)
    assert _ws(_cache(), batch=3, hq=4, mb=10, pps=33) == _ws(_cache(), batch=3, hq=4, mb=10, pps=48)
    assert _ws(_cache(), mb=0)[0] == INVALID
    assert _ws(_cache(), pps=-1)[0] == INVALID
    assert _ws(_cache(), hq=3)[0] == SHAPE                  # not a multiple of n_kv_heads
    assert _ws(_cache(), mb=1 << 26)[0] == SHAPE            # 2^30 tokens in one block-table row
    assert _ws(_cache(), batch=1 << 25, mb=64)[0] == SHAPE  # 2^30 tiles in the call


def test_decode_argument_errors():
    L = kvq.lib()
    c = _cache()

    def dec(batch=2, hq=4, mb=4, scale=0.0, pps=0, ws=FAKE, wsb=1 << 30, q=FAKE):
        return L.kvq_decode_attn(ctypes.byref(c), q, FAKE, mb, FAKE, batch, hq, scale, pps, FAKE, ws, wsb, None)

    assert dec(hq=3) == SHAPE            # not a multiple of n_kv_heads
    assert dec(hq=2 * 17) == UNSUPPORTED  # G > 16
    assert dec(scale=-1.0) == INVALID
    assert dec(scale=float("nan")) == INVALID
    assert dec(ws=None) == WORKSPACE
    assert dec(wsb=16) == WORKSPACE
    assert dec(ws=ctypes.c_void_p(0x1004)) == WORKSPACE  # not 16-byte aligned
    assert dec(q=None) == INVALID
    assert dec(batch=0) == OK            # empty batch: nothing to do
    assert dec(mb=0) == INVALID
    c = _cache(k_dtype=3)
    assert dec(batch=0) == OK            # INT4 group-32 keys decode


def test_prefill_accepts_int4_group32_keys():
    # an empty chunk batch over INT4 group-32 keys passes every check
    c = _cache(k_dtype=3)
    rc = kvq.lib().kvq_prefill_attn(ctypes.byref(c), FAKE, FAKE, FAKE, 4, FAKE, 0, 0, 4, 4, 0.1, FAKE, FAKE,
                                    1 << 30, None)
    assert rc == OK


@pytest.mark.skipif(kvq.binding.torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_call_without_device_reports_no_device():
    assert _write(_cache()) == NO_DEVICE


def test_fastdiv_constants_match_integer_division(tmp_path):
    # The write kernel divides row indices by n_kv_heads with the round-up
    # multiplier method.  Build the library's own constants (make_fastdiv in
    # csrc/kvq_fastdiv.h) with the host compiler and check the quotient the
    # kernel forms from them against integer division, exhaustively near the
    # multiples of d and on random rows below 2^31.
    import shutil
    import subprocess
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "fastdiv_check.cc"
    src.write_text(r"""
#include <cstdio>
#include <random>
#include "kvq_fastdiv.h"
int main() {
  unsigned ds[] = {96, 128, 255, 1000, 65535, 65536, 1u << 20, 2147483647u};
  std::mt19937 rng(7);
  long bad = 0, checked = 0;
  auto check = [&](unsigned d) {
    const kvq::FastDiv f = kvq::make_fastdiv(d);
    auto one = [&](unsigned n) { ++checked; if (kvq::fastdiv_host(n, f) != n / d) ++bad; };
    for (unsigned n = 0; n < 4096; ++n) one(n);
    for (unsigned k = 1; k < 2000; ++k) {
      const unsigned long long base = (unsigned long long)k * d;
      if (base >= (1ull << 31)) break;
      one((unsigned)base - 1); one((unsigned)base); one((unsigned)base + 1);
    }
    one(2147483647u); one(2147483647u - d);
    for (int i = 0; i < 20000; ++i) one(rng() & 0x7FFFFFFFu);
  };
  for (unsigned d = 1; d < 70; ++d) check(d);
  for (unsigned d : ds) check(d);
  printf("%ld %ld\n", checked, bad);
  return bad != 0;
}
""")
    exe = tmp_path / "fastdiv_check"
    inc = os.path.join(ROOT, "quantized_paged_kv_write_amd", "csrc")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", inc, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    checked, bad = map(int, r.stdout.split())
    assert r.returncode == 0 and bad == 0 and checked > 1_000_000, r.stdout


def test_bench_quality_statistic_matches_the_oracle_attention():
    # bench.py's quality statistic (float64 attention over the unquantized
    # fp16 K/V, in torch) against the oracle's float64 attention over the
    # same K/V, on CPU tensors.
    import sys

    import numpy as np
    import torch

    import oracle as o
    from quantized_paged_kv_write_amd import workloads as wl
    sys.path.insert(0, ROOT)
    import bench
    w = wl.Workload("small", 3, 8, 2, 64, 16, "int8", "int8", ("fixed", 0), 2, sink_tokens=4)
    inp = wl.make_inputs(w, 5, "cpu", ctx_lens=[40, 0, 75])
    out = torch.randn(inp.q.shape, generator=torch.Generator().manual_seed(1)).half()
    got = bench.quality(w, inp, out)
    num = den = mx = 0.0
    for b in (0, 2):
        st, L = inp.seq_start[b], inp.ctx_lens[b]
        ref = o.attention_fp64(inp.q[b].numpy(), inp.k[st:st + L].numpy().astype(np.float64),
                               inp.v[st:st + L].numpy().astype(np.float64))
        d = out[b].double().numpy() - ref
        mx = max(mx, float(np.abs(d).max()))
        num += float((d * d).sum())
        den += float((ref * ref).sum())
    assert abs(got["max_abs"] - mx) <= 1e-12 and abs(got["rel_l2"] - (num / den) ** 0.5) <= 1e-12


def test_copy_blocks_argument_errors():
    L = kvq.lib()
    a, b = _cache(), _cache(num_blocks=4)
    ids = (ctypes.c_int32 * 2)(0, 3)
    bad = (ctypes.c_int32 * 2)(0, 4)  # 4 is past b's 4 blocks

    def cp(s, d, si=ids, di=ids, n=2, engine=0):
        return L.kvq_copy_blocks(ctypes.byref(s), ctypes.byref(d), si, di, n, engine, None)

    assert L.kvq_copy_blocks(None, ctypes.byref(b), ids, ids, 2, 0, None) == INVALID
    assert cp(a, b, engine=3) == INVALID                # unknown engine
    assert cp(a, _cache(head_dim=64)) == SHAPE          # geometries differ
    assert cp(a, _cache(v_dtype=2)) == SHAPE            # formats differ
    assert cp(a, b, di=bad) == INVALID                  # id out of range, nothing copied
    assert cp(a, b, n=-1) == INVALID
    assert cp(a, b, n=0) == OK                          # nothing to do
    assert cp(a, _cache(num_blocks=4, v_scales=None)) == INVALID
    assert L.kvq_copy_blocks(ctypes.byref(a), ctypes.byref(b), None, ids, 2, 1, None) == INVALID
