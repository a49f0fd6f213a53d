"""Every code depends on the kernels' quotient x / s equalling the IEEE
binary32 quotient (the write kernels compute it from a reciprocal with one
Newton step and one correction step).  These sweeps put that to the test
through the C ABI, bit-exactly against the oracle:

* kvq_write_static with 64 KV heads per call, each head with its own
  calibrated scale and holding every finite fp16 value as its rows: every
  fp16 x against every subnormal scale, every power of two and its two fp16
  neighbours, the largest fp16, and 1000 seeded random normal scales, for
  INT8, INT4 group-32, FP8 E4M3FN and FP8 E5M2 codes;
* KIVI key pages whose channels are built so that (x - min) / s lands on
  k + 1/2 exactly (scales of few significant bits) or on the fp16 values
  nearest to it and their neighbours, with minima and ranges spread over the
  whole fp16 exponent range (subnormal and zero scales included)."""

import numpy as np
import pytest
import torch

import oracle as o
import quantized_paged_kv_write_amd as kvq
from kvq_testlib import compare_buffers, new_caches

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _finite_fp16():
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return h[np.isfinite(h)]


def _scale_set():
    bits = set(range(0x0001, 0x0400))  # every subnormal
    for e in range(-14, 16):  # normal powers of two and their neighbours
        b = int(np.float16(2.0 ** e).view(np.uint16))
        bits.update((b - 1, b, b + 1))
    bits.add(0x7BFF)  # 65504
    rng = np.random.default_rng(2024)
    bits.update(int(x) for x in rng.integers(0x0400, 0x7C00, 1000))
    bits = sorted(b for b in bits if 0 < b < 0x7C00)
    return np.array(bits, np.uint16).view(np.float16)


@pytest.mark.parametrize("kf,vf", [("int8", "int4_g32"), ("fp8_e4m3fn", "fp8_e5m2")])
def test_static_divisor_sweep(kf, vf):
    H, D, bs = 64, 128, 16
    x = _finite_fp16()
    T = x.size // D  # 63488 = 496 rows of 128
    assert T * D == x.size
    k = np.broadcast_to(x.reshape(T, 1, D), (T, H, D)).copy()
    v = np.broadcast_to(x[::-1].reshape(T, 1, D), (T, H, D)).copy()
    slots = np.arange(T, dtype=np.int64)
    nb = -(-T // bs)
    scales = _scale_set()
    dev, orc = new_caches(nb, bs, H, D, kf, vf, 1, DEV, seed=3, garbage=False)
    kd, vd, sd = torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV), torch.from_numpy(slots).to(DEV)
    n = 0
    for c0 in range(0, scales.size, H):
        ks = scales[c0:c0 + H]
        if ks.size < H:
            ks = np.concatenate([ks, scales[:H - ks.size]])
        vs = np.roll(ks, 17)
        kvq.write_static(dev, kd, vd, sd, torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV))
        o.write_static(orc, k, v, slots, ks, vs)
        torch.cuda.synchronize()
        bad = compare_buffers(dev, orc)
        assert bad == {}, (c0, bad)
        n += 2 * k.size
    print(f"[sweep] {kf}/{vf}: {scales.size} scales x {x.size} fp16 values, {n} quotients bit-exact", flush=True)


def _kivi_channels(n, rng):
    """n channel pages (32 values each, fp16) for the KIVI numerator sweep."""
    f16 = np.float16
    out = np.empty((n, 32), np.float16)
    i = 0
    while i < n:
        if i % 2 == 0:
            # exact ties: s = m 2^e with few significant bits, min on the 2^(e-1)
            # grid, max = min + 15 s, x = min + (k + 1/2) s
            e = int(rng.integers(-22, 11))
            m = int(rng.choice([1, 3, 5, 7, 9, 15, 17, 31, 63]))
            s = m * 2.0 ** e
            mn = float(rng.integers(-64, 65)) * 2.0 ** (e - 1) * int(rng.choice([1, 3, 7]))
            vals = [mn, mn + 15 * s] + [mn + (kk + 0.5) * s for kk in range(15)]
            vals += [mn + kk * s for kk in rng.integers(0, 16, 4)]
            if not all(abs(vv) <= 65504 and float(f16(vv)) == vv for vv in vals):
                continue  # not representable in fp16: draw again
            vals = np.array(vals, np.float64)
            near = []
            for vv in vals[2:17]:
                b = int(np.array([vv], np.float16).view(np.uint16)[0])
                for d in (-1, 1):
                    nb_ = np.array([(b + d) & 0xFFFF], np.uint16).view(np.float16)[0]
                    if np.isfinite(nb_) and mn <= float(nb_) <= mn + 15 * s:
                        near.append(float(nb_))
            pool = np.concatenate([vals, near])
        else:
            # random minimum and range over the whole exponent range; x near
            # the half-integer quotients of the scale the range gives
            sign = -1.0 if rng.random() < 0.5 else 1.0
            mn = float(f16(sign * 2.0 ** rng.uniform(-24, 15.9)))
            width = 2.0 ** rng.uniform(-26, 16.9)
            mx = float(f16(min(mn + width, 65504.0)))
            if mx < mn:
                mn, mx = mx, mn
            s16 = float(f16((np.float32(mx) - np.float32(mn)) / np.float32(15)))
            targets = [mn + (kk + 0.5) * s16 for kk in range(15)] if s16 > 0 else []
            near = []
            for tv in targets:
                b = int(np.array([tv], np.float16).view(np.uint16)[0])
                for d in (-1, 0, 1):
                    nb_ = np.array([(b + d) & 0xFFFF], np.uint16).view(np.float16)[0]
                    if np.isfinite(nb_) and mn <= float(nb_) <= mx:
                        near.append(float(nb_))
            rnd = [float(f16(mn + (mx - mn) * u)) for u in rng.random(8)]
            pool = np.array([mn, mx] + near + rnd, np.float64)
        row = np.empty(32)
        row[:2] = pool[:2]
        rest = pool[2:]
        row[2:] = rest[rng.integers(0, rest.size, 30)] if rest.size else pool[0]
        row[2:] = np.clip(row[2:], pool[0], pool[1])
        out[i] = rng.permutation(row.astype(np.float16))
        i += 1
    return out


def test_kivi_numerator_sweep():
    H, D, bs = 8, 128, 32
    pages = 80
    rng = np.random.default_rng(77)
    ch = _kivi_channels(pages * H * D, rng)  # (pages H D, 32)
    k = ch.reshape(pages, H, D, 32).transpose(0, 3, 1, 2).reshape(pages * 32, H, D).copy()
    v = k[::-1].copy()
    T = pages * 32
    slots = np.arange(T, dtype=np.int64)
    seq = np.zeros(T, np.int32)
    dev, orc = new_caches(pages, bs, H, D, "int4_kivi", "int4_g32", 1, DEV, seed=8, garbage=False)
    # a call of more than 2048 tokens (one seal wave per 32 tokens), then a
    # small one (one seal wave per token)
    for sl in (slice(0, 70 * 32), slice(70 * 32, T)):
        kvq.write(dev, torch.from_numpy(k[sl]).to(DEV), torch.from_numpy(v[sl]).to(DEV),
                  torch.from_numpy(slots[sl]).to(DEV), torch.from_numpy(seq[sl]).to(DEV))
        o.write(orc, k[sl], v[sl], slots[sl], seq[sl])
    torch.cuda.synchronize()
    s16 = orc.k_scales
    assert np.count_nonzero(s16 == 0) > 0 and np.count_nonzero((s16 > 0) & (s16 < 2 ** -14)) > 0
    bad = compare_buffers(dev, orc)
    assert bad == {}, bad
