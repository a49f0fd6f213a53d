"""ctypes binding of libkvq.so (see include/kvq.h for the contract).

This layer only marshals arguments: it turns torch tensors into device
pointers and the current torch stream into a hipStream_t, and allocates the
caller-owned cache buffers with torch.  Every step of the computation runs in
the HIP kernels; if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_OK = 0
STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID_ARG", -2: "KVQ_ERR_UNSUPPORTED", -3: "KVQ_ERR_SHAPE",
          -4: "KVQ_ERR_WORKSPACE", -5: "KVQ_ERR_NO_DEVICE", -6: "KVQ_ERR_HIP"}
DTYPES = {"int8": 1, "fp8_e4m3fn": 2, "int4_g32": 3, "int4_kivi": 4, "fp8_e5m2": 5}

# Functions declared in include/kvq.h (the symbol test checks this list
# against the header).
EXPORTS = ("kvq_write", "kvq_write_static", "kvq_decode_workspace_bytes", "kvq_decode_attn", "kvq_status_string",
           "kvq_get_device_error", "kvq_decode_attn_noalloc", "kvq_copy_blocks", "kvq_prefill_workspace_bytes",
           "kvq_prefill_attn")
NOALLOC_WORKSPACE_BYTES = 64 << 20  # KVQ_NOALLOC_WORKSPACE_BYTES
# Bits of kvq_get_device_error (kvq_device_error in include/kvq.h).
DEVERR = {"slot": 1, "seq": 2, "block": 4, "ctx": 8, "qlen": 16}


class KvqCacheStruct(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k_dtype", ctypes.c_int32), ("v_dtype", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
        ("k_zeros", ctypes.c_void_p), ("k_tail", ctypes.c_void_p), ("v_tail", ctypes.c_void_p),
        ("rot_signs", ctypes.c_uint32 * 8),
    ]


ROTATE_K, ROTATE_V = 1, 2  # kvq_cache_flags
COPY_ENGINES = {"kernel": 0, "dma": 1, "narrow": 2}  # kvq_copy_engine
COPY_NARROW_WORKGROUPS = 16  # KVQ_COPY_NARROW_WORKGROUPS


class KvqError(RuntimeError):
    def __init__(self, rc: int, what: str):
        self.rc = rc
        super().__init__(f"{what}: {STATUS.get(rc, rc)} ({status_string(rc)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so from the package directory (built by build.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_paged_kv_write_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cp = ctypes.POINTER(KvqCacheStruct)
        L.kvq_write.argtypes = [cp, vp, vp, vp, vp, i64, vp]
        L.kvq_write.restype = ctypes.c_int
        L.kvq_write_static.argtypes = [cp, vp, vp, vp, i64, vp, vp, vp]
        L.kvq_write_static.restype = ctypes.c_int
        L.kvq_decode_workspace_bytes.argtypes = [cp, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.kvq_decode_workspace_bytes.restype = ctypes.c_int
        L.kvq_decode_attn.argtypes = [cp, vp, vp, i32, vp, i32, i32, ctypes.c_float, i32, vp, vp, sz, vp]
        L.kvq_decode_attn.restype = ctypes.c_int
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_decode_attn_noalloc.argtypes = [cp, vp, vp, i32, vp, i32, i32, ctypes.c_float, i32, vp, vp]
        L.kvq_decode_attn_noalloc.restype = ctypes.c_int
        L.kvq_copy_blocks.argtypes = [cp, cp, vp, vp, i32, i32, vp]
        L.kvq_copy_blocks.restype = ctypes.c_int
        L.kvq_prefill_workspace_bytes.argtypes = [cp, i64, i32, ctypes.POINTER(sz)]
        L.kvq_prefill_workspace_bytes.restype = ctypes.c_int
        L.kvq_prefill_attn.argtypes = [cp, vp, vp, vp, i32, vp, i32, i64, i32, i32, ctypes.c_float, vp, vp, sz, vp]
        L.kvq_prefill_attn.restype = ctypes.c_int
        L.kvq_get_device_error.argtypes = [vp]
        L.kvq_get_device_error.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return lib().kvq_status_string(rc).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, dtype, name, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


class PagedKVCache:
    """One layer's quantized paged KV cache: caller-owned device buffers in
    the layouts of include/kvq.h (codes uint8, scales/zeros/tails fp16)."""

    def __init__(self, num_blocks, block_size, n_kv_heads, head_dim, k_dtype, v_dtype, max_seqs=0,
                 device="cuda", pin_memory=False, rotate_k=False, rotate_v=False, rot_signs=None):
        """rotate_k / rotate_v: Walsh-Hadamard rotation of keys / values with
        the signs rot_signs (8 uint32 words: bit c set negates channel c)."""
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.n_kv_heads, self.head_dim = int(n_kv_heads), int(head_dim)
        self.k_dtype, self.v_dtype, self.max_seqs = k_dtype, v_dtype, int(max_seqs)
        self.flags = (ROTATE_K if rotate_k else 0) | (ROTATE_V if rotate_v else 0)
        words = [0] * 8 if rot_signs is None else [int(x) & 0xFFFFFFFF for x in rot_signs]
        if len(words) != 8:
            raise ValueError("rot_signs must hold 8 uint32 words")
        self.rot_signs = words
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        nb, bs, H, D = self.num_blocks, self.block_size, self.n_kv_heads, self.head_dim
        # device="cpu", pin_memory=True: a pool of pages in pinned host memory
        # (for kvq_copy_blocks), laid out like the device cache
        self.pinned = bool(pin_memory)
        z = lambda *shape, dt: torch.zeros(shape, dtype=dt, device=self.device, pin_memory=self.pinned)  # noqa: E731
        half_row = lambda f: D // 2 if f in ("int4_g32", "int4_kivi") else D  # noqa: E731
        groups = lambda f: D // 32 if f == "int4_g32" else 1  # noqa: E731
        self.k_codes = z(nb, bs, H, half_row(k_dtype), dt=torch.uint8)
        self.v_codes = z(nb, bs, H, half_row(v_dtype), dt=torch.uint8)
        self.v_scales = z(nb, bs, H, groups(v_dtype), dt=torch.float16)
        if k_dtype == "int4_kivi":
            self.k_scales = z(nb, H, D, dt=torch.float16)
            self.k_zeros = z(nb, H, D, dt=torch.float16)
            self.k_tail = z(max(self.max_seqs, 1), bs, H, D, dt=torch.float16)
            self.v_tail = z(max(self.max_seqs, 1), bs, H, D, dt=torch.float16)
        else:
            self.k_scales = z(nb, bs, H, groups(k_dtype), dt=torch.float16)
            self.k_zeros = self.k_tail = self.v_tail = None

    def struct(self) -> KvqCacheStruct:
        return KvqCacheStruct(
            self.num_blocks, self.block_size, self.n_kv_heads, self.head_dim,
            DTYPES[self.k_dtype], DTYPES[self.v_dtype], self.max_seqs, self.flags,
            _ptr(self.k_codes), _ptr(self.v_codes), _ptr(self.k_scales), _ptr(self.v_scales),
            _ptr(self.k_zeros), _ptr(self.k_tail), _ptr(self.v_tail), (ctypes.c_uint32 * 8)(*self.rot_signs))

    def buffers(self) -> dict:
        out = {"k_codes": self.k_codes, "v_codes": self.v_codes, "k_scales": self.k_scales,
               "v_scales": self.v_scales}
        if self.k_dtype == "int4_kivi":
            out.update(k_zeros=self.k_zeros, k_tail=self.k_tail, v_tail=self.v_tail)
        return out


def write(cache: PagedKVCache, k, v, slot_mapping, seq_idx=None, stream=None):
    """kvq_write: quantize fp16 k, v (T, H, D) into the cache at slot_mapping."""
    dev = cache.device
    _check(k, torch.float16, "k", dev)
    _check(v, torch.float16, "v", dev)
    _check(slot_mapping, torch.int64, "slot_mapping", dev)
    if seq_idx is not None:
        _check(seq_idx, torch.int32, "seq_idx", dev)
    T = slot_mapping.numel()
    if k.shape != (T, cache.n_kv_heads, cache.head_dim) or v.shape != k.shape:
        raise ValueError(f"k/v must be ({T}, {cache.n_kv_heads}, {cache.head_dim})")
    c = cache.struct()
    rc = lib().kvq_write(ctypes.byref(c), _ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(seq_idx), T, _stream(stream))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_write")


def write_static(cache: PagedKVCache, k, v, slot_mapping, k_scale, v_scale, stream=None):
    """kvq_write_static: quantize fp16 k, v (T, H, D) with calibrated fp16
    scales k_scale, v_scale (H,) per KV head."""
    dev = cache.device
    _check(k, torch.float16, "k", dev)
    _check(v, torch.float16, "v", dev)
    _check(slot_mapping, torch.int64, "slot_mapping", dev)
    _check(k_scale, torch.float16, "k_scale", dev)
    _check(v_scale, torch.float16, "v_scale", dev)
    T = slot_mapping.numel()
    if k.shape != (T, cache.n_kv_heads, cache.head_dim) or v.shape != k.shape:
        raise ValueError(f"k/v must be ({T}, {cache.n_kv_heads}, {cache.head_dim})")
    if k_scale.shape != (cache.n_kv_heads,) or v_scale.shape != (cache.n_kv_heads,):
        raise ValueError(f"k_scale/v_scale must be ({cache.n_kv_heads},)")
    c = cache.struct()
    rc = lib().kvq_write_static(ctypes.byref(c), _ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_scale),
                                _ptr(v_scale), _stream(stream))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_write_static")


def copy_blocks(src: PagedKVCache, dst: PagedKVCache, src_blocks, dst_blocks, stream=None, engine="kernel"):
    """kvq_copy_blocks: page dst_blocks[i] of `dst` becomes a copy of page
    src_blocks[i] of `src` (either cache on the device or in pinned host
    memory), enqueued on the stream by the copy kernel or the DMA engines.
    The id lists are host sequences."""
    import numpy as np
    s_ids = np.ascontiguousarray(np.asarray(src_blocks, dtype=np.int32).ravel())
    d_ids = np.ascontiguousarray(np.asarray(dst_blocks, dtype=np.int32).ravel())
    if s_ids.size != d_ids.size:
        raise ValueError("src_blocks and dst_blocks differ in length")
    cs, cd = src.struct(), dst.struct()
    rc = lib().kvq_copy_blocks(ctypes.byref(cs), ctypes.byref(cd), s_ids.ctypes.data_as(ctypes.c_void_p),
                               d_ids.ctypes.data_as(ctypes.c_void_p), int(s_ids.size), COPY_ENGINES[engine],
                               _stream(stream))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_copy_blocks")


def get_device_error(stream=None) -> int:
    """kvq_get_device_error: the kvq_device_error bits recorded on the current
    device since the previous call (DEVERR), cleared by the read.  Orders
    after the work on `stream` and synchronizes it."""
    rc = lib().kvq_get_device_error(_stream(stream))
    if rc < 0:
        raise KvqError(rc, "kvq_get_device_error")
    return rc


def decode_workspace_bytes(cache: PagedKVCache, batch, n_q_heads, max_blocks_per_seq, split_tokens=0) -> int:
    out = ctypes.c_size_t(0)
    c = cache.struct()
    rc = lib().kvq_decode_workspace_bytes(ctypes.byref(c), batch, n_q_heads, max_blocks_per_seq, split_tokens,
                                          ctypes.byref(out))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_decode_workspace_bytes")
    return out.value


def decode_attn(cache: PagedKVCache, q, block_table, ctx_lens, sm_scale=0.0, split_tokens=0, out=None,
                workspace=None, stream=None):
    """kvq_decode_attn: one decode step over the cache; returns out (B, Hq, D) fp16."""
    dev = cache.device
    _check(q, torch.float16, "q", dev)
    _check(block_table, torch.int32, "block_table", dev)
    _check(ctx_lens, torch.int32, "ctx_lens", dev)
    B, Hq, D = q.shape
    if D != cache.head_dim or block_table.dim() != 2 or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("shape mismatch between q, block_table and ctx_lens")
    if out is None:
        out = torch.empty_like(q)
    _check(out, torch.float16, "out", dev)
    if out.shape != q.shape:
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    need = decode_workspace_bytes(cache, B, Hq, block_table.shape[1], split_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, torch.uint8, "workspace", dev)
    c = cache.struct()
    rc = lib().kvq_decode_attn(ctypes.byref(c), _ptr(q), _ptr(block_table), block_table.shape[1], _ptr(ctx_lens),
                               B, Hq, float(sm_scale), split_tokens, _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_decode_attn")
    return out


def decode_attn_noalloc(cache: PagedKVCache, q, block_table, ctx_lens, out, sm_scale=0.0, split_tokens=0,
                        stream=None):
    """kvq_decode_attn_noalloc: decode into the caller's `out` (B, Hq, D) fp16
    with the library's fixed per-device workspace (nothing is allocated)."""
    dev = cache.device
    _check(q, torch.float16, "q", dev)
    _check(block_table, torch.int32, "block_table", dev)
    _check(ctx_lens, torch.int32, "ctx_lens", dev)
    _check(out, torch.float16, "out", dev)
    B, Hq, D = q.shape
    if D != cache.head_dim or block_table.dim() != 2 or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("shape mismatch between q, block_table and ctx_lens")
    if out.shape != q.shape:
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    c = cache.struct()
    rc = lib().kvq_decode_attn_noalloc(ctypes.byref(c), _ptr(q), _ptr(block_table), block_table.shape[1],
                                       _ptr(ctx_lens), B, Hq, float(sm_scale), split_tokens, _ptr(out),
                                       _stream(stream))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_decode_attn_noalloc")
    return out


def prefill_workspace_bytes(cache: PagedKVCache, total_q, n_q_heads) -> int:
    """kvq_prefill_workspace_bytes (0 unless the cache stores rotated keys)."""
    n = ctypes.c_size_t(0)
    c = cache.struct()
    rc = lib().kvq_prefill_workspace_bytes(ctypes.byref(c), int(total_q), int(n_q_heads), ctypes.byref(n))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_prefill_workspace_bytes")
    return n.value


def prefill_attn(cache: PagedKVCache, q, q_start, block_table, ctx_lens, max_q_len, sm_scale=0.0, out=None,
                 workspace=None, stream=None):
    """kvq_prefill_attn: causal attention of the chunks q (total_q, Hq, D)
    fp16, sequence b's rows q_start[b] .. q_start[b + 1] - 1 (int32, B + 1),
    over the cache; returns out (total_q, Hq, D) fp16."""
    dev = cache.device
    _check(q, torch.float16, "q", dev)
    _check(q_start, torch.int32, "q_start", dev)
    _check(block_table, torch.int32, "block_table", dev)
    _check(ctx_lens, torch.int32, "ctx_lens", dev)
    Tq, Hq, D = q.shape
    B = ctx_lens.shape[0]
    if (D != cache.head_dim or block_table.dim() != 2 or block_table.shape[0] != B or ctx_lens.dim() != 1
            or q_start.shape != (B + 1,)):
        raise ValueError("shape mismatch between q, q_start, block_table and ctx_lens")
    if out is None:
        out = torch.empty_like(q)
    _check(out, torch.float16, "out", dev)
    if out.shape != q.shape:
        raise ValueError(f"out must have q's shape {tuple(q.shape)}, got {tuple(out.shape)}")
    need = prefill_workspace_bytes(cache, Tq, Hq)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check(workspace, torch.uint8, "workspace", dev)
    c = cache.struct()
    ws_bytes = 0 if workspace is None else workspace.numel()
    rc = lib().kvq_prefill_attn(ctypes.byref(c), _ptr(q), _ptr(q_start), _ptr(block_table), block_table.shape[1],
                                _ptr(ctx_lens), B, Tq, Hq, int(max_q_len), float(sm_scale), _ptr(out),
                                _ptr(workspace), ws_bytes, _stream(stream))
    if rc != KVQ_OK:
        raise KvqError(rc, "kvq_prefill_attn")
    return out


class DecodeCall:
    """kvq_decode_attn with its arguments checked and marshalled once, for
    loops that issue the same decode step many times (serving loops, double-
    buffered pipelines): calling it only calls into the library.  The tensors
    must stay alive and keep their storage while the object is used."""

    def __init__(self, cache: PagedKVCache, q, block_table, ctx_lens, out, workspace, sm_scale=0.0, split_tokens=0):
        decode_attn(cache, q, block_table, ctx_lens, sm_scale=sm_scale, split_tokens=split_tokens, out=out,
                    workspace=workspace)  # validates every argument (and runs once)
        self._c = cache.struct()
        self._args = (ctypes.byref(self._c), _ptr(q), _ptr(block_table), block_table.shape[1], _ptr(ctx_lens),
                      q.shape[0], q.shape[1], float(sm_scale), split_tokens, _ptr(out), _ptr(workspace),
                      workspace.numel() * workspace.element_size())
        self._refs = (cache, q, block_table, ctx_lens, out, workspace)

    def __call__(self, stream=None):
        rc = lib().kvq_decode_attn(*self._args, _stream(stream))
        if rc != KVQ_OK:
            raise KvqError(rc, "kvq_decode_attn")


class CopyCall:
    """kvq_copy_blocks with its arguments marshalled once (see DecodeCall)."""

    def __init__(self, src: PagedKVCache, dst: PagedKVCache, src_blocks, dst_blocks, engine="kernel"):
        import numpy as np
        self._s = np.ascontiguousarray(np.asarray(src_blocks, dtype=np.int32).ravel())
        self._d = np.ascontiguousarray(np.asarray(dst_blocks, dtype=np.int32).ravel())
        if self._s.size != self._d.size:
            raise ValueError("src_blocks and dst_blocks differ in length")
        self._cs, self._cd = src.struct(), dst.struct()
        self._args = (ctypes.byref(self._cs), ctypes.byref(self._cd), self._s.ctypes.data_as(ctypes.c_void_p),
                      self._d.ctypes.data_as(ctypes.c_void_p), int(self._s.size), COPY_ENGINES[engine])
        self._refs = (src, dst)

    def __call__(self, stream=None):
        rc = lib().kvq_copy_blocks(*self._args, _stream(stream))
        if rc != KVQ_OK:
            raise KvqError(rc, "kvq_copy_blocks")
