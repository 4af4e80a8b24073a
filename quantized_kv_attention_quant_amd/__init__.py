"""Python binding of libkvq: quantized-KV decode/verify attention on MI355X.

Thin ctypes layer over the C ABI declared in ``include/kvq.h``.  The entry
points keep the C names (``kv_cache_layout``, ``kv_quant_append``,
``kv_rollback``, ``kv_attn_verify``, ``kv_topk``, ``kv_dequant_gather``,
``kv_attn_verify_exact``, ``kv_fetch_rows`` and the workspace sizers);
this module only checks tensor shapes/dtypes, passes device pointers and the
current HIP stream, and turns non-zero return codes into ``KvqError``.  All
computation happens in the HIP kernels of ``libkvq.so``; PyTorch is used for
device memory and streams only.  There is no fallback: without the built
library every call raises.

``QuantKVCache`` owns the device buffers of one cache (allocated with torch)
and the ``kvq_cache`` struct that describes them.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "KVQ_TARGET", "KVQ_DRAFT4", "KvqError", "KvqCacheStruct", "lib",
    "kv_cache_layout", "kv_quant_append", "kv_rollback",
    "kv_attn_workspace_bytes", "kv_attn_verify", "kv_topk_workspace_bytes",
    "kv_topk", "kv_dequant_gather", "kv_attn_verify_exact", "kv_fetch_rows",
    "kv_last_error", "QuantKVCache", "HostMirror", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_ECAPACITY, KVQ_EROLLBACK = 0, -1, -2, -3
KVQ_EWORKSPACE, KVQ_EUNSUPPORTED, KVQ_EHIP = -4, -5, -6
KVQ_TARGET, KVQ_DRAFT4 = 0, 1
_PATHS = {"target": KVQ_TARGET, "draft4": KVQ_DRAFT4}


def _path(p) -> int:
    """Path name ("target", "draft4") or the raw KVQ_* integer."""
    return _PATHS[p] if isinstance(p, str) else int(p)


class KvqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libkvq error {code}: {msg}")
        self.code = code


class KvqCacheStruct(ctypes.Structure):
    """Mirror of ``struct kvq_cache`` in include/kvq.h (field order and
    types must match)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("G", ctypes.c_int32), ("Gv", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("R", ctypes.c_int32), ("L_max", ctypes.c_int32),
        ("max_append", ctypes.c_int32), ("ring", ctypes.c_int32),
        ("bytes_k_plane", ctypes.c_int64), ("bytes_v_plane", ctypes.c_int64),
        ("bytes_k_sz", ctypes.c_int64), ("bytes_v_sz", ctypes.c_int64),
        ("bytes_k_res", ctypes.c_int64), ("bytes_v_res", ctypes.c_int64),
        ("n_q", ctypes.c_int64), ("n_r", ctypes.c_int64),
        ("k_hi", ctypes.c_void_p), ("k_lo", ctypes.c_void_p),
        ("v_hi", ctypes.c_void_p), ("v_lo", ctypes.c_void_p),
        ("k_sz", ctypes.c_void_p), ("v_sz", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(hipcc, gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(KvqCacheStruct)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.kv_cache_layout.argtypes = [P]
    L.kv_quant_append.argtypes = [P, vp, vp, i32, vp]
    L.kv_rollback.argtypes = [P, i32]
    L.kv_attn_workspace_bytes.argtypes = [P, i32, i32]
    L.kv_attn_workspace_bytes.restype = sz
    L.kv_attn_verify.argtypes = [P, vp, i32, i32, i32, f32, vp, vp, vp, sz, vp]
    L.kv_attn_verify_noalloc.argtypes = [P, vp, i32, i32, i32, f32, vp, vp, vp]
    L.kv_topk_workspace_bytes.argtypes = [P, i32, i32]
    L.kv_topk_workspace_bytes.restype = sz
    L.kv_topk.argtypes = [P, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    L.kv_dequant_gather.argtypes = [P, vp, i32, i32, vp, vp, vp]
    L.kv_attn_verify_exact.argtypes = [P, vp, i32, i32, i32, f32, i32, vp, i32,
                                       vp, vp, vp, vp, vp, sz, vp, vp]
    L.kv_fetch_rows.argtypes = [P, vp, vp, ctypes.c_int64, vp, i32, vp, vp, vp]
    L.kv_last_error.argtypes = []
    L.kv_last_error.restype = ctypes.c_char_p
    for name in ("kv_cache_layout", "kv_quant_append", "kv_rollback",
                 "kv_attn_verify", "kv_attn_verify_noalloc", "kv_topk",
                 "kv_dequant_gather",
                 "kv_attn_verify_exact", "kv_fetch_rows"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def kv_last_error() -> str:
    return lib().kv_last_error().decode()


def _check(rc: int):
    if rc != KVQ_OK:
        raise KvqError(rc, kv_last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ---- the C entry points, same names ------------------------------------------

def kv_cache_layout(c: KvqCacheStruct) -> None:
    _check(lib().kv_cache_layout(ctypes.byref(c)))


def kv_quant_append(c: KvqCacheStruct, k_new, v_new, n: int, stream=None):
    _check(lib().kv_quant_append(ctypes.byref(c), _ptr(k_new), _ptr(v_new), n,
                                 _stream(stream)))


def kv_rollback(c: KvqCacheStruct, m: int) -> None:
    _check(lib().kv_rollback(ctypes.byref(c), m))


def kv_attn_workspace_bytes(c: KvqCacheStruct, T: int, Hq: int) -> int:
    return lib().kv_attn_workspace_bytes(ctypes.byref(c), T, Hq)


def kv_attn_verify(c: KvqCacheStruct, q, T: int, Hq: int, path, sm_scale: float,
                   out, lse, ws, stream=None) -> None:
    _check(lib().kv_attn_verify(
        ctypes.byref(c), _ptr(q), T, Hq, _path(path), float(sm_scale),
        _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream(stream)))


def kv_attn_verify_noalloc(c: KvqCacheStruct, q, T: int, Hq: int, path,
                           sm_scale: float, out, lse, stream=None) -> None:
    _check(lib().kv_attn_verify_noalloc(
        ctypes.byref(c), _ptr(q), T, Hq, _path(path), float(sm_scale),
        _ptr(out), _ptr(lse), _stream(stream)))


def kv_topk_workspace_bytes(c: KvqCacheStruct, Hq: int, k: int) -> int:
    return lib().kv_topk_workspace_bytes(ctypes.byref(c), Hq, k)


def kv_topk(c: KvqCacheStruct, q_spec, Hq: int, path, k: int, idx, key, ws,
            stream=None) -> None:
    _check(lib().kv_topk(
        ctypes.byref(c), _ptr(q_spec), Hq, _path(path), k, _ptr(idx),
        _ptr(key), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def kv_dequant_gather(c: KvqCacheStruct, idx, n: int, path, k_out, v_out,
                      stream=None) -> None:
    _check(lib().kv_dequant_gather(
        ctypes.byref(c), _ptr(idx), n, _path(path), _ptr(k_out), _ptr(v_out),
        _stream(stream)))


def kv_attn_verify_exact(c: KvqCacheStruct, q, T: int, Hq: int, path,
                         sm_scale: float, t_exact: int, idx, n: int, k_exact,
                         v_exact, out, lse, ws, stream=None,
                         rows_ready=None) -> None:
    """rows_ready: None, or an event (torch.cuda.Event or a raw hipEvent_t)
    recorded after k_exact/v_exact were written."""
    ev = getattr(rows_ready, "cuda_event", rows_ready)
    _check(lib().kv_attn_verify_exact(
        ctypes.byref(c), _ptr(q), T, Hq, _path(path), float(sm_scale), t_exact,
        _ptr(idx), n, _ptr(k_exact), _ptr(v_exact), _ptr(out), _ptr(lse),
        _ptr(ws), 0 if ws is None else ws.numel(), ev, _stream(stream)))


def kv_fetch_rows(c: KvqCacheStruct, host_k, host_v, host_len: int, idx, n: int,
                  k_out, v_out, stream=None) -> None:
    _check(lib().kv_fetch_rows(
        ctypes.byref(c), _ptr(host_k), _ptr(host_v), host_len, _ptr(idx), n,
        _ptr(k_out), _ptr(v_out), _stream(stream)))


# ---- torch-owned cache -----------------------------------------------------

@dataclass
class Shape:
    B: int
    Hkv: int
    d: int
    G: int
    Gv: int
    bits: int
    R: int
    L_max: int
    max_append: int = 32


class QuantKVCache:
    """Device buffers of one quantized cache, allocated with torch.

    Every buffer is a flat uint8 tensor of the byte size kv_cache_layout
    reports; the struct holds their addresses.  Methods only marshal
    arguments to the C entry points.
    """

    def __init__(self, shape: Shape, device="cuda"):
        import torch
        self.shape = shape
        c = KvqCacheStruct()
        for f in ("B", "Hkv", "d", "G", "Gv", "bits", "R", "L_max",
                  "max_append"):
            setattr(c, f, getattr(shape, f))
        kv_cache_layout(c)
        self.c = c
        u8 = dict(dtype=torch.uint8, device=device)
        self.k_hi = torch.zeros(c.bytes_k_plane, **u8)
        self.v_hi = torch.zeros(c.bytes_v_plane, **u8)
        self.k_lo = torch.zeros(c.bytes_k_plane, **u8) if shape.bits == 8 else None
        self.v_lo = torch.zeros(c.bytes_v_plane, **u8) if shape.bits == 8 else None
        self.k_sz = torch.zeros(c.bytes_k_sz, **u8)
        self.v_sz = torch.zeros(c.bytes_v_sz, **u8)
        self.k_res = torch.zeros(c.bytes_k_res, **u8)
        self.v_res = torch.zeros(c.bytes_v_res, **u8)
        for name in ("k_hi", "k_lo", "v_hi", "v_lo", "k_sz", "v_sz", "k_res",
                     "v_res"):
            setattr(c, name, _ptr(getattr(self, name)))

    # counters
    @property
    def n_q(self) -> int:
        return self.c.n_q

    @property
    def n_r(self) -> int:
        return self.c.n_r

    @property
    def ring(self) -> int:
        return self.c.ring

    def clone(self) -> "QuantKVCache":
        """A second cache with its own buffers holding the same contents."""
        import torch
        other = QuantKVCache.__new__(QuantKVCache)
        other.shape = self.shape
        other.c = KvqCacheStruct()
        ctypes.pointer(other.c)[0] = self.c
        for name in ("k_hi", "k_lo", "v_hi", "v_lo", "k_sz", "v_sz", "k_res",
                     "v_res"):
            t = getattr(self, name)
            t2 = None if t is None else t.clone()
            setattr(other, name, t2)
            setattr(other.c, name, _ptr(t2))
        return other

    def _tokens(self, x, name):
        import torch
        s = self.shape
        if (x.dtype != torch.float16 or not x.is_cuda or not x.is_contiguous()
                or x.dim() != 4 or x.shape[0] != s.B or x.shape[2] != s.Hkv
                or x.shape[3] != s.d):
            raise ValueError(f"{name} must be contiguous fp16 CUDA "
                             f"[B={s.B}][n][Hkv={s.Hkv}][d={s.d}]")
        return x

    def append(self, k_new, v_new, stream=None) -> None:
        """kv_quant_append of fp16 [B][n][Hkv][d] tokens."""
        self._tokens(k_new, "k_new")
        self._tokens(v_new, "v_new")
        if k_new.shape != v_new.shape:
            raise ValueError("k_new and v_new shapes differ")
        kv_quant_append(self.c, k_new, v_new, k_new.shape[1], stream)

    def rollback(self, m: int) -> None:
        kv_rollback(self.c, m)

    def attn_workspace(self, T: int, Hq: int):
        import torch
        n = kv_attn_workspace_bytes(self.c, T, Hq)
        return torch.zeros(n, dtype=torch.uint8, device=self.k_hi.device)

    def verify(self, q, path="target", sm_scale=None, out=None, lse=None,
               ws=None, want_lse=False, stream=None):
        """kv_attn_verify for fp16 q [B][T][Hq][d]; returns (out, lse)."""
        import torch
        s = self.shape
        if (q.dtype != torch.float16 or not q.is_cuda or not q.is_contiguous()
                or q.dim() != 4 or q.shape[0] != s.B or q.shape[3] != s.d):
            raise ValueError("q must be contiguous fp16 CUDA [B][T][Hq][d]")
        B, T, Hq, d = q.shape
        if sm_scale is None:
            sm_scale = d ** -0.5
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.attn_workspace(T, Hq)
        kv_attn_verify(self.c, q, T, Hq, path, sm_scale, out, lse, ws, stream)
        return out, lse

    def verify_exact(self, q, idx, k_exact, v_exact, t_exact=0, path="target",
                     sm_scale=None, out=None, lse=None, ws=None, want_lse=False,
                     stream=None, rows_ready=None):
        """kv_attn_verify_exact: like ``verify``, with query row t_exact
        reading k_exact/v_exact [B][Hkv][n][d] at positions idx
        [B][Hkv][n]; rows_ready: an event recorded after k_exact/v_exact
        were written (they may still be in flight on another stream), or
        None; returns (out, lse)."""
        import torch
        s = self.shape
        if (q.dtype != torch.float16 or not q.is_cuda or not q.is_contiguous()
                or q.dim() != 4 or q.shape[0] != s.B or q.shape[3] != s.d):
            raise ValueError("q must be contiguous fp16 CUDA [B][T][Hq][d]")
        if (idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous()
                or idx.dim() != 3 or tuple(idx.shape[:2]) != (s.B, s.Hkv)):
            raise ValueError("idx must be contiguous int32 CUDA [B][Hkv][n]")
        n = idx.shape[2]
        for t, name in ((k_exact, "k_exact"), (v_exact, "v_exact")):
            if (t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous()
                    or tuple(t.shape) != (s.B, s.Hkv, n, s.d)):
                raise ValueError(f"{name} must be contiguous fp16 CUDA "
                                 f"[B][Hkv][n][d]")
        B, T, Hq, d = q.shape
        if sm_scale is None:
            sm_scale = d ** -0.5
        if out is None:
            out = torch.empty_like(q)
        if lse is None and want_lse:
            lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.attn_workspace(T, Hq)
        kv_attn_verify_exact(self.c, q, T, Hq, path, sm_scale, t_exact, idx, n,
                             k_exact, v_exact, out, lse, ws, stream, rows_ready)
        return out, lse

    def topk_workspace(self, Hq: int, k: int):
        import torch
        n = kv_topk_workspace_bytes(self.c, Hq, k)
        return torch.zeros(n, dtype=torch.uint8, device=self.k_hi.device)

    def topk(self, q_spec, k: int, path="target", idx=None, key=None, ws=None,
             stream=None):
        """kv_topk for fp16 q_spec [B][Hq][d]; returns (idx, key)."""
        import torch
        s = self.shape
        if (q_spec.dtype != torch.float16 or not q_spec.is_cuda
                or not q_spec.is_contiguous() or q_spec.dim() != 3
                or q_spec.shape[0] != s.B or q_spec.shape[2] != s.d):
            raise ValueError("q_spec must be contiguous fp16 CUDA [B][Hq][d]")
        Hq = q_spec.shape[1]
        dev = q_spec.device
        if idx is None:
            idx = torch.empty((s.B, s.Hkv, k), dtype=torch.int32, device=dev)
        if key is None:
            key = torch.empty((s.B, s.Hkv, k), dtype=torch.float32, device=dev)
        if ws is None:
            ws = self.topk_workspace(Hq, k)
        kv_topk(self.c, q_spec, Hq, path, k, idx, key, ws, stream)
        return idx, key

    def gather(self, idx, path="target", k_out=None, v_out=None, stream=None):
        """kv_dequant_gather for int32 positions idx [B][Hkv][n]; returns the
        fp16 rows (k_out, v_out), each [B][Hkv][n][d]."""
        import torch
        s = self.shape
        if (idx.dtype != torch.int32 or not idx.is_cuda
                or not idx.is_contiguous() or idx.dim() != 3
                or idx.shape[0] != s.B or idx.shape[1] != s.Hkv):
            raise ValueError("idx must be contiguous int32 CUDA [B][Hkv][n]")
        n = idx.shape[2]
        shape = (s.B, s.Hkv, n, s.d)
        for t, name in ((k_out, "k_out"), (v_out, "v_out")):
            if t is not None and (t.dtype != torch.float16 or not t.is_cuda
                                  or not t.is_contiguous()
                                  or tuple(t.shape) != shape):
                raise ValueError(f"{name} must be contiguous fp16 CUDA {shape}")
        if k_out is None:
            k_out = torch.empty(shape, dtype=torch.float16, device=idx.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=torch.float16, device=idx.device)
        kv_dequant_gather(self.c, idx, n, path, k_out, v_out, stream)
        return k_out, v_out


class HostMirror:
    """Full-precision copy of a cache's tokens in pinned host memory, fp16
    [B][Hkv][L_max][d] for K and V, filled by the caller alongside its
    appends.  ``fetch`` runs kv_fetch_rows: the rows at positions idx
    [B][Hkv][n] come back as device fp16 [B][Hkv][n][d]."""

    def __init__(self, shape: Shape, length: int):
        import torch
        self.shape, self.length = shape, length
        dims = (shape.B, shape.Hkv, length, shape.d)
        self.k = torch.zeros(dims, dtype=torch.float16, pin_memory=True)
        self.v = torch.zeros(dims, dtype=torch.float16, pin_memory=True)

    def write(self, p0: int, k_tokens, v_tokens) -> None:
        """Store host fp16 tokens [B][n][Hkv][d] at positions p0.."""
        import torch
        n = k_tokens.shape[1]
        self.k[:, :, p0:p0 + n] = torch.as_tensor(k_tokens).permute(0, 2, 1, 3)
        self.v[:, :, p0:p0 + n] = torch.as_tensor(v_tokens).permute(0, 2, 1, 3)

    def fetch(self, cache: "QuantKVCache", idx, k_out=None, v_out=None,
              stream=None):
        import torch
        s = self.shape
        if (idx.dtype != torch.int32 or not idx.is_cuda or not idx.is_contiguous()
                or idx.dim() != 3 or tuple(idx.shape[:2]) != (s.B, s.Hkv)):
            raise ValueError("idx must be contiguous int32 CUDA [B][Hkv][n]")
        n = idx.shape[2]
        shape = (s.B, s.Hkv, n, s.d)
        if k_out is None:
            k_out = torch.empty(shape, dtype=torch.float16, device=idx.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=torch.float16, device=idx.device)
        kv_fetch_rows(cache.c, self.k, self.v, self.length, idx, n, k_out, v_out,
                      stream)
        return k_out, v_out
