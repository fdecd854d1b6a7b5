"""ctypes binding of libtq.so: argument checks and marshalling only.

torch is used for device memory and the current HIP stream; no computation
of the method happens here.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

TQ_F32, TQ_BF16 = 0, 1
TQ_CODEBOOK_GAUSSIAN, TQ_CODEBOOK_BETA = 0, 1
_KINDS = {"gaussian": TQ_CODEBOOK_GAUSSIAN, "beta": TQ_CODEBOOK_BETA}
_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libtq.so")

# Every entry point declared in include/tq.h.
EXPORTED_SYMBOLS = (
    "tq_codebook_tables", "tq_make_codebook", "tq_free_codebook", "tq_codebook_export",
    "tq_codebook_info", "tq_packed_bytes", "tq_encode_keys", "tq_append_keys",
    "tq_score_workspace_bytes", "tq_score_logits", "tq_score_cache", "tq_score_topk_workspace_bytes", "tq_score_topk", "tq_decode_mse",
    "tq_dense_logits_bf16", "tq_status_string", "tq_last_hip_error",
    "tq_value_packed_bytes", "tq_encode_values", "tq_attention_workspace_bytes",
    "tq_attention_decode", "tq_codebook_tables_ex", "tq_make_codebook_ex", "tq_rotation_dim",
    "tq_clock_probe", "tq_stream_probe", "tq_score_stream_probe",
    "tq_attention_decode_noalloc", "tq_attention_noalloc_max_bytes",
    "tq_paged_append_keys", "tq_paged_score", "tq_append_values", "tq_attention_cache",
    "tq_paged_append_values", "tq_paged_attention",
)

_c_i32, _c_i64, _c_u64, _c_sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
_SIGS = {
    "tq_codebook_tables": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_u64, _vp, _vp, _vp, _vp, _vp]),
    "tq_make_codebook": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_u64, ctypes.POINTER(_vp)]),
    "tq_codebook_tables_ex": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_u64, _c_i32, _vp, _vp, _vp, _vp,
                                             _vp]),
    "tq_make_codebook_ex": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_u64, _c_i32, ctypes.POINTER(_vp)]),
    "tq_free_codebook": (None, [_vp]),
    "tq_rotation_dim": (_c_i32, [_c_i32]),
    "tq_codebook_export": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "tq_codebook_info": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp]),
    "tq_packed_bytes": (_c_sz, [_vp, _c_i64, _c_i64]),
    "tq_encode_keys": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _vp]),
    "tq_append_keys": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp]),
    "tq_score_cache": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _c_i64, _c_i64, _vp, _vp]),
    "tq_score_workspace_bytes": (_c_sz, [_vp, _c_i64, _c_i32]),
    "tq_score_logits": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _c_i64, _vp, _vp,
                                       _c_sz, _vp]),
    "tq_score_topk_workspace_bytes": (_c_sz, [_vp, _c_i64, _c_i32, _c_i64, _c_i32]),
    "tq_score_topk": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _c_i64, _c_i32, _vp, _vp,
                                     _vp, _c_sz, _vp]),
    "tq_decode_mse": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i32, _vp]),
    "tq_dense_logits_bf16": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i32, _c_i64, _c_i32, _vp, _vp]),
    "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tq_value_packed_bytes": (_c_sz, [_vp, _c_i64, _c_i64]),
    "tq_encode_values": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _vp]),
    "tq_attention_workspace_bytes": (_c_sz, [_vp, _c_i64, _c_i32, _c_i64]),
    "tq_attention_decode": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _vp, _c_i64,
                                           ctypes.c_float, _vp, _vp, _c_sz, _vp]),
    "tq_append_values": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _c_i64, _c_i64, _vp]),
    "tq_attention_cache": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _vp, _c_i64, _c_i64,
                                          ctypes.c_float, _vp, _vp, _c_sz, _vp]),
    "tq_last_hip_error": (ctypes.c_int, []),
    "tq_attention_decode_noalloc": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _vp, _c_i64,
                                                   ctypes.c_float, _vp, _vp]),
    "tq_attention_noalloc_max_bytes": (_c_sz, []),
    "tq_paged_append_keys": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _c_i64, _c_i32, _vp,
                                            _c_i32, _vp, _vp]),
    "tq_paged_score": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _c_i64, _c_i32, _vp, _c_i32,
                                      _vp, _c_i64, _vp, _vp]),
    "tq_paged_append_values": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i64, _vp, _c_i64, _c_i32, _vp,
                                              _c_i32, _vp, _vp]),
    "tq_paged_attention": (ctypes.c_int, [_vp, _vp, _c_i32, _c_i64, _c_i32, _vp, _vp, _c_i64, _c_i32, _vp,
                                          _c_i32, _vp, _c_i64, ctypes.c_float, _vp, _vp, _c_sz, _vp]),
    "tq_clock_probe": (ctypes.c_int, [_vp, _c_i32, _vp]),
    "tq_stream_probe": (ctypes.c_int, [_vp, _c_sz, _vp, _c_sz, _c_i32, _vp]),
    "tq_score_stream_probe": (ctypes.c_int, [_vp, _c_i64, _c_i32, _vp, _c_i64, _vp, _vp]),
}

_lib = None


class TQError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = what
        if _lib is not None and status != 0:
            msg = f"{what}: {_lib.tq_status_string(status).decode()} (status {status}"
            if status == -4:
                msg += f", hipError {_lib.tq_last_hip_error()}"
            msg += ")"
        super().__init__(msg)


def library():
    """Load libtq.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise TQError(-1, f"{library_path} is missing; build it with "
                              "`python -m kv_cache_vector_rotate_amd.build`")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise TQError(rc, what)


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data if isinstance(a, np.ndarray) else a.data_ptr())


def rotation_dim(d: int) -> int:
    """The power of two the method runs in for d-element vectors (d, or the
    next power of two for a zero-padded d); 0 when unsupported."""
    return int(library().tq_rotation_dim(d))


def codebook_tables(d: int, bits: int, m: int | None = None, seed: int = 42, kind: str = "gaussian"):
    """Host-only quantizer tables (no GPU): levels, thresholds, delta, S, S R^T
    (kind: "gaussian" = N(0, 1/D) Lloyd-Max, "beta" = the exact coordinate law;
    D = rotation_dim(d), the arrays are D-dimensional)."""
    D = rotation_dim(d)
    if D == 0:
        raise TQError(-2, "tq_rotation_dim")
    m = D if m is None else m
    L = 1 << (bits - 1)
    out = dict(levels=np.empty(L, np.float64), thresholds=np.empty(L - 1, np.float64),
               delta=np.empty(D, np.int8), S=np.empty((m, D), np.float64),
               S_rot=np.empty((m, D), np.float64))
    _check(library().tq_codebook_tables_ex(d, bits, m, seed, _KINDS[kind], *(_ptr(out[k]) for k in
                                           ("levels", "thresholds", "delta", "S", "S_rot"))),
           "tq_codebook_tables_ex")
    return out


class Codebook:
    """Device-resident quantizer state for (d, bits, m, seed).  d is the
    length of the caller's vectors; D = rotation_dim(d) the dimension the
    method runs in (m defaults to D)."""

    def __init__(self, d: int = 128, bits: int = 3, m: int | None = None, seed: int = 42,
                 kind: str = "gaussian"):
        lib = library()
        self.D = rotation_dim(d)
        self.d, self.bits, self.m, self.seed = d, bits, (self.D or d) if m is None else m, seed
        self.kind = kind
        h = ctypes.c_void_p()
        _check(lib.tq_make_codebook_ex(d, bits, self.m, seed, _KINDS[kind], ctypes.byref(h)),
               "tq_make_codebook_ex")
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            library().tq_free_codebook(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass

    def export(self):
        L = 1 << (self.bits - 1)
        out = dict(levels=np.empty(L, np.float64), thresholds=np.empty(L - 1, np.float64),
                   delta=np.empty(self.D, np.int8), S=np.empty((self.m, self.D), np.float64),
                   S_rot=np.empty((self.m, self.D), np.float64))
        _check(library().tq_codebook_export(self._h, *(_ptr(out[k]) for k in
                                            ("levels", "thresholds", "delta", "S", "S_rot"))),
               "tq_codebook_export")
        return out


def packed_nbytes(cb: Codebook, G: int, N: int) -> int:
    return int(library().tq_packed_bytes(cb.handle, G, N))


def score_workspace_nbytes(cb: Codebook, G: int, Qg: int) -> int:
    return int(library().tq_score_workspace_bytes(cb.handle, G, Qg))


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    if t.dtype == torch.float32:
        return TQ_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need_cuda(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def _need_bytes(t, nbytes: int, name: str):
    """The C ABI takes raw pointers and cannot see allocation sizes: refuse a
    buffer smaller than what the kernels will read or write."""
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")


def _need_rows(t, name: str, G: int, d: int):
    if t.dim() != 3 or t.shape[0] != G or t.shape[2] != d:
        raise ValueError(f"{name} must be [G={G}, n, d={d}], got {tuple(t.shape)}")


def encode_keys(cb: Codebook, keys, out=None):
    """keys [G, N, d] (float32/bfloat16, device) -> packed uint8 [packed_nbytes]."""
    torch = _torch()
    _need_cuda(keys, "keys")
    G, N, d = keys.shape
    if d != cb.d:
        raise ValueError("key dimension does not match the codebook")
    nb = packed_nbytes(cb, G, N)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=keys.device)
    elif out.numel() * out.element_size() < nb:
        raise ValueError("packed buffer too small")
    _check(library().tq_encode_keys(cb.handle, _ptr(keys), _dtype_code(keys), G, N, _ptr(out),
                                    _stream()), "tq_encode_keys")
    return out


def _need_out(out, n: int):
    torch = _torch()
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() < n:
        raise ValueError("logits must be a contiguous float32 tensor of G*Qg*N elements")


def append_keys(cb: Codebook, keys, packed, Ncap: int, pos: int):
    """Encode keys [G, T, d] into records pos .. pos+T-1 of each group of a
    packed cache holding Ncap records per group (in place)."""
    _need_cuda(keys, "keys")
    _need_cuda(packed, "packed")
    G, T, d = keys.shape
    if d != cb.d:
        raise ValueError("key dimension does not match the codebook")
    if packed.numel() * packed.element_size() < packed_nbytes(cb, G, Ncap):
        raise ValueError("packed buffer too small for Ncap records per group")
    _check(library().tq_append_keys(cb.handle, _ptr(keys), _dtype_code(keys), G, T, _ptr(packed),
                                    Ncap, pos, _stream()), "tq_append_keys")
    return packed


def score_cache(cb: Codebook, q, packed, Ncap: int, length: int, out=None):
    """q [G, Qg, d] against the first `length` records of a packed cache of
    Ncap records per group -> float32 [G, Qg, length]."""
    torch = _torch()
    _need_cuda(q, "q")
    _need_cuda(packed, "packed")
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    if not 0 <= length <= Ncap:
        raise ValueError("length must lie in [0, Ncap]")
    _need_bytes(packed, packed_nbytes(cb, G, Ncap), "packed cache (Ncap records per group)")
    if out is None:
        out = torch.empty((G, Qg, length), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * length)
    _check(library().tq_score_cache(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(packed), Ncap,
                                    length, _ptr(out), _stream()), "tq_score_cache")
    return out


def _need_i32(t, n: int, name: str):
    torch = _torch()
    _need_cuda(t, name)
    if t.dtype != torch.int32 or t.numel() < n:
        raise ValueError(f"{name} must be a device int32 tensor of at least {n} elements")


def paged_pool_nbytes(cb: Codebook, num_pages: int, page_size: int) -> int:
    """Bytes of a pool of num_pages pages of page_size records."""
    return packed_nbytes(cb, num_pages, page_size)


def paged_append_keys(cb: Codebook, keys, pool, page_size: int, page_table, pos):
    """Encode keys [G, T, d] into a paged pool: key t of group g goes to
    logical position pos[g] + t through page_table [G, pages_per_group]
    (device int32); pos is a device int32 [G].  In place."""
    _need_cuda(keys, "keys")
    _need_cuda(pool, "pool")
    G, T, d = keys.shape
    if d != cb.d:
        raise ValueError("key dimension does not match the codebook")
    per_page = packed_nbytes(cb, 1, page_size)
    num_pages = (pool.numel() * pool.element_size()) // per_page if per_page else 0
    if page_table.dim() != 2 or page_table.shape[0] != G:
        raise ValueError("page_table must be [G, pages_per_group]")
    _need_i32(page_table, G * page_table.shape[1], "page_table")
    _need_i32(pos, G, "pos")
    _check(library().tq_paged_append_keys(cb.handle, _ptr(keys), _dtype_code(keys), G, T, _ptr(pool),
                                          num_pages, page_size, _ptr(page_table), page_table.shape[1],
                                          _ptr(pos), _stream()), "tq_paged_append_keys")
    return pool


def paged_score(cb: Codebook, q, pool, page_size: int, page_table, lens, Lmax: int, out=None):
    """q [G, Qg, d] against the first lens[g] records of each group of a
    paged pool -> float32 [G, Qg, Lmax] (entries past lens[g] untouched)."""
    torch = _torch()
    _need_cuda(q, "q")
    _need_cuda(pool, "pool")
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    per_page = packed_nbytes(cb, 1, page_size)
    num_pages = (pool.numel() * pool.element_size()) // per_page if per_page else 0
    if page_table.dim() != 2 or page_table.shape[0] != G:
        raise ValueError("page_table must be [G, pages_per_group]")
    _need_i32(page_table, G * page_table.shape[1], "page_table")
    _need_i32(lens, G, "lens")
    if out is None:
        out = torch.zeros((G, Qg, Lmax), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * Lmax)
    _check(library().tq_paged_score(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(pool), num_pages,
                                    page_size, _ptr(page_table), page_table.shape[1], _ptr(lens), Lmax,
                                    _ptr(out), _stream()), "tq_paged_score")
    return out


def value_packed_nbytes(cb: Codebook, G: int, N: int) -> int:
    return int(library().tq_value_packed_bytes(cb.handle, G, N))


def paged_value_pool_nbytes(cb: Codebook, num_pages: int, page_size: int) -> int:
    """Bytes of a value pool of num_pages pages of page_size value records."""
    return value_packed_nbytes(cb, num_pages, page_size)


def _pages(nbytes_of_one, t, page_size):
    per_page = nbytes_of_one(page_size)
    return (t.numel() * t.element_size()) // per_page if per_page else 0


def paged_append_values(cb: Codebook, values, pool, page_size: int, page_table, pos):
    """Encode values [G, T, d] into a paged value pool: value t of group g
    goes to logical position pos[g] + t through page_table [G,
    pages_per_group] (device int32); pos is a device int32 [G].  In place."""
    _need_cuda(values, "values")
    _need_cuda(pool, "pool")
    G, T, d = values.shape
    if d != cb.d:
        raise ValueError("value dimension does not match the codebook")
    num_pages = _pages(lambda ps: value_packed_nbytes(cb, 1, ps), pool, page_size)
    if page_table.dim() != 2 or page_table.shape[0] != G:
        raise ValueError("page_table must be [G, pages_per_group]")
    _need_i32(page_table, G * page_table.shape[1], "page_table")
    _need_i32(pos, G, "pos")
    _check(library().tq_paged_append_values(cb.handle, _ptr(values), _dtype_code(values), G, T, _ptr(pool),
                                            num_pages, page_size, _ptr(page_table), page_table.shape[1],
                                            _ptr(pos), _stream()), "tq_paged_append_values")
    return pool


def paged_attention(cb: Codebook, q, kpool, vpool, page_size: int, page_table, lens, Lmax: int, scale=None,
                    out=None, ws=None):
    """Decode attention of q [G, Qg, d] over the first lens[g] (at most Lmax)
    positions of each group of a paged key pool and value pool that share
    page_table -> float32 [G, Qg, d] (zeros for a group without keys)."""
    torch = _torch()
    for t, name in ((q, "q"), (kpool, "kpool"), (vpool, "vpool")):
        _need_cuda(t, name)
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    num_pages = _pages(lambda ps: packed_nbytes(cb, 1, ps), kpool, page_size)
    _need_bytes(vpool, paged_value_pool_nbytes(cb, num_pages, page_size), "vpool (as many pages as kpool)")
    if page_table.dim() != 2 or page_table.shape[0] != G:
        raise ValueError("page_table must be [G, pages_per_group]")
    _need_i32(page_table, G * page_table.shape[1], "page_table")
    _need_i32(lens, G, "lens")
    if out is None:
        out = torch.empty((G, Qg, d), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * d)
    wsb = attention_workspace_nbytes(cb, G, Qg, Lmax)
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check(library().tq_paged_attention(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(kpool), _ptr(vpool),
                                        num_pages, page_size, _ptr(page_table), page_table.shape[1],
                                        _ptr(lens), Lmax, scale, _ptr(out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream()), "tq_paged_attention")
    return out


def encode_values(cb: Codebook, values, out=None):
    """values [G, N, d] (float32/bfloat16, device) -> value records uint8."""
    torch = _torch()
    _need_cuda(values, "values")
    G, N, d = values.shape
    if d != cb.d:
        raise ValueError("value dimension does not match the codebook")
    nb = value_packed_nbytes(cb, G, N)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=values.device)
    elif out.numel() * out.element_size() < nb:
        raise ValueError("value buffer too small")
    _check(library().tq_encode_values(cb.handle, _ptr(values), _dtype_code(values), G, N, _ptr(out),
                                      _stream()), "tq_encode_values")
    return out


def append_values(cb: Codebook, values, vpacked, Ncap: int, pos: int):
    """Encode values [G, T, d] into records pos .. pos+T-1 of each group of a
    value cache holding Ncap records per group (in place)."""
    _need_cuda(values, "values")
    _need_cuda(vpacked, "vpacked")
    G, T, d = values.shape
    if d != cb.d:
        raise ValueError("value dimension does not match the codebook")
    _need_bytes(vpacked, value_packed_nbytes(cb, G, Ncap), "vpacked (Ncap records per group)")
    _check(library().tq_append_values(cb.handle, _ptr(values), _dtype_code(values), G, T, _ptr(vpacked),
                                      Ncap, pos, _stream()), "tq_append_values")
    return vpacked


def attention_workspace_nbytes(cb: Codebook, G: int, Qg: int, N: int) -> int:
    return int(library().tq_attention_workspace_bytes(cb.handle, G, Qg, N))


def attention_decode(cb: Codebook, q, kpacked, vpacked, N: int, scale=None, out=None, ws=None):
    """softmax(scale * estimated logits) @ v_mse for q [G, Qg, d] over N packed
    keys and values per group -> float32 [G, Qg, d] (scale 1/sqrt(d) by default)."""
    torch = _torch()
    for t, name in ((q, "q"), (kpacked, "kpacked"), (vpacked, "vpacked")):
        _need_cuda(t, name)
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    _need_bytes(kpacked, packed_nbytes(cb, G, N), "kpacked")
    _need_bytes(vpacked, value_packed_nbytes(cb, G, N), "vpacked")
    if out is None:
        out = torch.empty((G, Qg, d), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * d)
    wsb = attention_workspace_nbytes(cb, G, Qg, N)
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check(library().tq_attention_decode(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(kpacked),
                                         _ptr(vpacked), N, scale, _ptr(out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream()),
           "tq_attention_decode")
    return out


def attention_cache(cb: Codebook, q, kpacked, vpacked, Ncap: int, length: int, scale=None, out=None,
                    ws=None):
    """attention_decode over the first `length` records of a key cache and a
    value cache of Ncap records per group each -> float32 [G, Qg, d]."""
    torch = _torch()
    for t, name in ((q, "q"), (kpacked, "kpacked"), (vpacked, "vpacked")):
        _need_cuda(t, name)
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    if not 0 < length <= Ncap:
        raise ValueError("length must lie in [1, Ncap]")
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    _need_bytes(kpacked, packed_nbytes(cb, G, Ncap), "kpacked (Ncap records per group)")
    _need_bytes(vpacked, value_packed_nbytes(cb, G, Ncap), "vpacked (Ncap records per group)")
    if out is None:
        out = torch.empty((G, Qg, d), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * d)
    wsb = attention_workspace_nbytes(cb, G, Qg, length)
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check(library().tq_attention_cache(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(kpacked),
                                        _ptr(vpacked), Ncap, length, scale, _ptr(out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream()),
           "tq_attention_cache")
    return out


def attention_decode_noalloc(cb: Codebook, q, kpacked, vpacked, N: int, scale=None, out=None):
    """attention_decode working in the library's static device scratch (no
    workspace argument, nothing allocated by the library); out must be given
    by callers that cannot allocate."""
    torch = _torch()
    for t, name in ((q, "q"), (kpacked, "kpacked"), (vpacked, "vpacked")):
        _need_cuda(t, name)
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    scale = 1.0 / d ** 0.5 if scale is None else float(scale)
    _need_bytes(kpacked, packed_nbytes(cb, G, N), "kpacked")
    _need_bytes(vpacked, value_packed_nbytes(cb, G, N), "vpacked")
    if out is None:
        out = torch.empty((G, Qg, d), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * d)
    _check(library().tq_attention_decode_noalloc(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(kpacked),
                                                 _ptr(vpacked), N, scale, _ptr(out), _stream()),
           "tq_attention_decode_noalloc")
    return out


def attention_noalloc_max_nbytes() -> int:
    return int(library().tq_attention_noalloc_max_bytes())


def score_logits(cb: Codebook, q, packed, N: int, out=None, ws=None):
    """q [G, Qg, d] against packed keys of N per group -> float32 [G, Qg, N]."""
    torch = _torch()
    _need_cuda(q, "q")
    _need_cuda(packed, "packed")
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    _need_bytes(packed, packed_nbytes(cb, G, N), "packed")
    if out is None:
        out = torch.empty((G, Qg, N), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * N)
    wsb = score_workspace_nbytes(cb, G, Qg)
    if ws is None:
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check(library().tq_score_logits(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(packed), N,
                                     _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream()), "tq_score_logits")
    return out


def score_topk_workspace_nbytes(cb: Codebook, G: int, Qg: int, N: int, k: int) -> int:
    return int(library().tq_score_topk_workspace_bytes(cb.handle, G, Qg, N, k))


def score_topk(cb: Codebook, q, packed, N: int, k: int = 10, ws=None):
    """Best k keys per query by the estimated inner product: q [G, Qg, d]
    against packed keys of N per group -> (int32 idx [G, Qg, k], float32
    scores [G, Qg, k]), best first, ties to the smaller index."""
    torch = _torch()
    _need_cuda(q, "q")
    _need_cuda(packed, "packed")
    G, Qg, d = q.shape
    if d != cb.d:
        raise ValueError("query dimension does not match the codebook")
    _need_bytes(packed, packed_nbytes(cb, G, N), "packed")
    idx = torch.empty((G, Qg, k), dtype=torch.int32, device=q.device)
    scores = torch.empty((G, Qg, k), dtype=torch.float32, device=q.device)
    if ws is None:
        wsb = score_topk_workspace_nbytes(cb, G, Qg, N, k)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    _check(library().tq_score_topk(cb.handle, _ptr(q), _dtype_code(q), G, Qg, _ptr(packed), N, k,
                                   _ptr(idx), _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream()), "tq_score_topk")
    return idx, scores


def decode_mse(cb: Codebook, packed, G: int, N: int, dtype=None, out=None):
    """packed keys -> nu~ R^T c[code], [G, N, d] float32 (default) or bfloat16."""
    torch = _torch()
    _need_cuda(packed, "packed")
    _need_bytes(packed, packed_nbytes(cb, G, N), "packed")
    dtype = torch.float32 if dtype is None else dtype
    if out is None:
        out = torch.empty((G, N, cb.d), dtype=dtype, device=packed.device)
    _need_cuda(out, "out")
    _dtype_code(out)
    if out.numel() < G * N * cb.d:
        raise ValueError(f"out must hold G*N*d = {G * N * cb.d} elements")
    _check(library().tq_decode_mse(cb.handle, _ptr(packed), G, N, _ptr(out), _dtype_code(out),
                                   _stream()), "tq_decode_mse")
    return out


def dense_logits_bf16(q, keys, out=None):
    """Unquantised comparator: bf16 q [G, Qg, d] . bf16 keys [G, N, d] -> float32 [G, Qg, N]."""
    torch = _torch()
    _need_cuda(q, "q")
    _need_cuda(keys, "keys")
    G, Qg, d = q.shape
    _need_rows(keys, "keys", G, d)
    if q.dtype != torch.bfloat16 or keys.dtype != torch.bfloat16:
        raise TypeError("q and keys must be bfloat16")
    N = keys.shape[1]
    if out is None:
        out = torch.empty((G, Qg, N), dtype=torch.float32, device=q.device)
    _need_out(out, G * Qg * N)
    _check(library().tq_dense_logits_bf16(_ptr(q), _ptr(keys), G, Qg, N, d, _ptr(out), _stream()),
           "tq_dense_logits_bf16")
    return out


# ---- measurement helpers (not part of the method)

def clock_probe(ticks: int = 4000):
    """(core-clock cycles, reference ticks) counted by one wave over `ticks`
    reference ticks, as a device tensor of two int64 (read it after a sync)."""
    torch = _torch()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    _check(library().tq_clock_probe(_ptr(out), ticks, _stream()), "tq_clock_probe")
    return out


def stream_probe(src, dst=None, src_bytes=None, dst_bytes=None, grid: int = 0):
    """Stream src (read) and dst (write) device buffers: read-only when dst is
    None, a copy when both are the same size."""
    sb = src.numel() * src.element_size() if src_bytes is None else src_bytes
    db = 0 if dst is None else (dst.numel() * dst.element_size() if dst_bytes is None else dst_bytes)
    _need_cuda(src, "src")
    _need_bytes(src, sb, "src")
    if dst is not None:
        _need_cuda(dst, "dst")
        _need_bytes(dst, db, "dst")
    _check(library().tq_stream_probe(_ptr(src), sb, _ptr(dst), db, grid, _stream()), "tq_stream_probe")


def score_stream_probe(cb: Codebook, G: int, Qg: int, packed, N: int, out):
    """The scorer's loads and stores without its arithmetic (a ceiling)."""
    _need_cuda(packed, "packed")
    _need_bytes(packed, packed_nbytes(cb, G, N), "packed")
    _need_out(out, G * Qg * N)
    _check(library().tq_score_stream_probe(cb.handle, G, Qg, _ptr(packed), N, _ptr(out), _stream()),
           "tq_score_stream_probe")
