"""ctypes marshalling for libdsa.so (argument conversion only; no compute here)."""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    """The in-tree build, or the library named by DSA_LIBRARY (for alternative builds)."""
    return os.environ.get("DSA_LIBRARY") or os.path.join(_HERE, "libdsa.so")


if not os.path.exists(lib_path()):
    raise ImportError(
        f"{lib_path()} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python deepseek_sparse_attention_indexer_amd/build.py)")

_lib = C.CDLL(lib_path())

DSA_OK, DSA_ERR_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, -1, -2, -3, -4
DSA_ERR_SCRATCH_LIMIT = -5
STATIC_SCRATCH_BYTES = 64 << 20   # DSA_STATIC_SCRATCH_BYTES of include/dsa.h
ENTRY_TOPK, ENTRY_MLA_DECODE, ENTRY_MLA_PREFILL, ENTRY_DECODE, ENTRY_MLA_BACKWARD = 1, 2, 3, 4, 5
KEY_BF16, KEY_FP8 = 0, 1
KV_BF16, KV_FP8_UNIFORM, KV_FP8_DS_MLA, KV_FP8_UNIFORM_FNUZ = 0, 1, 2, 3


class _Paging(C.Structure):
    _fields_ = [("page_size", C.c_int32), ("_pad0", C.c_int32), ("block_table", C.c_void_p),
                ("bt_stride", C.c_int64), ("req_base", C.c_void_p)]


class _KeyCache(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("_pad0", C.c_int32), ("data", C.c_void_p),
                ("scale", C.c_void_p), ("n_slots", C.c_int64), ("paging", _Paging)]


class _KVCache(C.Structure):
    _fields_ = [("format", C.c_int32), ("d_nope", C.c_int32), ("d_rope", C.c_int32),
                ("_pad0", C.c_int32), ("data", C.c_void_p), ("scales", C.c_void_p),
                ("n_slots", C.c_int64), ("paging", _Paging)]


class _Rows(C.Structure):
    _fields_ = [("T", C.c_int32), ("n_req", C.c_int32), ("row_req", C.c_void_p),
                ("row_len", C.c_void_p), ("n_max", C.c_int32), ("_pad0", C.c_int32)]


class _AttnOpts(C.Structure):
    _fields_ = [("sink", C.c_void_p), ("lse_log2", C.c_int32), ("_pad0", C.c_int32)]


class _Problem(C.Structure):
    _fields_ = [("T", C.c_int32), ("n_max", C.c_int32), ("topk", C.c_int32), ("H", C.c_int32),
                ("n_idx", C.c_int32), ("n_slots", C.c_int32)]


_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_F = C.c_float
_SZ = C.c_size_t

_sigs = {
    "dsa_index_scores": [_P, _I64, _P, _I64, C.POINTER(_KeyCache), C.POINTER(_Rows), _I32, _I32, _F,
                         _P, _I64, _P],
    "dsa_topk": [_P, _I64, C.POINTER(_Rows), _I32, _P, _I64, _P, _P, _SZ, _P],
    "dsa_sparse_mla_decode": [_P, _I64, C.POINTER(_KVCache), _P, _I64, _I32, C.POINTER(_KVCache), _P,
                              _I64, _I32, _I32, _I32, _I32, _I32, _F, _P, _I64, _P,
                              C.POINTER(_AttnOpts), _P, _SZ, _P],
    "dsa_sparse_mla_prefill": [_P, _I64, C.POINTER(_KVCache), _P, _I64, _I32, C.POINTER(_KVCache), _P,
                               _I64, _I32, C.POINTER(_Rows), _I32, _I32, _I32, _F, _P, _I64, _P,
                               C.POINTER(_AttnOpts), _P, _SZ, _P],
    "dsa_sparse_mla_backward": [_P, _I64, C.POINTER(_KVCache), _P, _I64, _I32, C.POINTER(_Rows), _I32,
                                _I32, _I32, _F, _P, _I64, _P, _P, _I64, C.POINTER(_AttnOpts), _P,
                                _I64, _P, _P, _P, _SZ, _P],
    "dsa_decode": [_P, _I64, _P, _I64, _P, _I64, C.POINTER(_KeyCache), C.POINTER(_KVCache),
                   C.POINTER(_Rows), _I32, _I32, _I32, _I32, _I32, _I32, _F, _F, _P, _I64, _P,
                   C.POINTER(_AttnOpts), _P, _I64, _P, _P, _SZ, _P],
    "dsa_decode_static": [_P, _I64, _P, _I64, _P, _I64, C.POINTER(_KeyCache), C.POINTER(_KVCache),
                          C.POINTER(_Rows), _I32, _I32, _I32, _I32, _I32, _I32, _F, _F, _P, _I64, _P,
                          C.POINTER(_AttnOpts), _P, _I64, _P, _P],
    "dsa_workspace_init": [_P, _SZ, _P],
    "dsa_kv_cache_write": [_P, _I64, _I32, _P, C.POINTER(_KVCache), _P],
    "dsa_key_cache_write": [_P, _I64, _I32, _P, C.POINTER(_KeyCache), _I32, _P],
}
for _name, _args in _sigs.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = C.c_int32
_lib.dsa_workspace_size.argtypes = [_I32, C.POINTER(_Problem)]
_lib.dsa_workspace_size.restype = _SZ
_lib.dsa_status_string.argtypes = [_I32]
_lib.dsa_status_string.restype = C.c_char_p
_lib.dsa_abi_version.argtypes = []
_lib.dsa_abi_version.restype = _I32
ABI_VERSION = 7   # the signatures above
if _lib.dsa_abi_version() != ABI_VERSION:
    raise ImportError(f"{lib_path()} has ABI version {_lib.dsa_abi_version()}, this binding needs "
                      f"{ABI_VERSION}: rebuild the library")


class _KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 40), ("count", C.c_int32), ("total_ms", C.c_float),
                ("min_ms", C.c_float), ("max_ms", C.c_float)]


_lib.dsa_profile_enable.argtypes = [_I32]
_lib.dsa_profile_enable.restype = _I32
_lib.dsa_profile_collect.argtypes = [C.POINTER(_KernelTime), _I32]
_lib.dsa_profile_collect.restype = _I32
_lib.dsa_launch_override.argtypes = [_I32, _I32]
_lib.dsa_launch_override.restype = _I32


class DSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dsa_status_string(status)} (status {status})")


def dsa_status_string(status: int) -> str:
    return _lib.dsa_status_string(int(status)).decode()


def dsa_abi_version() -> int:
    return int(_lib.dsa_abi_version())


def dsa_profile_enable(on: bool):
    _check(_lib.dsa_profile_enable(1 if on else 0), "dsa_profile_enable")


def dsa_launch_override(head_tiles: int = 0, n_split: int = 0):
    """Force the attention launch plan of later calls (0 = the compiled-in table's choice);
    (0, 0) restores the table. See include/dsa.h."""
    _check(_lib.dsa_launch_override(int(head_tiles), int(n_split)), "dsa_launch_override")


def dsa_profile_collect(max_entries: int = 32) -> dict:
    """{kernel name: {"count", "total_ms", "min_ms", "max_ms"}} of the launches recorded while
    profiling was enabled (waits for them)."""
    buf = (_KernelTime * max_entries)()
    n = _lib.dsa_profile_collect(buf, max_entries)
    if n < 0:
        raise DSAError(n, "dsa_profile_collect")
    return {buf[i].name.decode(): {"count": buf[i].count, "total_ms": buf[i].total_ms,
                                   "min_ms": buf[i].min_ms, "max_ms": buf[i].max_ms} for i in range(n)}


def _check(status: int, where: str):
    if status != DSA_OK:
        raise DSAError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _ld(t) -> int:
    """Row stride (elements) of a row-major [rows, ...] tensor. A single row's leading stride is
    free in torch (e.g. a broadcast view gives 0); the library then gets one full row."""
    if t is None:
        return 0
    if t.dim() >= 1 and t.shape[0] == 1:
        row = 1
        for d in t.shape[1:]:
            row *= int(d)
        return max(int(t.stride(0)), row)
    return int(t.stride(0))


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dev(t: Optional[torch.Tensor], name: str):
    if t is not None and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _paging(page_size, block_table, req_base) -> _Paging:
    _dev(block_table, "block_table")
    _dev(req_base, "req_base")
    stride = _ld(block_table) if block_table is not None else 0
    return _Paging(int(page_size), 0, _ptr(block_table), stride, _ptr(req_base))


class KeyCache:
    """Indexer key cache: data [slots, di] (bf16 or uint8 fp8 bytes), fp8 scale [slots] fp32."""

    def __init__(self, data: torch.Tensor, scale: Optional[torch.Tensor] = None, page_size: int = 1,
                 block_table: Optional[torch.Tensor] = None, req_base: Optional[torch.Tensor] = None):
        _dev(data, "data")
        _dev(scale, "scale")
        self.keep = (data, scale, block_table, req_base)
        self.dtype = KEY_FP8 if data.dtype == torch.uint8 else KEY_BF16
        self.c = _KeyCache(self.dtype, 0, _ptr(data), _ptr(scale), int(data.shape[0]),
                           _paging(page_size, block_table, req_base))


class KVCache:
    """Latent cache. fmt 'bf16': data [slots, D] bf16; 'fp8_uniform' (OCP e4m3) and
    'fp8_uniform_fnuz' (fnuz e4m3): uint8 [slots, D] + scales [slots, D/64] fp32; 'fp8_ds_mla':
    uint8 [pages, page_size * 584]."""

    def __init__(self, fmt: str, data: torch.Tensor, d_nope: int, d_rope: int, page_size: int = 1,
                 block_table: Optional[torch.Tensor] = None, req_base: Optional[torch.Tensor] = None,
                 scales: Optional[torch.Tensor] = None):
        _dev(data, "data")
        _dev(scales, "scales")
        self.keep = (data, scales, block_table, req_base)
        f = {"bf16": KV_BF16, "fp8_uniform": KV_FP8_UNIFORM, "fp8_ds_mla": KV_FP8_DS_MLA,
             "fp8_uniform_fnuz": KV_FP8_UNIFORM_FNUZ}[fmt]
        n_slots = int(data.shape[0]) * (page_size if fmt == "fp8_ds_mla" else 1)
        self.c = _KVCache(f, int(d_nope), int(d_rope), 0, _ptr(data), _ptr(scales), n_slots,
                          _paging(page_size, block_table, req_base))


class Rows:
    """Query rows: row_len [T] int32 (device), optional row_req [T] int32, n_req, n_max (host)."""

    def __init__(self, row_len: torch.Tensor, n_req: int, n_max: int,
                 row_req: Optional[torch.Tensor] = None):
        _dev(row_len, "row_len")
        _dev(row_req, "row_req")
        self.keep = (row_len, row_req)
        self.T = int(row_len.shape[0])
        self.c = _Rows(self.T, int(n_req), _ptr(row_req), _ptr(row_len), int(n_max), 0)


def _opts(sink, lse_log2: bool):
    """Attention options struct (None when both are defaults); sink: fp32 [H] device tensor."""
    if sink is None and not lse_log2:
        return None
    _dev(sink, "sink")
    return C.byref(_AttnOpts(_ptr(sink), 1 if lse_log2 else 0, 0))


def dsa_workspace_size(entry: int, T: int = 0, n_max: int = 0, topk: int = 0, H: int = 0,
                       n_idx: int = 0, n_slots: int = 0) -> int:
    p = _Problem(int(T), int(n_max), int(topk), int(H), int(n_idx), int(n_slots))
    n = int(_lib.dsa_workspace_size(int(entry), C.byref(p)))
    if n == (1 << 64) - 1:
        raise DSAError(DSA_ERR_ARG, "dsa_workspace_size")
    return n


def dsa_workspace_init(ws: torch.Tensor, stream=None):
    _check(_lib.dsa_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "dsa_workspace_init")


class Workspace:
    """A device byte buffer initialised for the library (grown on demand)."""

    def __init__(self, nbytes: int = 0, device="cuda"):
        self.device = device
        self.buf = None
        self.ensure(nbytes)

    def ensure(self, nbytes: int):
        nbytes = max(int(nbytes), 1 << 23)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            dsa_workspace_init(self.buf)
        return self

    @property
    def ptr(self):
        return _ptr(self.buf)

    @property
    def nbytes(self) -> int:
        return self.buf.numel()


def dsa_kv_cache_write(src, slots, kv: KVCache, stream=None):
    """Write bf16 rows src [n, D] (row stride src.stride(0)) into the latent cache at slots [n]
    (int32 device; -1 skips), in the cache's format."""
    _check(_lib.dsa_kv_cache_write(_ptr(src), _ld(src), int(src.shape[0]), _ptr(slots),
                                   C.byref(kv.c), _stream(stream)), "dsa_kv_cache_write")


def dsa_key_cache_write(src, slots, keys: KeyCache, di: int, stream=None):
    """Write bf16 index keys src [n, di] into the key cache at slots [n] (bf16 copy, or fp8 with
    one scale per token)."""
    _check(_lib.dsa_key_cache_write(_ptr(src), _ld(src), int(src.shape[0]), _ptr(slots),
                                    C.byref(keys.c), int(di), _stream(stream)), "dsa_key_cache_write")


def dsa_index_scores(q_idx, w, keys: KeyCache, rows: Rows, Hi: int, di: int, index_scale: float,
                     logits, stream=None):
    _check(_lib.dsa_index_scores(_ptr(q_idx), _ld(q_idx), _ptr(w), _ld(w),
                                 C.byref(keys.c), C.byref(rows.c), int(Hi), int(di),
                                 float(index_scale), _ptr(logits), _ld(logits),
                                 _stream(stream)), "dsa_index_scores")


def dsa_topk(logits, rows: Rows, topk: int, indices, lens, ws: Optional[Workspace], stream=None):
    _check(_lib.dsa_topk(_ptr(logits), _ld(logits), C.byref(rows.c), int(topk),
                         _ptr(indices), _ld(indices), _ptr(lens),
                         ws.ptr if ws else None, ws.nbytes if ws else 0, _stream(stream)),
           "dsa_topk")


def dsa_sparse_mla_decode(q, kv: KVCache, idx, extra_kv: Optional[KVCache], extra_idx, B: int,
                          H: int, d_qk: int, d_v: int, softmax_scale: float, out, lse,
                          ws: Optional[Workspace], stream=None, sink=None, lse_log2: bool = False):
    n_idx = int(idx.shape[1]) if idx is not None else 0
    n_extra = int(extra_idx.shape[1]) if extra_idx is not None else 0
    _check(_lib.dsa_sparse_mla_decode(
        _ptr(q), _ld(q), C.byref(kv.c), _ptr(idx), _ld(idx) if idx is not None else 0,
        n_idx, C.byref(extra_kv.c) if extra_kv else None, _ptr(extra_idx),
        _ld(extra_idx) if extra_idx is not None else 0, n_extra, int(B), int(H), int(d_qk),
        int(d_v), float(softmax_scale), _ptr(out), _ld(out), _ptr(lse), _opts(sink, lse_log2),
        ws.ptr if ws else None, ws.nbytes if ws else 0, _stream(stream)), "dsa_sparse_mla_decode")


def dsa_sparse_mla_prefill(q, kv: KVCache, idx, extra_kv: Optional[KVCache], extra_idx, rows: Rows,
                           H: int, d_qk: int, d_v: int, softmax_scale: float, out, lse,
                           ws: Optional[Workspace] = None, stream=None, sink=None,
                           lse_log2: bool = False):
    n_idx = int(idx.shape[1]) if idx is not None else 0
    n_extra = int(extra_idx.shape[1]) if extra_idx is not None else 0
    _check(_lib.dsa_sparse_mla_prefill(
        _ptr(q), _ld(q), C.byref(kv.c), _ptr(idx), _ld(idx) if idx is not None else 0,
        n_idx, C.byref(extra_kv.c) if extra_kv else None, _ptr(extra_idx),
        _ld(extra_idx) if extra_idx is not None else 0, n_extra, C.byref(rows.c), int(H),
        int(d_qk), int(d_v), float(softmax_scale), _ptr(out), _ld(out), _ptr(lse),
        _opts(sink, lse_log2), ws.ptr if ws else None, ws.nbytes if ws else 0, _stream(stream)),
        "dsa_sparse_mla_prefill")


def dsa_sparse_mla_backward(q, kv: KVCache, idx, rows: Rows, H: int, d_qk: int, d_v: int,
                            softmax_scale: float, out, lse, dout, dq, dkv, ws: "Workspace", dsink=None,
                            stream=None, sink=None, lse_log2: bool = False):
    n_idx = int(idx.shape[1]) if idx is not None else 0
    _check(_lib.dsa_sparse_mla_backward(
        _ptr(q), _ld(q), C.byref(kv.c), _ptr(idx), _ld(idx) if idx is not None else 0, n_idx,
        C.byref(rows.c), int(H), int(d_qk), int(d_v), float(softmax_scale), _ptr(out), _ld(out),
        _ptr(lse), _ptr(dout), _ld(dout), _opts(sink, lse_log2), _ptr(dq), _ld(dq), _ptr(dkv),
        _ptr(dsink), ws.ptr if ws else None, ws.nbytes if ws else 0, _stream(stream)),
        "dsa_sparse_mla_backward")


def dsa_decode(q, q_idx, w, keys: KeyCache, kv: KVCache, rows: Rows, H: int, d_qk: int, d_v: int,
               Hi: int, di: int, topk: int, index_scale: float, softmax_scale: float, out, lse,
               idx_out, lens_out, ws: Workspace, stream=None, sink=None, lse_log2: bool = False):
    _check(_lib.dsa_decode(
        _ptr(q), _ld(q), _ptr(q_idx), _ld(q_idx), _ptr(w), _ld(w),
        C.byref(keys.c), C.byref(kv.c), C.byref(rows.c), int(H), int(d_qk), int(d_v), int(Hi), int(di),
        int(topk), float(index_scale), float(softmax_scale), _ptr(out), _ld(out), _ptr(lse),
        _opts(sink, lse_log2), _ptr(idx_out), _ld(idx_out) if idx_out is not None else 0, _ptr(lens_out),
        ws.ptr, ws.nbytes, _stream(stream)), "dsa_decode")


def dsa_decode_static(q, q_idx, w, keys: KeyCache, kv: KVCache, rows: Rows, H: int, d_qk: int, d_v: int,
                      Hi: int, di: int, topk: int, index_scale: float, softmax_scale: float, out, lse,
                      idx_out, lens_out, stream=None, sink=None, lse_log2: bool = False):
    """dsa_decode on the library's static device scratch (no workspace argument)."""
    _check(_lib.dsa_decode_static(
        _ptr(q), _ld(q), _ptr(q_idx), _ld(q_idx), _ptr(w), _ld(w),
        C.byref(keys.c), C.byref(kv.c), C.byref(rows.c), int(H), int(d_qk), int(d_v), int(Hi), int(di),
        int(topk), float(index_scale), float(softmax_scale), _ptr(out), _ld(out), _ptr(lse),
        _opts(sink, lse_log2), _ptr(idx_out), _ld(idx_out) if idx_out is not None else 0, _ptr(lens_out),
        _stream(stream)), "dsa_decode_static")
