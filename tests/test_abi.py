"""The C ABI on the CPU: the library loads, exports every entry point include/dsa.h declares,
and rejects bad arguments with the documented status before touching the GPU (no compute
call is made here; the pointers are aligned dummies that are never dereferenced)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

dsa = pytest.importorskip("deepseek_sparse_attention_indexer_amd")
from deepseek_sparse_attention_indexer_amd import _binding as B  # noqa: E402

FAKE = C.c_void_p(0x10000)      # aligned, never dereferenced on the host
FAKE_ODD = C.c_void_p(0x10004)  # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"dsa_index_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
            "dsa_decode", "dsa_workspace_size", "dsa_workspace_init", "dsa_status_string"} <= set(names)
    lib = C.CDLL(B.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert dsa.dsa_abi_version() >= 1
    for s in (0, -1, -2, -3, -4):
        assert dsa.dsa_status_string(s) and dsa.dsa_status_string(s) != "unknown status"
    assert dsa.dsa_status_string(7) == "unknown status"


def _rows(T=1, n_max=1000, n_req=1, row_len=FAKE):
    return B._Rows(T, n_req, None, row_len, n_max, 0)


def _keys(dtype=B.KEY_BF16, data=FAKE, scale=None, page=64, bt=FAKE, stride=16, n_slots=1024):
    return B._KeyCache(dtype, 0, data, scale, n_slots, B._Paging(page, 0, bt, stride, None))


def _kv(fmt=B.KV_BF16, d_nope=512, d_rope=64, data=FAKE, scales=None, page=64, n_slots=1024):
    return B._KVCache(fmt, d_nope, d_rope, 0, data, scales, n_slots, B._Paging(page, 0, FAKE, 16, None))


def scores(**kw):
    a = dict(q_idx=FAKE, ld_q=64 * 128, w=FAKE, ld_w=64, keys=_keys(), rows=_rows(), Hi=64, di=128,
             scale=1.0, logits=FAKE, ld_logits=1024)
    a.update(kw)
    return B._lib.dsa_index_scores(a["q_idx"], a["ld_q"], a["w"], a["ld_w"], C.byref(a["keys"]),
                                   C.byref(a["rows"]), a["Hi"], a["di"], a["scale"], a["logits"],
                                   a["ld_logits"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_idx=None), B.DSA_ERR_ARG),
    (dict(q_idx=FAKE_ODD), B.DSA_ERR_ARG),
    (dict(ld_q=64 * 128 - 8), B.DSA_ERR_ARG),
    (dict(ld_q=64 * 128 + 4), B.DSA_ERR_ARG),
    (dict(w=None), B.DSA_ERR_ARG),
    (dict(ld_w=63), B.DSA_ERR_ARG),
    (dict(logits=None), B.DSA_ERR_ARG),
    (dict(ld_logits=999), B.DSA_ERR_ARG),
    (dict(Hi=0), B.DSA_ERR_ARG),
    (dict(Hi=65), B.DSA_ERR_UNSUPPORTED),
    (dict(di=96), B.DSA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), B.DSA_ERR_ARG),
    (dict(keys=_keys(dtype=B.KEY_FP8, scale=None)), B.DSA_ERR_ARG),
    (dict(keys=_keys(dtype=7)), B.DSA_ERR_UNSUPPORTED),
    (dict(keys=_keys(page=0)), B.DSA_ERR_ARG),
    (dict(keys=_keys(bt=None)), B.DSA_ERR_ARG),       # no table and no req_base
    (dict(keys=_keys(n_slots=1000)), B.DSA_ERR_ARG),  # not whole pages
    (dict(rows=_rows(T=-1)), B.DSA_ERR_ARG),
    (dict(rows=_rows(row_len=None)), B.DSA_ERR_ARG),
    (dict(rows=_rows(n_req=0)), B.DSA_ERR_ARG),
    (dict(rows=_rows(T=70000, n_req=70000)), B.DSA_ERR_UNSUPPORTED),
    (dict(rows=_rows(T=3, n_req=2)), B.DSA_ERR_ARG),   # row t is request t, but only 2 requests
])
def test_index_scores_rejects(kw, status):
    assert scores(**kw) == status


def test_index_scores_empty_rows_is_a_no_op():
    assert scores(rows=_rows(T=0), q_idx=None, w=None, logits=None) == B.DSA_OK


def topk(**kw):
    a = dict(logits=FAKE, ld=1024, rows=_rows(), k=128, idx=FAKE, ld_idx=128, lens=FAKE, ws=None, wsb=0)
    a.update(kw)
    return B._lib.dsa_topk(a["logits"], a["ld"], C.byref(a["rows"]), a["k"], a["idx"], a["ld_idx"],
                           a["lens"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), B.DSA_ERR_ARG),
    (dict(k=70000, ld_idx=70000), B.DSA_ERR_UNSUPPORTED),
    (dict(logits=None), B.DSA_ERR_ARG),
    (dict(ld=999), B.DSA_ERR_ARG),
    (dict(idx=None), B.DSA_ERR_ARG),
    (dict(ld_idx=127), B.DSA_ERR_ARG),
    (dict(lens=None), B.DSA_ERR_ARG),
    # long rows need the workspace
    (dict(rows=_rows(n_max=100000), ld=100000), B.DSA_ERR_WORKSPACE),
    (dict(rows=_rows(n_max=100000), ld=100000, ws=FAKE, wsb=1024), B.DSA_ERR_WORKSPACE),
])
def test_topk_rejects(kw, status):
    assert topk(**kw) == status


def mla(**kw):
    a = dict(q=FAKE, ld_q=16 * 576, kv=_kv(), idx=FAKE, ld_idx=128, n_idx=128, extra_kv=None,
             extra_idx=None, ld_extra=0, n_extra=0, B=1, H=16, d_qk=576, d_v=512, scale=0.04,
             out=FAKE, ld_out=16 * 512, lse=None, opts=None, ws=None, wsb=0)
    a.update(kw)
    return B._lib.dsa_sparse_mla_decode(
        a["q"], a["ld_q"], C.byref(a["kv"]), a["idx"], a["ld_idx"], a["n_idx"],
        C.byref(a["extra_kv"]) if a["extra_kv"] is not None else None, a["extra_idx"], a["ld_extra"],
        a["n_extra"], a["B"], a["H"], a["d_qk"], a["d_v"], a["scale"], a["out"], a["ld_out"], a["lse"],
        C.byref(a["opts"]) if a["opts"] is not None else None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=0), B.DSA_ERR_ARG),
    (dict(H=8, ld_q=8 * 576 - 8, ld_out=8 * 512), B.DSA_ERR_ARG),    # q row shorter than 8 heads
    (dict(d_v=256, ld_out=16 * 256), B.DSA_ERR_UNSUPPORTED),
    (dict(d_qk=640, ld_q=16 * 640), B.DSA_ERR_UNSUPPORTED),
    (dict(q=None), B.DSA_ERR_ARG),
    (dict(q=FAKE_ODD), B.DSA_ERR_ARG),
    (dict(out=None), B.DSA_ERR_ARG),
    (dict(ld_out=100), B.DSA_ERR_ARG),
    (dict(idx=None), B.DSA_ERR_ARG),
    (dict(ld_idx=100), B.DSA_ERR_ARG),
    (dict(kv=_kv(d_nope=448)), B.DSA_ERR_ARG),                   # 448 + 64 != d_qk
    (dict(kv=_kv(fmt=B.KV_FP8_UNIFORM)), B.DSA_ERR_ARG),         # uniform pool without scales
    (dict(kv=_kv(fmt=B.KV_FP8_DS_MLA)), B.DSA_ERR_UNSUPPORTED),  # ds_mla is 448 + 64 only
    (dict(kv=_kv(fmt=5)), B.DSA_ERR_UNSUPPORTED),
    (dict(n_extra=10, extra_idx=FAKE, ld_extra=10, extra_kv=None), B.DSA_ERR_ARG),
    (dict(n_extra=10, extra_idx=FAKE, ld_extra=10,
          extra_kv=_kv(fmt=B.KV_FP8_UNIFORM, scales=FAKE)), B.DSA_ERR_UNSUPPORTED),  # mixed formats
    (dict(scale=float("inf")), B.DSA_ERR_ARG),
    (dict(kv=_kv(fmt=B.KV_FP8_UNIFORM_FNUZ)), B.DSA_ERR_ARG),    # fnuz pool without scales
    (dict(n_extra=10, extra_idx=FAKE, ld_extra=10, kv=_kv(fmt=B.KV_FP8_UNIFORM, scales=FAKE),
          extra_kv=_kv(fmt=B.KV_FP8_UNIFORM_FNUZ, scales=FAKE)), B.DSA_ERR_UNSUPPORTED),  # OCP + fnuz
    (dict(opts=B._AttnOpts(None, 2, 0)), B.DSA_ERR_ARG),         # lse base flag is 0 or 1
    (dict(opts=B._AttnOpts(C.c_void_p(0x10002), 0, 0)), B.DSA_ERR_ARG),   # misaligned sink
    # a 2048-entry list over 64 heads splits across workgroups and needs the workspace
    (dict(H=64, ld_q=64 * 576, ld_out=64 * 512, n_idx=2048, ld_idx=2048), B.DSA_ERR_WORKSPACE),
])
def test_sparse_mla_rejects(kw, status):
    assert mla(**kw) == status


def test_workspace_sizes():
    hdr = dsa.dsa_workspace_size(dsa.ENTRY_TOPK, T=1, n_max=1000, topk=128)
    assert hdr > 0
    assert dsa.dsa_workspace_size(dsa.ENTRY_TOPK, T=1, n_max=1 << 20, topk=2048) >= hdr + 8 * (1 << 20)
    assert dsa.dsa_workspace_size(dsa.ENTRY_MLA_PREFILL, T=10, H=64, n_idx=2048) == 0
    dec = dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=1, n_max=131072, topk=2048, H=64)
    assert dec >= hdr + 131072 * 4
    with pytest.raises(dsa.DSAError):
        dsa.dsa_workspace_size(9, T=1)
    # a head count that is not whole 16-head tiles is padded inside: 8 heads split like 16
    assert dsa.dsa_workspace_size(dsa.ENTRY_MLA_DECODE, T=1, H=8, n_idx=2048) == \
        dsa.dsa_workspace_size(dsa.ENTRY_MLA_DECODE, T=1, H=16, n_idx=2048)
    assert dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=2, H=40, n_idx=256) == \
        dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=2, H=64, n_idx=256)
    with pytest.raises(dsa.DSAError):
        dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=1, H=129, n_idx=64)
    # the backward's owner map: one int32 per cache slot in whole 16-byte words, 256-aligned
    base = dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=2, H=64, n_idx=256)
    for n_slots, extra in ((1, 256), (64, 256), (65, 512), (4096, 16384), (4099, 16640)):
        assert dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=2, H=64, n_idx=256, n_slots=n_slots) == base + extra
    with pytest.raises(dsa.DSAError):
        dsa.dsa_workspace_size(dsa.ENTRY_MLA_BACKWARD, T=1, H=64, n_idx=64, n_slots=-1)


def test_launch_override():
    """The plan override is checked, moves the workspace size with the plan it forces, and a
    head-tile count that does not divide the heads is refused before any launch."""
    for bad in ((3, 0), (-1, 0), (8, 0), (0, -1)):
        with pytest.raises(dsa.DSAError):
            dsa.dsa_launch_override(*bad)
    base = dsa.dsa_workspace_size(dsa.ENTRY_MLA_DECODE, T=1, H=64, n_idx=2048)
    fused = dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=1, n_max=131072, topk=2048, H=64)
    try:
        dsa.dsa_launch_override(0, 8)       # 8 splits instead of the table's: fewer partials
        assert dsa.dsa_workspace_size(dsa.ENTRY_MLA_DECODE, T=1, H=64, n_idx=2048) < base
        assert dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=1, n_max=131072, topk=2048, H=64) < fused
        dsa.dsa_launch_override(4, 0)       # 64-head workgroups cannot serve 16 heads
        assert mla() == B.DSA_ERR_UNSUPPORTED
        dsa.dsa_launch_override(2, 0)       # 32-head workgroups: 48 heads are three 16-head tiles
        assert mla(H=48, ld_q=48 * 576, ld_out=48 * 512) == B.DSA_ERR_UNSUPPORTED
    finally:
        dsa.dsa_launch_override(0, 0)
    assert dsa.dsa_workspace_size(dsa.ENTRY_MLA_DECODE, T=1, H=64, n_idx=2048) == base


def test_workspace_init_rejects():
    assert B._lib.dsa_workspace_init(None, 1 << 24, None) == B.DSA_ERR_ARG
    assert B._lib.dsa_workspace_init(FAKE, 16, None) == B.DSA_ERR_WORKSPACE


def decode_static(**kw):
    a = dict(q=FAKE, ld_q=64 * 576, q_idx=FAKE, ld_q_idx=64 * 128, w=FAKE, ld_w=64, keys=_keys(n_slots=1 << 22),
             kv=_kv(n_slots=1 << 22), rows=_rows(n_max=131072), H=64, d_qk=576, d_v=512, Hi=64, di=128,
             topk=2048, index_scale=1.0, scale=0.04, out=FAKE, ld_out=64 * 512, lse=None, opts=None,
             idx_out=None, ld_idx_out=0, lens_out=None)
    a.update(kw)
    return B._lib.dsa_decode_static(
        a["q"], a["ld_q"], a["q_idx"], a["ld_q_idx"], a["w"], a["ld_w"], C.byref(a["keys"]), C.byref(a["kv"]),
        C.byref(a["rows"]), a["H"], a["d_qk"], a["d_v"], a["Hi"], a["di"], a["topk"], a["index_scale"],
        a["scale"], a["out"], a["ld_out"], a["lse"], C.byref(a["opts"]) if a["opts"] is not None else None,
        a["idx_out"], a["ld_idx_out"], a["lens_out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.DSA_ERR_ARG),
    (dict(topk=0), B.DSA_ERR_ARG),
    (dict(H=0), B.DSA_ERR_ARG),
    (dict(Hi=65), B.DSA_ERR_UNSUPPORTED),
    (dict(idx_out=FAKE, ld_idx_out=2047), B.DSA_ERR_ARG),        # idx_out row shorter than topk
    # more scratch than the static array holds: 64 rows of 1M candidates
    (dict(rows=_rows(T=64, n_req=64, n_max=1 << 20)), B.DSA_ERR_SCRATCH_LIMIT),
])
def test_decode_static_rejects_before_any_hip_call(kw, status):
    """Argument and size checks come before the scratch lookup (no GPU here: a HIP call would
    fail with DSA_ERR_HIP instead)."""
    assert decode_static(**kw) == status


def test_decode_static_limit_matches_the_workspace_size():
    need_1m = dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=1, n_max=1 << 20, topk=2048, H=64)
    assert need_1m <= dsa.STATIC_SCRATCH_BYTES       # one 1M-candidate row fits
    need_big = dsa.dsa_workspace_size(dsa.ENTRY_DECODE, T=64, n_max=1 << 20, topk=2048, H=64)
    assert need_big > dsa.STATIC_SCRATCH_BYTES
    assert dsa.dsa_status_string(dsa.DSA_ERR_SCRATCH_LIMIT) != "unknown status"
