"""Seeded workload generators for the DSA layer hot path (scores -> top-k -> sparse MLA).

Every tensor is drawn from numpy's PCG64 with the sub-stream ``default_rng([seed, tensor_id])``
and stored in the byte format the caches use:

* bf16 values as their uint16 bit patterns (round-to-nearest-even from float32, done by
  torch's dtype cast);
* fp8 e4m3 (OCP ``float8_e4m3fn``) as uint8 bytes, encoded once by torch's dtype cast after
  clamping to +-448 (the generator's quantisation is data preparation, not the method);
* the packed ``fp8_ds_mla`` page layout of aiter PR 4382 "Paged Sparse Attention Gluon Kernel",
  section "Packed fp8 fp8_ds_mla - 3D": per page, ``page_size`` tokens x 576 data bytes
  (448 NoPE fp8 + 64 RoPE bf16) followed by ``page_size`` x 8 scale bytes (7 UE8M0 exponents,
  one per 64 NoPE channels, and one pad byte);
* the uniform fp8 pool of the same page's section "Uniform fp8 pool - 2D": ``[slots, D]`` fp8
  with one fp32 scale per 64 channels, OCP bytes, or fnuz bytes (``float8_e4m3fnuz``, bias 8,
  torch's cast after clamping to +-240; section "fp8 flavors");
* DeepSeek-V4 attention sinks: one logit per head, drawn N(3, 2^2) (the pages give no
  distribution; with unit-variance logits over ~100 rows this puts the sink's share of the
  softmax mass anywhere from negligible to most of it).

Page tables are random permutations of physical pages ("shuffled page table").
Nothing here scores, selects, attends or dequantises.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0
FP8_FNUZ_MAX = 240.0
DS_MLA_NOPE = 448
DS_MLA_ROPE = 64
DS_MLA_DATA_BYTES = 576          # 448 fp8 + 64 * 2 bytes of bf16
DS_MLA_SCALE_BYTES = 8           # 7 UE8M0 exponents + 1 pad
DS_MLA_TOKEN_BYTES = DS_MLA_DATA_BYTES + DS_MLA_SCALE_BYTES  # 584


# --------------------------------------------------------------------------- containers
@dataclass
class KeyPool:
    """Lightning-indexer key cache, paged like the latent cache.

    dtype "bf16": data uint16 [slots, di]; dtype "fp8": data uint8 [slots, di] and a float32
    per-slot scale [slots]. A logical position s of request b lives in slot
    block_table[b, s // page_size] * page_size + s % page_size, or req_base[b] + s when there
    is no block table.
    """
    dtype: str
    data: np.ndarray
    scale: Optional[np.ndarray]
    page_size: int
    block_table: Optional[np.ndarray]
    req_base: Optional[np.ndarray]

    @property
    def di(self) -> int:
        return int(self.data.shape[1])


@dataclass
class KVPool:
    """Latent (MLA) KV cache.

    fmt "bf16":        data uint16 [slots, D]            (D = d_nope + d_rope, e.g. 512 + 64)
    fmt "fp8_uniform": data uint8  [slots, D], scales float32 [slots, D // 64]
    fmt "fp8_uniform_fnuz": the same with fnuz e4m3 bytes
    fmt "fp8_ds_mla":  data uint8  [pages, page_size * 584] (block-planar page layout)
    Addressing as for KeyPool (for fp8_ds_mla the slot splits into page = slot // page_size and
    in-page position = slot % page_size).
    """
    fmt: str
    data: np.ndarray
    scales: Optional[np.ndarray]
    page_size: int
    block_table: Optional[np.ndarray]
    req_base: Optional[np.ndarray]
    d_nope: int
    d_rope: int

    @property
    def dim(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def n_slots(self) -> int:
        if self.fmt == "fp8_ds_mla":
            return int(self.data.shape[0]) * self.page_size
        return int(self.data.shape[0])


@dataclass
class DSAProblem:
    """One batch of the DSA layer.

    Row t (a query token) belongs to request row_req[t] and sees the candidates
    [0, row_len[t]) of that request. q: uint16 [T, H, d_qk] (bf16); q_idx: uint16 [T, Hi, di];
    w: float32 [T, Hi]. Attention-only workloads carry explicit index lists instead of an
    indexer (idx_main [T, n_main], optionally idx_extra [T, n_extra] into a second pool).
    """
    name: str
    T: int
    H: int
    d_qk: int
    d_v: int
    topk: int
    q: np.ndarray
    kv: KVPool
    row_req: np.ndarray
    row_len: np.ndarray
    n_req: int
    softmax_scale: float
    Hi: int = 0
    di: int = 0
    q_idx: Optional[np.ndarray] = None
    w: Optional[np.ndarray] = None
    kpool: Optional[KeyPool] = None
    index_scale: float = 1.0
    idx_main: Optional[np.ndarray] = None
    extra_kv: Optional[KVPool] = None
    idx_extra: Optional[np.ndarray] = None
    sink: Optional[np.ndarray] = None       # float32 [H] per-head sink logit (DeepSeek-V4)
    lse_log2: bool = False                  # lse in base 2
    meta: dict = field(default_factory=dict)

    @property
    def n_max(self) -> int:
        return int(self.row_len.max()) if self.T else 0


# --------------------------------------------------------------------------- primitives
def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, tensor_id])


def _normal(seed: int, tid: int, shape, chunk: int = 1 << 26) -> np.ndarray:
    """float32 N(0,1) of the given shape, drawn in chunks from one sub-stream."""
    rng = _rng(seed, tid)
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp8_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn bytes (torch cast, RNE) after saturating to +-448."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def to_fp8_fnuz_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> fnuz e4m3 bytes (torch cast, RNE) after saturating to +-240."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_FNUZ_MAX, FP8_FNUZ_MAX)
    return torch.from_numpy(x).to(torch.float8_e4m3fnuz).view(torch.uint8).numpy()


def _bf16_normal(seed, tid, shape):
    return to_bf16_bits(_normal(seed, tid, shape))


def shuffled_pages(seed: int, tid: int, n_req: int, pages_per_req, n_phys: Optional[int] = None,
                   width: Optional[int] = None) -> tuple[np.ndarray, int]:
    """Block table int32 [n_req, width]: request b's logical pages map to distinct physical
    pages drawn from a random permutation; unused entries point at page 0."""
    pages_per_req = np.broadcast_to(np.asarray(pages_per_req, dtype=np.int64), (n_req,))
    total = int(pages_per_req.sum())
    n_phys = total if n_phys is None else n_phys
    width = int(pages_per_req.max()) if width is None else width
    perm = _rng(seed, tid).permutation(n_phys)[:total].astype(np.int32)
    bt = np.zeros((n_req, max(width, 1)), dtype=np.int32)
    o = 0
    for b in range(n_req):
        k = int(pages_per_req[b])
        bt[b, :k] = perm[o:o + k]
        o += k
    return bt, n_phys


def pack_ds_mla(values: np.ndarray, page_size: int) -> np.ndarray:
    """Quantise float32 [slots, 512] (448 NoPE + 64 RoPE) into fp8_ds_mla pages.

    NoPE: per 64-channel group, exponent e = ceil(log2(amax / 448)) + 127 (UE8M0, clamped to
    [1, 254]); bytes = fp8(x / 2^(e-127)). RoPE: bf16 bits, little-endian, after the NoPE
    bytes. Returns uint8 [slots // page_size, page_size * 584].
    """
    slots = values.shape[0]
    assert slots % page_size == 0 and values.shape[1] == DS_MLA_NOPE + DS_MLA_ROPE
    n_pages = slots // page_size
    out = np.zeros((n_pages, page_size * DS_MLA_TOKEN_BYTES), dtype=np.uint8)
    step = max(1, (1 << 22) // (page_size * 512))
    for p0 in range(0, n_pages, step):
        p1 = min(n_pages, p0 + step)
        v = values[p0 * page_size:p1 * page_size]
        nope = v[:, :DS_MLA_NOPE].reshape(-1, 7, 64)
        amax = np.abs(nope).max(axis=2).astype(np.float64)
        e = np.where(amax > 0, np.ceil(np.log2(np.maximum(amax, 1e-300) / FP8_MAX)) + 127, 127)
        e = np.clip(e, 1, 254).astype(np.int64)
        scale = np.ldexp(1.0, e - 127).astype(np.float32)
        q8 = to_fp8_bytes((nope / scale[:, :, None]).reshape(-1, DS_MLA_NOPE))
        rope = to_bf16_bits(v[:, DS_MLA_NOPE:]).view(np.uint8).reshape(-1, 2 * DS_MLA_ROPE)
        npg = p1 - p0
        data = np.concatenate([q8, rope], axis=1).reshape(npg, page_size * DS_MLA_DATA_BYTES)
        sc = np.zeros((npg * page_size, DS_MLA_SCALE_BYTES), dtype=np.uint8)
        sc[:, :7] = e.reshape(-1, 7).astype(np.uint8)
        out[p0:p1, :page_size * DS_MLA_DATA_BYTES] = data
        out[p0:p1, page_size * DS_MLA_DATA_BYTES:] = sc.reshape(npg, page_size * DS_MLA_SCALE_BYTES)
    return out


def quant_uniform(values: np.ndarray, fnuz: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """float32 [slots, D] -> (fp8 bytes [slots, D], float32 scales [slots, D // 64]),
    scale = amax over 64 channels / 448 (OCP bytes), or / 240 (fnuz bytes)."""
    slots, D = values.shape
    assert D % 64 == 0
    g = values.reshape(slots, D // 64, 64)
    amax = np.abs(g).max(axis=2)
    fmax = np.float32(FP8_FNUZ_MAX if fnuz else FP8_MAX)
    scale = np.where(amax > 0, amax / fmax, np.float32(1.0)).astype(np.float32)
    enc = to_fp8_fnuz_bytes if fnuz else to_fp8_bytes
    return enc((g / scale[:, :, None]).reshape(slots, D)), scale


def quant_rows(values: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float32 [slots, di] -> (fp8 bytes, float32 per-row scale = amax_row / 448)."""
    amax = np.abs(values).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    return to_fp8_bytes(values / scale[:, None]), scale


# --------------------------------------------------------------------------- workloads
# tensor ids of the sub-streams
_T_Q, _T_QIDX, _T_W, _T_KIDX, _T_KV, _T_BT, _T_EXTRA, _T_CTX, _T_LIST, _T_BT2, _T_KV2, _T_SINK = range(12)


def sinks(seed: int, H: int) -> np.ndarray:
    """Per-head attention-sink logits, float32 [H] ~ N(3, 2^2)."""
    return (3.0 + 2.0 * _rng(seed, _T_SINK).standard_normal(H)).astype(np.float32)


def glm_decode(n_ctx: int = 32768, B: int = 1, H: int = 64, Hi: int = 64, di: int = 128,
               topk: int = 2048, page_size: int = 64, d_nope: int = 512, d_rope: int = 64,
               key_dtype: str = "bf16", kv_fmt: str = "bf16", shuffled: bool = True,
               seed: int = 0, ctx_lens=None, w_low: float = 0.0, index_scale: float = 1.0,
               make_kv: bool = True, name: Optional[str] = None, q_len: int = 1) -> DSAProblem:
    """GLM-style decode: B requests, q_len query tokens each (1: plain decode; more:
    speculative verification or an extend chunk), n_ctx cached tokens per request (or
    per-request ctx_lens) that include the new tokens, MLA 512+64 latent rows, indexer
    Hi x di, weights ~U(w_low, 1). Rows are request-major; the i-th new token of a request
    sees its ctx - q_len + 1 + i first positions (causal among the new tokens).
    make_kv=False replaces the latent cache by one page of data (for indexer-only uses)."""
    ctx = np.full(B, n_ctx, dtype=np.int64) if ctx_lens is None else np.asarray(ctx_lens, np.int64)
    D = d_nope + d_rope
    ppr = (ctx + page_size - 1) // page_size
    if shuffled:
        bt, n_pages = shuffled_pages(seed, _T_BT, B, ppr)
    else:
        n_pages = int(ppr.sum())
        bt = np.zeros((B, int(ppr.max())), dtype=np.int32)
        o = 0
        for b in range(B):
            bt[b, :ppr[b]] = np.arange(o, o + ppr[b], dtype=np.int32)
            o += int(ppr[b])
    slots = n_pages * page_size
    T = B * q_len
    if np.any(ctx < q_len):
        raise ValueError("every context must hold the request's new tokens")
    q = _bf16_normal(seed, _T_Q, (T, H, D))
    q_idx = _bf16_normal(seed, _T_QIDX, (T, Hi, di))
    w = _rng(seed, _T_W).uniform(w_low, 1.0, size=(T, Hi)).astype(np.float32)
    row_req = np.repeat(np.arange(B, dtype=np.int32), q_len)
    row_len = (np.repeat(ctx, q_len) - (q_len - 1) + np.tile(np.arange(q_len), B)).astype(np.int32)
    kraw = _normal(seed, _T_KIDX, (slots, di))
    if key_dtype == "bf16":
        kpool = KeyPool("bf16", to_bf16_bits(kraw), None, page_size, bt, None)
    else:
        k8, ks = quant_rows(kraw)
        kpool = KeyPool("fp8", k8, ks, page_size, bt, None)
    del kraw
    if make_kv:
        kv = _make_kv(seed, _T_KV, kv_fmt, slots, d_nope, d_rope, page_size, bt, None)
    else:
        kv = _make_kv(seed, _T_KV, kv_fmt, page_size, d_nope, d_rope, page_size,
                      np.zeros_like(bt), None)
    return DSAProblem(
        name=name or f"glm_decode_{n_ctx}", T=T, H=H, d_qk=D, d_v=d_nope, topk=topk, q=q, kv=kv,
        row_req=row_req, row_len=row_len, n_req=B,
        softmax_scale=1.0 / math.sqrt(D), Hi=Hi, di=di, q_idx=q_idx, w=w, kpool=kpool,
        index_scale=index_scale)


def _make_kv(seed, tid, fmt, slots, d_nope, d_rope, page_size, bt, req_base) -> KVPool:
    D = d_nope + d_rope
    if fmt == "bf16":
        return KVPool("bf16", _bf16_normal(seed, tid, (slots, D)), None, page_size, bt, req_base,
                      d_nope, d_rope)
    vals = _normal(seed, tid, (slots, D))
    if fmt in ("fp8_uniform", "fp8_uniform_fnuz"):
        data, sc = quant_uniform(vals, fnuz=fmt == "fp8_uniform_fnuz")
        return KVPool(fmt, data, sc, page_size, bt, req_base, d_nope, d_rope)
    if fmt == "fp8_ds_mla":
        assert d_nope == DS_MLA_NOPE and d_rope == DS_MLA_ROPE
        return KVPool("fp8_ds_mla", pack_ds_mla(vals, page_size), None, page_size, bt, req_base,
                      d_nope, d_rope)
    raise ValueError(fmt)


def tiny_decode(seed: int = 0, topk: int = 128) -> DSAProblem:
    """Tiny decode: 1 request, 1 query token, context 512, 16 heads, MLA 576 (512 + 64), value
    dim 512, indexer 4 heads x 64, topk 128, bf16, softmax_scale 1/sqrt(576), page 64,
    identity page table."""
    p = glm_decode(n_ctx=512, B=1, H=16, Hi=4, di=64, topk=topk, page_size=64, shuffled=False,
                   seed=seed, name="tiny_decode")
    return p


def causal_prefill(seg_lens=(8192, 1), H: int = 64, Hi: int = 64, di: int = 128,
                   topk: int = 2048, d_nope: int = 512, d_rope: int = 64, seed: int = 0,
                   name: Optional[str] = None, make_attn: bool = True) -> DSAProblem:
    """Packed causal prefill: segments laid out back to back in one contiguous cache
    (req_base = segment offsets, no page table). Row at segment position p sees [0, p].
    make_attn=False leaves out the attention inputs (q, latent cache): indexer only."""
    seg = np.asarray(seg_lens, dtype=np.int64)
    T = int(seg.sum())
    D = d_nope + d_rope
    base = np.concatenate([[0], np.cumsum(seg)[:-1]]).astype(np.int32)
    row_req = np.repeat(np.arange(len(seg), dtype=np.int32), seg)
    row_len = np.concatenate([np.arange(1, s + 1) for s in seg]).astype(np.int32)
    q = _bf16_normal(seed, _T_Q, (T, H, D)) if make_attn else None
    q_idx = _bf16_normal(seed, _T_QIDX, (T, Hi, di))
    w = _rng(seed, _T_W).uniform(0.0, 1.0, size=(T, Hi)).astype(np.float32)
    kpool = KeyPool("bf16", _bf16_normal(seed, _T_KIDX, (T, di)), None, 1, None, base)
    kv = _make_kv(seed, _T_KV, "bf16", T, d_nope, d_rope, 1, None, base) if make_attn else None
    return DSAProblem(
        name=name or "causal_prefill_" + "_".join(str(int(s)) for s in seg), T=T, H=H, d_qk=D,
        d_v=d_nope, topk=topk, q=q, kv=kv, row_req=row_req, row_len=row_len, n_req=len(seg),
        softmax_scale=1.0 / math.sqrt(D), Hi=Hi, di=di, q_idx=q_idx, w=w, kpool=kpool)


def long_decode(n_ctx: int = 1 << 20, seed: int = 0, **kw) -> DSAProblem:
    """Long-context decode: 1 request, context 1,048,576, 64 heads, MLA 512+64 bf16, indexer
    64 x 128 with fp8 e4m3 keys and an fp32 per-token scale, topk 2048, page 64 shuffled."""
    return glm_decode(n_ctx=n_ctx, key_dtype="fp8", seed=seed,
                      name=kw.pop("name", f"long_decode_{n_ctx}"), **kw)


def dsv4_fp8_decode(B: int = 64, H: int = 16, window: int = 128, n_extra: int = 1024,
                    ratio: int = 4, ctx_lo: int = 16384, ctx_hi: int = 131072,
                    page_size: int = 256, seed: int = 0, name: Optional[str] = None) -> DSAProblem:
    """DeepSeek-V4-style fp8 paged decode (attention stage on given indices).

    B requests with ctx_b ~ U[ctx_lo, ctx_hi]. Main (sliding-window) list: positions
    ctx_b - window .. ctx_b - 1 in a main fp8_ds_mla cache whose table backs only the window's
    pages (every other entry points at one dummy page). Extra (top-k) list: n_extra distinct
    positions ~U[0, ceil(ctx_b / ratio)) in a compressed fp8_ds_mla cache of
    ceil(ctx_b / ratio) tokens per request. Pages of 256 tokens, shuffled. D = 512
    (448 NoPE fp8 + 64 RoPE bf16); value = the whole 512-wide row; scale 1/sqrt(512).
    """
    rng = _rng(seed, _T_CTX)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=B).astype(np.int64)
    D = DS_MLA_NOPE + DS_MLA_ROPE
    # main cache: page 0 is the dummy page; window pages get fresh physical pages
    width_main = int((ctx.max() + page_size - 1) // page_size)
    win_pages = []
    for b in range(B):
        first = (int(ctx[b]) - window) // page_size
        last = (int(ctx[b]) - 1) // page_size
        win_pages.append(list(range(first, last + 1)))
    n_main_pages = 1 + sum(len(p) for p in win_pages)
    perm = _rng(seed, _T_BT).permutation(np.arange(1, n_main_pages)).astype(np.int32)
    bt_main = np.zeros((B, width_main), dtype=np.int32)
    o = 0
    for b in range(B):
        for lp in win_pages[b]:
            bt_main[b, lp] = perm[o]
            o += 1
    main_vals = _normal(seed, _T_KV, (n_main_pages * page_size, D))
    main = KVPool("fp8_ds_mla", pack_ds_mla(main_vals, page_size), None, page_size, bt_main, None,
                  DS_MLA_NOPE, DS_MLA_ROPE)
    del main_vals
    # compressed cache
    n_c = (ctx + ratio - 1) // ratio
    ppr = (n_c + page_size - 1) // page_size
    bt_c, n_cp = shuffled_pages(seed, _T_BT2, B, ppr)
    extra = KVPool("fp8_ds_mla", pack_ds_mla(_normal(seed, _T_KV2, (n_cp * page_size, D)), page_size),
                   None, page_size, bt_c, None, DS_MLA_NOPE, DS_MLA_ROPE)
    idx_main = (ctx[:, None] - window + np.arange(window)[None, :]).astype(np.int32)
    lrng = _rng(seed, _T_LIST)
    idx_extra = np.stack([lrng.choice(int(n_c[b]), size=n_extra, replace=False) for b in range(B)])
    idx_extra = idx_extra.astype(np.int32)
    q = _bf16_normal(seed, _T_Q, (B, H, D))
    return DSAProblem(
        name=name or "dsv4_fp8_decode", T=B, H=H, d_qk=D, d_v=D, topk=n_extra, q=q, kv=main,
        row_req=np.arange(B, dtype=np.int32), row_len=ctx.astype(np.int32), n_req=B,
        softmax_scale=1.0 / math.sqrt(D), idx_main=idx_main, extra_kv=extra, idx_extra=idx_extra,
        meta={"ctx": ctx, "n_compressed": n_c})


def attention_case(fmt: str = "bf16", B: int = 2, H: int = 16, n_ctx: int = 700, n_idx: int = 96,
                   pad: str = "tail", n_pad: int = 10, page_size: int = 64, seed: int = 0,
                   n_extra: int = 0, extra_fmt: Optional[str] = None, d_nope: Optional[int] = None,
                   d_rope: int = 64, d_v: Optional[int] = None, name: Optional[str] = None,
                   sink: bool = False, lse_log2: bool = False) -> DSAProblem:
    """Attention-only case with explicit index lists.

    Each request b has n_ctx cached tokens; its list holds n_idx distinct positions drawn at
    random, with n_pad of them replaced by -1 ("tail": the last n_pad entries; "shuffled":
    random places; "all": every entry). fmt chooses the pool format. bf16 defaults to the GLM
    row (512 latent + 64 RoPE, value = the 512 latent columns); the fp8 formats default to the
    DeepSeek-V4 row (448 NoPE + 64 RoPE, value = the whole 512-wide row). sink draws per-head
    sink logits; lse_log2 asks for the base-2 lse."""
    if d_nope is None:
        d_nope = 512 if fmt == "bf16" else DS_MLA_NOPE
    if fmt == "fp8_ds_mla" or extra_fmt == "fp8_ds_mla":
        assert d_nope == DS_MLA_NOPE
    D = d_nope + d_rope
    if d_v is None:
        d_v = d_nope if fmt == "bf16" else D
    ctx = np.full(B, n_ctx, dtype=np.int64)
    ppr = (ctx + page_size - 1) // page_size
    bt, n_pages = shuffled_pages(seed, _T_BT, B, ppr)
    kv = _make_kv(seed, _T_KV, fmt, n_pages * page_size, d_nope, d_rope, page_size, bt, None)
    lrng = _rng(seed, _T_LIST)

    def lists(n):
        idx = np.stack([lrng.choice(n_ctx, size=n, replace=False) for _ in range(B)]).astype(np.int32)
        if pad == "tail" and n_pad:
            idx[:, n - n_pad:] = -1
        elif pad == "shuffled" and n_pad:
            for b in range(B):
                idx[b, lrng.choice(n, size=n_pad, replace=False)] = -1
        elif pad == "all":
            idx[:] = -1
        return idx

    idx_main = lists(n_idx)
    extra = None
    idx_extra = None
    if n_extra:
        efmt = extra_fmt or fmt
        bt2, n_pages2 = shuffled_pages(seed, _T_BT2, B, ppr)
        extra = _make_kv(seed, _T_KV2, efmt, n_pages2 * page_size, d_nope, d_rope, page_size, bt2, None)
        idx_extra = lists(n_extra)
    q = _bf16_normal(seed, _T_Q, (B, H, D))
    return DSAProblem(
        name=name or f"attn_{fmt}_{B}x{H}_{n_idx}_{pad}", T=B, H=H, d_qk=D,
        d_v=d_v, topk=n_idx, q=q, kv=kv,
        row_req=np.arange(B, dtype=np.int32), row_len=ctx.astype(np.int32), n_req=B,
        softmax_scale=1.0 / math.sqrt(D), idx_main=idx_main, extra_kv=extra, idx_extra=idx_extra,
        sink=sinks(seed, H) if sink else None, lse_log2=lse_log2)


# Named workloads (the five the measurement plan covers, plus the 128k headline shape).
WORKLOADS = {
    "tiny_decode": lambda seed=0: tiny_decode(seed=seed),
    "glm_decode_32k": lambda seed=0: glm_decode(n_ctx=32768, seed=seed, name="glm_decode_32k"),
    "glm_decode_128k": lambda seed=0: glm_decode(n_ctx=131072, seed=seed, name="glm_decode_128k"),
    "causal_prefill_8k": lambda seed=0: causal_prefill((8192, 1), seed=seed, name="causal_prefill_8k"),
    "dsv4_fp8_decode": lambda seed=0: dsv4_fp8_decode(seed=seed),
    "long_decode_1m": lambda seed=0: long_decode(seed=seed, name="long_decode_1m"),
    # several query tokens per request: speculative verification, and a 64-token extend chunk
    "spec_decode_b16_q4_32k": lambda seed=0: glm_decode(n_ctx=32768, B=16, q_len=4, seed=seed,
                                                        name="spec_decode_b16_q4_32k"),
    "extend_64_128k": lambda seed=0: glm_decode(n_ctx=131072, q_len=64, seed=seed, name="extend_64_128k"),
}


def make_workload(name: str, seed: int = 0) -> DSAProblem:
    return WORKLOADS[name](seed=seed)


# The row layouts of the prefill correctness grid (radixark/miles PR 3608, section
# "Correctness": packed, 1-token segments, causal, batch 2).
GRID_LAYOUTS = {
    "causal": dict(seg_lens=(200,)),                         # one causal sequence
    "packed": dict(seg_lens=(90, 57, 33)),                   # sequences back to back
    "one_token": dict(seg_lens=(1,) * 6 + (40,) + (1,) * 6),  # packed, with 1-token segments
    "batch2": dict(seg_lens=(120, 100), paged=True),         # two requests in a paged cache
}


def grid_base(layout: str, H: int, seed: int = 0, d_nope: int = 512, d_rope: int = 64) -> DSAProblem:
    """Rows and caches of one layout of the grid (no lists yet): causal rows (the row at
    position p of its sequence sees [0, p]); packed layouts share one contiguous cache through
    req_base, "batch2" puts each request in its own pages of a shuffled 64-token page table."""
    spec = GRID_LAYOUTS[layout]
    seg = np.asarray(spec["seg_lens"], dtype=np.int64)
    T = int(seg.sum())
    D = d_nope + d_rope
    row_req = np.repeat(np.arange(len(seg), dtype=np.int32), seg)
    row_len = np.concatenate([np.arange(1, s + 1) for s in seg]).astype(np.int32)
    if spec.get("paged"):
        page = 64
        ppr = (seg + page - 1) // page
        bt, n_pages = shuffled_pages(seed, _T_BT, len(seg), ppr)
        kv = _make_kv(seed, _T_KV, "bf16", n_pages * page, d_nope, d_rope, page, bt, None)
    else:
        base = np.concatenate([[0], np.cumsum(seg)[:-1]]).astype(np.int32)
        kv = _make_kv(seed, _T_KV, "bf16", T, d_nope, d_rope, 1, None, base)
    q = _bf16_normal(seed, _T_Q, (T, H, D))
    return DSAProblem(name=f"grid_{layout}_h{H}", T=T, H=H, d_qk=D, d_v=d_nope, topk=0, q=q, kv=kv,
                      row_req=row_req, row_len=row_len, n_req=len(seg),
                      softmax_scale=1.0 / math.sqrt(D))


def grid_lists(base: DSAProblem, topk: int, pad: str, seed: int = 0) -> np.ndarray:
    """Index lists int32 [T, topk] for the grid: row t lists m distinct positions of [0, n_t)
    drawn at random, m = min(topk, n_t) when n_t < topk and topk - topk // 8 otherwise (so every
    row has some -1 padding); pad "tail" puts the m positions first, "shuffled" scatters them
    over the row's topk slots."""
    rng = _rng(seed, _T_LIST)
    idx = np.full((base.T, topk), -1, dtype=np.int32)
    for t in range(base.T):
        n = int(base.row_len[t])
        m = n if n < topk else topk - topk // 8
        pos = rng.choice(n, size=m, replace=False).astype(np.int32)
        where = np.arange(m) if pad == "tail" else np.sort(rng.choice(topk, size=m, replace=False))
        idx[t, where] = pos
    return idx
