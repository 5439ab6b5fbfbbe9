"""Cache writes on the GPU (dsa_kv_cache_write, dsa_key_cache_write) against the oracle.

Quantisation is byte work: every written byte (fp8 codes, exponent bytes, RoPE bytes) and every
fp32 scale must equal the oracle's exactly; slots that are skipped (-1, out of range) and
slots no row maps to keep their previous contents.
"""
import numpy as np
import pytest
import torch

from oracle import cache_write as CW
from dev import dsa, need_gpu, say
from workloads.gen import to_bf16_bits

pytestmark = [pytest.mark.gpu, need_gpu]

SENT = 0xAB


def _rows(rng, n, D):
    """bf16 rows with mixed magnitudes: per-row spread, an all-zero group, a tiny group, a huge
    group and exact values on e4m3 ties."""
    x = rng.standard_normal((n, D)).astype(np.float32) * rng.lognormal(0, 3, (n, 1)).astype(np.float32)
    if n > 4:
        x[1, :64] = 0.0
        x[2, 64:128] *= np.float32(1e-30)
        x[3, :64] *= np.float32(1e30)
        x[4, :16] = np.float32(448.0) * np.array([1, 0.5, 0.25, 0.3125, 1.0625, 0.96875, 0, -1] * 2, np.float32)
    return to_bf16_bits(x)


def _slots(rng, n, n_slots):
    s = rng.permutation(n_slots)[:n].astype(np.int32)
    s[::11] = -1                                   # skipped rows
    s[5::13] = n_slots + 3                         # out of range: skipped
    return s


def _src(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("fnuz", [False, True], ids=["ocp", "fnuz"])
@pytest.mark.parametrize("D", [512, 576])
def test_kv_uniform(D, fnuz):
    m = dsa()
    rng = np.random.default_rng(D + fnuz)
    n, n_slots = 300, 1000
    bits = _rows(rng, n, D)
    if fnuz:   # values on the fnuz ties near the top (232 between 224 and 240) and tiny ones
        x = np.array([240, 232, -232, 233, 224, 228, -240, 2.0 ** -11, -(2.0 ** -11), -1e-6,
                      3 * 2.0 ** -12, 0, -0.0, 1, 100, 16] * 4, np.float32)
        bits[6, :64] = to_bf16_bits(x)
    slots = _slots(rng, n, n_slots)
    data = torch.full((n_slots, D), SENT, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_slots, D // 64), -7.0, dtype=torch.float32, device="cuda")
    kv = m.KVCache("fp8_uniform_fnuz" if fnuz else "fp8_uniform", data, D - 64, 64, scales=scales)
    say("cache write uniform", D, "fnuz" if fnuz else "ocp")
    m.dsa_kv_cache_write(_src(bits), torch.from_numpy(slots).cuda(), kv)
    torch.cuda.synchronize()
    q, s = CW.write_uniform(bits, fnuz=fnuz)
    got, gs = data.cpu().numpy(), scales.cpu().numpy()
    ok = (slots >= 0) & (slots < n_slots)
    assert np.array_equal(got[slots[ok]], q[ok])
    assert np.array_equal(gs[slots[ok]], s[ok])
    untouched = np.setdiff1d(np.arange(n_slots), slots[ok])
    assert np.all(got[untouched] == SENT) and np.all(gs[untouched] == -7.0)


@pytest.mark.parametrize("page", [256, 33])
def test_kv_ds_mla(page):
    m = dsa()
    rng = np.random.default_rng(page)
    n_pages = 7
    n_slots = n_pages * page
    n = min(400, n_slots)
    bits = _rows(rng, n, 512)
    slots = _slots(rng, n, n_slots)
    data = torch.full((n_pages, page * 584), SENT, dtype=torch.uint8, device="cuda")
    kv = m.KVCache("fp8_ds_mla", data, 448, 64, page_size=page)
    say("cache write ds_mla", page)
    m.dsa_kv_cache_write(_src(bits), torch.from_numpy(slots).cuda(), kv)
    torch.cuda.synchronize()
    rows, sc = CW.write_ds_mla(bits)
    got = data.cpu().numpy()
    written = np.zeros(n_slots, bool)
    for i, sl in enumerate(slots):
        if not 0 <= sl < n_slots:
            continue
        p, pos = divmod(int(sl), page)
        assert np.array_equal(got[p, pos * 576:(pos + 1) * 576], rows[i]), f"row {i} data"
        assert np.array_equal(got[p, page * 576 + pos * 8: page * 576 + pos * 8 + 8], sc[i]), f"row {i} exponents"
        written[sl] = True
    for sl in np.flatnonzero(~written):
        p, pos = divmod(int(sl), page)
        assert np.all(got[p, pos * 576:(pos + 1) * 576] == SENT)
        assert np.all(got[p, page * 576 + pos * 8: page * 576 + pos * 8 + 8] == SENT)


def test_kv_bf16_copy():
    m = dsa()
    rng = np.random.default_rng(5)
    n, n_slots, D = 200, 500, 576
    bits = _rows(rng, n, D)
    slots = _slots(rng, n, n_slots)
    data = torch.full((n_slots, D), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    kv = m.KVCache("bf16", data, 512, 64)
    m.dsa_kv_cache_write(_src(bits), torch.from_numpy(slots).cuda(), kv)
    torch.cuda.synchronize()
    got = data.view(torch.int16).cpu().numpy().view(np.uint16)
    ok = (slots >= 0) & (slots < n_slots)
    assert np.array_equal(got[slots[ok]], bits[ok])
    untouched = np.setdiff1d(np.arange(n_slots), slots[ok])
    assert np.all(got[untouched] == 0xFFFF)


@pytest.mark.parametrize("di,fp8", [(128, True), (64, True), (128, False)])
def test_index_keys(di, fp8):
    m = dsa()
    rng = np.random.default_rng(di + fp8)
    n, n_slots = 333, 800
    bits = _rows(rng, n, di)
    slots = _slots(rng, n, n_slots)
    if fp8:
        data = torch.full((n_slots, di), SENT, dtype=torch.uint8, device="cuda")
        scale = torch.full((n_slots,), -7.0, dtype=torch.float32, device="cuda")
    else:
        data = torch.full((n_slots, di), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        scale = None
    keys = m.KeyCache(data, scale=scale)
    m.dsa_key_cache_write(_src(bits), torch.from_numpy(slots).cuda(), keys, di)
    torch.cuda.synchronize()
    ok = (slots >= 0) & (slots < n_slots)
    if fp8:
        q, s = CW.write_index_keys(bits)
        got, gs = data.cpu().numpy(), scale.cpu().numpy()
        assert np.array_equal(got[slots[ok]], q[ok]) and np.array_equal(gs[slots[ok]], s[ok])
        untouched = np.setdiff1d(np.arange(n_slots), slots[ok])
        assert np.all(got[untouched] == SENT) and np.all(gs[untouched] == -7.0)
    else:
        got = data.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got[slots[ok]], bits[ok])


def test_written_cache_feeds_the_attention_kernel():
    """A ds_mla cache filled by the write kernel gives the same attention as the oracle reading
    those bytes (the written format is the one the attention kernel reads)."""
    import oracle
    from workloads.gen import KVPool
    m = dsa()
    rng = np.random.default_rng(9)
    page, n_pages, H, n_idx = 64, 4, 16, 100
    n_slots = page * n_pages
    bits = to_bf16_bits(rng.standard_normal((n_slots, 512)).astype(np.float32))
    data = torch.zeros((n_pages, page * 584), dtype=torch.uint8, device="cuda")
    bt = torch.arange(n_pages, dtype=torch.int32, device="cuda")[None, :]
    kv = m.KVCache("fp8_ds_mla", data, 448, 64, page_size=page, block_table=bt)
    m.dsa_kv_cache_write(_src(bits), torch.arange(n_slots, dtype=torch.int32, device="cuda"), kv)
    q = to_bf16_bits(rng.standard_normal((1, H, 512)).astype(np.float32))
    idx = np.ascontiguousarray(rng.permutation(n_slots)[:n_idx].astype(np.int32)[None, :])
    out = torch.empty((1, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws = m.Workspace(m.dsa_workspace_size(m.ENTRY_MLA_DECODE, T=1, H=H, n_idx=n_idx))
    m.dsa_sparse_mla_decode(_src(q.reshape(1, H * 512)).view(1, H, 512), kv, torch.from_numpy(idx).cuda(),
                            None, None, 1, H, 512, 512, 1 / np.sqrt(512), out, lse, ws)
    torch.cuda.synchronize()
    pool = KVPool("fp8_ds_mla", data.cpu().numpy(), None, page, bt.cpu().numpy(), None, 448, 64)

    class P:
        pass
    p = P()
    p.q, p.kv, p.extra_kv, p.H, p.d_qk, p.d_v = q, pool, None, H, 512, 512
    p.softmax_scale, p.row_req, p.n_req = 1 / np.sqrt(512), np.zeros(1, np.int32), 1
    o_ref, l_ref = oracle.attention_row(p, 0, idx[0])
    assert np.abs(out[0].float().cpu().numpy() - o_ref).max() < 5e-2
    assert np.abs(lse[0].cpu().numpy() - l_ref).max() < 1e-3
