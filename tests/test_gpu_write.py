"""GPU parity of the write path and the FP4 dequant: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from oracle import OracleCache, dequantise_blocks, unpack_nibbles
from synth import make_decode_case, small_decode
from tests.helpers import bits, cache_bytes_equal, gpu_cache_for, oracle_cache_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def test_dequant_every_code_byte_at_every_scale(fk):
    n = 255
    pages = (n + 63) // 64
    bt = torch.arange(pages, dtype=torch.int32)[None]
    oc = OracleCache(pages, bt.numpy())
    u = np.arange(n, dtype=np.uint8)
    for j in range(n):
        p, s = j // 64, j % 64
        oc.lat_codes[p, s] = np.arange(256, dtype=np.uint8)
        oc.lat_scales[p, s] = u[j]
        oc.idx_codes[p, s] = (np.arange(32) * 7 + j).astype(np.uint8)
        oc.idx_scales[p, s] = [u[j], 254 - u[j]]
    cache = fk.PagedCache(*(torch.from_numpy(getattr(oc, f)).cuda() for f in
                            ("lat_codes", "lat_scales", "idx_codes", "idx_scales")), bt.cuda())
    idx = torch.arange(n, dtype=torch.int32, device="cuda")[None]
    lat, key = fk.debug_gather(cache, idx)
    torch.cuda.synchronize()
    want_lat = oc.latent(0, np.arange(n)).astype(np.float32)
    want_key = oc.index_keys(0, np.arange(n)).astype(np.float32)
    got_lat = lat[0].cpu().numpy()
    got_key = key[0].cpu().numpy()
    bad = np.nonzero((got_lat.view(np.uint32) != want_lat.view(np.uint32)).any(axis=1))[0]
    print("latent rows with a mismatch (scale byte):", bad.tolist()[:20])
    assert bad.size == 0
    assert np.array_equal(got_key.view(np.uint32), want_key.view(np.uint32))


def test_debug_gather_bad_ids_give_nan(fk):
    bt = torch.tensor([[0, 5, -1]], dtype=torch.int32)
    cache = fk.PagedCache.allocate(2, bt)
    idx = torch.tensor([[0, -1, 64, 130, 10 ** 6]], dtype=torch.int32, device="cuda")
    lat, key = fk.debug_gather(cache, idx)
    torch.cuda.synchronize()
    lat = lat.cpu()
    assert torch.all(lat[0, 0] == 0)
    assert torch.isnan(lat[0, 1:]).all()


@pytest.mark.parametrize("pages,ctx,heavy", [
    ("random", (4096, 778, 130), 0.05),
    ("identity", (2048,), 0.0),
    ("fragmented", (6002, 2, 190, 1024), 0.05),
])
def test_write_matches_oracle_bytes(fk, pages, ctx, heavy):
    cfg = small_decode(1, B=len(ctx), ctx=ctx, pages=pages, heavy_frac=heavy, append=0)
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff


def _bf16_from_f64(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def test_write_extremes_zeros_and_offsets(fk):
    rng = np.random.default_rng(5)
    T = 2 * 70
    x = rng.standard_normal((T, 512)) * np.ldexp(1.0, rng.integers(-60, 60, size=(T, 1)))
    x[0:2, :64] = 0.0                        # all-zero blocks
    x[2:4, 64:96] = -0.0                     # negative-zero block
    x[4, :] = 2.0 ** -130                    # subnormal-range merges
    x[6:8, 100] = 1e30                       # a huge channel
    x[8:10, 200:232] = rng.standard_normal((2, 32)) * 2.0 ** -126
    w = rng.uniform(-2, 2, size=(T, 512))
    w[10:12] = 0.0
    k = rng.standard_normal((T // 2, 64)) * np.ldexp(1.0, rng.integers(-40, 40, size=(T // 2, 1)))
    k[3] = 0.0
    xb, wb, kb = _bf16_from_f64(x), _bf16_from_f64(w), _bf16_from_f64(k)
    bt = torch.tensor([[2, 0, 1]], dtype=torch.int32)
    oc = OracleCache(3, bt.numpy())
    start = 38                               # entries 19..88 straddle two pages
    oc.write(0, start, bits(xb), bits(wb), bits(kb))
    gc = fk.PagedCache.allocate(3, bt)
    fk.write_kv(gc, torch.tensor([start], dtype=torch.int32, device="cuda"), xb.cuda()[None].contiguous(),
                wb.cuda()[None].contiguous(), kb.cuda()[None].contiguous())
    torch.cuda.synchronize()
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff


def test_batched_append_with_per_sequence_starts(fk):
    cfg = small_decode(4, B=5, ctx=(700, 64, 4000, 130, 2048), append=64)
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case, recipe="sum")
    gc = gpu_cache_for(case, recipe="sum")
    x, w, k, start = case.append_tokens()
    for b in range(case.B):
        oc.write(b, int(start[b]), bits(x[b]), bits(w[b]), bits(k[b]))
    fk.write_kv(gc, start.cuda(), x.cuda(), w.cuda(), k.cuda())
    torch.cuda.synchronize()
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff


def test_write_quantiser_ties_and_neighbours(fk):
    """Every e2m1 decision point (ties and grid points), each exact and one step above and
    below, both signs, at seven scale exponents: the stored codes and scales must be the
    oracle's bit for bit.  Entry values are y = x0 + x1 (weights 1): x0 = +-v 2^k and x1 =
    +-2^(k-20) when the value is offset, so y sits 2^-20 of the scale from the point."""
    points = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]
    combos = [(s * v, o) for v in points for o in (0, 1, -1) for s in (1.0, -1.0)]   # 90
    ks = [-100, -40, -7, 0, 3, 30, 90]
    n_ent = 64
    x = np.zeros((2 * n_ent, 512))
    w = np.ones((2 * n_ent, 512))
    kk = np.zeros((n_ent, 64))
    for i in range(n_ent):
        k = ks[i % len(ks)]
        for blk in range(16):
            c0 = 32 * blk
            x[2 * i, c0] = 7.0 * 2.0 ** k            # block maximum: scale exponent k
            for j in range(31):
                v, o = combos[(i * 7 + blk * 31 + j) % len(combos)]
                x[2 * i, c0 + 1 + j] = v * 2.0 ** k
                x[2 * i + 1, c0 + 1 + j] = o * np.copysign(1.0, v) * 2.0 ** (k - 20)
        for blk in range(2):
            c0 = 32 * blk
            kk[i, c0] = -7.0 * 2.0 ** k
            for j in range(31):
                v, o = combos[(i * 5 + blk * 31 + j) % len(combos)]
                step = 2.0 ** (np.floor(np.log2(abs(v))) - 7)               # one bf16 step at |v|
                kk[i, c0 + 1 + j] = (v + o * np.copysign(step, v)) * 2.0 ** k
    xb, wb, kb = _bf16_from_f64(x), _bf16_from_f64(w), _bf16_from_f64(kk)
    assert np.array_equal(xb.float().numpy().astype(np.float64), x)    # every input is exact in bf16
    assert np.array_equal(kb.float().numpy().astype(np.float64), kk)
    bt = torch.tensor([[1, 0]], dtype=torch.int32)
    oc = OracleCache(2, bt.numpy())
    start = 2 * 32                           # entries 32..95: both pages
    oc.write(0, start, bits(xb), bits(wb), bits(kb))
    gc = fk.PagedCache.allocate(2, bt)
    fk.write_kv(gc, torch.tensor([start], dtype=torch.int32, device="cuda"), xb.cuda()[None].contiguous(),
                wb.cuda()[None].contiguous(), kb.cuda()[None].contiguous())
    torch.cuda.synchronize()
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff
