"""GPU parity of the write with indexer keys projected from the entries
(csa2_write_kv_proj): every cache byte equals the oracle's."""
import numpy as np
import pytest
import torch

from oracle import OracleCache
from tests.helpers import bits, cache_bytes_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _setup(rng, starts, T, ratio):
    """Random page table covering every sequence's entries up to start/ratio + T/ratio."""
    per = [(s // ratio + T // ratio + 63) // 64 for s in starts]
    n_pages = sum(per)
    perm = rng.permutation(n_pages)
    bt = np.full((len(starts), max(per)), -1, np.int32)
    o = 0
    for b, n in enumerate(per):
        bt[b, :n] = perm[o:o + n]
        o += n
    return n_pages, torch.from_numpy(bt)


def _write_both(fk, rng, starts, T, ratio, x, w, p):
    n_pages, bt = _setup(rng, starts, T, ratio)
    oc = OracleCache(n_pages, bt.numpy(), ratio=ratio)
    for b, s in enumerate(starts):
        oc.write_projected(b, s, bits(x[b]), None if w is None else bits(w[b]), bits(p))
    gc = fk.PagedCache.allocate(n_pages, bt, ratio=ratio)
    fk.write_kv_proj(gc, torch.tensor(starts, dtype=torch.int32, device="cuda"), x.cuda().contiguous(),
                     None if w is None else w.cuda().contiguous(), p.cuda().contiguous())
    torch.cuda.synchronize()
    return gc, oc


@pytest.mark.parametrize("ratio", [2, 1])
@pytest.mark.parametrize("spread", [0, 24], ids=["normal", "wide-exponents"])
def test_projected_write_matches_oracle_bytes(fk, ratio, spread):
    # spread > 0: every token row and every weight gets its own power-of-two factor
    # in 2^-spread .. 2^spread, so the float64 sums round in most steps and only the
    # channel order keeps the two sides equal.
    rng = np.random.default_rng(101 + 10 * ratio + spread)
    starts, T = [0, 40, 130], 300
    f = (lambda *s: np.ldexp(1.0, rng.integers(-spread, spread + 1, size=s))) if spread else (lambda *s: 1.0)
    x = _bf16(rng.standard_normal((3, T, 512)) * f(3, T, 1))
    w = _bf16(rng.uniform(0, 1, (3, T, 512))) if ratio == 2 else None
    p = _bf16(rng.standard_normal((64, 512)) / np.sqrt(512) * f(64, 512))
    gc, oc = _write_both(fk, rng, starts, T, ratio, x, w, p)
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff


def test_many_entries_through_the_grid_stride_loop(fk):
    # more entries than the launch has waves (512 workgroups x 4 waves)
    rng = np.random.default_rng(7)
    starts, T = [0, 64], 5000
    x = _bf16(rng.standard_normal((2, T, 512)))
    p = _bf16(rng.standard_normal((64, 512)) / np.sqrt(512))
    gc, oc = _write_both(fk, rng, starts, T, 1, x, None, p)
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff


def test_selection_weights_reproduce_the_supplied_key_write(fk):
    # Weights that pick channels 0..63: the projected key of a ratio-1 entry is its
    # token's first 64 channels, so both GPU write paths store the same bytes.
    rng = np.random.default_rng(8)
    starts, T = [6, 0], 200
    x = _bf16(rng.standard_normal((2, T, 512)) * 3.0)
    sel = torch.zeros((64, 512), dtype=torch.bfloat16)
    sel[torch.arange(64), torch.arange(64)] = 1.0
    n_pages, bt = _setup(rng, starts, T, 1)
    a = fk.PagedCache.allocate(n_pages, bt, ratio=1)
    b = fk.PagedCache.allocate(n_pages, bt, ratio=1)
    st = torch.tensor(starts, dtype=torch.int32, device="cuda")
    fk.write_kv_proj(a, st, x.cuda(), None, sel.cuda())
    fk.write_kv(b, st, x.cuda(), None, x[:, :, :64].contiguous().cuda())
    torch.cuda.synchronize()
    for f in ("lat_codes", "lat_scales", "idx_codes", "idx_scales"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_accumulation_follows_channel_order(fk):
    # 2^60 + 1 rounds to 2^60 in float64, so over channels 0, 1, 2 in order the sum
    # 2^60 + 1 - 2^60 is 0, where the exact value (or another order) gives 1.  Output
    # 1 picks channel 1 alone (= 1), so the key block's scale is set by it.
    x = torch.zeros((1, 64, 512), dtype=torch.bfloat16)
    x[0, :, 0], x[0, :, 1], x[0, :, 2] = 2.0 ** 60, 1.0, -(2.0 ** 60)
    p = torch.zeros((64, 512), dtype=torch.bfloat16)
    p[0, :3] = 1.0
    p[1, 1] = 1.0
    n_pages, bt = 1, torch.zeros((1, 1), dtype=torch.int32)
    oc = OracleCache(n_pages, bt.numpy(), ratio=1)
    oc.write_projected(0, 0, bits(x[0]), None, bits(p))
    gc = fk.PagedCache.allocate(n_pages, bt, ratio=1)
    fk.write_kv_proj(gc, torch.zeros(1, dtype=torch.int32, device="cuda"), x.cuda(), None, p.cuda())
    torch.cuda.synchronize()
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), diff
    keys = oc.index_keys(0, np.arange(64))
    assert np.all(keys[:, 0] == 0.0) and np.all(keys[:, 1] == 1.0)
