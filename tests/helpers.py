"""Test-side glue between synth inputs, the oracle and the HIP binding."""
from __future__ import annotations

import numpy as np
import torch

from oracle import OracleCache


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (on the host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def gpu_available() -> bool:
    return torch.cuda.is_available()


def oracle_cache_for(case, recipe: str = "l2", seqs=None) -> OracleCache:
    """Oracle cache holding the pre-built part of every sequence of a DecodeCase."""
    ratio = getattr(case.cfg, "ratio", 2)
    oc = OracleCache(case.n_pages, case.block_table.numpy(), ratio=ratio)
    for b in (range(case.B) if seqs is None else seqs):
        if case.prebuilt[b] == 0:
            continue
        x, w, k = case.seq_tokens(b, recipe)
        oc.write(b, 0, bits(x), None if w is None else bits(w), bits(k))
    return oc


def gpu_cache_for(case, recipe: str = "l2", device="cuda"):
    """PagedCache filled by csa2_write_kv with the same pre-built tokens, one sequence at a time."""
    import fp4_kv_cache_write_amd as fk
    ratio = getattr(case.cfg, "ratio", 2)
    cache = fk.PagedCache.allocate(case.n_pages, case.block_table, device=device, ratio=ratio)
    for b in range(case.B):
        T = case.prebuilt[b]
        if T == 0:
            continue
        x, w, k = case.seq_tokens(b, recipe)
        sub = cache.rows(b, b + 1)
        start = torch.zeros(1, dtype=torch.int32, device=device)
        fk.write_kv(sub, start, x.to(device)[None].contiguous(),
                    None if w is None else w.to(device)[None].contiguous(), k.to(device)[None].contiguous())
    torch.cuda.synchronize()
    return cache


def cache_bytes_equal(gc, oc) -> dict:
    """Per-field equality of the GPU cache bytes and the oracle's."""
    res = {}
    for name in ("lat_codes", "lat_scales", "idx_codes", "idx_scales"):
        g = getattr(gc, name).cpu().numpy()
        o = getattr(oc, name)
        res[name] = int((g != o).sum())
    return res


def check_topk_set(gpu_ids, domain, scores, k: int, tol: float = 1e-3) -> dict:
    """Compare a GPU top-K against the oracle's scores over `domain` (entry ids).

    The sets must agree except for entries whose oracle score is within `tol` of
    the K-th largest score; sizes must agree; GPU ids must be distinct members of
    the domain, ascending, and padded with -1.
    """
    g = np.asarray(gpu_ids)
    valid = g[g >= 0]
    assert np.all(g[len(valid):] == -1), "padding must follow the ids"
    assert np.all(np.diff(valid) > 0), "ids must be ascending and distinct"
    domain = np.asarray(domain)
    s = dict(zip(domain.tolist(), np.asarray(scores).tolist()))
    assert set(valid.tolist()) <= set(s), "id outside the visible domain"
    n_sel = min(k, len(domain))
    assert len(valid) == n_sel, (len(valid), n_sel)
    order = np.lexsort((domain, -np.asarray(scores)))
    want = set(domain[order[:n_sel]].tolist())
    diff = want.symmetric_difference(set(valid.tolist()))
    if n_sel == len(domain):
        assert not diff
        return {"diff": 0}
    s_k = float(np.asarray(scores)[order[n_sel - 1]])
    far = [j for j in diff if abs(s[j] - s_k) > tol]
    assert not far, f"{len(far)} entries differ beyond {tol} of the K-th score {s_k}: {far[:5]}"
    return {"diff": len(diff)}


def check_attention_rows(o_gpu_bits, o_ref, tol: float = 2e-3) -> float:
    """Per output row (one head): max_d (|o_gpu - o_ref| - 2^-8 |o_gpu|)_+ <= tol * max_d |o_ref|.

    o_gpu_bits: bf16 bit patterns [..., 512]; o_ref: float64 [..., 512].  The
    2^-8 |o_gpu| term is the bf16 rounding of the output; what remains is the
    fp32-accumulation error the bar limits.  Returns the worst ratio seen.
    """
    from oracle import bf16_bits_to_f64
    og = bf16_bits_to_f64(o_gpu_bits)
    err = np.maximum(np.abs(og - o_ref) - 2.0 ** -8 * np.abs(og), 0.0).max(axis=-1)
    ref = np.abs(o_ref).max(axis=-1)
    ratio = err / np.maximum(ref, 1e-300)
    worst = float(ratio.max())
    assert np.all(err <= tol * ref), f"worst ratio {worst:.3e} > {tol}"
    return worst


def check_pool_set(gpu_pool, s, n_vis: int, cand_block: int, pool_blocks: int) -> dict:
    """A GPU HSI pool row ([pool_blocks] block ids, -1 padded) against the oracle's
    entry scores s: block maxima over cand_block entries (last block padded with
    -inf), the block of entry n_vis-1 forced to +inf, the best pool_blocks blocks
    up to near-ties (check_topk_set)."""
    nb = (n_vis + cand_block - 1) // cand_block
    pad = np.full(nb * cand_block, -np.inf)
    pad[:n_vis] = s
    beta = pad.reshape(nb, cand_block).max(axis=1)
    if nb:
        beta[(n_vis - 1) // cand_block] = np.inf
    return check_topk_set(gpu_pool, np.arange(nb), beta, pool_blocks)


def attention_errors(o_gpu_bits, o_ref) -> dict:
    """Raw elementwise error of a bf16 output against the float64 reference, with no
    allowance for the output's bf16 rounding: max |o_gpu - o_ref|; the largest
    |o_gpu - o_ref| / |o_ref| over elements at least 1% of their row's max |o_ref|
    (smaller elements are dominated by rounding of the larger ones); and per row
    max_d |o_gpu - o_ref| / max_d |o_ref|."""
    from oracle import bf16_bits_to_f64
    og = bf16_bits_to_f64(o_gpu_bits)
    d = np.abs(og - o_ref)
    a = np.abs(o_ref)
    rowmax = a.max(axis=-1, keepdims=True)
    big = a >= 1e-2 * rowmax
    rel = d[big] / a[big]
    return dict(max_abs=float(d.max()), max_rel=float(rel.max()) if rel.size else 0.0,
                max_rel_row=float((d.max(axis=-1) / np.maximum(rowmax[..., 0], 1e-300)).max()))


class AttentionReport:
    """Checks attention outputs against the bar (check_attention_rows) and lse within
    1e-4, and keeps the worst bar ratio and raw elementwise errors over every output
    checked, for the test's printed summary."""

    def __init__(self, tol: float = 2e-3):
        self.tol, self.n, self.ratio = tol, 0, 0.0
        self.raw = dict(max_abs=0.0, max_rel=0.0, max_rel_row=0.0)
        self.lse = 0.0

    def check(self, o_gpu_bits, o_ref, lse_gpu=None, lse_ref=None) -> None:
        self.ratio = max(self.ratio, check_attention_rows(o_gpu_bits, o_ref, self.tol))
        for k, v in attention_errors(o_gpu_bits, o_ref).items():
            self.raw[k] = max(self.raw[k], v)
        if lse_gpu is not None:
            d = float(np.abs(np.asarray(lse_gpu, np.float64) - lse_ref).max())
            assert d <= 1e-4, f"lse differs by {d:.3e}"
            self.lse = max(self.lse, d)
        self.n += 1

    def __str__(self) -> str:
        return (f"{self.n} outputs checked, worst {self.ratio / self.tol:.4f} of the bar; raw max abs "
                f"{self.raw['max_abs']:.3e}, max rel {self.raw['max_rel']:.3e} (elements >= 1% of row max), "
                f"row-relative {self.raw['max_rel_row']:.3e}, lse {self.lse:.1e}")


def prefill_caches(case, device="cuda", oracle_seqs=(), k_override=None, oracle_latent=True):
    """GPU cache and oracle cache of a PrefillCase: prior tokens, then the chunk.

    The GPU cache receives every sequence; the oracle writes only `oracle_seqs`, and
    with oracle_latent=False only their indexer keys (latent rows are then written
    later, for the entries a check reads, with write_entry_rows).
    k_override(b, kidx) may replace the indexer keys (both sides get the same).
    Returns (gpu_cache, oracle_cache, chunk dict of CPU tensors).
    """
    import fp4_kv_cache_write_amd as fk
    cfg = case.cfg
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device=device)
    oc = OracleCache(case.n_pages, case.block_table.numpy())
    bt = case.block_table.to(device)
    ch = case.chunk()
    if k_override is not None:
        ch["k_idx"] = torch.stack([k_override(b, ch["k_idx"][b]) for b in range(case.B)])
    for b in range(case.B):
        if cfg.prior > 0:
            x, w, k = case.prior_tokens(b)
            if k_override is not None:
                k = k_override(b, k)
            sub = fk.PagedCache(gc.lat_codes, gc.lat_scales, gc.idx_codes, gc.idx_scales, bt[b:b + 1].contiguous())
            fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device=device), x.to(device)[None].contiguous(),
                        w.to(device)[None].contiguous(), k.to(device)[None].contiguous())
            if b in oracle_seqs:
                oc.write(b, 0, bits(x), bits(w), bits(k), latent=oracle_latent)
    fk.write_kv(gc, ch["start_tok"].to(device), ch["x"].to(device), ch["w"].to(device), ch["k_idx"].to(device))
    for b in oracle_seqs:
        oc.write(b, cfg.prior, bits(ch["x"][b]), bits(ch["w"][b]), bits(ch["k_idx"][b]), latent=oracle_latent)
    torch.cuda.synchronize()
    return gc, oc, ch


def write_entry_rows(oc, b: int, js, x_bits, w_bits, k_bits) -> None:
    """Store entries js of sequence b (ratio 2) in the oracle cache from the whole
    sequence's write inputs (x_bits, w_bits [T,512], k_bits [T/2,64]), one oracle write
    per run of consecutive entries."""
    js = np.unique(np.asarray(js, dtype=np.int64))
    if js.size == 0:
        return
    for run in np.split(js, np.nonzero(np.diff(js) != 1)[0] + 1):
        j0, j1 = int(run[0]), int(run[-1]) + 1
        oc.write(b, 2 * j0, x_bits[2 * j0:2 * j1], w_bits[2 * j0:2 * j1], k_bits[j0:j1])
