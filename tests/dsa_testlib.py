"""Shared helpers for the DSA tests: run the HIP path on a synthetic batch and compute the
oracle's answers for chosen rows.  No arithmetic of the method lives here beyond calling
the oracle (references) or the library (results)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

# Tolerances.  Indexer score: |g - o| <= 1e-3 * max(|o|, A) where A is the same head sum with
# |w| (guards cancellation near zero).  Attention: |g - o| <= 2e-2 + 1e-2 |o| for O (bf16 out),
# 1e-4 + 1e-5 |lse| for the LSE: its logits are accumulated in fp32 from 576 FP8 products,
# so their absolute rounding grows with their magnitude (a large common offset, as with
# latents that share a large mean, moves every logit by the same large amount).
SCORE_RTOL = 1e-3
O_ATOL, O_RTOL = 2e-2, 1e-2
LSE_ATOL, LSE_RTOL = 1e-4, 1e-5


def host(batch):
    """numpy views of a synth.Batch's host-needed arrays."""
    return dict(
        key_pool=batch.key_pool.cpu().numpy(),
        latent_pool=batch.latent_pool.cpu().numpy(),
        bt=batch.block_table.cpu().numpy(),
        q_idx=batch.q_idx.cpu().double().numpy(),
        w=batch.head_w.cpu().numpy(),
        q_mla=batch.q_mla.cpu().double().numpy(),
    )


def request_keys(batch, b, key_pool=None, bt=None):
    """Oracle-read index keys of request b: (codes, scales) for E4M3 keys, or the key values
    [L, 128] for MXFP4 keys."""
    mx = batch.wl.key_format == "mxfp4"
    read = O.read_index_keys_mxfp4 if mx else O.read_index_keys
    if key_pool is None:
        # pull only this request's pages from the device
        pages = batch.block_table[b, : (batch.wl.seq_lens[b] + 63) // 64].long()
        sub = batch.key_pool[pages].cpu().numpy()
        return read(sub, np.arange(len(pages)), batch.wl.seq_lens[b])
    return read(key_pool, bt[b], batch.wl.seq_lens[b])


def oracle_scores(batch, row, keys=None):
    """Oracle fp32 scores of query row `row` over its visible tokens, plus the magnitude
    bound A used by the tolerance."""
    b, pos = batch.wl.row_positions()[row]
    keys = keys if keys is not None else request_keys(batch, b)
    q = batch.q_idx[row].cpu().double().numpy()
    w = batch.head_w[row].cpu().numpy()
    if batch.wl.key_format == "mxfp4":
        kv = keys[: pos + 1]
        return O.index_scores_values(q, w, kv), O.index_scores_values(q, np.abs(w), kv)
    kc, ks = keys
    s = O.index_scores(q, w, kc[: pos + 1], ks[: pos + 1])
    a = O.index_scores(q, np.abs(w), kc[: pos + 1], ks[: pos + 1])
    return s, a


def check_scores(got, ref, mag, where=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = SCORE_RTOL * np.maximum(np.abs(ref), np.asarray(mag, np.float64)) + 1e-30
    err = np.abs(got - ref)
    bad = np.nonzero(~(err <= bound))[0]
    assert bad.size == 0, (f"{where}: {bad.size} scores out of tolerance, first at {bad[:5]}: "
                           f"got {got[bad[:5]]} ref {ref[bad[:5]]}")
    return float(np.max(err / np.maximum(np.abs(ref), 1e-30))) if err.size else 0.0


def check_attention(o_got, lse_got, o_ref, lse_ref, where=""):
    o_got = np.asarray(o_got, np.float64)
    lse_got = np.asarray(lse_got, np.float64)
    d = np.abs(o_got - o_ref)
    bad = d > O_ATOL + O_RTOL * np.abs(o_ref)
    assert not bad.any(), f"{where}: {int(bad.sum())} outputs out of tolerance, max err {d.max()}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_got), fin), f"{where}: LSE finiteness differs"
    if fin.any():
        dl = np.abs(lse_got[fin] - lse_ref[fin])
        lim = LSE_ATOL + LSE_RTOL * np.abs(lse_ref[fin])
        assert (dl <= lim).all(), f"{where}: LSE max err {dl.max()} (|lse| up to {np.abs(lse_ref[fin]).max():.1f})"
    return float(d.max()), float(np.abs(lse_got[fin] - lse_ref[fin]).max()) if fin.any() else 0.0


def topk_is_valid_for(scores_row_f32, sel, k):
    """Property check of a top-k answer against the scores it was computed from: the set
    has min(k, n) distinct members and, under (score desc, index asc), no unselected token
    beats a selected one."""
    s = np.asarray(scores_row_f32, np.float64) + 0.0
    n = s.shape[0]
    sel = np.asarray(sel)
    sel = sel[sel >= 0]
    assert sel.size == min(k, n) and np.unique(sel).size == sel.size
    if sel.size == n:
        return True
    mask = np.zeros(n, bool)
    mask[sel] = True
    worst_sel = min(((s[t], -t) for t in sel))
    best_unsel = max(((s[t], -t) for t in np.nonzero(~mask)[0]))
    return best_unsel < worst_sel


def latent_rows(batch, slots):
    """Oracle-read latent codes for physical slots (only the pages needed are copied)."""
    slots = np.asarray(slots, np.int64)
    pages = np.unique(slots // 64)
    sub = batch.latent_pool[torch.from_numpy(pages).to(batch.latent_pool.device)].cpu().numpy()
    remap = {int(p): i for i, p in enumerate(pages)}
    local = np.array([remap[int(s // 64)] * 64 + int(s % 64) for s in slots], np.int64)
    return O.read_latents(sub, local)
