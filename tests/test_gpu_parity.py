"""GPU parity: every stage of the HIP path against the CPU oracle on the same seeded inputs.

Small ragged batches span several tiles and group tails; the named workloads run at full
size with sampled rows.  Top-k is compared bit for bit on identical fp32 scores (scores the
oracle computed, uploaded to both sides); the indexer within 1e-3 relative; attention
outputs within 2e-2 abs + 1e-2 rel and the LSE within 1e-4 + 1e-5 |lse|.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
import sparse_attention_decode_score_amd as dsa
from dsa_testlib import (check_attention, check_scores, host, latent_rows, oracle_scores,
                         request_keys, topk_is_valid_for)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def run_scores(batch):
    wl = batch.wl
    scores = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, scores, max_seq_len=wl.max_seq_len,
                        max_q_per_seq=max(wl.q_per_seq), key_format=wl.key_format)
    torch.cuda.synchronize()
    return scores


def run_topk(batch, scores, k, with_slots=True):
    wl = batch.wl
    idx = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV) if with_slots else None
    ws = torch.empty(dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, k), dtype=torch.uint8,
                     device=DEV)
    dsa.dsa_topk(batch.cu_q, batch.seq_lens, scores, k, batch.block_table if with_slots else None,
                 idx, slot, ws, max_seq_len=wl.max_seq_len)
    torch.cuda.synchronize()
    return idx, slot


def run_mla(batch, slots, num_splits):
    """fp32 split partials merged by dsa_lse_combine (one split: the direct output)."""
    n_q = batch.wl.n_q
    if num_splits == 1:
        out = torch.empty((n_q, 96, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((n_q, 96), dtype=torch.float32, device=DEV)
        dsa.dsa_sparse_mla_decode(batch.q_mla, batch.latent_pool, batch.latent_scale, slots,
                                  batch.softmax_scale, 1, out=out, lse=lse)
        torch.cuda.synchronize()
        return out, lse, None, None
    op = torch.full((num_splits, n_q, 96, 512), float("nan"), device=DEV)
    lp = torch.full((num_splits, n_q, 96), float("nan"), device=DEV)
    dsa.dsa_sparse_mla_decode(batch.q_mla, batch.latent_pool, batch.latent_scale, slots,
                              batch.softmax_scale, num_splits, o_part=op, lse_part=lp)
    out = torch.empty((n_q, 96, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n_q, 96), dtype=torch.float32, device=DEV)
    dsa.dsa_lse_combine(op, lp, out, lse)
    torch.cuda.synchronize()
    return out, lse, op, lp


def run_mla_merged(batch, slots, num_splits, prepared=False):
    """(out, lse) from one call: fp16 partials merged inside it when num_splits > 1;
    prepared: the query quantised beforehand by dsa_quantize_q."""
    n_q = batch.wl.n_q
    out = torch.full((n_q, 96, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((n_q, 96), float("nan"), dtype=torch.float32, device=DEV)
    kw = {}
    if prepared:
        q8 = torch.empty((n_q, 96, 576), dtype=torch.uint8, device=DEV)
        qs = torch.empty((n_q, 96), dtype=torch.float32, device=DEV)
        dsa.dsa_quantize_q(batch.q_mla, q8, qs)
        kw = dict(q8=q8, q_scale=qs)
    dsa.dsa_sparse_mla_decode(None if prepared else batch.q_mla, batch.latent_pool,
                              batch.latent_scale, slots, batch.softmax_scale, num_splits,
                              out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return out, lse


# ------------------------------------------------------------------------ a0: quantisation
@pytest.mark.parametrize("dim,heads", [(128, 32), (576, 96)])
def test_query_quantisation_bit_exact(dim, heads):
    say("quantise", dim)
    g = torch.Generator().manual_seed(dim)
    q = torch.randn((6, heads, dim), generator=g) * torch.logspace(-6, 4, 6).view(6, 1, 1)
    q[0, 0] = 0.0                     # all-zero head -> scale 1
    q[1, 1, :] = 1e-3
    q[1, 1, 5] = -448.0 * 2.0 ** -7   # absmax exactly on a power-of-two boundary
    qb = q.to(torch.bfloat16)
    codes = torch.empty((6, heads, dim), dtype=torch.uint8, device=DEV)
    scales = torch.empty((6, heads), device=DEV)
    dsa.dsa_quantize_q(qb.to(DEV), codes, scales)
    torch.cuda.synchronize()
    vals = qb.double().numpy()
    for r in range(6):
        ref_c, ref_s = O.quantize_heads(vals[r])
        np.testing.assert_array_equal(scales[r].cpu().numpy().astype(np.float64), ref_s)
        np.testing.assert_array_equal(codes[r].cpu().numpy(), ref_c)


# ------------------------------------------------------------------------ a2: indexer
SMALL = [
    synth.custom([300, 64, 129, 1000], [1, 2, 3, 8], topk=128, seed=21, name="ragged"),
    synth.custom([5000, 4097], [4, 5], topk=2048, seed=22, name="spec-small"),
    synth.custom([1, 63, 65], [1, 1, 1], topk=16, seed=23, name="tiny-tails"),
    synth.custom([2100], [20], topk=64, seed=24, name="many-rows"),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_index_scores_small(wl):
    say("index", wl.name)
    batch = synth.make_batch(wl, DEV)
    scores = run_scores(batch).cpu().numpy()
    h = host(batch)
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref, mag = oracle_scores(batch, row, keys=request_keys(batch, b, h["key_pool"], h["bt"]))
        check_scores(scores[row, : pos + 1], ref, mag, f"{wl.name} row {row}")


def test_index_scores_block_table_permutation_is_bit_identical():
    wl = synth.custom([3000, 777], [2, 1], seed=25)
    batch = synth.make_batch(wl, DEV)
    s1 = run_scores(batch)
    # move every page to a new physical location (and a packed stride of 8448 + 64)
    P = batch.num_pages
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5)).to(DEV)
    stride = 8448 + 64
    pool2 = torch.full((P, stride), 0x7F, dtype=torch.uint8, device=DEV)
    pool2[perm, :8448] = batch.key_pool
    bt2 = torch.where(batch.block_table >= 0, perm[batch.block_table.long().clamp(min=0)].int(),
                      batch.block_table)
    scores = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, pool2, bt2.contiguous(),
                        scores, max_seq_len=wl.max_seq_len, max_q_per_seq=2, key_page_stride=stride)
    torch.cuda.synchronize()
    for row, (b, pos) in enumerate(wl.row_positions()):
        assert torch.equal(s1[row, : pos + 1], scores[row, : pos + 1])


# ------------------------------------------------------------------------ a3: top-k
def _topk_case(lens, q_per, k, kind, seed):
    """A batch whose score matrix is oracle-free synthetic data of a given structure."""
    wl = synth.custom(lens, q_per, topk=k, seed=seed)
    batch = synth.make_batch(wl, DEV)
    sc = synth.random_scores(wl.n_q, wl.max_seq_len, seed, kind)
    return wl, batch, sc


TOPK_CASES = [
    ([131072, 9000], [1, 2], 2048, "normal"),
    ([8192, 8193, 16385, 2047], [1, 1, 1, 1], 2048, "normal"),
    ([40000], [3], 4096, "ties"),
    ([30000], [1], 2048, "equal"),
    ([20000], [2], 1000, "signed_zero"),
    ([50000], [1], 2048, "increasing"),
    ([70000], [1], 100, "neg_inf_tail"),
    ([5000, 3000], [1, 1], 1, "normal"),
    ([3000], [1], 4096, "normal"),          # k >= visible: everything, then -1
    ([60000, 131072], [2, 1], 2048, "extremes"),
    ([60000], [1], 64, "extremes"),
    ([100000], [2], 2048, "huge"),
]


@pytest.mark.parametrize("lens,q_per,k,kind", TOPK_CASES)
def test_topk_bit_exact_on_identical_scores(lens, q_per, k, kind):
    say("topk", lens, k, kind)
    wl, batch, sc = _topk_case(lens, q_per, k, kind, seed=len(lens) * 100 + k)
    idx, slot = run_topk(batch, sc.to(DEV), k)
    idx, slot = idx.cpu().numpy(), slot.cpu().numpy()
    bt = batch.block_table.cpu().numpy()
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref = O.topk_indices(sc[row, : pos + 1].numpy(), k)
        got = idx[row]
        n = min(k, pos + 1)
        assert (got[n:] == -1).all()
        assert np.array_equal(got[:n], np.sort(ref)), f"row {row}"
        assert np.array_equal(slot[row, :n], O.physical_slot(bt[b], got[:n]))
        assert (slot[row, n:] == -1).all()


def test_topk_winners_in_few_groups_are_resent_in_full():
    # the top 2,048 sit in ~10 consecutive 256-token groups, each of which may send only 16
    # candidates: the exactness check flags them and they are re-read in full
    L = 131072
    wl = synth.custom([L], [1], topk=2048, seed=31)
    batch = synth.make_batch(wl, DEV)
    sc = torch.randn((1, L), generator=torch.Generator().manual_seed(3))
    sc[0, 3 * 8192: 3 * 8192 + 2500] += 100.0
    idx, _ = run_topk(batch, sc.to(DEV), 2048)
    ref = np.sort(O.topk_indices(sc[0].numpy(), 2048))
    assert np.array_equal(idx[0].cpu().numpy(), ref)


def test_topk_resend_too_large_keeps_only_elements_ranked_above_the_candidate_kth():
    # 40 boosted tokens in each of 128 groups: the groups hold 2,048 winners between them,
    # ~16 each, and send their best 16; all but one are flagged, and re-reading them in full
    # would not fit on chip: only their elements ranked at or above the candidates' k-th are
    # kept, and selected again
    L = 131072
    wl = synth.custom([L], [1], topk=2048, seed=33)
    batch = synth.make_batch(wl, DEV)
    sc = torch.randn((1, L), generator=torch.Generator().manual_seed(4))
    for g in range(0, 512, 4):
        sc[0, g * 256: g * 256 + 40] += 100.0
    idx, _ = run_topk(batch, sc.to(DEV), 2048)
    ref = np.sort(O.topk_indices(sc[0].numpy(), 2048))
    assert np.array_equal(idx[0].cpu().numpy(), ref)


def test_topk_ranked_resend_too_large_falls_back_to_the_whole_row():
    # every fourth group holds 256 equal scores far above the rest: each sends its first 16,
    # the candidates' k-th is the last of those, and every other boosted group is flagged
    # with all 256 elements tied with it, so even the ranked resend (32,528) does not fit on
    # chip: the whole row is filtered by the k-th key and selected again
    L = 131072
    wl = synth.custom([L], [1], topk=2048, seed=34)
    batch = synth.make_batch(wl, DEV)
    sc = torch.randn((1, L), generator=torch.Generator().manual_seed(5))
    for g in range(0, 512, 4):
        sc[0, g * 256: (g + 1) * 256] = 100.0
    idx, _ = run_topk(batch, sc.to(DEV), 2048)
    ref = np.sort(O.topk_indices(sc[0].numpy(), 2048))
    assert np.array_equal(ref, np.concatenate([np.arange(g * 256, (g + 1) * 256) for g in range(0, 32, 4)]))
    assert np.array_equal(idx[0].cpu().numpy(), ref)


def test_topk_on_oracle_scores_of_a_real_batch():
    wl = synth.custom([20000, 9000], [5, 1], topk=2048, seed=32)
    batch = synth.make_batch(wl, DEV)
    h = host(batch)
    sc = torch.full((wl.n_q, wl.max_seq_len), -1e30)
    for row, (b, pos) in enumerate(wl.row_positions()):
        s, _ = oracle_scores(batch, row, keys=request_keys(batch, b, h["key_pool"], h["bt"]))
        sc[row, : pos + 1] = torch.from_numpy(s)
    idx, _ = run_topk(batch, sc.to(DEV), 2048)
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref = np.sort(O.topk_indices(sc[row, : pos + 1].numpy(), 2048))
        assert np.array_equal(idx[row].cpu().numpy(), ref)


# ------------------------------------------------------------------------ a4 + a5: attention
def _oracle_attention(batch, row, slots_row, num_splits):
    slots_row = np.asarray(slots_row)
    qm = batch.q_mla[row].cpu().double().numpy()
    c, sm = batch.latent_scale, batch.softmax_scale
    k = slots_row.shape[0]
    parts = []
    for a, e in O.split_ranges(k, num_splits):
        seg = slots_row[a:e]
        seg = seg[seg >= 0]
        lat = latent_rows(batch, seg) if seg.size else np.zeros((0, 576), np.uint8)
        parts.append(O.mla_attend(qm, lat, c, sm))
    return parts


def _mla_small_case(num_splits):
    wl = synth.custom([3000, 700, 64], [2, 1, 1], topk=256, seed=41)
    batch = synth.make_batch(wl, DEV)
    # selections: random distinct visible tokens, the short request padded with -1
    rng = np.random.default_rng(num_splits)
    bt = batch.block_table.cpu().numpy()
    slots = np.full((wl.n_q, 256), -1, np.int32)
    for row, (b, pos) in enumerate(wl.row_positions()):
        n = min(256, pos + 1)
        t = np.sort(rng.choice(pos + 1, size=n, replace=False))
        slots[row, :n] = O.physical_slot(bt[b], t)
    return wl, batch, slots


@pytest.mark.parametrize("num_splits", [1, 3, 16, 40, 64])
def test_sparse_mla_small(num_splits):
    say("mla", num_splits)
    wl, batch, slots = _mla_small_case(num_splits)
    slots_d = torch.from_numpy(slots).to(DEV)
    out, lse, op, lp = run_mla(batch, slots_d, num_splits)
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for row in range(wl.n_q):
        parts = _oracle_attention(batch, row, slots[row], num_splits)
        o_ref, l_ref = O.lse_combine(parts)
        check_attention(out[row], lse[row], o_ref, l_ref, f"row {row} S={num_splits}")
        if num_splits > 1:
            for s_, (po, pl) in enumerate(parts):
                check_attention(op[s_, row].cpu().numpy(), lp[s_, row].cpu().numpy(), po, pl,
                                f"row {row} split {s_}")


@pytest.mark.parametrize("num_splits", [1, 3, 16, 40, 64])
@pytest.mark.parametrize("prepared", [False, True], ids=["bf16-query", "prepared-query"])
def test_sparse_mla_merged_in_call(num_splits, prepared):
    # fp16 split partials merged inside the call, against the oracle; and the prepared
    # query gives bitwise the output of the query quantised in the kernel
    say("mla merged", num_splits, prepared)
    wl, batch, slots = _mla_small_case(num_splits)
    slots_d = torch.from_numpy(slots).to(DEV)
    out, lse = run_mla_merged(batch, slots_d, num_splits, prepared)
    o_np, l_np = out.float().cpu().numpy(), lse.cpu().numpy()
    for row in range(wl.n_q):
        o_ref, l_ref = O.lse_combine(_oracle_attention(batch, row, slots[row], num_splits))
        check_attention(o_np[row], l_np[row], o_ref, l_ref, f"row {row} S={num_splits} merged")
    if prepared:
        out2, lse2 = run_mla_merged(batch, slots_d, num_splits, False)
        assert torch.equal(out, out2) and torch.equal(lse, lse2)


def _adversarial_mla_case(case):
    """Latents with a large common mean (every E4M3 latent shifted by +2 and re-encoded) and,
    for row 0, a query aligned with one selected token's latent so that this token carries
    almost all the softmax weight (a second one close behind for "two_dominant")."""
    wl = synth.custom([4096, 3000], [2, 1], topk=2048, seed=95)
    batch = synth.make_batch(wl, DEV)
    pool = batch.latent_pool
    vals = pool.view(torch.float8_e4m3fn).float()
    batch.latent_pool.copy_((vals + 2.0).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
    rng = np.random.default_rng(96)
    bt = batch.block_table.cpu().numpy()
    slots = np.full((wl.n_q, 2048), -1, np.int32)
    for row, (b, pos) in enumerate(wl.row_positions()):
        n = min(2048, pos + 1)
        t = np.sort(rng.choice(pos + 1, size=n, replace=False))
        slots[row, :n] = O.physical_slot(bt[b], t)
    if case != "large_mean":
        lat = latent_rows(batch, slots[0]).view(np.uint8)
        lv = torch.from_numpy(lat.copy()).view(torch.float8_e4m3fn).double().numpy()  # [2048, 576]
        star = 1234
        q = lv[star] - lv.mean(axis=0)          # aligned with the chosen token's latent
        # scale so that the chosen token's logit leads the next one by about 25 nats
        lg = (lv @ q) * batch.latent_scale * batch.softmax_scale
        gap = lg[star] - np.max(np.delete(lg, star))
        q = q * (25.0 / max(gap, 1e-6))
        qm = np.repeat(q[None], 96, axis=0)
        if case == "two_dominant":
            second = 77
            q2 = lv[second] - lv.mean(axis=0)
            qm[::2] = 0.5 * qm[::2] + q2 * (25.0 / max(gap, 1e-6)) * 0.5
        batch.q_mla[0].copy_(torch.from_numpy(qm).to(torch.bfloat16))
    return wl, batch, slots


@pytest.mark.parametrize("case", ["dominant", "two_dominant", "large_mean"])
@pytest.mark.parametrize("num_splits", [1, 4])
def test_sparse_mla_adversarial_softmax(case, num_splits):
    # probabilities spanning many orders of magnitude within and across 32-token blocks,
    # and values with a large common mean: the two-term E4M3 probabilities stay within the
    # parity tolerance (the oracle takes the exact softmax of the same quantised inputs)
    say("mla adversarial", case, num_splits)
    wl, batch, slots = _adversarial_mla_case(case)
    slots_d = torch.from_numpy(slots).to(DEV)
    out, lse = run_mla_merged(batch, slots_d, num_splits)
    o_np, l_np = out.float().cpu().numpy(), lse.cpu().numpy()
    for row in range(wl.n_q):
        o_ref, l_ref = O.lse_combine(_oracle_attention(batch, row, slots[row], num_splits))
        check_attention(o_np[row], l_np[row], o_ref, l_ref, f"{case} row {row} S={num_splits}")


def test_sparse_mla_topk_equal_to_context_is_dense_mla():
    wl = synth.custom([2048], [1], topk=2048, seed=42)
    batch = synth.make_batch(wl, DEV)
    bt = batch.block_table.cpu().numpy()
    slots = torch.from_numpy(O.physical_slot(bt[0], np.arange(2048)).astype(np.int32)[None]).to(DEV)
    out, lse, _, _ = run_mla(batch, slots, 1)
    lat = latent_rows(batch, slots[0].cpu().numpy())
    o_d, l_d = O.dense_mla(batch.q_mla[0].cpu().double().numpy(), lat, batch.latent_scale,
                           batch.softmax_scale)
    check_attention(out[0].float().cpu().numpy(), lse[0].cpu().numpy(), o_d, l_d, "dense")


def test_lse_combine_matches_oracle_with_empty_splits():
    rng = np.random.default_rng(7)
    S, n_q = 5, 3
    o = rng.normal(size=(S, n_q, 96, 512)).astype(np.float32)
    l = rng.normal(size=(S, n_q, 96)).astype(np.float32) * 3
    l[1] = -np.inf
    o[1] = 0
    l[3, 2] = -np.inf
    o[3, 2] = 0
    l[:, 0, 7] = -np.inf                # one head empty in every split
    o[:, 0, 7] = 0
    out = torch.empty((n_q, 96, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n_q, 96), device=DEV)
    dsa.dsa_lse_combine(torch.from_numpy(o).to(DEV), torch.from_numpy(l).to(DEV), out, lse)
    torch.cuda.synchronize()
    for r in range(n_q):
        ref_o, ref_l = O.lse_combine([(o[s, r].astype(np.float64), l[s, r].astype(np.float64))
                                      for s in range(S)])
        check_attention(out[r].float().cpu().numpy(), lse[r].cpu().numpy(), ref_o, ref_l, f"row {r}")


# ------------------------------------------------------------------------ whole path
def _end_to_end(wl, rows, num_splits=None, query_prep=None):
    S = num_splits or wl.num_splits
    say("e2e", wl.name, "rows", rows, "S", S, "query", query_prep or "default")
    batch = synth.make_batch(wl, DEV)
    step = dsa.DecodeStep(wl.n_q, wl.max_seq_len, wl.topk, S, key_format=wl.key_format,
                          query_prep=query_prep)
    out, lse = step.run(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, batch.q_mla, batch.latent_pool, batch.latent_scale,
                        batch.softmax_scale, max(wl.q_per_seq))
    torch.cuda.synchronize()
    # the default step stores no scores (the final pass recomputes what it re-reads); the
    # scores come from a stored-score indexer call, whose candidates are bitwise the same
    scores = step.scores if step.store_scores else run_scores(batch)
    idx = step.topk_idx.cpu().numpy()
    slots = step.topk_slot.cpu().numpy()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rowpos = wl.row_positions()
    for row in rows:
        b, pos = rowpos[row]
        keys = request_keys(batch, b)
        ref, mag = oracle_scores(batch, row, keys=keys)
        got_s = scores[row, : pos + 1].cpu().numpy()
        check_scores(got_s, ref, mag, f"{wl.name} row {row}")
        # the GPU's selection is a valid top-k of the GPU's own scores ...
        assert topk_is_valid_for(got_s, idx[row], wl.topk)
        # ... and agrees with the oracle's selection except where the two score sets differ
        # within tolerance at the selection boundary
        ref_sel = set(O.topk_indices(ref, wl.topk).tolist())
        gsel = set(int(t) for t in idx[row] if t >= 0)
        diff = ref_sel ^ gsel
        if diff:
            kth = np.sort(ref.astype(np.float64))[::-1][min(wl.topk, pos + 1) - 1]
            for t in diff:
                assert abs(float(ref[t]) - kth) <= 2e-3 * max(abs(kth), float(mag[t])), (row, t)
        assert len(diff) <= 8, (row, len(diff))
        # attention on the GPU's own selection, oracle from the same slots
        parts = _oracle_attention(batch, row, slots[row], S)
        o_ref, l_ref = O.lse_combine(parts)
        check_attention(out[row], lse[row], o_ref, l_ref, f"{wl.name} row {row}")
    return batch


def test_end_to_end_tiny():
    _end_to_end(synth.workload("tiny"), rows=[0])


@pytest.mark.parametrize("num_splits", [1, 8])
def test_end_to_end_degenerate_contexts(num_splits):
    # a request of one token (its row sees only token 0), rows at positions 0 and 1 of a
    # two-token request, a partial first page, exactly one page, one page and one token,
    # and a context just above k: the whole default step (fused first pass, no stored
    # scores, final pass inside the attention), splits with no selected token included
    wl = synth.custom([1, 2, 63, 64, 65, 2049], [1, 2, 1, 1, 1, 1], topk=2048,
                      num_splits=num_splits, seed=71, name="degenerate")
    _end_to_end(wl, rows=list(range(wl.n_q)))


@pytest.mark.parametrize("query_prep", ["fused", "first", "side"])
def test_end_to_end_with_a_prepared_query(query_prep):
    # the MLA query quantised by the indexer's launch, by its own launch, or on a side
    # stream: the attention kernel then reads the prepared codes
    wl = synth.custom([20000, 9000, 2049], [5, 1, 3], topk=2048, num_splits=4, seed=88,
                      name="e2e-prepared")
    _end_to_end(wl, rows=[0, 4, 5, 8], query_prep=query_prep)


def test_end_to_end_spec_full_size():
    wl = synth.workload("spec")
    _end_to_end(wl, rows=[0, 4, 77, 159])


def test_end_to_end_long_full_size():
    wl = synth.workload("long")
    _end_to_end(wl, rows=[0, 13, 31])


def test_end_to_end_long_full_size_16_splits():
    # the 16 contiguous chunks of the pages' reading of the long decode: each split
    # attends 128 of the row's 2,048 selected tokens
    wl = synth.workload("long")
    _end_to_end(wl, rows=[0, 31], num_splits=16)


@pytest.mark.slow
def test_end_to_end_million_full_size():
    wl = synth.workload("million")
    _end_to_end(wl, rows=[0, 4])


@pytest.mark.slow
def test_end_to_end_prefill_full_size():
    wl = synth.workload("prefill")
    _end_to_end(wl, rows=[0, 1000, 2047])


def test_batch_composition_does_not_change_a_row():
    """A request's outputs are bitwise identical alone and inside a larger batch."""
    lens, q_per = [6000, 9000, 3000], [1, 5, 2]
    wl = synth.custom(lens, q_per, topk=2048, num_splits=4, seed=51)
    big = synth.make_batch(wl, DEV)
    step = dsa.DecodeStep(wl.n_q, wl.max_seq_len, 2048, 4)
    out_big, lse_big = step.run(big.cu_q, big.seq_lens, big.q_idx, big.head_w, big.key_pool,
                                big.block_table, big.q_mla, big.latent_pool, big.latent_scale,
                                big.softmax_scale, 5)
    out_big, lse_big = out_big.clone(), lse_big.clone()
    # request 1 alone, same pools and block-table row
    rows = slice(1, 6)
    one = dsa.DecodeStep(5, wl.max_seq_len, 2048, 4)
    cu = torch.tensor([0, 5], dtype=torch.int32, device=DEV)
    out1, lse1 = one.run(cu, big.seq_lens[1:2].contiguous(), big.q_idx[rows].contiguous(),
                         big.head_w[rows].contiguous(), big.key_pool, big.block_table[1:2].contiguous(),
                         big.q_mla[rows].contiguous(), big.latent_pool, big.latent_scale,
                         big.softmax_scale, 5)
    torch.cuda.synchronize()
    out1, lse1 = out1.clone(), lse1.clone()
    assert torch.equal(out1, out_big[rows]) and torch.equal(lse1, lse_big[rows])
    # and a repeat run is bitwise identical
    out2, lse2 = one.run(cu, big.seq_lens[1:2].contiguous(), big.q_idx[rows].contiguous(),
                         big.head_w[rows].contiguous(), big.key_pool, big.block_table[1:2].contiguous(),
                         big.q_mla[rows].contiguous(), big.latent_pool, big.latent_scale,
                         big.softmax_scale, 5)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


# ------------------------------------------------------------------------ fused stages 1 + 2
FUSED = SMALL + [
    synth.custom([20000, 9000, 2049], [5, 1, 3], topk=2048, seed=61, name="fused-spec"),
    synth.custom([131072], [1], topk=2048, seed=62, name="fused-128k"),
    synth.custom([3000], [1], topk=4096, seed=63, name="fused-k-above-context"),
]


def _stage_by_stage(batch, k):
    wl = batch.wl
    scores = run_scores(batch)
    idx, slot = run_topk(batch, scores, k)
    return scores, idx, slot


def _fused(batch, k):
    wl = batch.wl
    scores = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    idx = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    ws = dsa.workspace(dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, k))
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, scores, max_seq_len=wl.max_seq_len,
                        max_q_per_seq=max(wl.q_per_seq), cand_k=k, cand_workspace=ws,
                        key_format=wl.key_format)
    dsa.dsa_topk(batch.cu_q, batch.seq_lens, scores, k, batch.block_table, idx, slot, ws,
                 max_seq_len=wl.max_seq_len, from_candidates=True)
    torch.cuda.synchronize()
    return scores, idx, slot


@pytest.mark.parametrize("wl", FUSED, ids=lambda w: w.name)
def test_fused_index_topk_is_bitwise_the_stage_by_stage_path(wl):
    say("fused", wl.name)
    batch = synth.make_batch(wl, DEV)
    s1, i1, t1 = _stage_by_stage(batch, wl.topk)
    s2, i2, t2 = _fused(batch, wl.topk)
    for row, (b, pos) in enumerate(wl.row_positions()):
        assert torch.equal(s1[row, : pos + 1], s2[row, : pos + 1]), row
    assert torch.equal(i1, i2) and torch.equal(t1, t2)


def test_final_pass_selects_nothing_from_candidates_of_another_layout():
    # the indexer writes candidates for a top-2,048; a final pass asked for a top-1,024 would
    # read them with another row and group layout: it selects nothing, and the workspace
    # record reports it; calls that agree select the exact top-k and leave the record clean
    say("workspace layout record")
    wl = synth.custom([5000, 3000], [2, 1], topk=2048, seed=71, name="layout")
    batch = synth.make_batch(wl, DEV)
    k_idx = 2048
    ws = dsa.workspace(max(dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, kk)
                           for kk in (1024, 2048)))
    scores = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)

    def index():
        dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                            batch.block_table, scores, max_seq_len=wl.max_seq_len,
                            max_q_per_seq=max(wl.q_per_seq), cand_k=k_idx, cand_workspace=ws)

    def final(k):
        idx = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
        slot = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
        dsa.dsa_topk(batch.cu_q, batch.seq_lens, scores, k, batch.block_table, idx, slot, ws,
                     max_seq_len=wl.max_seq_len, from_candidates=True)
        torch.cuda.synchronize()
        return idx, slot

    def attend(k):
        out = torch.full((wl.n_q, 96, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((wl.n_q, 96), float("nan"), dtype=torch.float32, device=DEV)
        dsa.dsa_topk_sparse_mla(batch.cu_q, batch.seq_lens, scores, k, batch.block_table, ws,
                                batch.q_mla, batch.latent_pool, batch.latent_scale,
                                batch.softmax_scale, 2, max_seq_len=wl.max_seq_len, out=out,
                                lse=lse)
        torch.cuda.synchronize()
        return out, lse

    index()
    idx, slot = final(1024)
    assert bool((idx == -1).all()) and bool((slot == -1).all())
    with pytest.raises(dsa.DsaError):
        dsa.dsa_topk_workspace_status(ws)
    index()
    out, lse = attend(1024)
    assert bool((out.float() == 0).all()) and bool(torch.isneginf(lse).all())
    with pytest.raises(dsa.DsaError):
        dsa.dsa_topk_workspace_status(ws)
    index()
    idx, slot = final(k_idx)
    dsa.dsa_topk_workspace_status(ws)
    for row, (b, pos) in enumerate(wl.row_positions()):
        n = min(k_idx, pos + 1)
        ref = np.sort(O.topk_indices(scores[row, : pos + 1].cpu().numpy(), k_idx))
        assert np.array_equal(idx[row, :n].cpu().numpy(), ref), row


def test_full_row_boundary_selects_the_exact_topk():
    # rows of up to 32,768 visible tokens send every key to the final pass (full rows); a row
    # of 32,769 goes through the first-pass groups: both give the exact top-k of the scores,
    # with and without stored scores
    say("full-row boundary")
    wl = synth.custom([32768, 32769, 16385], [2, 2, 1], topk=2048, seed=66, name="full-row-edge")
    batch = synth.make_batch(wl, DEV)
    s1, i1, t1 = _stage_by_stage(batch, 2048)
    s2, i2, t2 = _fused(batch, 2048)
    assert torch.equal(i1, i2) and torch.equal(t1, t2)
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref = np.sort(O.topk_indices(s2[row, : pos + 1].cpu().numpy(), 2048))
        assert np.array_equal(i2[row].cpu().numpy(), ref), row
    _check_no_scores_matches(batch, 2048, expect_rescored=None)


@pytest.mark.parametrize("wl", [
    SMALL[0], SMALL[3], FUSED[4], FUSED[5],
    synth.custom([5000, 4097], [4, 5], topk=2048, seed=87, name="mx-prep", key_format="mxfp4"),
], ids=lambda w: w.name)
def test_index_with_query_prep_is_bitwise_both_calls(wl):
    """dsa_index_score_quantize_q = dsa_index_score (scores and candidates, bit for bit) +
    dsa_quantize_q of the MLA query (codes and scales, bit for bit), for row groups of 1, 2,
    4 and 8 rows per request and both key formats."""
    say("index+query prep", wl.name)
    batch = synth.make_batch(wl, DEV)
    k = wl.topk
    ws1 = dsa.workspace(dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, k))
    ws2 = dsa.workspace(dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, k))
    s1 = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    s2 = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    q8_ref = torch.empty((wl.n_q, 96, 576), dtype=torch.uint8, device=DEV)
    qs_ref = torch.empty((wl.n_q, 96), device=DEV)
    q8 = torch.full((wl.n_q, 96, 576), 0x5A, dtype=torch.uint8, device=DEV)
    qs = torch.full((wl.n_q, 96), float("nan"), device=DEV)
    common = dict(max_seq_len=wl.max_seq_len, max_q_per_seq=max(wl.q_per_seq), cand_k=k,
                  key_format=wl.key_format)
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, s1, cand_workspace=ws1, **common)
    dsa.dsa_quantize_q(batch.q_mla, q8_ref, qs_ref)
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, s2, cand_workspace=ws2,
                        mla_query=(batch.q_mla, q8, qs), **common)
    torch.cuda.synchronize()
    assert torch.equal(q8, q8_ref) and torch.equal(qs, qs_ref)
    for row, (b, pos) in enumerate(wl.row_positions()):
        assert torch.equal(s1[row, : pos + 1], s2[row, : pos + 1]), row
    # the candidates: the final pass over each workspace selects bitwise the same
    idx1 = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    idx2 = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(batch.cu_q, batch.seq_lens, s1, k, None, idx1, None, ws1,
                 max_seq_len=wl.max_seq_len, from_candidates=True)
    dsa.dsa_topk(batch.cu_q, batch.seq_lens, s2, k, None, idx2, None, ws2,
                 max_seq_len=wl.max_seq_len, from_candidates=True)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)


def test_fused_topk_resends_groups_that_hold_the_winners():
    wl = synth.custom([40000], [2], topk=2048, seed=64, name="fused-skew")
    batch = synth.make_batch(wl, DEV)
    # multiply the key scales of tokens 5,120 .. 6,143 (four 256-token groups) by 1000: the
    # groups then hold ~500 of the best scores but may send only 56 candidates each
    bt = batch.block_table.cpu().numpy()
    for page in range(80, 96):
        phys = int(bt[0, page])
        sc = batch.key_pool[phys, 8192:].view(torch.float32)
        sc.mul_(1000.0)
    torch.cuda.synchronize()
    s1, i1, t1 = _stage_by_stage(batch, 2048)
    s2, i2, t2 = _fused(batch, 2048)
    assert torch.equal(i1, i2) and torch.equal(t1, t2)
    h = host(batch)
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref, mag = oracle_scores(batch, row, keys=request_keys(batch, b, h["key_pool"], h["bt"]))
        got = s2[row, : pos + 1].cpu().numpy()
        check_scores(got, ref, mag, f"skew row {row}")
        assert topk_is_valid_for(got, i2[row].cpu().numpy(), 2048)
        in_groups = ((i2[row] >= 5120) & (i2[row] < 6144)).sum().item()
        assert in_groups > 200, in_groups


# ------------------------------------------------------------- stage 2's final pass in stage 3
def _select_attend(batch, k, num_splits, prepared=False, outputs=True):
    """Indexer with candidates, then dsa_topk_sparse_mla: (idx, slot, out, lse)."""
    wl = batch.wl
    scores = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    ws = dsa.workspace(dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, k))
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, scores, max_seq_len=wl.max_seq_len,
                        max_q_per_seq=max(wl.q_per_seq), cand_k=k, cand_workspace=ws,
                        key_format=wl.key_format)
    idx = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    out = torch.full((wl.n_q, 96, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((wl.n_q, 96), float("nan"), dtype=torch.float32, device=DEV)
    kw = {}
    if prepared:
        q8 = torch.empty((wl.n_q, 96, 576), dtype=torch.uint8, device=DEV)
        qs = torch.empty((wl.n_q, 96), dtype=torch.float32, device=DEV)
        dsa.dsa_quantize_q(batch.q_mla, q8, qs)
        kw = dict(q8=q8, q_scale=qs)
    dsa.dsa_topk_sparse_mla(batch.cu_q, batch.seq_lens, scores, k, batch.block_table, ws,
                            None if prepared else batch.q_mla, batch.latent_pool,
                            batch.latent_scale, batch.softmax_scale, num_splits,
                            max_seq_len=wl.max_seq_len, out=out, lse=lse,
                            topk_idx=idx if outputs else None,
                            topk_slot=slot if outputs else None, **kw)
    torch.cuda.synchronize()
    return idx, slot, out, lse


def _two_calls(batch, k, num_splits):
    _, idx, slot = _fused(batch, k)
    out, lse = run_mla_merged(batch, slot, num_splits)
    return idx, slot, out, lse


@pytest.mark.parametrize("num_splits", [1, 4])
@pytest.mark.parametrize("wl", FUSED, ids=lambda w: w.name)
def test_select_in_attention_is_bitwise_the_two_call_path(wl, num_splits):
    say("select+attend", wl.name, num_splits)
    batch = synth.make_batch(wl, DEV)
    i1, t1, o1, l1 = _two_calls(batch, wl.topk, num_splits)
    i2, t2, o2, l2 = _select_attend(batch, wl.topk, num_splits)
    assert torch.equal(i1, i2) and torch.equal(t1, t2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_select_in_attention_without_selection_outputs_and_with_prepared_query():
    wl = FUSED[1]
    say("select+attend variants", wl.name)
    batch = synth.make_batch(wl, DEV)
    _, _, o1, l1 = _select_attend(batch, wl.topk, 3)
    i2, t2, o2, l2 = _select_attend(batch, wl.topk, 3, prepared=True, outputs=False)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert bool((i2 == -7).all()) and bool((t2 == -7).all())   # not written


def test_select_in_attention_matches_the_oracle():
    # the selection is a valid exact top-k of the row's scores (checked against the oracle's
    # scores), its slots follow the block table, and the attention over them matches the
    # oracle's MLA + LSE merge
    wl = SMALL[0]
    say("select+attend oracle", wl.name)
    batch = synth.make_batch(wl, DEV)
    idx, slot, out, lse = _select_attend(batch, wl.topk, 2)
    scores = run_scores(batch)
    h = host(batch)
    o_np, l_np = out.float().cpu().numpy(), lse.cpu().numpy()
    idx_np, slots = idx.cpu().numpy(), slot.cpu().numpy()
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref, mag = oracle_scores(batch, row, keys=request_keys(batch, b, h["key_pool"], h["bt"]))
        got = scores[row, : pos + 1].cpu().numpy()
        check_scores(got, ref, mag, f"row {row}")
        assert topk_is_valid_for(got, idx_np[row], wl.topk), row
        sel = idx_np[row][idx_np[row] >= 0]
        assert np.array_equal(slots[row][: sel.size], O.physical_slot(h["bt"][b], sel)), row
        assert (slots[row][sel.size:] == -1).all(), row
        o_ref, l_ref = O.lse_combine(_oracle_attention(batch, row, slots[row], 2))
        check_attention(o_np[row], l_np[row], o_ref, l_ref, f"row {row} select+attend")


def test_select_in_attention_resends_groups_that_hold_the_winners():
    wl = synth.custom([40000], [2], topk=2048, seed=64, name="fused-skew")
    batch = synth.make_batch(wl, DEV)
    bt = batch.block_table.cpu().numpy()
    for page in range(80, 96):
        batch.key_pool[int(bt[0, page]), 8192:].view(torch.float32).mul_(1000.0)
    torch.cuda.synchronize()
    i1, t1, o1, l1 = _two_calls(batch, 2048, 2)
    i2, t2, o2, l2 = _select_attend(batch, 2048, 2)
    assert torch.equal(i1, i2) and torch.equal(t1, t2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert ((i2[0] >= 5120) & (i2[0] < 6144)).sum().item() > 200


# --------------------------------------------- candidates with no stored scores (recomputed)
def _index(batch, k, store_scores, ws_fill=0):
    wl = batch.wl
    scores = torch.full((wl.n_q, wl.max_seq_len), float("nan"), device=DEV)
    ws = torch.full((dsa.dsa_topk_workspace_size(wl.n_q, wl.max_seq_len, k),), ws_fill,
                    dtype=torch.uint8, device=DEV)
    dsa.dsa_index_score(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                        batch.block_table, scores if store_scores else None,
                        max_seq_len=wl.max_seq_len, max_q_per_seq=max(wl.q_per_seq),
                        cand_k=k, cand_workspace=ws, key_format=wl.key_format)
    torch.cuda.synchronize()
    return scores, ws


def _final(batch, k, scores, ws, rescore):
    wl = batch.wl
    idx = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(batch.cu_q, batch.seq_lens, scores, k, batch.block_table, idx, slot, ws,
                 max_seq_len=wl.max_seq_len, from_candidates=True,
                 rescore=(batch.q_idx, batch.head_w, batch.key_pool) if rescore else None,
                 key_format=wl.key_format)
    torch.cuda.synchronize()
    return idx, slot


def _boost_pages(batch, b, pages, factor=1000.0):
    """Multiplies the key scales of logical pages `pages` of request b (scores scale too):
    fp32 scales by `factor`; MXFP4 E8M0 block scales by 2^10."""
    bt = batch.block_table.cpu().numpy()
    for page in pages:
        if batch.wl.key_format == "mxfp4":
            sc = batch.key_pool[int(bt[b, page]), 4096:4352]
            assert int(sc.max().item()) <= 244          # stays below the NaN code 0xFF
            sc.add_(10)
        else:
            batch.key_pool[int(bt[b, page]), 8192:].view(torch.float32).mul_(factor)
    torch.cuda.synchronize()


def _check_no_scores_matches(batch, k, expect_rescored):
    """Stored-scores path vs no-scores path: candidates, selection and the recomputed
    scores (bitwise), and whether anything was recomputed."""
    wl = batch.wl
    s_ref, ws_ref = _index(batch, k, True)
    s_none, ws_none = _index(batch, k, False)
    assert bool(torch.isnan(s_none).all())          # the indexer stored nothing
    assert torch.equal(ws_ref, ws_none)             # same candidates, byte for byte
    i1, t1 = _final(batch, k, s_ref, ws_ref, False)
    i2, t2 = _final(batch, k, s_none, ws_none, True)
    assert torch.equal(i1, i2) and torch.equal(t1, t2)
    n_rescored = 0
    for row, (b, pos) in enumerate(wl.row_positions()):
        got = s_none[row, : pos + 1]
        done = ~torch.isnan(got)
        n_rescored += int(done.sum().item())
        assert torch.equal(got[done], s_ref[row, : pos + 1][done]), row
    if expect_rescored is not None:
        assert (n_rescored > 0) == expect_rescored, n_rescored
    return i2, n_rescored


@pytest.mark.parametrize("wl", FUSED, ids=lambda w: w.name)
def test_no_stored_scores_is_bitwise_the_stored_scores_path(wl):
    say("no scores", wl.name)
    batch = synth.make_batch(wl, DEV)
    _check_no_scores_matches(batch, wl.topk, expect_rescored=False)


def test_no_stored_scores_recomputes_flagged_groups_exactly():
    # four groups hold ~500 of the winners but send 56 candidates each: flagged, recomputed
    wl = synth.custom([40000], [2], topk=2048, seed=64, name="rescore-skew")
    batch = synth.make_batch(wl, DEV)
    _boost_pages(batch, 0, range(80, 96))
    idx, n = _check_no_scores_matches(batch, 2048, expect_rescored=True)
    assert n <= 2 * 4 * 256                          # only the flagged groups (both rows)
    assert ((idx[0] >= 5120) & (idx[0] < 6144)).sum().item() > 200


def test_no_stored_scores_recomputes_only_flagged_groups_when_the_resend_is_too_large():
    # one boosted page in every fourth group: 128 groups each hold ~32 winners and send 16,
    # so nearly all are flagged and their full resend would not fit on chip: only they are
    # recomputed, and their elements ranked at or above the candidates' k-th are kept
    L = 131072
    wl = synth.custom([L], [1], topk=2048, seed=65, name="rescore-ranked")
    batch = synth.make_batch(wl, DEV)
    _boost_pages(batch, 0, range(0, L // 64, 16))
    idx, n = _check_no_scores_matches(batch, 2048, expect_rescored=True)
    assert 0 < n <= 128 * 256


def _copy_token_to_pages(batch, b, t_src, pages, factor):
    """Writes the E4M3 index key of token t_src of request b into every token of logical
    pages `pages` of request b, with its fp32 scale multiplied by `factor`."""
    bt = batch.block_table.cpu().numpy()
    src = batch.key_pool[int(bt[b, t_src // 64])]
    o = t_src % 64
    codes = src[:8192].view(8, 64, 16)[:, o, :].clone()          # [column block][16 bytes]
    scale = float(src[8192:].view(torch.float32)[o].item()) * factor
    for page in pages:
        pg = batch.key_pool[int(bt[b, page])]
        pg[:8192].view(8, 64, 16).copy_(codes[:, None, :].expand(8, 64, 16))
        pg[8192:].view(torch.float32).fill_(scale)
    torch.cuda.synchronize()


def test_no_stored_scores_recomputes_the_whole_row_when_even_the_ranked_resend_is_too_large():
    # every token of every fourth group gets the key of the row's best token, with its scale
    # raised: 128 groups of 256 tied scores far above the rest, so even the ranked resend does
    # not fit on chip and the whole row is recomputed, filtered and selected again
    L = 131072
    wl = synth.custom([L], [1], topk=2048, seed=67, name="rescore-all")
    batch = synth.make_batch(wl, DEV)
    s0 = run_scores(batch)
    t_best = int(torch.argmax(s0[0, :L]).item())
    assert s0[0, t_best].item() > 0
    _copy_token_to_pages(batch, 0, t_best, [p for g in range(0, 512, 4) for p in range(4 * g, 4 * g + 4)],
                         1000.0)
    idx, n = _check_no_scores_matches(batch, 2048, expect_rescored=True)
    assert n == L
    want = np.concatenate([np.arange(g * 256, (g + 1) * 256) for g in range(0, 32, 4)])
    assert np.array_equal(np.sort(idx[0].cpu().numpy()), want)


def test_resend_beyond_4096_groups_rereads_the_whole_row():
    # 1,049,000 tokens = 4,098 groups of 256, more group starts than the final pass holds in
    # LDS: a flagged group (one boosted page holds the positive-scoring of its tokens among
    # the winners, the group sends 4) makes it recompute and re-read the whole row; the selection is bitwise the stored-scores path's
    # and the exact top-k of those scores
    L = 1049000
    wl = synth.custom([L], [1], topk=2048, seed=68, name="resend-4098-groups")
    batch = synth.make_batch(wl, DEV)
    _boost_pages(batch, 0, [9000])
    idx, n = _check_no_scores_matches(batch, 2048, expect_rescored=True)
    assert n == L
    s_ref, _ = _index(batch, 2048, True)
    ref = np.sort(O.topk_indices(s_ref[0, :L].cpu().numpy(), 2048))
    assert np.array_equal(idx[0].cpu().numpy(), ref)
    # more winners from the boosted page than its group's 4 candidates: the resend counted
    assert ((idx[0] >= 9000 * 64) & (idx[0] < 9001 * 64)).sum().item() > 4


@pytest.mark.parametrize("key_format", ["e4m3", "mxfp4"])
@pytest.mark.parametrize("num_splits", [1, 4])
def test_select_in_attention_with_no_stored_scores(num_splits, key_format):
    say("select+attend no scores", num_splits, key_format)
    wl = synth.custom([40000, 9000], [2, 1], topk=2048, seed=66, name="rescore-attend",
                      key_format=key_format)
    batch = synth.make_batch(wl, DEV)
    _boost_pages(batch, 0, range(80, 96))
    i1, t1, o1, l1 = _select_attend(batch, 2048, num_splits)
    k = 2048
    s_none, ws = _index(batch, k, False)
    idx = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((wl.n_q, k), -7, dtype=torch.int32, device=DEV)
    out = torch.full((wl.n_q, 96, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((wl.n_q, 96), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_topk_sparse_mla(batch.cu_q, batch.seq_lens, s_none, k, batch.block_table, ws,
                            batch.q_mla, batch.latent_pool, batch.latent_scale,
                            batch.softmax_scale, num_splits, max_seq_len=wl.max_seq_len,
                            out=out, lse=lse, topk_idx=idx, topk_slot=slot,
                            rescore=(batch.q_idx, batch.head_w, batch.key_pool),
                            key_format=key_format)
    torch.cuda.synchronize()
    assert torch.equal(i1, idx) and torch.equal(t1, slot)
    assert torch.equal(o1, out) and torch.equal(l1, lse)


# ------------------------------------------------------------------------ cache append
def _bf16_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("n,key_mag,lat_sat,pad", [(1, 1.0, False, 0), (37, 1.0, True, 0),
                                                   (300, 1e-3, False, 64), (64, 300.0, True, 16)])
def test_cache_append_bit_exact(n, key_mag, lat_sat, pad):
    say("append", n, key_mag, lat_sat, pad)
    pages = 24
    g = torch.Generator().manual_seed(n)
    key_pool = torch.full((pages, 8448 + pad), 0x7F, dtype=torch.uint8)
    key_pool[:, 8192:8448] = torch.full((pages, 64), float("nan")).view(torch.uint8)
    lat_pool = torch.full((pages, 64 * 576 + pad), 0x7F, dtype=torch.uint8)
    slots = torch.randperm(pages * 64, generator=g)[:n].to(torch.int32)
    if n > 2:
        slots[1] = -1
    key = (torch.randn((n, 128), generator=g) * key_mag).to(torch.bfloat16)
    if n > 3:
        key[3] = 0.0
    lat = (torch.randn((n, 576), generator=g) * torch.logspace(-3, 2, n).view(n, 1)).to(torch.bfloat16)
    lat_scale = float(np.float32(lat.float().abs().max() / (1000.0 if lat_sat else 448.0)))
    kp_ref, lp_ref = key_pool.numpy().copy(), lat_pool.numpy().copy()
    O.cache_append(kp_ref, lp_ref, slots.numpy(), _bf16_bits(key), _bf16_bits(lat), lat_scale)
    kp, lp = key_pool.to(DEV), lat_pool.to(DEV)
    dsa.dsa_cache_append(slots.to(DEV), key.to(DEV), lat.to(DEV), lat_scale, kp, lp)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), kp_ref)
    assert np.array_equal(lp.cpu().numpy(), lp_ref)


def test_cache_append_keys_only_leaves_latents_and_feeds_the_indexer():
    # append the last token of each request into a batch's caches, then score: the new
    # token's score equals the oracle's on the appended (oracle-quantised) key
    wl = synth.custom([1000, 70], [1, 1], topk=64, seed=71)
    batch = synth.make_batch(wl, DEV)
    bt = batch.block_table.cpu().numpy()
    g = torch.Generator().manual_seed(71)
    key = torch.randn((2, 128), generator=g).to(torch.bfloat16)
    slots = torch.tensor([O.physical_slot(bt[b], np.array([L - 1]))[0]
                          for b, L in enumerate(wl.seq_lens)], dtype=torch.int32)
    lat_before = batch.latent_pool.clone()
    kp_ref = batch.key_pool.cpu().numpy().copy()
    O.cache_append(kp_ref, None, slots.numpy(), _bf16_bits(key), None, 1.0)
    dsa.dsa_cache_append(slots.to(DEV), key.to(DEV), None, 1.0, batch.key_pool, None)
    torch.cuda.synchronize()
    assert np.array_equal(batch.key_pool.cpu().numpy(), kp_ref)
    assert torch.equal(batch.latent_pool, lat_before)
    scores = run_scores(batch)
    for row, (b, pos) in enumerate(wl.row_positions()):
        kc, ks = O.read_index_keys(kp_ref, bt[b], pos + 1)
        ref = O.index_scores(batch.q_idx[row].cpu().double().numpy(), batch.head_w[row].cpu().numpy(),
                             kc, ks)
        mag = O.index_scores(batch.q_idx[row].cpu().double().numpy(),
                             np.abs(batch.head_w[row].cpu().numpy()), kc, ks)
        check_scores(scores[row, : pos + 1].cpu().numpy(), ref, mag, f"append row {row}")


def _mx_edge_keys(n, g):
    """bf16 keys [n, 128] with the MXFP4 append's edge cases: E2M1 tie points and saturation
    on a block's own grid, all-zero and -0 blocks, fp32-subnormal (bf16) blocks that reach the
    E8M0 floor, huge magnitudes, and negative values that round to -0."""
    k = torch.randn((n, 128), generator=g) * torch.logspace(-4, 4, n).view(n, 1)
    ties = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.5, 5.5, -0.75, -0.1, 4.0])
    for i in range(0, n, 7):
        blk = i % 4
        e = float(2.0 ** ((i % 21) - 10))
        k[i, 32 * blk:32 * blk + 32] = 0.0
        k[i, 32 * blk:32 * blk + len(ties)] = ties * e
    if n > 3:
        k[1] = 0.0
        k[2, :32] = -0.0
        k[3, 32:64] = torch.linspace(-1, 1, 32) * 1e-39   # bf16 subnormals
        k[3, 64:96] = torch.linspace(-1, 1, 32) * 3e38
    return k.to(torch.bfloat16)


@pytest.mark.parametrize("n,pad", [(1, 0), (40, 0), (300, 48)])
def test_cache_append_mxfp4_bit_exact(n, pad):
    say("append mxfp4", n, pad)
    pages = 20
    g = torch.Generator().manual_seed(100 + n)
    key_pool = torch.full((pages, 4352 + pad), 0x77, dtype=torch.uint8)
    key_pool[:, 4096:4352] = 0xFF
    lat_pool = torch.full((pages, 64 * 576), 0x7F, dtype=torch.uint8)
    slots = torch.randperm(pages * 64, generator=g)[:n].to(torch.int32)
    if n > 4:
        slots[4] = -1
    key = _mx_edge_keys(n, g)
    lat = torch.randn((n, 576), generator=g).to(torch.bfloat16)
    lat_scale = float(np.float32(lat.float().abs().max() / 448.0))
    kp_ref, lp_ref = key_pool.numpy().copy(), lat_pool.numpy().copy()
    O.cache_append(kp_ref, lp_ref, slots.numpy(), _bf16_bits(key), _bf16_bits(lat), lat_scale,
                   key_format="mxfp4")
    kp, lp = key_pool.to(DEV), lat_pool.to(DEV)
    dsa.dsa_cache_append_mxfp4(slots.to(DEV), key.to(DEV), lat.to(DEV), lat_scale, kp, lp)
    torch.cuda.synchronize()
    got = kp.cpu().numpy()
    bad = np.argwhere(got != kp_ref)
    assert bad.size == 0, (bad[:5].tolist(), got[tuple(bad[0])], kp_ref[tuple(bad[0])])
    assert np.array_equal(lp.cpu().numpy(), lp_ref)


def test_cache_append_mxfp4_keys_feed_the_mxfp4_indexer():
    wl = synth.custom([1000, 70], [1, 1], topk=64, seed=72, key_format="mxfp4")
    batch = synth.make_batch(wl, DEV)
    bt = batch.block_table.cpu().numpy()
    g = torch.Generator().manual_seed(72)
    key = torch.randn((2, 128), generator=g).to(torch.bfloat16)
    slots = torch.tensor([O.physical_slot(bt[b], np.array([L - 1]))[0]
                          for b, L in enumerate(wl.seq_lens)], dtype=torch.int32)
    lat_before = batch.latent_pool.clone()
    kp_ref = batch.key_pool.cpu().numpy().copy()
    O.cache_append(kp_ref, None, slots.numpy(), _bf16_bits(key), None, 1.0, key_format="mxfp4")
    dsa.dsa_cache_append_mxfp4(slots.to(DEV), key.to(DEV), None, 1.0, batch.key_pool, None)
    torch.cuda.synchronize()
    assert np.array_equal(batch.key_pool.cpu().numpy(), kp_ref)
    assert torch.equal(batch.latent_pool, lat_before)
    scores = run_scores(batch)
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref, mag = oracle_scores(batch, row, keys=request_keys(batch, b, kp_ref, bt))
        check_scores(scores[row, : pos + 1].cpu().numpy(), ref, mag, f"mx append row {row}")


# ------------------------------------------------------------------------ MXFP4 index keys
MX_SMALL = [
    synth.custom([300, 64, 129, 1000], [1, 2, 3, 8], topk=128, seed=81, name="mx-ragged",
                 key_format="mxfp4"),
    synth.custom([5000, 4097], [4, 5], topk=2048, seed=82, name="mx-spec-small",
                 key_format="mxfp4"),
    synth.custom([1, 63, 65], [1, 1, 1], topk=16, seed=83, name="mx-tiny-tails",
                 key_format="mxfp4"),
]


@pytest.mark.parametrize("wl", MX_SMALL, ids=lambda w: w.name)
def test_index_scores_mxfp4_small(wl):
    say("mx index", wl.name)
    batch = synth.make_batch(wl, DEV)
    scores = run_scores(batch)
    h = host(batch)
    for row, (b, pos) in enumerate(wl.row_positions()):
        ref, mag = oracle_scores(batch, row, keys=request_keys(batch, b, h["key_pool"], h["bt"]))
        check_scores(scores[row, : pos + 1].cpu().numpy(), ref, mag, f"{wl.name} row {row}")


@pytest.mark.parametrize("wl", MX_SMALL[:2] + [synth.custom([131072], [1], topk=2048, seed=84,
                                                             name="mx-128k", key_format="mxfp4")],
                         ids=lambda w: w.name)
def test_index_mxfp4_fused_candidates_are_bitwise_the_stage_by_stage_path(wl):
    say("mx fused", wl.name)
    batch = synth.make_batch(wl, DEV)
    s1, i1, t1 = _stage_by_stage(batch, wl.topk)
    s2, i2, t2 = _fused(batch, wl.topk)
    for row, (b, pos) in enumerate(wl.row_positions()):
        assert torch.equal(s1[row, : pos + 1], s2[row, : pos + 1]), row
    assert torch.equal(i1, i2) and torch.equal(t1, t2)


@pytest.mark.parametrize("wl", MX_SMALL[:2] + [synth.custom([131072], [1], topk=2048, seed=85,
                                                             name="mx-128k", key_format="mxfp4")],
                         ids=lambda w: w.name)
def test_no_stored_scores_mxfp4_is_bitwise_the_stored_scores_path(wl):
    say("mx no scores", wl.name)
    batch = synth.make_batch(wl, DEV)
    _check_no_scores_matches(batch, wl.topk, expect_rescored=None)


def test_no_stored_scores_mxfp4_recomputes_flagged_groups_exactly():
    wl = synth.custom([40000], [2], topk=2048, seed=86, name="mx-rescore-skew",
                      key_format="mxfp4")
    batch = synth.make_batch(wl, DEV)
    _boost_pages(batch, 0, range(80, 96))
    idx, n = _check_no_scores_matches(batch, 2048, expect_rescored=True)
    assert n <= 2 * 4 * 256
    assert ((idx[0] >= 5120) & (idx[0] < 6144)).sum().item() > 200


def test_no_stored_scores_mxfp4_recomputes_only_flagged_groups_when_the_resend_is_too_large():
    L = 131072
    wl = synth.custom([L], [1], topk=2048, seed=87, name="mx-rescore-ranked", key_format="mxfp4")
    batch = synth.make_batch(wl, DEV)
    _boost_pages(batch, 0, range(0, L // 64, 16))
    idx, n = _check_no_scores_matches(batch, 2048, expect_rescored=True)
    assert 0 < n <= 128 * 256


def test_mxfp4_cache_with_the_e4m3_rescore_format_is_refused():
    # an MXFP4 pool (4,352-byte pages) read as E4M3 keys (8,448-byte pages) fails the host check
    wl = MX_SMALL[1]
    batch = synth.make_batch(wl, DEV)
    assert batch.key_pool.stride(0) == 4352
    s_none, ws = _index(batch, wl.topk, False)
    idx = torch.empty((wl.n_q, wl.topk), dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DsaError, match="key_page_stride"):
        dsa.dsa_topk(batch.cu_q, batch.seq_lens, s_none, wl.topk, batch.block_table, idx, None,
                     ws, max_seq_len=wl.max_seq_len, from_candidates=True,
                     rescore=(batch.q_idx, batch.head_w, batch.key_pool), key_format="e4m3")


def test_end_to_end_tiny_mxfp4():
    _end_to_end(synth.workload("tiny-mxfp4"), rows=[0])


def test_end_to_end_long_mxfp4_full_size():
    _end_to_end(synth.workload("long-mxfp4"), rows=[0, 17])
