"""The allocation-free attention entry point (dsa_sparse_mla_decode_noalloc) against the
workspace one (dsa_sparse_mla_decode) on the same inputs: bitwise the same outputs, on two
calls in a row whose second is smaller (the static scratch keeps the first call's partials),
and the oracle's answer within the attention tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
import sparse_attention_decode_score_amd as dsa
from dsa_testlib import check_attention, latent_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seq_lens, q_per_seq, k, seed):
    wl = synth.custom(seq_lens, q_per_seq, topk=k, seed=seed)
    batch = synth.make_batch(wl, DEV)
    rng = np.random.default_rng(seed)
    bt = batch.block_table.cpu().numpy()
    slots = np.full((wl.n_q, k), -1, np.int32)
    for row, (b, pos) in enumerate(wl.row_positions()):
        n = min(k, pos + 1)
        t = np.sort(rng.choice(pos + 1, size=n, replace=False))
        slots[row, :n] = O.physical_slot(bt[b], t)
    return wl, batch, slots


def _both(batch, slots_d, S):
    n_q = slots_d.shape[0]
    outs = []
    for fn in (dsa.dsa_sparse_mla_decode, dsa.dsa_sparse_mla_decode_noalloc):
        out = torch.full((n_q, 96, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((n_q, 96), float("nan"), device=DEV)
        fn(batch.q_mla, batch.latent_pool, batch.latent_scale, slots_d, batch.softmax_scale, S,
           out=out, lse=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # first call: 12 rows x 16 splits of 2,048 tokens; second: 3 rows x 5 splits of 700
    cases = [(([20000, 9000, 4096], [5, 4, 3], 2048, 71), 16), (([3000, 700], [2, 1], 700, 72), 5)]
    for (lens, qps, k, seed), S in cases:
        say("noalloc", lens, qps, k, S)
        wl, batch, slots = _case(lens, qps, k, seed)
        slots_d = torch.from_numpy(slots).to(DEV)
        (o_ws, l_ws), (o_na, l_na) = _both(batch, slots_d, S)
        assert torch.equal(o_ws, o_na), "O differs from the workspace entry point"
        assert torch.equal(l_ws, l_na), "LSE differs from the workspace entry point"
        o_np, l_np = o_na.float().cpu().numpy(), l_na.cpu().numpy()
        for row in (0, wl.n_q - 1):
            sl = slots[row]
            lat = latent_rows(batch, sl[sl >= 0])
            parts = [O.mla_attend(batch.q_mla[row].cpu().double().numpy(), lat[a:e],
                                  batch.latent_scale, batch.softmax_scale)
                     for a, e in O.split_ranges(k, S)]
            o_ref, l_ref = O.lse_combine(parts)
            check_attention(o_np[row], l_np[row], o_ref, l_ref, f"noalloc row {row} S={S}")


def test_noalloc_single_split_and_fp32_partials_need_no_scratch():
    wl, batch, slots = _case([3000, 700], [2, 1], 256, 73)
    slots_d = torch.from_numpy(slots).to(DEV)
    (o_ws, l_ws), (o_na, l_na) = _both(batch, slots_d, 1)
    assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
    op = [torch.full((4, wl.n_q, 96, 512), float("nan"), device=DEV) for _ in range(2)]
    lp = [torch.full((4, wl.n_q, 96), float("nan"), device=DEV) for _ in range(2)]
    dsa.dsa_sparse_mla_decode(batch.q_mla, batch.latent_pool, batch.latent_scale, slots_d,
                              batch.softmax_scale, 4, o_part=op[0], lse_part=lp[0])
    dsa.dsa_sparse_mla_decode_noalloc(batch.q_mla, batch.latent_pool, batch.latent_scale, slots_d,
                                      batch.softmax_scale, 4, o_part=op[1], lse_part=lp[1])
    torch.cuda.synchronize()
    assert torch.equal(op[0], op[1]) and torch.equal(lp[0], lp[1])


def test_noalloc_rejects_more_than_its_scratch():
    # 720 rows x 64 splits need ~4.5 GB of partials: refused on the host, nothing launched
    n_q, S, k = 720, 64, 64
    slots = torch.full((n_q, k), -1, dtype=torch.int32, device=DEV)
    q = torch.zeros((n_q, 96, 576), dtype=torch.bfloat16, device=DEV)
    pool = torch.zeros((1, 36864), dtype=torch.uint8, device=DEV)
    out = torch.empty((n_q, 96, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((n_q, 96), device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_sparse_mla_decode_noalloc(q, pool, 1.0, slots, 0.04, S, out=out, lse=lse)
    assert e.value.status == 3 and "static scratch" in str(e.value)
