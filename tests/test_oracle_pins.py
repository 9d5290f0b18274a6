"""Pins for the CPU oracle: library routines, closed forms, brute force, invariants.

Every check here compares the oracle against something that is not the oracle:
torch's own FP8/bf16 codecs, pure-Python loops over tiny inputs, torch CPU fp64
softmax attention, closed forms, and invariants of the method.  A dropped term, a
wrong sign or a transposed operand anywhere in the oracle fails at least one.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth


# ------------------------------------------------------------------------------ codecs
def test_e4m3_table_matches_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.E4M3_TABLE
    nan_ref, nan_mine = np.isnan(ref), np.isnan(mine)
    assert (nan_ref == nan_mine).all()
    assert np.array_equal(ref[~nan_ref], mine[~nan_mine])


def test_e4m3_special_values():
    # OCP E4M3FN: max normal 0x7E = 448, 0x7F NaN, min subnormal 2^-9, min normal 2^-6
    assert O.E4M3_TABLE[0x7E] == 448.0
    assert math.isnan(O.E4M3_TABLE[0x7F]) and math.isnan(O.E4M3_TABLE[0xFF])
    assert O.E4M3_TABLE[0x01] == 2.0 ** -9
    assert O.E4M3_TABLE[0x08] == 2.0 ** -6
    assert O.E4M3_TABLE[0x38] == 1.0
    assert O.E4M3_TABLE[0xB8] == -1.0
    pos = O.E4M3_TABLE[:0x7F]
    assert (np.diff(pos) > 0).all()


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_grid_midpoints_and_random():
    pos = O.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    eps = np.float64(2.0 ** -20)
    probes = np.concatenate([pos, mids, mids * (1 + eps), mids * (1 - eps)])
    probes = np.concatenate([probes, -probes])
    rng = np.random.default_rng(0)
    probes = np.concatenate([probes, rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 20000)])
    probes = probes.astype(np.float32).astype(np.float64)   # torch path takes fp32
    mine = O.e4m3_encode(probes)
    ref = _torch_e4m3(probes)
    # torch keeps the sign of zero results; so does the oracle
    assert np.array_equal(mine, ref)


def test_e4m3_encode_ties_to_even_and_saturates():
    assert O.e4m3_encode([1.0625])[0] == 0x38          # between 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode([1.1875])[0] == 0x3A          # between 1.125 and 1.25 -> even 0x3A
    assert O.e4m3_encode([500.0, -1e9])[0] == 0x7E
    assert O.e4m3_encode([-1e9])[0] == 0xFE
    assert O.e4m3_encode([2.0 ** -10])[0] == 0x00      # half of min subnormal -> 0 (even)
    assert O.e4m3_encode([-0.0])[0] == 0x80


def test_bf16_value_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.bf16_value(bits)
    ok = ~np.isnan(t)
    assert np.array_equal(np.isnan(mine), ~ok)
    assert np.array_equal(mine[ok], t[ok])


# ------------------------------------------------------------------ query quantisation
@pytest.mark.parametrize("a", [1e-30, 2.0 ** -20, 0.3, 1.0, 3.5, 3.7, 7.0, 448.0, 448.0 * 2 ** 5,
                               448.0 * 2 ** 5 * (1 + 2 ** -40), 1234.5, 1e30])
def test_pow2_scale_is_smallest_power_of_two(a):
    s = O.pow2_scale(a)
    m, e = math.frexp(s)
    assert m == 0.5                          # a power of two
    assert a <= 448.0 * s
    assert a > 448.0 * s / 2                 # minimal


def test_pow2_scale_zero():
    assert O.pow2_scale(0.0) == 1.0


def test_quantize_heads_error_bound_and_exact_cases():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(32, 128)).astype(np.float32).astype(np.float64)
    codes, sq = O.quantize_heads(q)
    deq = O.e4m3_decode(codes) * sq[:, None]
    amax = np.abs(q).max(axis=1)
    assert (amax <= 448 * sq).all() and (amax > 224 * sq).all()
    # round-to-nearest: error at most half a step; steps are 2^-3 relative for normals,
    # 2^-9 * sq absolute for subnormals
    tol = np.maximum(np.abs(q) * 2.0 ** -4, (2.0 ** -10) * sq[:, None])
    assert (np.abs(deq - q) <= tol * (1 + 1e-12)).all()
    # values already on the scaled grid come back exactly
    grid = O.E4M3_TABLE[rng.integers(0, 0x7F, size=(4, 128))] * 2.0 ** -3
    grid[:, 0] = 448 * 2.0 ** -3
    c2, s2 = O.quantize_heads(grid)
    assert np.array_equal(O.e4m3_decode(c2) * s2[:, None], grid)
    z, sz = O.quantize_heads(np.zeros((2, 8)))
    assert (sz == 1.0).all() and (O.e4m3_decode(z) == 0).all()


def _query_by_definition(q):
    """The dequantised query q_hat = E4M3(q / sq) * sq written from the definition, without
    the oracle: sq = the smallest 2^e with max|q_h| <= 448 * 2^e (found by stepping e over
    exact powers of two, 1 for an all-zero head), codes by torch's float8_e4m3fn conversion
    of q / sq (exact in fp32 for bf16 inputs), decoded by torch."""
    q = np.asarray(q, np.float64)
    out = np.empty_like(q)
    for h in range(q.shape[0]):
        a = float(np.max(np.abs(q[h])))
        sq = 1.0
        if a > 0.0:
            e = -160
            while a > 448.0 * math.ldexp(1.0, e):
                e += 1
            sq = math.ldexp(1.0, e)
        codes = torch.from_numpy((q[h] / sq).astype(np.float32)).to(torch.float8_e4m3fn)
        out[h] = codes.to(torch.float64).numpy() * sq
    return out


def _bf16_heads(rng, heads, dim):
    """bf16 query heads whose magnitudes span many powers of two (one head all zero)."""
    q = rng.normal(size=(heads, dim)) * np.exp2(rng.integers(-30, 30, size=(heads, 1)))
    q[heads // 2] = 0.0
    return torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).double().numpy()


def test_dequantized_query_matches_definition():
    # Query quantisation of the fused indexer front ("Fused low-latency decode for DSA
    # layers"): every value of the oracle's q_hat equals the definition, bit for bit.
    rng = np.random.default_rng(21)
    for heads, dim in ((32, 128), (96, 576)):
        q = _bf16_heads(rng, heads, dim)
        assert np.array_equal(O.dequantized_query(q), _query_by_definition(q))
    # a head that is already on the E4M3 grid times a power of two comes back unchanged
    g = O.E4M3_TABLE[rng.integers(0, 0x7F, size=(1, 128))] * 2.0 ** 7
    g[0, 5] = 448.0 * 2.0 ** 7
    assert np.array_equal(O.dequantized_query(g), g)


def test_index_scores_with_quantised_query_brute_force():
    # score_t = sum_h w_h ReLU(q_hat_h . k_t s_t) with q_hat from the definition above
    rng = np.random.default_rng(22)
    q = _bf16_heads(rng, 32, 128)
    _, w, codes, sc = _rand_idx_inputs(23, 24)
    got = O.index_scores(q, w, codes, sc).astype(np.float64)
    ref = _brute_scores(_query_by_definition(q).tolist(), w, codes, sc)
    np.testing.assert_allclose(got, ref, rtol=2e-7, atol=1e-30)


def test_mla_attend_with_quantised_query_matches_torch_softmax_attention():
    rng = np.random.default_rng(24)
    q = torch.from_numpy(rng.normal(size=(96, 576)).astype(np.float32) * 3.0).to(torch.bfloat16)
    q = q.double().numpy()
    x = rng.normal(size=(60, 576)).astype(np.float32)
    c = np.float32(np.abs(x).max() / 448)
    codes = _torch_e4m3(x / c)
    sm = float(np.float32(1 / math.sqrt(576)))
    o, lse = O.mla_attend(q, codes, float(c), sm)
    kv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double() * float(c)
    logits = (torch.from_numpy(_query_by_definition(q)) @ kv.T) * sm
    np.testing.assert_allclose(o, (torch.softmax(logits, -1) @ kv[:, :512]).numpy(), rtol=1e-12,
                               atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), rtol=1e-12, atol=1e-12)
    # and the dense-MLA routine on the same query
    o_d, l_d = O.dense_mla(q, codes, float(c), sm)
    np.testing.assert_allclose(o_d, o, rtol=1e-11, atol=1e-14)


# -------------------------------------------------------------------------- paging
@pytest.fixture(scope="module")
def small_batch():
    wl = synth.custom([300, 130, 64], [1, 3, 2], topk=64, seed=7)
    return synth.make_batch(wl, "cpu", keep_logical=True)


def test_paged_key_and_latent_readers_match_logical(small_batch):
    b = small_batch
    pool = b.key_pool.numpy()
    lat = b.latent_pool.numpy()
    bt = b.block_table.numpy()
    for r, L in enumerate(b.wl.seq_lens):
        codes, scales = O.read_index_keys(pool, bt[r], L)
        assert np.array_equal(codes, b.keys_logical[r].numpy())
        assert np.array_equal(scales, b.scales_logical[r].numpy().astype(np.float64))
        slots = O.physical_slot(bt[r], np.arange(L))
        assert np.array_equal(O.read_latents(lat, slots), b.latents_logical[r].numpy())
    # pages no request owns are poisoned
    owned = set(int(x) for x in bt.ravel() if x >= 0)
    spare = [p for p in range(pool.shape[0]) if p not in owned]
    assert spare and (pool[spare[0], :8192] == 0x7F).all()


# ---------------------------------------------------------------- indexer score
def _brute_scores(q_vals, w, key_codes, key_scales):
    """Pure-Python triple loop; values decoded by torch's E4M3 decoder."""
    kv = torch.from_numpy(np.ascontiguousarray(key_codes)).view(torch.float8_e4m3fn).double().tolist()
    out = []
    for t in range(len(kv)):
        acc = 0.0
        for h in range(32):
            dot = 0.0
            for d in range(128):
                dot += q_vals[h][d] * kv[t][d]
            dot *= float(key_scales[t])
            acc += float(w[h]) * (dot if dot > 0 else 0.0)
        out.append(acc)
    return np.array(out)


def _rand_idx_inputs(seed, n):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(32, 128)).astype(np.float32)
    q = torch.from_numpy(q).to(torch.bfloat16).double().numpy()
    w = (rng.normal(size=32) / math.sqrt(32)).astype(np.float32)
    k = rng.normal(size=(n, 128)).astype(np.float32)
    sc = (np.abs(k).max(axis=1) / np.float32(448)).astype(np.float32)
    codes = _torch_e4m3(k / sc[:, None])
    return q, w, codes, sc


def test_index_scores_brute_force():
    q, w, codes, sc = _rand_idx_inputs(2, 40)
    got = O.index_scores(q, w, codes, sc).astype(np.float64)
    qhat = O.dequantized_query(q).tolist()
    ref = _brute_scores(qhat, w, codes, sc)
    np.testing.assert_allclose(got, ref, rtol=2e-7, atol=1e-9)
    # without query quantisation the brute force on raw q must match too
    got_raw = O.index_scores(q, w, codes, sc, quantize_query=False).astype(np.float64)
    np.testing.assert_allclose(got_raw, _brute_scores(q.tolist(), w, codes, sc), rtol=2e-7, atol=1e-9)


def test_index_scores_one_hot_weight_is_relu_matmul():
    q, _, codes, sc = _rand_idx_inputs(3, 200)
    kv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for h in (0, 17, 31):
        w = np.zeros(32, np.float32)
        w[h] = 1.0
        got = O.index_scores(q, w, codes, sc, quantize_query=False).astype(np.float64)
        ref = np.maximum(kv @ q[h] * sc, 0.0)
        np.testing.assert_allclose(got, ref, rtol=2e-7, atol=1e-9)


def test_index_scores_nonnegative_linear_closed_form():
    q, _, codes, sc = _rand_idx_inputs(4, 100)
    q = np.abs(q)
    codes = codes & 0x7F                                  # |k|
    kv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    w = np.ones(32, np.float32)
    got = O.index_scores(q, w, codes, sc, quantize_query=False).astype(np.float64)
    ref = sc * (kv @ q.sum(axis=0))                       # s_t * (sum_h q_h) . k_t
    np.testing.assert_allclose(got, ref, rtol=2e-7)


def test_index_scores_negative_weight_flips_sign():
    q, w, codes, sc = _rand_idx_inputs(5, 64)
    a = O.index_scores(q, w, codes, sc).astype(np.float64)
    b = O.index_scores(q, -w, codes, sc).astype(np.float64)
    np.testing.assert_array_equal(a, -b)


# ------------------------------------------------------------------------- top-k
def test_topk_brute_force_definition():
    rng = np.random.default_rng(6)
    for n, k in [(50, 7), (300, 64), (64, 64), (10, 40)]:
        s = rng.integers(-5, 5, size=n).astype(np.float32) * 0.5   # many ties
        got = O.topk_indices(s, k).tolist()
        ref = sorted(range(n), key=lambda t: (-float(s[t]), t))[:min(k, n)]
        assert got == ref


def test_topk_special_cases():
    eq = np.full(100, 2.5, np.float32)
    assert O.topk_indices(eq, 10).tolist() == list(range(10))
    inc = np.arange(100, dtype=np.float32)
    assert sorted(O.topk_indices(inc, 10).tolist()) == list(range(90, 100))
    assert sorted(O.topk_indices(inc, 500).tolist()) == list(range(100))
    z = np.array([-0.0, 0.0, -0.0, 0.0], np.float32)
    assert O.topk_indices(z, 2).tolist() == [0, 1]
    ninf = np.array([-np.inf, 1.0, -np.inf, -np.inf], np.float32)
    assert O.topk_indices(ninf, 3).tolist() == [1, 0, 2]


# --------------------------------------------------------------- sparse MLA
def _rand_mla(seed, n):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.normal(size=(96, 576)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    x = rng.normal(size=(n, 576)).astype(np.float32)
    c = np.float32(np.abs(x).max() / 448)
    codes = _torch_e4m3(x / c)
    return q, codes, float(c), float(np.float32(1 / math.sqrt(576)))


def test_mla_attend_matches_torch_softmax_attention():
    q, codes, c, sm = _rand_mla(8, 150)
    o, lse = O.mla_attend(q, codes, c, sm, quantize_query=False)
    kv = torch.from_numpy(codes).view(torch.float8_e4m3fn).double() * c
    qt = torch.from_numpy(q)
    logits = (qt @ kv.T) * sm
    ref_o = torch.softmax(logits, dim=-1) @ kv[:, :512]
    ref_lse = torch.logsumexp(logits, dim=-1)
    np.testing.assert_allclose(o, ref_o.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def test_mla_attend_special_cases():
    q, codes, c, sm = _rand_mla(9, 40)
    kv = O.e4m3_decode(codes) * c
    # one token: output is that token's value, LSE its logit
    o, lse = O.mla_attend(q, codes[3:4], c, sm, quantize_query=False)
    np.testing.assert_allclose(o, np.broadcast_to(kv[3, :512], o.shape), rtol=1e-13)
    np.testing.assert_allclose(lse, sm * (q @ kv[3]), rtol=1e-12)
    # zero query: equal logits -> mean of values, LSE = ln n
    o, lse = O.mla_attend(np.zeros_like(q), codes, c, sm)
    np.testing.assert_allclose(o, np.broadcast_to(kv[:, :512].mean(0), o.shape), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(40.0), rtol=1e-14)
    # order of the selected rows does not matter
    perm = np.random.default_rng(0).permutation(40)
    o1, l1 = O.mla_attend(q, codes, c, sm)
    o2, l2 = O.mla_attend(q, codes[perm], c, sm)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    # empty selection
    o, lse = O.mla_attend(q, codes[:0], c, sm)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_topk_equal_to_context_reproduces_dense_mla():
    q, codes, c, sm = _rand_mla(10, 97)
    sel = O.topk_indices(np.random.default_rng(1).normal(size=97).astype(np.float32), 97)
    o_s, l_s = O.mla_attend(q, codes[sel], c, sm)
    o_d, l_d = O.dense_mla(q, codes, c, sm)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-13)


# --------------------------------------------------------------- LSE combine
@pytest.mark.parametrize("num_splits", [1, 2, 5, 16])
def test_split_then_combine_equals_unsplit(num_splits):
    q, codes, c, sm = _rand_mla(11, 70)
    full = O.mla_attend(q, codes, c, sm)
    parts = [O.mla_attend(q, codes[a:b], c, sm) for a, b in O.split_ranges(70, num_splits)]
    o, lse = O.lse_combine(parts)
    np.testing.assert_allclose(o, full[0], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lse, full[1], rtol=1e-13)


def test_combine_with_empty_parts_and_two_split_closed_form():
    q, codes, c, sm = _rand_mla(12, 30)
    full = O.mla_attend(q, codes, c, sm)
    parts = [O.mla_attend(q, codes[:0], c, sm), O.mla_attend(q, codes[:12], c, sm),
             O.mla_attend(q, codes[12:12], c, sm), O.mla_attend(q, codes[12:], c, sm)]
    o, lse = O.lse_combine(parts)
    np.testing.assert_allclose(o, full[0], rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lse, full[1], rtol=1e-13)
    (o1, l1), (o2, l2) = parts[1], parts[3]
    # two splits: O = (e^l1 O1 + e^l2 O2) / (e^l1 + e^l2), LSE = ln(e^l1 + e^l2)
    ref_l = np.log(np.exp(l1) + np.exp(l2))
    ref_o = (np.exp(l1)[:, None] * o1 + np.exp(l2)[:, None] * o2) / (np.exp(l1) + np.exp(l2))[:, None]
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13)
    np.testing.assert_allclose(o, ref_o, rtol=1e-11, atol=1e-14)
    allempty = O.lse_combine([parts[0], parts[2]])
    assert (allempty[0] == 0).all() and np.isneginf(allempty[1]).all()


def test_split_ranges_partition():
    for n, s in [(2048, 16), (2048, 7), (5, 8), (0, 3)]:
        r = O.split_ranges(n, s)
        assert len(r) == s and r[0][0] == 0 and r[-1][1] == n
        assert all(a <= b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(s - 1))


# ---------------------------------------------------------------- whole row
def test_decode_row_small_batch(small_batch):
    b = small_batch
    pool, lat, bt = b.key_pool.numpy(), b.latent_pool.numpy(), b.block_table.numpy()
    qi = b.q_idx.double().numpy()
    qm = b.q_mla.double().numpy()
    w = b.head_w.numpy()
    rows = b.wl.row_positions()
    for i, (r, pos) in enumerate(rows):
        L = b.wl.seq_lens[r]
        kc, ks = O.read_index_keys(pool, bt[r], L)
        lc = O.read_latents(lat, O.physical_slot(bt[r], np.arange(L)))
        out = O.decode_row(qi[i], w[i], qm[i], kc, ks, lc, b.latent_scale, b.softmax_scale,
                           pos, b.wl.topk, bt[r])
        assert len(out["topk"]) == min(b.wl.topk, pos + 1)
        assert out["topk"].max() <= pos
        assert np.isfinite(out["o"]).all() and np.isfinite(out["lse"]).all()
        if pos + 1 <= b.wl.topk:   # every visible token selected: sparse == dense
            o_d, l_d = O.dense_mla(qm[i], lc[:pos + 1], b.latent_scale, b.softmax_scale)
            np.testing.assert_allclose(out["o"], o_d, rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(out["lse"], l_d, rtol=1e-12)


# ------------------------------------------------------------------------ cache append
def _append_inputs(seed, n, scale_mag=1.0):
    rng = np.random.default_rng(seed)
    k = (rng.normal(size=(n, 128)) * scale_mag).astype(np.float32)
    x = rng.normal(size=(n, 576)).astype(np.float32)
    kb = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return kb, xb


def test_cache_append_codes_scales_and_layout():
    pages, n = 6, 40
    key_pool = np.full((pages, 8448), 0x7F, dtype=np.uint8)
    key_pool[:, 8192:] = np.full((pages, 64), np.nan, dtype=np.float32).view(np.uint8)
    lat_pool = np.full((pages, 64 * 576), 0x7F, dtype=np.uint8)
    rng = np.random.default_rng(3)
    slots = rng.choice(pages * 64, size=n, replace=False).astype(np.int64)
    slots[5] = -1                                      # skipped
    kb, xb = _append_inputs(4, n)
    kb[7] = 0                                          # all-zero key: scale 1, codes 0
    kb[9] = torch.tensor([1e-30] * 128).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lat_scale = np.float32(0.0123)
    key_before, lat_before = key_pool.copy(), lat_pool.copy()
    O.cache_append(key_pool, lat_pool, slots, kb, xb, float(lat_scale))
    kf = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).float().numpy()
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    touched_k = np.zeros_like(key_pool, dtype=bool)
    touched_l = np.zeros_like(lat_pool, dtype=bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        page, o = int(slot // 64), int(slot % 64)
        codes, scales = O.read_index_keys(key_pool, np.array([page]), 64)
        a = np.float32(np.abs(kf[i]).max())
        sc = np.float32(a / np.float32(448)) if a > 0 else np.float32(1)
        assert scales[o] == sc
        # the codes are torch's own E4M3 conversion of k / s in fp32
        assert np.array_equal(codes[o], _torch_e4m3(kf[i] / sc)), i
        lat = O.read_latents(lat_pool, np.array([slot]))[0]
        assert np.array_equal(lat, _torch_e4m3(xf[i] / lat_scale)), i
        for d in range(128):
            touched_k[page, (d // 16) * 1024 + o * 16 + d % 16] = True
        touched_k[page, 8192 + 4 * o: 8192 + 4 * o + 4] = True
        touched_l[page, o * 576:(o + 1) * 576] = True
    # nothing else changed
    assert np.array_equal(key_pool[~touched_k], key_before[~touched_k])
    assert np.array_equal(lat_pool[~touched_l], lat_before[~touched_l])
    # the zero key and the absmax element
    p7, o7 = int(slots[7] // 64), int(slots[7] % 64)
    c7, s7 = O.read_index_keys(key_pool, np.array([p7]), 64)
    assert s7[o7] == 1.0 and (c7[o7] == 0).all()
    c0, s0 = O.read_index_keys(key_pool, np.array([int(slots[0] // 64)]), 64)
    assert np.abs(O.e4m3_decode(c0[int(slots[0] % 64)])).max() == 448.0


# ------------------------------------------------------------------------ MXFP4 index keys
def test_e8m0_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).double().numpy()
    got = O.e8m0_value(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e2m1_decode_is_the_ocp_table():
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]     # OCP MX v1.0, E2M1 magnitudes
    got = O.e2m1_decode(np.arange(16))
    assert np.array_equal(got[:8], table)
    assert np.array_equal(got[8:], [-v for v in table])
    assert np.signbit(got[8])                               # -0


def _mx_reference(raw):
    """Brute-force OCP MX quantisation of fp32 keys [n, 128] -> dequantised values: per
    block of 32 the scale 2^(floor(log2 absmax) - 2) (exactly, via frexp), each element the
    nearest E2M1 value of x / scale (ties to the even code), saturated at 6."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = np.empty(raw.shape, dtype=np.float64)
    for t in range(raw.shape[0]):
        for blk in range(4):
            x = raw[t, 32 * blk:32 * blk + 32].astype(np.float64)
            amax = np.abs(x).max()
            e = (math.frexp(amax)[1] - 1 - 2) if amax > 0 else 0
            sc = 2.0 ** e
            for j, v in enumerate(x):
                a = min(abs(v) / sc, 6.0)
                best = min(range(8), key=lambda c: (abs(grid[c] - a), c % 2))
                out[t, 32 * blk + j] = math.copysign(grid[best] * sc, v)
    return out


def test_mxfp4_cache_reader_matches_reference_quantisation():
    wl = synth.custom([130, 64], [1, 1], topk=16, seed=17, key_format="mxfp4")
    b = synth.make_batch(wl, "cpu", keep_logical=True)
    pool, bt = b.key_pool.numpy(), b.block_table.numpy()
    for r, L in enumerate(wl.seq_lens):
        got = O.read_index_keys_mxfp4(pool, bt[r], L)
        raw = b.keys_logical[r].numpy()
        ref = _mx_reference(raw)
        assert np.array_equal(got, ref), r
        # within the MX error: half a grid step, or the saturation at 6 * scale
        assert np.isfinite(got).all()


def test_mxfp4_encode_ties_saturation_and_scales():
    # one block per row of this table: (values, expected magnitudes after decoding)
    x = np.zeros((1, 128))
    # block 0: absmax 5 -> floor(log2 5) = 2 -> scale 2^0; the E2M1 grid's tie points go to
    # the even code: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    x[0, :11] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0, -0.75, -0.1, 0.2]
    # block 1: absmax 7.5 -> scale 2^0 and saturation at 6; 5.5 is nearest 6
    x[0, 32:35] = [7.5, -5.5, 0.5]
    # block 2: absmax 0.3 -> floor(log2 0.3) = -2 -> scale 2^-4 (0.3 / 2^-4 = 4.8 -> 4)
    x[0, 64:66] = [0.3, -0.03125]
    # block 3: all zero except a -0.0: scale 2^0, codes 0 and -0
    x[0, 96] = -0.0
    nib, sb = O.mxfp4_encode(x)
    assert sb.tolist() == [[127, 127, 123, 127]]
    dec = O.e2m1_decode(nib[0]) * O.e8m0_value(np.repeat(sb[0], 32))
    assert dec[:11].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 4.0, -1.0, -0.0, 0.0]
    assert nib[0, 9] == 8 and nib[0, 10] == 0          # -0.1 rounds to -0, 0.2 to +0
    assert dec[32:35].tolist() == [6.0, -6.0, 0.5]
    assert dec[64:66].tolist() == [0.25, -0.03125]
    assert nib[0, 96] == 8 and (nib[0, 97:] == 0).all()
    # the E8M0 floor: a block of fp32 subnormals keeps the scale 2^-127
    tiny = np.zeros((1, 128))
    tiny[0, 0] = 2.0 ** -140
    nib, sb = O.mxfp4_encode(tiny)
    assert sb[0, 0] == 0 and nib[0, 0] == 0            # 2^-140 / 2^-127 = 2^-13 -> 0


def test_mxfp4_encode_reproduces_grid_values():
    # values on a block's own E2M1 grid (one element of magnitude 4 or 6 fixing the scale)
    # come back bit for bit
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=(20, 128))
    codes[:, ::32] = rng.choice([6, 7, 14, 15], size=(20, 4))
    e = rng.integers(-30, 30, size=(20, 4))
    x = O.e2m1_decode(codes) * np.repeat(2.0 ** e, 32, axis=1)
    nib, sb = O.mxfp4_encode(x)
    assert np.array_equal(sb, (e + 127).astype(np.uint8))
    assert np.array_equal(nib, codes)


def test_mxfp4_encode_matches_brute_force_and_the_input_generator():
    rng = np.random.default_rng(12)
    raw = (rng.normal(size=(6, 128)) * 2.0 ** rng.integers(-8, 8, size=(6, 1))).astype(np.float32)
    nib, sb = O.mxfp4_encode(raw)
    got = O.e2m1_decode(nib) * np.repeat(O.e8m0_value(sb), 32, axis=1)
    assert np.array_equal(got, _mx_reference(raw))
    # the synthetic MXFP4 pool is written by an independent quantiser: same bytes
    wl = synth.custom([100], [1], topk=16, seed=19, key_format="mxfp4")
    b = synth.make_batch(wl, "cpu", keep_logical=True)
    pool, bt = b.key_pool.numpy(), b.block_table.numpy()
    nib, sb = O.mxfp4_encode(b.keys_logical[0].numpy())
    for t in range(100):
        page, o = bt[0, t // 64], t % 64
        for d in range(0, 128, 2):
            assert pool[page, (d // 32) * 1024 + o * 16 + (d % 32) // 2] == nib[t, d] | (nib[t, d + 1] << 4)
        assert np.array_equal(pool[page, 4096 + 4 * o:4100 + 4 * o], sb[t])


def test_cache_append_mxfp4_keys_and_layout():
    pages, n = 5, 30
    key_pool = np.full((pages, O.MX_PAGE_BYTES), 0x77, dtype=np.uint8)
    key_pool[:, O.MX_PAGE_KEY_BYTES:] = 0xFF
    rng = np.random.default_rng(13)
    slots = rng.choice(pages * 64, size=n, replace=False).astype(np.int64)
    slots[4] = -1                                      # skipped
    kb, _ = _append_inputs(14, n)
    kb[6] = 0                                          # all-zero key: scale 2^0, codes 0
    before = key_pool.copy()
    O.cache_append(key_pool, None, slots, kb, None, 1.0, key_format="mxfp4")
    kf = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).float().numpy()
    touched = np.zeros_like(key_pool, dtype=bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        page, o = int(slot // 64), int(slot % 64)
        vals = O.read_index_keys_mxfp4(key_pool, np.array([page]), 64)[o]
        assert np.array_equal(vals, _mx_reference(kf[i:i + 1])[0]), i
        for blk in range(4):
            touched[page, blk * 1024 + o * 16:blk * 1024 + o * 16 + 16] = True
        touched[page, 4096 + 4 * o:4100 + 4 * o] = True
    assert np.array_equal(key_pool[~touched], before[~touched])
    p6, o6 = int(slots[6] // 64), int(slots[6] % 64)
    assert (key_pool[p6, 4096 + 4 * o6:4100 + 4 * o6] == 127).all()


def test_index_scores_values_brute_force():
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.normal(size=(32, 128)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    w = (rng.normal(size=32) / math.sqrt(32)).astype(np.float32)
    kv = O.e2m1_decode(rng.integers(0, 16, size=(12, 128))) * 2.0 ** rng.integers(-3, 3, size=(12, 1))
    got = O.index_scores_values(q, w, kv).astype(np.float64)
    qd = O.dequantized_query(q).tolist()
    for t in range(12):
        acc = 0.0
        for h in range(32):
            dot = 0.0
            for d in range(128):
                dot += qd[h][d] * kv[t][d]
            acc += float(w[h]) * (dot if dot > 0 else 0.0)
        assert abs(got[t] - acc) <= 1e-6 * max(1.0, abs(acc)), t
