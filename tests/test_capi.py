"""Host-side checks of the C ABI: the library loads, exports every declared entry point,
and rejects bad host arguments with the documented status before launching anything.
None of these calls reaches the GPU."""
import ctypes
import os
import re

import pytest

import sparse_attention_decode_score_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.LIB_PATH):
        from sparse_attention_decode_score_amd import build
        build.build()
    return dsa.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"dsa_index_score", "dsa_topk", "dsa_topk_workspace_size", "dsa_sparse_mla_decode",
            "dsa_sparse_mla_workspace_size", "dsa_topk_sparse_mla", "dsa_lse_combine", "dsa_cache_append", "dsa_cache_append_mxfp4", "dsa_quantize_q", "dsa_last_error",
            "dsa_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version(L):
    assert "gfx950" in dsa.dsa_version()


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every call below fails validation
FAKE_ODD = ctypes.c_void_p(0x1001)


def _err():
    return dsa.lib().dsa_last_error().decode()


def test_index_score_rejects_bad_host_args(L):
    f = L.dsa_index_score
    cand_need = L.dsa_topk_workspace_size(3, 1000, 2048)
    assert cand_need > 0
    ok_args = [2, 3, 1000, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 8448, FAKE, 16, FAKE, 1000, 2048,
               ctypes.c_void_p(0x10000), cand_need, None]
    bad = dict(enumerate(ok_args))
    cases = [({0: 0}, 1, "num_seqs"), ({1: 1}, 1, "n_q"), ({2: 0}, 1, "max_seq_len"),
             ({3: 0}, 1, "max_q_per_seq"), ({4: None}, 1, "cu_q"), ({8: None}, 1, "key_pages"),
             ({9: 8447}, 1, "key_page_stride"), ({9: 8456}, 1, "key_page_stride"),
             ({11: 15}, 1, "bt_stride"), ({13: 999}, 1, "score_stride"),
             ({6: FAKE_ODD}, 1, "aligned"), ({14: 0}, 2, "cand_k"), ({14: 4097}, 2, "cand_k"),
             ({16: cand_need - 1}, 3, "workspace"), ({12: None, 15: None}, 1, "scores"),
             ({15: ctypes.c_void_p(0x10010)}, 1, "aligned")]
    for patch, status, word in cases:
        args = list(ok_args)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == status, patch
        assert word in _err(), (patch, _err())


def test_topk_rejects_bad_host_args(L):
    f = L.dsa_topk
    for fused in (0, 1):
        need = L.dsa_topk_workspace_size(3, 1000, 2048)
        assert need > 0
        base = [2, 3, 1000, FAKE, FAKE, FAKE, 1000, 2048, FAKE, 16, FAKE, FAKE,
                ctypes.c_void_p(0x10000), need, fused, None, None, None, 0, 0, None]
        for patch, status in [({7: 0}, 2), ({7: 4097}, 2), ({8: None}, 1), ({6: 10}, 1),
                              ({13: need - 1}, 3), ({12: None}, 3),
                              ({12: ctypes.c_void_p(0x10010)}, 1)]:
            args = list(base)
            for i, v in patch.items():
                args[i] = v
            assert f(*args) == status, (fused, patch, _err())
    # recomputation inputs: all or none, only with candidates, with a block table
    base = [2, 3, 1000, FAKE, FAKE, FAKE, 1000, 2048, FAKE, 16, FAKE, FAKE,
            ctypes.c_void_p(0x10000), L.dsa_topk_workspace_size(3, 1000, 2048), 1,
            FAKE, FAKE, FAKE, 8448, 0, None]
    for patch, status, word in [
            ({16: None}, 1, "all"), ({14: 0}, 1, "from_candidates"),
            ({8: None, 11: None}, 1, "block_table"), ({18: 8447}, 1, "key_page_stride"),
            ({15: FAKE_ODD}, 1, "aligned"), ({19: 2}, 2, "key_format"),
            ({19: -1}, 2, "key_format"),
            # MXFP4 keys: 4,352-byte pages; E4M3 keys need 8,448
            ({18: 4351, 19: 1}, 1, "key_page_stride"), ({18: 4352}, 1, "key_page_stride")]:
        args = list(base)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == status, (patch, _err())
        assert word in _err(), (patch, _err())
    assert L.dsa_topk_workspace_size(0, 10, 10) == 0
    assert L.dsa_topk_workspace_size(4, 10, 5000) == 0


def test_sparse_mla_and_combine_reject_bad_host_args(L):
    f = L.dsa_sparse_mla_decode
    need = L.dsa_sparse_mla_workspace_size(4, 4)
    assert need >= 4 * 4 * 96 * 512 * 2
    assert L.dsa_sparse_mla_workspace_size(0, 4) == 0 and L.dsa_sparse_mla_workspace_size(4, 65) == 0
    WS = ctypes.c_void_p(0x10000)
    # n_q, q_bf16, q8, q_scale, latent, stride, lat_scale, slots, k, sm, S, out, lse, o_part,
    # lse_part, workspace, ws_bytes, stream: merged output through the workspace
    base = [4, FAKE, None, None, FAKE, 36864, ctypes.c_float(0.01), FAKE, 2048,
            ctypes.c_float(0.04), 4, FAKE, FAKE, None, None, WS, need, None]
    for patch, status in [({0: 0}, 1), ({8: 0}, 2), ({10: 0}, 2), ({10: 65}, 2), ({5: 36863}, 1),
                          ({6: ctypes.c_float(0.0)}, 1), ({7: None}, 1), ({4: FAKE_ODD}, 1),
                          ({16: need - 1}, 3), ({15: None}, 3), ({15: ctypes.c_void_p(0x10010)}, 1),
                          ({1: None}, 1), ({2: FAKE}, 1), ({1: FAKE_ODD}, 1), ({11: None}, 1),
                          ({13: FAKE}, 1)]:
        args = list(base)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == status, (patch, _err())
    args = list(base)
    args[8], args[10] = 3, 4                     # more splits than selected tokens
    assert f(*args) == 1
    args = list(base)                            # fp32 partials: no workspace needed
    args[11] = args[12] = None
    args[13] = args[14] = FAKE
    args[15], args[16] = None, 0
    args[0] = 0                                  # (stopped by n_q, after the layout checks)
    assert f(*args) == 1 and "n_q" in _err()
    g = L.dsa_lse_combine
    assert g(0, 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert g(65, 4, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert g(4, 0, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert g(4, 4, None, FAKE, FAKE, FAKE, None) == 1


def test_topk_sparse_mla_rejects_bad_host_args(L):
    f = L.dsa_topk_sparse_mla
    cand = L.dsa_topk_workspace_size(4, 1000, 512)
    need = L.dsa_sparse_mla_workspace_size(4, 4)
    CW, WS = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    # num_seqs, n_q, max_seq_len, cu_q, seq_lens, scores, score_stride, k, block_table,
    # bt_stride, cand_ws, cand_bytes, q_idx, head_w, key_pages, key_stride, key_format,
    # topk_idx, topk_slot, q_bf16, q8, q_scale, latent, latent_stride, latent_scale,
    # softmax_scale, S, out, lse, workspace, ws_bytes, stream
    base = [2, 4, 1000, FAKE, FAKE, FAKE, 1000, 512, FAKE, 16, CW, cand, None, None, None, 0, 0,
            None, None, FAKE, None, None, FAKE, 36864, ctypes.c_float(0.01),
            ctypes.c_float(0.04), 4, FAKE, FAKE, WS, need, None]
    RS = {12: FAKE, 13: FAKE, 14: FAKE}
    cases = [({0: 0}, 1, "num_seqs"), ({7: 0}, 2, "k"), ({7: 4097}, 2, "k"),
             ({26: 65}, 2, "num_splits"), ({8: None}, 1, "block_table"),
             ({5: None}, 1, "scores"), ({6: 999}, 1, "score_stride"), ({9: 15}, 1, "bt_stride"),
             ({10: None}, 3, "candidate"), ({11: cand - 1}, 3, "candidate"),
             ({10: ctypes.c_void_p(0x10010)}, 1, "cand_workspace"),
             ({12: FAKE}, 1, "all"), ({**RS, 15: 100}, 1, "key_page_stride"),
             ({**RS, 15: 8448, 16: 3}, 2, "key_format"),
             ({**RS, 15: 4351, 16: 1}, 1, "key_page_stride"),
             ({19: None}, 1, "query"), ({20: FAKE}, 1, "q8"), ({22: None}, 1, "latent_pages"),
             ({23: 36863}, 1, "latent_page_stride"), ({27: None}, 1, "out_bf16"),
             ({29: None}, 3, "workspace"), ({30: need - 1}, 3, "workspace")]
    for patch, status, word in cases:
        args = list(base)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == status, (patch, _err())
        assert word in _err(), (patch, _err())
    args = list(base)
    args[7], args[26] = 3, 4                     # more splits than selected tokens
    assert f(*args) == 1 and "num_splits" in _err()


def test_quantize_rejects_bad_dim(L):
    assert L.dsa_quantize_q(1, 1, 100, FAKE, FAKE, FAKE, None) == 2
    assert "dim" in _err()
    assert L.dsa_quantize_q(1, 1, 128, None, FAKE, FAKE, None) == 1


def test_python_binding_refuses_host_tensors(L):
    import torch
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dsa.dsa_quantize_q(q, torch.zeros((1, 32, 128), dtype=torch.uint8), torch.zeros((1, 32)))


def test_cache_append_rejects_bad_host_args(L):
    f = L.dsa_cache_append
    base = [4, FAKE, FAKE, FAKE, ctypes.c_float(0.01), FAKE, 8448, FAKE, 36864, None]
    for patch, word in [({0: -1}, "n_tok"), ({1: None}, "slots"), ({2: None, 3: None}, "give"),
                        ({5: None}, "key_pages"), ({6: 8447}, "key_page_stride"),
                        ({7: None}, "latent_pages"), ({8: 100}, "latent_page_stride"),
                        ({4: ctypes.c_float(0.0)}, "latent_scale"), ({2: FAKE_ODD}, "aligned")]:
        args = list(base)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == 1, (patch, _err())
        assert word in _err(), (patch, _err())
    # a cache that is not given is not checked
    args = list(base)
    args[3], args[7], args[8] = None, None, 0
    args[0] = -1
    assert f(*args) == 1 and "n_tok" in _err()


def test_cache_append_mxfp4_rejects_bad_host_args(L):
    f = L.dsa_cache_append_mxfp4
    base = [4, FAKE, FAKE, FAKE, ctypes.c_float(0.01), FAKE, 4352, FAKE, 36864, None]
    for patch, word in [({0: -1}, "n_tok"), ({1: None}, "slots"), ({2: None, 3: None}, "give"),
                        ({5: None}, "key_pages"), ({6: 4351}, "key_page_stride"),
                        ({6: 4360}, "key_page_stride"), ({2: FAKE_ODD}, "aligned"),
                        ({4: ctypes.c_float(0.0)}, "latent_scale")]:
        args = list(base)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == 1, (patch, _err())
        assert word in _err(), (patch, _err())
    # any stride of at least 4352 (a multiple of 16) is accepted; no tokens launch nothing
    args = list(base)
    args[0], args[6] = 0, 8448
    assert f(*args) == 0, _err()


def test_index_score_mxfp4_rejects_bad_host_args(L):
    f = L.dsa_index_score_mxfp4
    ok_args = [2, 3, 1000, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 4352, FAKE, 16, FAKE, 1000, 0,
               None, 0, None]
    for patch, word in [({9: 4351}, "key_page_stride"), ({12: None}, "scores"),
                        ({9: 4360}, "key_page_stride")]:
        args = list(ok_args)
        for i, v in patch.items():
            args[i] = v
        assert f(*args) == 1, (patch, _err())
        assert word in _err(), (patch, _err())


# ------------------------------------------------------------------ host-side validators
def _valid_batch():
    import numpy as np
    import synth
    import oracle as O
    wl = synth.custom([300, 130, 64], [1, 3, 2], topk=64, seed=7)
    b = synth.make_batch(wl, "cpu")
    bt = b.block_table.numpy()
    slots = np.full((wl.n_q, 64), -1, dtype=np.int32)
    for row, (r, pos) in enumerate(wl.row_positions()):
        sel = np.sort(np.random.default_rng(row).permutation(pos + 1)[:64])
        slots[row, :len(sel)] = O.physical_slot(bt[r], sel)
    return wl, b, slots


def test_validate_batch_accepts_a_valid_batch_and_names_each_violation(L):
    import numpy as np
    wl, b, slots = _valid_batch()
    cu, sl, bt = b.cu_q.numpy(), b.seq_lens.numpy(), b.block_table.numpy()
    kw = dict(max_seq_len=wl.max_seq_len, max_q_per_seq=3)
    dsa.dsa_validate_batch(cu, sl, bt, b.num_pages, topk_slot=slots, **kw)
    dsa.dsa_validate_batch(cu, sl, bt, b.num_pages, **kw)

    def bad(word, **over):
        args = dict(cu_q=cu, seq_lens=sl, block_table=bt, num_pages=b.num_pages, topk_slot=slots)
        args.update(over)
        with pytest.raises(dsa.DsaError) as e:
            dsa.dsa_validate_batch(args["cu_q"], args["seq_lens"], args["block_table"],
                                   args["num_pages"], topk_slot=args["topk_slot"], **kw)
        assert e.value.status == 1 and word in str(e.value), str(e.value)

    c2 = cu.copy(); c2[2] = c2[1]
    bad("query rows", cu_q=c2)                       # a request with no row
    s2 = sl.copy(); s2[1] = wl.max_seq_len + 1
    bad("seq_lens[1]", seq_lens=s2)
    s3 = sl.copy(); s3[2] = 1
    bad("only 1 tokens", seq_lens=s3)                # 2 rows on 1 token
    bt2 = bt.copy(); bt2[0, 4] = b.num_pages
    bad("block_table[0][4]", block_table=bt2)
    bt3 = bt.copy(); bt3[1, 1] = -1
    bad("block_table[1][1]", block_table=bt3)
    t2 = slots.copy(); t2[0, 5] = t2[0, 6]
    bad("twice", topk_slot=t2)
    t3 = slots.copy(); t3[0, 0] = -7
    bad("neither -1", topk_slot=t3)
    # a slot of the request's own pages but past the row's position (row 1 sits at 127;
    # token 129 is offset 1 of its third page)
    t4 = slots.copy(); t4[1, 0] = int(bt[1][2]) * 64 + 1
    bad("not a token row 1 sees", topk_slot=t4)
    # a slot of another request's page
    t5 = slots.copy(); t5[4, 0] = int(bt[0][0]) * 64
    bad("not a token row 4 sees", topk_slot=t5)
    with pytest.raises(dsa.DsaError):
        dsa.dsa_validate_batch(cu, sl, bt[:, :2], b.num_pages, **kw)  # bt_stride too small
    assert "bt_stride" in _err()


def test_topk_workspace_status_rejects_bad_host_args(L):
    # argument checks run before any device access, so they need no GPU
    L.dsa_topk_workspace_status.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert L.dsa_topk_workspace_status(None, 4096, None) == 1
    assert b"non-null" in L.dsa_last_error()
    assert L.dsa_topk_workspace_status(ctypes.c_void_p(256), 64, None) == 1
    assert b">= 256" in L.dsa_last_error()


def test_validate_slots(L):
    import numpy as np
    dsa.dsa_validate_slots(np.array([0, 5, -1, 64 * 9 + 63], np.int32), 10)
    dsa.dsa_validate_slots(np.zeros(0, np.int32), 1)
    for slots, word in (([3, 3], "twice"), ([640], "neither -1"), ([-2], "neither -1")):
        with pytest.raises(dsa.DsaError) as e:
            dsa.dsa_validate_slots(np.array(slots, np.int32), 10)
        assert word in str(e.value)
