"""Pins against figures the K3.1 page prints (tests/golden/k31_page_figures.json): the
per-token byte widths of the two caches, the indexer's head count and k, the MXFP4 saving
and the DSA / dense-MLA byte ratio at long context.  They check the oracle's page readers,
the seeded input generator's pools, the C header's layout constants and the benchmark's
byte model against the page, not against themselves."""
import json
import os
import re

import numpy as np
import torch

import bench
import oracle as O
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def figures():
    d = json.load(open(os.path.join(HERE, "golden", "k31_page_figures.json")))
    return {f["name"]: f["value"] for f in d["figures"]}


def header_defines():
    txt = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (DSA_\w+) (\d+)", txt)}


def test_header_page_sizes_are_64_tokens_of_the_page_widths():
    f, h = figures(), header_defines()
    assert h["DSA_IDX_PAGE_BYTES"] == 64 * f["index_key_fp8_bytes_per_token"]
    assert h["DSA_IDX_MXFP4_PAGE_BYTES"] == 64 * f["index_key_mxfp4_bytes_per_token"]
    assert h["DSA_LATENT_PAGE_BYTES"] == 64 * f["latent_fp8_bytes_per_token"]
    assert h["DSA_LATENT_DIM"] == f["latent_fp8_bytes_per_token"]   # one E4M3 byte per dim


def test_oracle_page_layouts_match_the_page_widths():
    f = figures()
    # E4M3 key page: 128 code bytes + one fp32 scale per token
    assert O.IDX_PAGE_KEY_BYTES + O.PAGE * 4 == O.PAGE * f["index_key_fp8_bytes_per_token"]
    assert O.MX_PAGE_BYTES == O.PAGE * f["index_key_mxfp4_bytes_per_token"]
    assert O.LAT_ROW == f["latent_fp8_bytes_per_token"]
    # the oracle's E4M3 reader takes pages of exactly that width: one page whose token o has
    # every code 0x38 (1.0) and scale o + 1 reads back as keys of value o + 1
    page = np.zeros((1, O.PAGE * f["index_key_fp8_bytes_per_token"]), dtype=np.uint8)
    page[0, : O.IDX_PAGE_KEY_BYTES] = 0x38
    page[0, O.IDX_PAGE_KEY_BYTES:] = np.arange(1, O.PAGE + 1, dtype=np.float32).view(np.uint8)
    codes, scales = O.read_index_keys(page, np.array([0]), O.PAGE)
    vals = O.e4m3_decode(codes) * scales[:, None]
    assert np.array_equal(vals, np.repeat(np.arange(1, O.PAGE + 1, dtype=np.float64)[:, None], 128, 1))


def test_generator_pools_have_the_page_widths():
    f = figures()
    wl = synth.custom([100], [1], topk=64, seed=7)
    b = synth.make_batch(wl, "cpu")
    assert b.key_pool.shape[1] == 64 * f["index_key_fp8_bytes_per_token"]
    assert b.latent_pool.shape[1] == 64 * f["latent_fp8_bytes_per_token"]
    assert b.q_idx.shape[1] == f["indexer_heads"]
    wl = synth.custom([100], [1], topk=64, seed=7, key_format="mxfp4")
    assert synth.make_batch(wl, "cpu").key_pool.shape[1] == 64 * f["index_key_mxfp4_bytes_per_token"]


def test_workloads_use_the_page_topk():
    f = figures()
    for name in synth.WORKLOADS:
        assert synth.workload(name).topk == f["topk"]


def test_mxfp4_saving_matches_the_page():
    f = figures()
    saving = 1 - f["index_key_mxfp4_bytes_per_token"] / f["index_key_fp8_bytes_per_token"]
    assert round(saving, 3) == f["mxfp4_index_storage_reduction"]
    assert bench.MX_IDX_BYTES_PER_TOKEN == f["index_key_mxfp4_bytes_per_token"]
    assert bench.IDX_BYTES_PER_TOKEN == f["index_key_fp8_bytes_per_token"]


def test_dsa_bytes_are_about_23_percent_of_dense_at_long_context():
    # the byte model of the benchmark on the longest workload (1,048,576 tokens): index keys
    # of every token plus the latents of the selected 2,048, over every token's latent
    f = figures()
    L = synth.workload("million").seq_lens[0]
    ab = bench.algorithmic_bytes([L], [1], f["topk"])
    ratio = (ab["index_keys"] + ab["latents"]) / bench.dense_mla_bytes([L], [1])
    assert round(ratio, 2) == f["dsa_bytes_fraction_of_dense_long_context"]
