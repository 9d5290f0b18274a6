"""How far the E4M3 query quantisation moves the path's results from a bf16-exact query.

TEST INFRASTRUCTURE ONLY (CPU, oracle and the seeded input generator; nothing of the HIP
library).  The K3.1 page's fused indexer front quantises the indexer query to FP8 before
scoring ("Fused low-latency decode for DSA layers" / DSA層のための融合低レイテンシデコード)
and is silent on the MLA query; the kernels quantise both (one power-of-two scale per
(row, head)).  This script measures, on seeded inputs drawn like the decode workloads
(bf16 N(0,1) queries, N(0, 1/32) head weights, E4M3 keys and latents from N(0,1)), the
deviation of every stage from the same stage evaluated on the unquantised bf16 query:

  indexer   |s_q - s_x| / max(|s_x|, A_t), with A_t the same head sum over |w| (the
            tolerance form of the parity tests), and the plain relative error
  top-k     overlap of the two top-2048 sets
  MLA       |O_q - O_x| and |LSE_q - LSE_x| over the exact query's selected tokens

Usage: python -m oracle.query_quantisation_report [--rows 4] [--context 131072]
"""
from __future__ import annotations

import argparse
import json

import numpy as np

from oracle import dsa_oracle as O


def _row_inputs(batch, row, b):
    L = batch.wl.seq_lens[b]
    bt = batch.block_table[b].numpy()
    kc, ks = O.read_index_keys(batch.key_pool.numpy(), bt, L)
    lat = O.read_latents(batch.latent_pool.numpy(), O.physical_slot(bt, np.arange(L)))
    return (batch.q_idx[row].double().numpy(), batch.head_w[row].numpy(),
            batch.q_mla[row].double().numpy(), kc, ks, lat)


def report(rows: int = 4, context: int = 131072, topk: int = 2048, seed: int = 31) -> dict:
    import synth  # seeded generator shared by the tests and the benchmark

    wl = synth.custom([context] * rows, [1] * rows, topk=topk, seed=seed)
    batch = synth.make_batch(wl, "cpu")
    score_tol, score_rel, overlap, d_o, d_lse = [], [], [], [], []
    for row, (b, pos) in enumerate(wl.row_positions()):
        qi, w, qm, kc, ks, lat = _row_inputs(batch, row, b)
        n = pos + 1
        s_q = O.index_scores(qi, w, kc[:n], ks[:n]).astype(np.float64)
        s_x = O.index_scores(qi, w, kc[:n], ks[:n], quantize_query=False).astype(np.float64)
        a_t = O.index_scores(qi, np.abs(w), kc[:n], ks[:n], quantize_query=False).astype(np.float64)
        score_tol.append(np.abs(s_q - s_x) / np.maximum(np.abs(s_x), a_t))
        nz = np.abs(s_x) > 0
        score_rel.append(np.abs(s_q - s_x)[nz] / np.abs(s_x)[nz])
        sel_q = O.topk_indices(s_q.astype(np.float32), topk)
        sel_x = O.topk_indices(s_x.astype(np.float32), topk)
        overlap.append(len(np.intersect1d(sel_q, sel_x)) / len(sel_x))
        o_q, l_q = O.mla_attend(qm, lat[sel_x], batch.latent_scale, batch.softmax_scale)
        o_x, l_x = O.mla_attend(qm, lat[sel_x], batch.latent_scale, batch.softmax_scale,
                                quantize_query=False)
        d_o.append(np.abs(o_q - o_x).ravel())
        d_lse.append(np.abs(l_q - l_x))
    st, sr, do, dl = (np.concatenate(x) for x in (score_tol, score_rel, d_o, d_lse))
    return {
        "rows": rows, "context": context, "topk": topk, "seed": seed,
        "score_dev_over_max_abs_and_A": {"median": float(np.median(st)), "p99": float(np.quantile(st, 0.99)),
                                         "max": float(st.max())},
        "score_plain_rel_err": {"median": float(np.median(sr)), "p99": float(np.quantile(sr, 0.99))},
        "topk_set_overlap": {"min": float(min(overlap)), "mean": float(np.mean(overlap))},
        "mla_abs_dO": {"median": float(np.median(do)), "max": float(do.max())},
        "mla_abs_dLSE": {"median": float(np.median(dl)), "max": float(dl.max())},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=4)
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--topk", type=int, default=2048)
    ap.add_argument("--seed", type=int, default=31)
    a = ap.parse_args()
    print(json.dumps(report(a.rows, a.context, a.topk, a.seed), indent=1))


if __name__ == "__main__":
    main()
