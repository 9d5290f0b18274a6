"""Benchmark of the MI355X DSA decode hot path: one step = indexer scores -> top-2048 ->
sparse MLA over the selected latents -> LSE combine of the split partials, for every query
row of one synthetic batch (the four library calls on one stream).

Default workload: decode of 32 requests x 1 query row at 131,072 tokens of context each
(FP8 index keys 132 B/token, FP8 latents 576 B/token, top-2048, 8 attention splits).  Prints ONE
JSON line.  `value` is the whole step's algorithmic HBM traffic divided by its time (GB/s);
the JSON also carries us/layer, the indexer kernel's roofline, and the CPU oracle timed on
a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long|spec|...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, vendor figure
PAGE = 64
IDX_BYTES_PER_TOKEN = 132        # 128 B E4M3 key + 4 B fp32 scale
MX_IDX_BYTES_PER_TOKEN = 68      # MXFP4 key: 64 B of E2M1 codes + 4 E8M0 block scales


def idx_bytes_per_token(key_format):
    return MX_IDX_BYTES_PER_TOKEN if key_format == "mxfp4" else IDX_BYTES_PER_TOKEN
LAT_BYTES_PER_TOKEN = 576        # E4M3 latent
QIDX_BYTES_PER_ROW = 32 * 128 * 2 + 32 * 4     # bf16 indexer query + fp32 head weights
QMLA_BYTES_PER_ROW = 96 * 576 * 2              # bf16 MLA query
OUT_BYTES_PER_ROW = 96 * 512 * 2 + 96 * 4      # bf16 output + fp32 LSE
BT_BYTES_PER_PAGE = 4


def algorithmic_bytes(seq_lens, q_per_seq, topk, key_format="e4m3"):
    """Bytes the method itself must move for one step (the byte model of the K3.1 page's
    "Sparse attention cuts long-context decode bandwidth" section: the whole context's
    132-byte index keys (68 with MXFP4 keys) once per request, 576 bytes for each selected
    token of each row, plus queries, outputs and the block table).  Returns a dict of parts
    and the total."""
    keys = sum(L * idx_bytes_per_token(key_format) for L in seq_lens)
    lat = 0
    n_rows = 0
    for L, nq in zip(seq_lens, q_per_seq):
        for j in range(nq):
            pos = L - nq + j
            lat += min(topk, pos + 1) * LAT_BYTES_PER_TOKEN
        n_rows += nq
    bt = sum(((L + PAGE - 1) // PAGE) * BT_BYTES_PER_PAGE for L in seq_lens)
    q = n_rows * (QIDX_BYTES_PER_ROW + QMLA_BYTES_PER_ROW)
    out = n_rows * OUT_BYTES_PER_ROW
    parts = {"index_keys": keys, "latents": lat, "queries": q, "outputs": out, "block_table": bt}
    parts["total"] = sum(parts.values())
    return parts


def index_score_bytes(seq_lens, key_format="e4m3"):
    """Algorithmic bytes of one dsa_index_score launch: 132 B (MXFP4: 68 B) per context
    token of every request (keys are read once and shared by that request's rows)."""
    return sum(L * idx_bytes_per_token(key_format) for L in seq_lens)


FP8_MFMA_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 matrix peak (no sparsity), vendor figure
IDX_FLOP_PER_ROW_TOKEN = 32 * 128 * 2      # indexer q.k over 32 heads x 128 dims
MLA_FLOP_PER_ROW_TOKEN = 96 * (576 + 512) * 2  # logits over 576 dims + values over 512, 96 heads


def index_score_flops(wl):
    """Algorithmic FLOPs of one dsa_index_score launch: 8,192 per (row, visible token)."""
    return sum((pos + 1) * IDX_FLOP_PER_ROW_TOKEN for _, pos in wl.row_positions())


def sparse_mla_flops(wl):
    """Algorithmic FLOPs of the sparse MLA: 208,896 per (row, selected token)."""
    return sum(min(wl.topk, pos + 1) * MLA_FLOP_PER_ROW_TOKEN for _, pos in wl.row_positions())


def dense_mla_bytes(seq_lens, q_per_seq):
    """Bytes a dense-MLA decode reads for the same batch: every context token's latent."""
    return sum(L * LAT_BYTES_PER_TOKEN for L in seq_lens)


def _source_hash(name):
    p = os.path.join(ROOT, "sparse_attention_decode_score_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _traffic_from_profile():
    """HBM bytes per launch of the indexer from the committed counter summary, if it was
    taken on the current kernel sources; None otherwise."""
    p = os.path.join(ROOT, "profiles", "index_score_long_counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    hashes = d.get("source_sha256_16")
    if not isinstance(hashes, dict) or any(_source_hash(f) != v for f, v in hashes.items()):
        return None
    return d.get("hbm_bytes_per_launch")


def cache_append_timing(torch, dsa, batch, wl, steps):
    """dsa_cache_append (dsa_cache_append_mxfp4 for MXFP4 keys) of one new token per query
    row (its own position), timed with events over `steps` calls; run after everything else
    (it rewrites those tokens)."""
    import numpy as np
    bt = batch.block_table.cpu().numpy()
    slots = []
    for b, pos in wl.row_positions():
        slots.append(int(bt[b][pos // PAGE]) * PAGE + pos % PAGE)
    n = len(slots)
    slots_d = torch.tensor(slots, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(99)
    key = torch.randn((n, 128), generator=g, device="cuda").to(torch.bfloat16)
    lat = torch.randn((n, 576), generator=g, device="cuda").to(torch.bfloat16)
    mx = wl.key_format == "mxfp4"
    append = dsa.dsa_cache_append_mxfp4 if mx else dsa.dsa_cache_append
    for _ in range(3):
        append(slots_d, key, lat, batch.latent_scale, batch.key_pool, batch.latent_pool)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        append(slots_d, key, lat, batch.latent_scale, batch.key_pool, batch.latent_pool)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    return {"tokens": n, "us_per_call": round(us, 2),
            "note": ("one new token per query row: " +
                     ("its MXFP4 index key (68 B)" if mx else "its index key (132 B)") +
                     " and latent (576 B)" +
                     " quantised into the paged caches; calls back to back from Python, caches "
                     "warm")}


def cpu_baseline(batch, rows, budget_s=12.0, max_passes=64):
    """Times the oracle (as it stands) on a bounded sample of the same workload: the rows are
    taken in turn (cycling) until budget_s seconds of oracle time have been spent, and the
    throughput is returned in the benchmark's unit (algorithmic GB/s)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle as O

    wl = batch.wl
    rowpos = wl.row_positions()
    done, t_total, byts = 0, 0.0, 0
    stage_s = [0.0, 0.0, 0.0, 0.0]  # indexer, top-k, sparse MLA, LSE combine
    rows = list(rows)
    host = {}  # each sampled row's inputs, copied to the host once (outside the timing)
    for i in range(len(rows) * max_passes):
        row = rows[i % len(rows)]
        b, pos = rowpos[row]
        L = wl.seq_lens[b]
        if row not in host:
            pages = batch.block_table[b, : (L + 63) // 64].long()
            host[row] = (batch.key_pool[pages].cpu().numpy(), np.arange(len(pages)),
                         batch.q_idx[row].cpu().double().numpy(),
                         batch.head_w[row].cpu().numpy(),
                         batch.q_mla[row].cpu().double().numpy(),
                         batch.latent_pool[pages].cpu().numpy())
        key_pages, bt_local, qi, w, qm, lat_pages = host[row]
        t0 = time.perf_counter()
        if wl.key_format == "mxfp4":
            kv = O.read_index_keys_mxfp4(key_pages, bt_local, L)
            scores = O.index_scores_values(qi, w, kv[: pos + 1])
        else:
            kc, ks = O.read_index_keys(key_pages, bt_local, L)
            scores = O.index_scores(qi, w, kc[: pos + 1], ks[: pos + 1])
        t1 = time.perf_counter()
        sel = O.topk_indices(scores, wl.topk)
        t2 = time.perf_counter()
        lat = O.read_latents(lat_pages, O.physical_slot(bt_local, sel))
        parts = [O.mla_attend(qm, lat[a:e], batch.latent_scale, batch.softmax_scale)
                 for a, e in O.split_ranges(len(sel), wl.num_splits)]
        t3 = time.perf_counter()
        O.lse_combine(parts)
        t4 = time.perf_counter()
        stage_s[0] += t1 - t0
        stage_s[1] += t2 - t1
        stage_s[2] += t3 - t2
        stage_s[3] += t4 - t3
        t_total += t4 - t0
        # the row's share of the algorithmic bytes: its request's keys divided over the
        # request's rows, its selected latents, its query / output
        nq = wl.q_per_seq[b]
        byts += (L * idx_bytes_per_token(wl.key_format)) / nq + min(wl.topk, pos + 1) * LAT_BYTES_PER_TOKEN \
            + QIDX_BYTES_PER_ROW + QMLA_BYTES_PER_ROW + OUT_BYTES_PER_ROW
        done += 1
        if t_total > budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(byts / t_total / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "cores_note": "one Python process; cores = the BLAS threads numpy may use in the "
                          "oracle's matrix products (the rest of it runs on one core)",
            "cpu_model": cpu_model(), "kind": "oracle",
            "stage_s": {"index_score": round(stage_s[0], 3), "topk": round(stage_s[1], 3),
                        "sparse_mla": round(stage_s[2], 3), "lse_combine": round(stage_s[3], 3)},
            "sample": f"{done} query-row passes over the {len(rows)} rows of the {wl.name} "
                      f"workload taken in turn, whole path per row, {t_total:.1f} s of CPU "
                      f"time; GB/s = those rows' share of the algorithmic bytes / time"}


def _probe_lib():
    import ctypes
    import sparse_attention_decode_score_amd as dsa
    path = os.path.join(dsa.PKG, "lib", "libdsa_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the package first")
    L = ctypes.CDLL(path)
    L.dsa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    L.dsa_probe_page_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.dsa_probe_page_read_mx.argtypes = L.dsa_probe_page_read.argtypes
    return L


def page_read_ceiling(torch, batch):
    """Rate at which this GPU reads the workload's own index-key pages through its block
    table with the indexer's load pattern and no arithmetic (our probe kernel): the ceiling
    of the indexer's key stream, for E4M3 (8,448-byte) or MXFP4 (4,352-byte) pages."""
    wl = batch.wl
    L = _probe_lib()
    mx = wl.key_format == "mxfp4"
    read = L.dsa_probe_page_read_mx if mx else L.dsa_probe_page_read
    page_bytes = PAGE * (MX_IDX_BYTES_PER_TOKEN if mx else IDX_BYTES_PER_TOKEN)
    pages = torch.cat([batch.block_table[b, : (wl.seq_lens[b] + PAGE - 1) // PAGE]
                       for b in range(wl.num_seqs)]).contiguous()
    n = pages.numel()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    stride = batch.key_pool.stride(0)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        read(batch.key_pool.data_ptr(), stride, pages.data_ptr(), n, sink.data_ptr(), st)
    ts = []
    for _ in range(5):
        L.dsa_probe_stream_read(flush.data_ptr(), flush.numel(), sink.data_ptr(), 8192, st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        read(batch.key_pool.data_ptr(), stride, pages.data_ptr(), n, sink.data_ptr(), st)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del flush
    ts.sort()
    return n * page_bytes / ts[len(ts) // 2] / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def stream_read_ceiling(torch, n_bytes=4 << 30):
    """Achievable streaming-read rate of this GPU with ordinary loads (our probe kernel)."""
    L = _probe_lib()
    x = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        L.dsa_probe_stream_read(x.data_ptr(), n_bytes, sink.data_ptr(), 8192, st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        L.dsa_probe_stream_read(x.data_ptr(), n_bytes, sink.data_ptr(), 8192, st)
    e1.record()
    torch.cuda.synchronize()
    gbps = 5 * n_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x
    return gbps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--splits", type=int, default=0, help="sparse-attention splits (0 = workload default)")
    ap.add_argument("--no-flush", action="store_true", help="keep the 256 MB last-level cache warm")
    ap.add_argument("--unfused", action="store_true",
                    help="run stage 2 as both top-k passes instead of taking the indexer's "
                         "per-chunk candidates")
    ap.add_argument("--query-prep", choices=("fused", "inline", "first", "side"), default=None,
                    help="where the MLA query is quantised: inside the attention kernel "
                         "(default), by the indexer's launch, by its own launch ahead of stage 1, "
                         "or on a side stream during stages 1-2")
    ap.add_argument("--query-side-stream", action="store_true",
                    help="quantise the MLA query on a side stream during stages 1-2 instead of "
                         "inside the attention kernel")
    ap.add_argument("--store-scores", action="store_true",
                    help="have the indexer store its scores (by default with candidates it "
                         "stores none and the final pass recomputes what it re-reads)")
    ap.add_argument("--separate-topk", action="store_true",
                    help="run stage 2's final pass as its own kernel instead of inside the "
                         "attention kernel")
    ap.add_argument("--also-splits", type=int, nargs="*", default=None,
                    help="also time the step at these split counts (default: 16 for the long "
                         "workload, the split count of the pages' 16-chunk reading)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 512 MiB device copy (reference dispatch for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import sparse_attention_decode_score_amd as dsa

    wl = synth.workload(args.workload)
    S = args.splits or wl.num_splits
    torch.cuda.set_device(0)
    batch = synth.make_batch(wl, "cuda")
    def make_step(n_splits):
        return dsa.DecodeStep(wl.n_q, wl.max_seq_len, wl.topk, n_splits, fused=not args.unfused,
                              query_on_side_stream=args.query_side_stream,
                              query_prep=args.query_prep,
                              select_in_attention=not (args.separate_topk or args.unfused),
                              store_scores=True if (args.store_scores or args.unfused) else None,
                              key_format=wl.key_format,
                              write_selection=False)

    step = make_step(S)
    stream = torch.cuda.current_stream()
    probe = _probe_lib()
    flush_buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    flush_sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def flush():
        # evict the 256 MB last-level cache by streaming 1 GiB of reads: clean lines, so the
        # next kernel pays no write-back for the flush
        probe.dsa_probe_stream_read(flush_buf.data_ptr(), flush_buf.numel(), flush_sink.data_ptr(),
                                    8192, stream.cuda_stream)

    def one_step(evs=None, step=step):
        # stage 3's query quantisation runs on a side stream while stages 1 and 2 run; the
        # step starts at evs[0] on the main stream, which the side stream waits for
        if evs:
            evs[0].record(stream)
        if step.query_prep == "first":
            step.prepare_query(batch.q_mla, stream=stream)
        if step.query_on_side_stream:
            step._ev_start.record(stream)
            step.side.wait_event(step._ev_start)
            step.prepare_query(batch.q_mla, stream=step.side)
            step._ev_query.record(step.side)
        step.index(batch.cu_q, batch.seq_lens, batch.q_idx, batch.head_w, batch.key_pool,
                   batch.block_table, max(wl.q_per_seq), stream, q_mla=batch.q_mla)
        if evs:
            evs[1].record(stream)
        if not step.select_in_attention:
            step.select(batch.cu_q, batch.seq_lens, batch.block_table, stream)
        if evs:
            evs[2].record(stream)
        if step.query_on_side_stream:
            stream.wait_event(step._ev_query)
        if step.select_in_attention:
            step.select_attend(batch.cu_q, batch.seq_lens, batch.block_table, batch.q_mla,
                               batch.latent_pool, batch.latent_scale, batch.softmax_scale, stream)
        else:
            step.attend(batch.q_mla, batch.latent_pool, batch.latent_scale, batch.softmax_scale,
                        stream)
        if evs:
            evs[3].record(stream)

    for _ in range(args.warmup):
        if not args.no_flush:
            flush()
        one_step()
    torch.cuda.synchronize()

    def timed_steps(with_stages, stp=step):
        per = []
        for _ in range(args.steps):
            if not args.no_flush:
                flush()                     # outside the events
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            if with_stages:
                one_step(evs, stp)
            else:
                evs[0].record(stream)
                one_step(None, stp)
                evs[3].record(stream)
            per.append(evs)
        torch.cuda.synchronize()
        return per

    # the timed steps carry only a start and an end event (each event between kernels adds a
    # few microseconds); the same steps are then run again with events between the stages
    # for the per-stage times and the indexer's launch duration
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    per_step = timed_steps(False)
    t_wall = time.perf_counter() - t_wall0
    step_us = [evs[0].elapsed_time(evs[3]) * 1e3 for evs in per_step]
    stage = [[], [], []]
    for evs in timed_steps(True):
        for i in range(3):
            stage[i].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)   # us
    also = args.also_splits if args.also_splits is not None else ([16] if wl.name == "long" else [])
    also_us = {}
    for s2 in also:
        if s2 == S:
            continue
        st2 = make_step(s2)
        for _ in range(args.warmup):
            if not args.no_flush:
                flush()
            one_step(None, st2)
        per2 = timed_steps(False, st2)
        also_us[str(s2)] = round(sum(e[0].elapsed_time(e[3]) * 1e3 for e in per2) / len(per2), 2)
        del st2
    step_us_sorted = sorted(step_us)
    med = step_us_sorted[len(step_us_sorted) // 2]
    p10 = step_us_sorted[int(0.1 * (len(step_us_sorted) - 1))]
    p90 = step_us_sorted[int(round(0.9 * (len(step_us_sorted) - 1)))]
    mean_us = sum(step_us) / len(step_us)
    stage_mean = [sum(s) / len(s) for s in stage]

    ab = algorithmic_bytes(wl.seq_lens, wl.q_per_seq, wl.topk, wl.key_format)
    value = ab["total"] / (mean_us * 1e-6) / 1e9
    idx_bytes = index_score_bytes(wl.seq_lens, wl.key_format)
    idx_gbps = idx_bytes / (stage_mean[0] * 1e-6) / 1e9
    idx_flops = index_score_flops(wl)
    idx_tflops = idx_flops / (stage_mean[0] * 1e-6) / 1e12
    # the indexer is MFMA-bound when its FLOP per byte exceeds the FP8 ridge (peak FLOP/s over
    # peak B/s = 625): many query rows per request, as in a prefill append
    mfma_bound = idx_flops / idx_bytes > FP8_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    traffic = _traffic_from_profile() if wl.name == "long" else None  # counted on `long`
    ceiling = stream_read_ceiling(torch)
    page_ceiling = page_read_ceiling(torch, batch)
    if args.copy_calibration:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        del flush_buf
        rows = list(range(0, wl.n_q, max(1, wl.n_q // 8)))
        cpu = cpu_baseline(batch, rows, budget_s=args.cpu_budget)

    append = cache_append_timing(torch, dsa, batch, wl, steps=args.steps)

    rec = {
        "metric": "DSA decode µs/layer & HBM GB/s (%peak) at 128K ctx, batch 32",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 x mxfp4 MFMA (indexer), fp8e4m3 MFMA (attention), fp32 accumulate, "
                  "bf16 in/out" if wl.key_format == "mxfp4" else
                  "fp8e4m3 MFMA, fp32 accumulate, bf16 in/out"),
        "data": ("synthetic (seeded N(0,1) queries/keys/latents, MXFP4 index keys, E4M3 "
                 "latents, shuffled 64-token pages)" if wl.key_format == "mxfp4" else
                 "synthetic (seeded N(0,1) queries/keys/latents, E4M3-quantised caches, "
                 "shuffled 64-token pages)"),
        "config": {"workload": wl.name, "batch": wl.num_seqs, "query_rows": wl.n_q,
                   "context": wl.max_seq_len if len(set(wl.seq_lens)) == 1 else "ragged",
                   "topk": wl.topk, "num_splits": S, "page_size": PAGE,
                   "index_key_format": wl.key_format,
                   "indexer_emits_topk_candidates": not args.unfused,
                   "scores_stored": step.store_scores,
                   "topk_final_in_attention": step.select_in_attention,
                   "mla_query_prep": step.query_prep,
                   "flush_llc_between_steps": not args.no_flush},
        "us_per_layer": round(mean_us, 2),
        "us_per_layer_at_other_splits": also_us or None,
        "us_per_layer_median": round(med, 2),
        "us_per_layer_p10_p90": [round(p10, 2), round(p90, 2)],
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
        "stage_us": ({"index_score": round(stage_mean[0], 2),
                      "topk_final_in_sparse_mla_and_merge": round(stage_mean[2], 2)}
                     if step.select_in_attention else
                     {"index_score": round(stage_mean[0], 2), "topk": round(stage_mean[1], 2),
                      "sparse_mla_and_merge": round(stage_mean[2], 2)}),
        "algorithmic_bytes": ab,
        "dsa_vs_dense_mla_bytes": round(ab["total"] / dense_mla_bytes(wl.seq_lens, wl.q_per_seq), 4),
        "roofline": ({"kernel": "dsa_index_score", "bound": "mfma", "achieved": round(idx_tflops, 1),
                      "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(idx_tflops / FP8_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                      "algorithmic_flops_per_launch": idx_flops,
                      "avg_launch_us": round(stage_mean[0], 2)} if mfma_bound else
                     {"kernel": "dsa_index_score", "bound": "hbm", "achieved": round(idx_gbps, 1),
                      "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(idx_gbps / HBM_PEAK_GBPS, 4),
                      "traffic": traffic, "algorithmic_bytes_per_launch": idx_bytes,
                      "avg_launch_us": round(stage_mean[0], 2)}),
        "algorithmic_tflop": {"index_score": round(idx_flops / 1e12, 4),
                              "sparse_mla": round(sparse_mla_flops(wl) / 1e12, 4)},
        "stream_read_ceiling_GBps": round(ceiling, 1),
        "index_page_read_ceiling_GBps": round(page_ceiling, 1) if page_ceiling else None,
        "index_score_frac_of_page_ceiling": (round(idx_gbps / page_ceiling, 4)
                                             if page_ceiling and not mfma_bound else None),
        "wall_s_timed_loop": round(t_wall, 4),
        "cpu_baseline": cpu,
        "cache_append": append,
    }
    print(json.dumps(rec, ensure_ascii=False))


if __name__ == "__main__":
    main()
