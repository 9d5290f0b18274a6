"""Seeded synthetic inputs for the DSA decode hot path.

This module only draws random numbers and lays the resulting cache contents out in
pages.  It holds none of the arithmetic of the method itself: indexer scoring, top-k,
attention and the combine live in the HIP library and, independently, in the oracle.
Quantising the *cache contents* (the FP8 index keys and FP8 latents that an earlier
layer step would have written) is input preparation and happens here.

Workloads (sizes from the DSA decode description of Kimi K3.1 Pro on the vLLM
day-0 page: 32 indexer heads x 128 dims with one FP8 key + fp32 scale per token,
top-2048, a 576-byte FP8 latent of which values use the first 512 dims, 96 heads):

  tiny     1 request, 1 query row, context 4,096
  spec     32 requests x 5 query rows (causal among the 5), context U{8,192..32,768}
  long     32 requests x 1 query row, context 131,072
  million  1 request x 5 query rows, context 1,048,576
  prefill  1 request x 2,048 query rows appended on a 150,000-token prefix

Distributions: indexer q ~ N(0,1) rounded to bf16; head weights ~ N(0, 1/32) fp32;
keys N(0,1) quantised to E4M3 with a per-token fp32 scale absmax/448; MLA q ~ N(0,1)
bf16; latents N(0,1) quantised to E4M3 with one per-tensor fp32 scale absmax/448
over the whole latent pool.  Pages hold 64 tokens and every request's logical pages
are scattered over the pool by a seeded permutation.  Token slots past the end of a
request and pages no request owns are poisoned with the E4M3 NaN byte 0x7F and NaN
scales, so that any read outside the visible context shows up as NaN.

Page formats (the library's documented cache layout):
  index-key page, 8,448 bytes: 8,192 bytes of E4M3 codes in 16-byte column blocks
      (byte d of token o lives at (d // 16) * 1024 + o * 16 + d % 16), then 64 fp32
      scales (scale of token o at 8192 + 4 * o);
  latent page, 36,864 bytes: token o's 576 E4M3 codes at o * 576.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE = 64
IDX_HEADS = 32
IDX_DIM = 128
MLA_HEADS = 96
LAT_DIM = 576
V_DIM = 512
IDX_PAGE_BYTES = PAGE * IDX_DIM + PAGE * 4   # 8448
MX_PAGE_BYTES = PAGE * IDX_DIM // 2 + PAGE * 4   # 4352: MXFP4 index keys, 68 B per token
LAT_PAGE_BYTES = PAGE * LAT_DIM              # 36864
E4M3_NAN = 0x7F
E4M3_MAX = 448.0

# sub-stream ids of the master seed
_S_KEYS, _S_LAT, _S_QIDX, _S_W, _S_QMLA, _S_PERM, _S_LENS = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seq_lens: tuple            # context length of each request (includes its query tokens)
    q_per_seq: tuple           # query rows per request: the last q tokens of the request
    topk: int = 2048
    num_splits: int = 1        # split count used for the sparse-attention stage
    seed: int = 0
    key_format: str = "e4m3"   # index-key cache: "e4m3" (132 B/token) or "mxfp4" (68 B/token)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def n_q(self) -> int:
        return int(sum(self.q_per_seq))

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens))

    def row_positions(self):
        """(request, absolute position) of every query row, rows grouped by request."""
        out = []
        for b, (L, nq) in enumerate(zip(self.seq_lens, self.q_per_seq)):
            for j in range(nq):
                out.append((b, L - nq + j))
        return out


def _spec_lens(seed: int):
    rng = np.random.default_rng([seed, _S_LENS])
    return tuple(int(x) for x in rng.integers(8192, 32768 + 1, size=32))


def workload(name: str) -> Workload:
    """The five named workloads.  Master seed = position in the list below."""
    if name == "tiny":
        return Workload("tiny", (4096,), (1,), 2048, 16, seed=0)
    if name == "spec":
        return Workload("spec", _spec_lens(1), (5,) * 32, 2048, 1, seed=1)
    if name == "long":
        return Workload("long", (131072,) * 32, (1,) * 32, 2048, 8, seed=2)
    if name == "million":
        return Workload("million", (1048576,), (5,), 2048, 16, seed=3)
    if name == "prefill":
        return Workload("prefill", (152048,), (2048,), 2048, 1, seed=4)
    if name.endswith("-mxfp4") and name[:-6] in WORKLOADS:
        return dataclasses.replace(workload(name[:-6]), name=name, key_format="mxfp4")
    raise KeyError(name)


WORKLOADS = ("tiny", "spec", "long", "million", "prefill")


def custom(seq_lens, q_per_seq, topk=2048, num_splits=1, seed=12345, name="custom",
           key_format="e4m3") -> Workload:
    return Workload(name, tuple(int(x) for x in seq_lens), tuple(int(x) for x in q_per_seq),
                    int(topk), int(num_splits), int(seed), key_format)


@dataclasses.dataclass
class Batch:
    wl: Workload
    device: str
    cu_q: torch.Tensor          # int32 [B+1]
    seq_lens: torch.Tensor      # int32 [B]
    block_table: torch.Tensor   # int32 [B, bt_stride], -1 past the last page
    key_pool: torch.Tensor      # uint8 [P, 8448] (E4M3 keys) or [P, 4352] (MXFP4 keys)
    latent_pool: torch.Tensor   # uint8 [P, 36864]
    latent_scale: float         # per-tensor fp32 scale of the latents
    q_idx: torch.Tensor         # bf16 [n_q, 32, 128]
    head_w: torch.Tensor        # fp32 [n_q, 32]
    q_mla: torch.Tensor         # bf16 [n_q, 96, 576]
    softmax_scale: float
    # logical (unpaged) copies, kept only when asked for (small workloads)
    keys_logical: Optional[list] = None      # per request uint8 [L, 128] codes (E4M3) or
                                             # the unquantised fp32 [L, 128] keys (MXFP4)
    scales_logical: Optional[list] = None    # per request fp32 [L]
    latents_logical: Optional[list] = None   # per request uint8 [L, 576]

    @property
    def num_pages(self) -> int:
        return int(self.key_pool.shape[0])


def _gen(device, seed, stream, idx):
    g = torch.Generator(device=device)
    # distinct 63-bit seed per (master seed, sub-stream, index)
    g.manual_seed((seed * 1_000_003 + stream * 10_007 + idx * 7919 + 0x5EED) & ((1 << 63) - 1))
    return g


def _to_e4m3(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> E4M3 codes (uint8); |x| is at most 448 here, so no saturation happens."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


_E2M1_TIES_ODD = (1, 3, 5)  # boundaries between codes i and i+1 where i is odd: ties go up


def _to_mxfp4(x: torch.Tensor):
    """fp32 [n, 128] -> (E2M1 codes [n, 128] as int, E8M0 scale bytes [n, 4]) by the OCP MX
    recipe: per block of 32, shared exponent floor(log2 absmax) - 2 (E2M1's largest
    exponent), elements rounded to nearest even on the E2M1 grid and saturated at 6; an
    all-zero block gets scale 2^0 and zero codes."""
    blk = x.view(x.shape[0], 4, 32)
    amax = blk.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                        # amax = m * 2^ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex.to(torch.int32) - 3, torch.zeros_like(ex, dtype=torch.int32))
    e = e.clamp(-127, 127)
    q = blk / torch.ldexp(torch.ones_like(amax), e.to(amax.dtype))[:, :, None]
    a = q.abs()
    bounds = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
    code = torch.zeros_like(a, dtype=torch.int32)
    for i, bnd in enumerate(bounds):
        code += (a > bnd).to(torch.int32)
        if i in _E2M1_TIES_ODD:
            code += (a == bnd).to(torch.int32)
    code = code | (torch.signbit(q).to(torch.int32) << 3)
    return code.view(x.shape[0], 128), (e + 127).to(torch.uint8)


def _chunks(n, step):
    for s in range(0, n, step):
        yield s, min(n, s + step)


def make_batch(wl: Workload, device: str = "cpu", keep_logical: bool = False,
               spare_pages: int = 3, chunk_tokens: int = 1 << 18) -> Batch:
    dev = torch.device(device)
    seed = wl.seed
    B = wl.num_seqs
    n_pages = [(L + PAGE - 1) // PAGE for L in wl.seq_lens]
    total = int(sum(n_pages)) + spare_pages
    bt_stride = max(n_pages)

    perm = torch.randperm(total, generator=_gen("cpu", seed, _S_PERM, 0))
    bt = torch.full((B, bt_stride), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        off += n

    mx = wl.key_format == "mxfp4"
    if mx:
        # poison: maximal codes and E8M0 NaN scales
        key_pool = torch.full((total, MX_PAGE_BYTES), 0x77, dtype=torch.uint8, device=dev)
        key_pool[:, PAGE * IDX_DIM // 2:] = 0xFF
    else:
        key_pool = torch.full((total, IDX_PAGE_BYTES), E4M3_NAN, dtype=torch.uint8, device=dev)
        nan_scales = torch.full((total, PAGE), float("nan"), dtype=torch.float32, device=dev)
        key_pool[:, PAGE * IDX_DIM:] = nan_scales.view(torch.uint8)
    latent_pool = torch.full((total, LAT_PAGE_BYTES), E4M3_NAN, dtype=torch.uint8, device=dev)

    keys_log, scales_log, lat_log = ([] if keep_logical else None for _ in range(3))

    # ---- index keys: MXFP4 (block scales) ------------------------------------------------
    for b, L in enumerate(wl.seq_lens if mx else ()):
        g = _gen(dev, seed, _S_KEYS, b)
        phys = bt[b, :n_pages[b]].to(dev).long()
        nb = torch.full((n_pages[b] * PAGE, 64), 0x77, dtype=torch.uint8, device=dev)
        sb = torch.full((n_pages[b] * PAGE, 4), 0xFF, dtype=torch.uint8, device=dev)
        raw = [] if keep_logical else None
        for s, e in _chunks(L, chunk_tokens):
            k = torch.randn((e - s, IDX_DIM), generator=g, device=dev, dtype=torch.float32)
            codes, scl = _to_mxfp4(k)
            pair = codes.view(e - s, 64, 2)
            nb[s:e] = (pair[:, :, 0] | (pair[:, :, 1] << 4)).to(torch.uint8)
            sb[s:e] = scl
            if keep_logical:
                raw.append(k.cpu())
        # 16-byte blocks (one per 32 dims): [page, token, 4, 16] -> [page, 4, token, 16]
        blk = nb.view(n_pages[b], PAGE, 4, 16).permute(0, 2, 1, 3)
        key_pool[phys, :PAGE * IDX_DIM // 2] = blk.reshape(n_pages[b], PAGE * IDX_DIM // 2)
        key_pool[phys, PAGE * IDX_DIM // 2:] = sb.view(n_pages[b], PAGE * 4)
        if keep_logical:
            keys_log.append(torch.cat(raw))     # the unquantised fp32 keys
            scales_log.append(None)

    # ---- index keys: per-token scale absmax/448 --------------------------------------
    for b, L in enumerate(() if mx else wl.seq_lens):
        g = _gen(dev, seed, _S_KEYS, b)
        phys = bt[b, :n_pages[b]].to(dev).long()
        codes_all = torch.empty((n_pages[b] * PAGE, IDX_DIM), dtype=torch.uint8, device=dev)
        codes_all.fill_(E4M3_NAN)
        scales_all = torch.full((n_pages[b] * PAGE,), float("nan"), dtype=torch.float32, device=dev)
        for s, e in _chunks(L, chunk_tokens):
            k = torch.randn((e - s, IDX_DIM), generator=g, device=dev, dtype=torch.float32)
            amax = k.abs().amax(dim=1)
            sc = amax / E4M3_MAX
            sc = torch.where(sc > 0, sc, torch.ones_like(sc))
            codes_all[s:e] = _to_e4m3(k / sc[:, None])
            scales_all[s:e] = sc
        # 16-byte column blocks: [page, token, 8, 16] -> [page, 8, token, 16]
        blk = codes_all.view(n_pages[b], PAGE, IDX_DIM // 16, 16).permute(0, 2, 1, 3)
        key_pool[phys, :PAGE * IDX_DIM] = blk.reshape(n_pages[b], PAGE * IDX_DIM)
        key_pool[phys, PAGE * IDX_DIM:] = scales_all.view(n_pages[b], PAGE).contiguous().view(torch.uint8)
        if keep_logical:
            keys_log.append(codes_all[:L].cpu())
            scales_log.append(scales_all[:L].cpu())

    # ---- latents: one per-tensor scale over the whole pool (two passes) ---------------
    amax = torch.zeros((), dtype=torch.float32, device=dev)
    for b, L in enumerate(wl.seq_lens):
        g = _gen(dev, seed, _S_LAT, b)
        for s, e in _chunks(L, chunk_tokens):
            x = torch.randn((e - s, LAT_DIM), generator=g, device=dev, dtype=torch.float32)
            amax = torch.maximum(amax, x.abs().amax())
    c = float(amax.item()) / E4M3_MAX
    c = float(np.float32(c))
    c_t = torch.tensor(c, dtype=torch.float32, device=dev)
    for b, L in enumerate(wl.seq_lens):
        g = _gen(dev, seed, _S_LAT, b)
        phys = bt[b, :n_pages[b]].to(dev).long()
        lat = torch.empty((n_pages[b] * PAGE, LAT_DIM), dtype=torch.uint8, device=dev)
        lat.fill_(E4M3_NAN)
        for s, e in _chunks(L, chunk_tokens):
            x = torch.randn((e - s, LAT_DIM), generator=g, device=dev, dtype=torch.float32)
            lat[s:e] = _to_e4m3(x / c_t)
        latent_pool[phys] = lat.view(n_pages[b], LAT_PAGE_BYTES)
        if keep_logical:
            lat_log.append(lat[:L].cpu())
        del lat

    n_q = wl.n_q
    q_idx = torch.randn((n_q, IDX_HEADS, IDX_DIM), generator=_gen(dev, seed, _S_QIDX, 0),
                        device=dev, dtype=torch.float32).to(torch.bfloat16)
    head_w = torch.randn((n_q, IDX_HEADS), generator=_gen(dev, seed, _S_W, 0),
                         device=dev, dtype=torch.float32) * float(1.0 / math.sqrt(IDX_HEADS))
    q_mla = torch.randn((n_q, MLA_HEADS, LAT_DIM), generator=_gen(dev, seed, _S_QMLA, 0),
                        device=dev, dtype=torch.float32).to(torch.bfloat16)

    cu = [0]
    for nq in wl.q_per_seq:
        cu.append(cu[-1] + nq)
    return Batch(
        wl=wl, device=str(dev),
        cu_q=torch.tensor(cu, dtype=torch.int32, device=dev),
        seq_lens=torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev),
        block_table=bt.to(dev),
        key_pool=key_pool, latent_pool=latent_pool, latent_scale=c,
        q_idx=q_idx, head_w=head_w, q_mla=q_mla,
        softmax_scale=float(np.float32(1.0 / math.sqrt(LAT_DIM))),
        keys_logical=keys_log, scales_logical=scales_log, latents_logical=lat_log,
    )


def random_scores(n_rows: int, n_cols: int, seed: int, kind: str = "normal") -> torch.Tensor:
    """fp32 score matrices for exercising top-k on its own (host tensor).

    kinds: normal, ties (few distinct values), equal (all the same), signed_zero
    (only +0.0 and -0.0), increasing, neg_inf_tail (normal with the second half -inf),
    extremes (normal with 1% each of +-inf, +-FLT_MAX and denormals), huge (all within a
    factor of two below FLT_MAX).
    """
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        return torch.randn((n_rows, n_cols), generator=g)
    if kind == "ties":
        return torch.randint(0, 7, (n_rows, n_cols), generator=g).float() * 0.25
    if kind == "equal":
        return torch.full((n_rows, n_cols), 1.5)
    if kind == "signed_zero":
        sgn = torch.randint(0, 2, (n_rows, n_cols), generator=g).bool()
        return torch.where(sgn, torch.tensor(-0.0), torch.tensor(0.0))
    if kind == "increasing":
        return torch.arange(n_cols, dtype=torch.float32).repeat(n_rows, 1) * 1e-3
    if kind == "neg_inf_tail":
        x = torch.randn((n_rows, n_cols), generator=g)
        x[:, n_cols // 2:] = float("-inf")
        return x
    if kind == "extremes":
        x = torch.randn((n_rows, n_cols), generator=g)
        pick = torch.randint(0, 100, (n_rows, n_cols), generator=g)
        fmax = torch.finfo(torch.float32).max
        for code, v in ((0, float("inf")), (1, fmax), (2, -fmax), (3, float("-inf")),
                        (4, 1e-40), (5, -1e-40)):
            x[pick == code] = v
        return x
    if kind == "huge":
        u = torch.rand((n_rows, n_cols), generator=g)
        return torch.finfo(torch.float32).max * (0.5 + 0.5 * u)
    raise KeyError(kind)
