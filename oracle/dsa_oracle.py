"""CPU oracle for the DSA (DeepSeek Sparse Attention) decode hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library.

Plain, slow and written to be checked by eye: numpy in fp64, full sorts, dense
softmax.  Every function names the passage it follows.  "The K3.1 page" below is
the vLLM blog page on Kimi K3.1 Pro day-0 support (sparse attention, DCP,
zero-mismatch RL); its section titles are given in English with the original.

Readings of points the pages leave open (each is listed in the design notes):
  * FP8 means OCP E4M3FN: 4 exponent bits (bias 7), 3 mantissa bits, max 448,
    0x7F/0xFF NaN, no infinities.  The cache scales are "absmax / 448".
  * Queries are quantised to E4M3 before both contractions, one power-of-two scale
    per (row, head): the K3.1 page's fused indexer front quantises the indexer query
    to FP8 ("Fused low-latency decode for DSA layers" / DSA層のための融合低レイテンシデコード).
    The power-of-two scale sq is the smallest 2^e with absmax <= 448 * 2^e, so
    q / sq is exact and one round-to-nearest-even gives the code.
  * A query row at absolute position pos sees tokens 0..pos inclusive.
  * Top-k ties are broken by the lower token index; -0.0 equals +0.0.
  * The LSE is the natural log-sum-exp of the scaled logits.
  * MXFP4 index keys follow the OCP microscaling recipe (mxfp4_encode): block scale
    2^(floor(log2 absmax) - 2), elements rounded to nearest even on the E2M1 grid and
    saturated at 6.
  * Softmax probabilities are not quantised here: this is the exact softmax.  The
    kernel's two-term FP8 probabilities in the value contraction deviate from it by a
    stated bound per probability, and the attention outputs are compared with this
    oracle at the attention tolerance; the encoding itself is modelled and checked in
    the tests (with torch's own E4M3 codec), not here.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

E4M3_MAX = 448.0
PAGE = 64
IDX_HEADS, IDX_DIM = 32, 128
MLA_HEADS, LAT_DIM, V_DIM = 96, 576, 512
IDX_PAGE_KEY_BYTES = PAGE * IDX_DIM           # 8192 bytes of codes, then 64 fp32 scales
LAT_ROW = LAT_DIM


# --------------------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------------------
def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN byte: sign s, exponent e (bias 7), mantissa m.

    e = 15 and m = 7 is NaN; e = 0 is subnormal m * 2^-9; else (1 + m/8) * 2^(e-7).
    The K3.1 page stores index keys and latents in FP8 ("What changed in Kimi K3.1
    Pro" / Kimi K3.1 Proの変更点, "Packed KV cache" / パック型KVキャッシュ).
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        v = m * 2.0 ** -9
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# magnitudes of codes 0x00..0x7E in increasing order (0 .. 448)
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even onto the E4M3 grid, saturating at +-448, sign kept.

    The nearest representable magnitude is looked up among the 127 finite
    non-negative codes; on an exact tie the code with the even mantissa (even code)
    wins.  Inputs must not be NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    lo = np.clip(np.searchsorted(_E4M3_POS, a, side="right") - 1, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code.astype(np.int64) | sign).astype(np.uint8)


# MXFP4 (OCP microscaling): E2M1 elements in blocks of 32 sharing one E8M0 scale.  The K3.1
# page's opt-in MXFP4 index key is 68 bytes with its scales ("Packed KV cache for three kinds
# of state" / パック型KVキャッシュ, "Native MXFP4 indexer" / ネイティブMXFP4インデクサー):
# 128 E2M1 values (64 bytes) and one E8M0 scale per 32 dimensions (4 bytes).
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(nibbles) -> np.ndarray:
    """E2M1 nibble -> value: bit 3 sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent 0
    is subnormal (m * 0.5), otherwise (1 + m/2) * 2^(e-1).  No NaN or infinity."""
    c = np.asarray(nibbles, dtype=np.int64) & 0xF
    e, m = (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.where(c & 8, -mag, mag)


def e8m0_value(b) -> np.ndarray:
    """E8M0 scale byte -> 2^(b - 127); 0xFF is NaN."""
    b = np.asarray(b, dtype=np.int64)
    with np.errstate(over="ignore"):
        return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def floor_log2(a: float) -> int:
    """The integer f with 2^f <= a < 2^(f+1), for a finite a > 0 (exact, by comparison)."""
    f = int(math.floor(math.log2(a)))
    while 2.0 ** f > a:
        f -= 1
    while 2.0 ** (f + 1) <= a:
        f += 1
    return f


def mxfp4_encode(x) -> Tuple[np.ndarray, np.ndarray]:
    """OCP MX quantisation of key values [n, 128] (finite) to E2M1 nibbles [n, 128] and
    E8M0 scale bytes [n, 4]: the 68-byte MXFP4 index key of the "Native MXFP4 indexer"
    section (ネイティブMXFP4インデクサー), blocks of 32 dimensions sharing one scale.

    Reading (the OCP microscaling recipe; the page names the format, not the rounding):
    block scale X = 2^(floor(log2 absmax) - 2), 2 being E2M1's largest exponent, kept in
    E8M0's range (exponent at least -127); an all-zero block takes X = 1.  Each element is
    the E2M1 value nearest |x| / X, a tie going to the value with an even code (mantissa bit
    0), capped at 6, the largest E2M1 value: round-to-nearest-even with saturation.  The
    sign bit is x's own, so a negative value that rounds to zero is -0 (nibble 8).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    nib = np.zeros((n, IDX_DIM), dtype=np.int64)
    sbytes = np.zeros((n, IDX_DIM // 32), dtype=np.uint8)
    for t in range(n):
        for b in range(IDX_DIM // 32):
            blk = x[t, 32 * b:32 * b + 32]
            amax = float(np.max(np.abs(blk)))
            e = max(floor_log2(amax) - 2, -127) if amax > 0 else 0
            sbytes[t, b] = e + 127
            for j, v in enumerate(blk):
                a = abs(v) / 2.0 ** e
                dist = np.abs(E2M1_MAG - a)
                near = np.flatnonzero(dist == dist.min())
                even = [c for c in near if c % 2 == 0]
                code = int(even[0] if even else near[0])
                nib[t, 32 * b + j] = code | (8 if np.signbit(v) else 0)
    return nib, sbytes


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: a bf16 is the top 16 bits of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# Query quantisation (reading of the fused indexer front, see module docstring)
# --------------------------------------------------------------------------------------
def pow2_scale(absmax: float) -> float:
    """Smallest power of two 2^e with absmax <= 448 * 2^e (1.0 when absmax is 0)."""
    if absmax == 0.0:
        return 1.0
    _, E = math.frexp(absmax)
    e = E - 12
    while absmax > E4M3_MAX * 2.0 ** e:
        e += 1
    return 2.0 ** e


def quantize_heads(q: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """q [H, D] real values -> (E4M3 codes [H, D], power-of-two scale [H]).

    Dequantised query = e4m3_decode(codes) * scale[:, None].
    """
    q = np.asarray(q, dtype=np.float64)
    sq = np.array([pow2_scale(float(np.max(np.abs(row)))) for row in q])
    codes = e4m3_encode(q / sq[:, None])
    return codes, sq


def dequantized_query(q: np.ndarray) -> np.ndarray:
    codes, sq = quantize_heads(q)
    return e4m3_decode(codes) * sq[:, None]


# --------------------------------------------------------------------------------------
# Paged caches: block table -> physical page -> bytes
# (the K3.1 page: block tables and cache slots are translated to kernel page
#  addresses before each step; kernels see small fixed-size pages; 132 B per index
#  key, 576 B per latent — "Packed KV cache" / パック型KVキャッシュ)
# --------------------------------------------------------------------------------------
def physical_slot(block_table_row: np.ndarray, t: np.ndarray) -> np.ndarray:
    t = np.asarray(t, dtype=np.int64)
    return block_table_row[t // PAGE].astype(np.int64) * PAGE + t % PAGE


def read_index_keys(key_pool: np.ndarray, block_table_row: np.ndarray, n: int):
    """Codes [n, 128] and scales [n] of logical tokens 0..n-1 of one request.

    Index-key page: byte d of token o at (d // 16) * 1024 + o * 16 + d % 16; the
    fp32 scale of token o at 8192 + 4 * o.
    """
    pool = np.asarray(key_pool, dtype=np.uint8)
    codes = np.empty((n, IDX_DIM), dtype=np.uint8)
    scales = np.empty(n, dtype=np.float64)
    for t in range(0, n, PAGE):
        page = pool[int(block_table_row[t // PAGE])]
        cnt = min(PAGE, n - t)
        blocks = page[:IDX_PAGE_KEY_BYTES].reshape(IDX_DIM // 16, PAGE, 16)   # [8, 64, 16]
        codes[t:t + cnt] = blocks.transpose(1, 0, 2).reshape(PAGE, IDX_DIM)[:cnt]
        sc = page[IDX_PAGE_KEY_BYTES:IDX_PAGE_KEY_BYTES + 4 * PAGE].view(np.float32)
        scales[t:t + cnt] = sc[:cnt]
    return codes, scales


MX_PAGE_KEY_BYTES = PAGE * IDX_DIM // 2   # 4096 bytes of E2M1 codes, then 64 x 4 scale bytes
MX_PAGE_BYTES = MX_PAGE_KEY_BYTES + PAGE * 4  # 4352 = 64 x 68


def read_index_keys_mxfp4(key_pool: np.ndarray, block_table_row: np.ndarray, n: int):
    """Key values [n, 128] (fp64) of logical tokens 0..n-1 of one request, MXFP4 cache.

    MXFP4 index-key page (4,352 B): block b (dims 32b .. 32b+31) of token o is 16 bytes at
    b * 1024 + o * 16, byte j holding dims 32b + 2j (low nibble) and 32b + 2j + 1 (high
    nibble); the E8M0 scale of block b of token o is the byte at 4096 + 4 * o + b.
    """
    pool = np.asarray(key_pool, dtype=np.uint8)
    vals = np.empty((n, IDX_DIM), dtype=np.float64)
    for t in range(0, n, PAGE):
        page = pool[int(block_table_row[t // PAGE])]
        cnt = min(PAGE, n - t)
        blocks = page[:MX_PAGE_KEY_BYTES].reshape(4, PAGE, 16)          # [block, token, byte]
        by = blocks.transpose(1, 0, 2)[:cnt].astype(np.int64)           # [tok, block, byte]
        nib = np.stack([by & 0xF, by >> 4], axis=-1).reshape(cnt, 4, 32)  # dims in order
        sc = page[MX_PAGE_KEY_BYTES:MX_PAGE_KEY_BYTES + 4 * PAGE].reshape(PAGE, 4)[:cnt]
        vals[t:t + cnt] = (e2m1_decode(nib) * e8m0_value(sc)[:, :, None]).reshape(cnt, IDX_DIM)
    return vals


def read_latents(latent_pool: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """Latent codes [len(slots), 576] of physical slots (page * 64 + offset)."""
    pool = np.asarray(latent_pool, dtype=np.uint8)
    slots = np.asarray(slots, dtype=np.int64)
    rows = pool.reshape(pool.shape[0], PAGE, LAT_ROW)
    return rows[slots // PAGE, slots % PAGE]


# --------------------------------------------------------------------------------------
# Cache append: the new tokens' index keys and latents into the paged caches
# --------------------------------------------------------------------------------------
def cache_append(key_pool: np.ndarray, latent_pool: np.ndarray, slots, key_bf16, latent_bf16,
                 latent_scale: float, key_format: str = "e4m3") -> None:
    """Quantises and writes tokens into the paged caches by physical slot (in place).

    The K3.1 page stores one FP8 index key per token, 132 bytes with its scale ("What
    changed in Kimi K3.1 Pro" / Kimi K3.1 Proの変更点), and a 576-byte FP8 latent ("Packed KV
    cache for three kinds of state" / パック型KVキャッシュ); its fused indexer front writes
    the new token's index key in the same kernel as the query prep ("Fused low-latency
    decode for DSA layers").  Readings (the page fixes neither): the key's scale is one
    fp32 per token, s = absmax / 448 (1 for an all-zero key), and its codes are the E4M3
    round-to-nearest-even (saturating) of k / s evaluated in fp32; the latent's codes are
    the E4M3 of x / latent_scale in fp32 with the cache's per-tensor scale.  Slot -1 is
    skipped.  key_bf16 [n, 128] / latent_bf16 [n, 576] are bf16 bit patterns (uint16);
    either may be None (that cache is left alone).  key_format "mxfp4": the index-key pool
    holds the page's opt-in 68-byte MXFP4 keys ("Native MXFP4 indexer"), and the key is
    mxfp4_encode of its bf16 values, written in the page layout of read_index_keys_mxfp4.
    """
    slots = np.asarray(slots, dtype=np.int64)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        page, o = int(slot // PAGE), int(slot % PAGE)
        if key_bf16 is not None and key_format == "mxfp4":
            nib, sb = mxfp4_encode(bf16_value(np.asarray(key_bf16)[i])[None, :])
            for d in range(0, IDX_DIM, 2):
                byte = int(nib[0, d]) | (int(nib[0, d + 1]) << 4)
                key_pool[page, (d // 32) * 1024 + o * 16 + (d % 32) // 2] = byte
            key_pool[page, MX_PAGE_KEY_BYTES + 4 * o:MX_PAGE_KEY_BYTES + 4 * o + 4] = sb[0]
        elif key_bf16 is not None:
            assert key_format == "e4m3", key_format
            k = bf16_value(np.asarray(key_bf16)[i]).astype(np.float32)
            a = np.float32(np.max(np.abs(k)))
            sc = np.float32(a / np.float32(E4M3_MAX)) if a > 0 else np.float32(1.0)
            codes = e4m3_encode((k / sc).astype(np.float32))
            for d in range(IDX_DIM):
                key_pool[page, (d // 16) * 1024 + o * 16 + d % 16] = codes[d]
            off = IDX_PAGE_KEY_BYTES + 4 * o
            key_pool[page, off:off + 4] = np.array([sc], dtype=np.float32).view(np.uint8)
        if latent_bf16 is not None:
            x = bf16_value(np.asarray(latent_bf16)[i]).astype(np.float32)
            latent_pool[page, o * LAT_ROW:(o + 1) * LAT_ROW] = e4m3_encode(
                (x / np.float32(latent_scale)).astype(np.float32))


# --------------------------------------------------------------------------------------
# Stage 1: lightning-indexer score
# --------------------------------------------------------------------------------------
def index_scores(q_idx: np.ndarray, head_w: np.ndarray, key_codes: np.ndarray,
                 key_scales: np.ndarray, quantize_query: bool = True) -> np.ndarray:
    """score_t = sum_h w_h * ReLU(q_h . k_t * s_t) for every given token, as fp32.

    The K3.1 page ("What changed in Kimi K3.1 Pro" / Kimi K3.1 Proの変更点) has 32
    light heads score every prior token against one FP8 key (with its scale) per
    token and defers the exact form to DeepSeek-V3.2's lightning indexer: a
    head-weighted sum of ReLU'd query-key dot products.  The "Native MXFP4
    indexer" section (ネイティブMXFP4インデクサー) adds FP32 accumulation and the
    head-weighted reduction.  q_h is the E4M3-quantised query (module docstring);
    k_t = decoded key codes, s_t = its fp32 scale.  Evaluated in fp64, rounded once.
    """
    q = dequantized_query(q_idx) if quantize_query else np.asarray(q_idx, np.float64)
    k = e4m3_decode(key_codes)                                  # [n, 128]
    logits = (q @ k.T) * np.asarray(key_scales, np.float64)[None, :]   # [32, n]
    w = np.asarray(head_w, dtype=np.float64)[:, None]           # [32, 1]
    score = np.sum(w * np.maximum(logits, 0.0), axis=0)
    return score.astype(np.float32)


def index_scores_values(q_idx: np.ndarray, head_w: np.ndarray, key_values: np.ndarray,
                        quantize_query: bool = True) -> np.ndarray:
    """The same score for keys given as values k_t [n, 128] (the MXFP4 keys of the "Native
    MXFP4 indexer" section, whose block scales are part of the values, so there is no
    per-token scale): score_t = sum_h w_h * ReLU(q_h . k_t), fp64, rounded once to fp32."""
    q = dequantized_query(q_idx) if quantize_query else np.asarray(q_idx, np.float64)
    logits = q @ np.asarray(key_values, np.float64).T                # [32, n]
    w = np.asarray(head_w, dtype=np.float64)[:, None]
    score = np.sum(w * np.maximum(logits, 0.0), axis=0)
    return score.astype(np.float32)


# --------------------------------------------------------------------------------------
# Stage 2: top-k
# --------------------------------------------------------------------------------------
def topk_indices(scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) best token indices under (score descending, index ascending).

    The K3.1 page keeps the top 2,048 tokens per query ("What changed in Kimi K3.1
    Pro") with exact selection ("Exact top-k merge" / 正確なtop-kマージ) and a
    consistent tie rule ("Inter-GPU communication" / GPU間通信).  A full sort:
    -0.0 is made +0.0 first, so the two zeros tie and the lower index wins.
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0
    assert not np.isnan(s).any(), "NaN score"
    t = np.arange(s.shape[0])
    order = np.lexsort((t, -s))
    return order[:min(k, s.shape[0])]


# --------------------------------------------------------------------------------------
# Stage 3: exact MLA over the selected tokens (NoPE, shared 576-dim latent)
# --------------------------------------------------------------------------------------
def mla_attend(q_mla: np.ndarray, latent_codes: np.ndarray, latent_scale: float,
               softmax_scale: float, quantize_query: bool = True):
    """Softmax attention of 96 heads over the given latent rows.

    The K3.1 page runs MLA exactly over only the selected tokens ("What changed in
    Kimi K3.1 Pro"), on a 576-byte FP8 latent ("Sparse attention cuts long-context
    decode bandwidth" / スパースアテンションが長いコンテキストのデコード帯域幅を削減)
    with no positional encoding (NoPE) and 96 heads ("Token-sharded prefill").
    Keys are all 576 dims of the decoded latent, values its first 512 dims.

    Returns O [96, 512] and LSE [96] in fp64.  No rows: O = 0, LSE = -inf.
    """
    q = dequantized_query(q_mla) if quantize_query else np.asarray(q_mla, np.float64)
    n = latent_codes.shape[0]
    if n == 0:
        return np.zeros((q.shape[0], V_DIM)), np.full(q.shape[0], -np.inf)
    kv = e4m3_decode(latent_codes) * float(latent_scale)       # [n, 576]
    x = float(softmax_scale) * (q @ kv.T)                      # [96, n]
    m = np.max(x, axis=1, keepdims=True)
    e = np.exp(x - m)
    z = np.sum(e, axis=1, keepdims=True)
    o = (e / z) @ kv[:, :V_DIM]
    lse = m[:, 0] + np.log(z[:, 0])
    return o, lse


def dense_mla(q_mla: np.ndarray, latent_codes_all: np.ndarray, latent_scale: float,
              softmax_scale: float, quantize_query: bool = True):
    """Dense MLA over every visible token, written independently of mla_attend.

    Uses the log-domain form: LSE = log(sum exp(x)), weights = exp(x - LSE).  It is
    the right-hand side of the check that a top-k equal to the context length
    reproduces dense attention.
    """
    q = dequantized_query(q_mla) if quantize_query else np.asarray(q_mla, np.float64)
    kv = e4m3_decode(latent_codes_all) * float(latent_scale)
    logits = float(softmax_scale) * np.einsum("hd,td->ht", q, kv)
    lse = np.logaddexp.reduce(logits, axis=1)
    weights = np.exp(logits - lse[:, None])
    o = np.einsum("ht,td->hd", weights, kv[:, :V_DIM])
    return o, lse


# --------------------------------------------------------------------------------------
# Stage 4: log-sum-exp combine of split partials
# --------------------------------------------------------------------------------------
def lse_combine(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Merge per-split (O_s normalised by its own sum, LSE_s) into (O, LSE).

    The K3.1 page merges partial attention outputs by log-sum-exp ("Decode context
    parallelism with the sparse indexer" / スパースインデクサーを使用したデコード
    コンテキスト並列処理, and the exchange-and-combine kernels of "Exact top-k
    merge").  LSE = m + ln sum_s exp(LSE_s - m), O = sum_s exp(LSE_s - LSE) O_s.
    An empty split has LSE_s = -inf and contributes nothing; all empty -> O = 0,
    LSE = -inf.
    """
    lses = np.stack([np.asarray(l, np.float64) for _, l in parts])      # [S, H]
    outs = np.stack([np.asarray(o, np.float64) for o, _ in parts])      # [S, H, D]
    m = np.max(lses, axis=0)                                           # [H]
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe[None, :]), 0.0)
    tot = np.sum(w, axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    coef = np.where(finite[None, :], w / np.where(finite, tot, 1.0)[None, :], 0.0)
    o = np.einsum("sh,shd->hd", coef, outs)
    return o, lse


def split_ranges(n: int, num_splits: int) -> List[Tuple[int, int]]:
    """Balanced contiguous ranges [s*n//S, (s+1)*n//S) of the selected list."""
    return [(s * n // num_splits, (s + 1) * n // num_splits) for s in range(num_splits)]


# --------------------------------------------------------------------------------------
# Whole row
# --------------------------------------------------------------------------------------
def decode_row(q_idx, head_w, q_mla, key_codes, key_scales, latent_codes, latent_scale,
               softmax_scale, pos: int, k: int, block_table_row=None):
    """Every stage for one query row that sees tokens 0..pos.

    key_codes / key_scales / latent_codes are the request's logical rows (at least
    pos + 1 of them).  Returns a dict with scores (fp32), the selected indices
    (sorted by score), O and LSE (fp64), and physical slots if a block table row
    is given.
    """
    n = pos + 1
    scores = index_scores(q_idx, head_w, key_codes[:n], key_scales[:n])
    sel = topk_indices(scores, k)
    o, lse = mla_attend(q_mla, latent_codes[sel], latent_scale, softmax_scale)
    out = {"scores": scores, "topk": sel, "o": o, "lse": lse}
    if block_table_row is not None:
        out["slots"] = physical_slot(block_table_row, sel)
    return out
