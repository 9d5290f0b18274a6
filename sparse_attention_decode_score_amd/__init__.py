"""Python binding of libdsa, the MI355X (gfx950) DSA decode hot path.

Argument marshalling only: every step of the path runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and the stream; each function passes raw
pointers, host scalars and `torch.cuda.current_stream().cuda_stream` to the C ABI
declared in include/dsa.h, under the same names.

The library is loaded from this package's lib/ folder (built by build.py).  There is
no fallback: if it is missing, or a tensor is not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libdsa.so")

PAGE = 64
IDX_HEADS, IDX_DIM, IDX_PAGE_BYTES = 32, 128, 8448
MLA_HEADS, LATENT_DIM, V_DIM, LATENT_PAGE_BYTES = 96, 576, 512, 36864
MAX_TOPK, MAX_SPLITS = 4096, 64

STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
          3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_LAUNCH"}


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libdsa (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python sparse_attention_decode_score_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        L.dsa_index_score.argtypes = [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P, _I32,
                                      _P, _I64, _I32, _P, _SZ, _P]
        L.dsa_index_score_mxfp4.argtypes = L.dsa_index_score.argtypes
        L.dsa_index_score_quantize_q.argtypes = [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _I64,
                                                 _I32, _P, _I32, _P, _I64, _I32, _P, _SZ, _P, _P,
                                                 _P, _P]
        L.dsa_topk_workspace_status.argtypes = [_P, _SZ, _P]
        L.dsa_topk_workspace_size.argtypes = [_I32, _I32, _I32]
        L.dsa_topk_workspace_size.restype = _SZ
        L.dsa_topk.argtypes = [_I32, _I32, _I32, _P, _P, _P, _I64, _I32, _P, _I32, _P, _P, _P, _SZ,
                               _I32, _P, _P, _P, _I64, _I32, _P]
        L.dsa_sparse_mla_workspace_size.argtypes = [_I32, _I32]
        L.dsa_sparse_mla_workspace_size.restype = _SZ
        L.dsa_sparse_mla_decode.argtypes = [_I32, _P, _P, _P, _P, _I64, _F32, _P, _I32, _F32, _I32,
                                            _P, _P, _P, _P, _P, _SZ, _P]
        L.dsa_topk_sparse_mla.argtypes = [_I32, _I32, _I32, _P, _P, _P, _I64, _I32, _P, _I32, _P,
                                          _SZ, _P, _P, _P, _I64, _I32, _P, _P, _P, _P, _P, _P, _I64,
                                          _F32, _F32, _I32, _P, _P, _P, _SZ, _P]
        L.dsa_lse_combine.argtypes = [_I32, _I32, _P, _P, _P, _P, _P]
        L.dsa_cache_append.argtypes = [_I32, _P, _P, _P, _F32, _P, _I64, _P, _I64, _P]
        L.dsa_cache_append_mxfp4.argtypes = [_I32, _P, _P, _P, _F32, _P, _I64, _P, _I64, _P]
        L.dsa_quantize_q.argtypes = [_I32, _I32, _I32, _P, _P, _P, _P]
        L.dsa_sparse_mla_decode_noalloc.argtypes = [_I32, _P, _P, _P, _P, _I64, _F32, _P, _I32,
                                                    _F32, _I32, _P, _P, _P, _P, _P]
        L.dsa_validate_batch.argtypes = [_I32, _I32, _I32, _I32, _P, _P, _P, _I32, _I64, _P, _I32]
        L.dsa_validate_slots.argtypes = [_I32, _P, _I64]
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_version.restype = ctypes.c_char_p
        for f in ("dsa_index_score", "dsa_index_score_mxfp4", "dsa_index_score_quantize_q", "dsa_topk", "dsa_sparse_mla_decode", "dsa_topk_sparse_mla",
                  "dsa_lse_combine", "dsa_quantize_q", "dsa_cache_append", "dsa_cache_append_mxfp4",
                  "dsa_validate_batch",
                  "dsa_validate_slots", "dsa_sparse_mla_decode_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise DsaError(status, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("DSA tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("DSA tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _expect(t: torch.Tensor, name: str, dtype, shape=None):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _host_i32(a, name):
    """A contiguous host int32 array (numpy or CPU tensor) and its address."""
    import numpy as np
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError(f"{name}: the validators take host copies (call .cpu() first)")
        a = a.numpy()
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data


def dsa_validate_batch(cu_q, seq_lens, block_table, num_pages: int, *, max_seq_len: int,
                       max_q_per_seq: int, topk_slot=None) -> None:
    """Checks host copies of a batch description, its block table and (optionally) selected
    slots [n_q, k] on the CPU; raises DsaError naming the first violation."""
    cu, cu_p = _host_i32(cu_q, "cu_q")
    sl, sl_p = _host_i32(seq_lens, "seq_lens")
    bt, bt_p = _host_i32(block_table, "block_table")
    ts, ts_p, k = None, None, 0
    if topk_slot is not None:
        ts, ts_p = _host_i32(topk_slot, "topk_slot")
        k = ts.shape[1]
    _check(lib().dsa_validate_batch(sl.shape[0], int(cu[-1]) if cu.size else 0, int(max_seq_len),
                                    int(max_q_per_seq), cu_p, sl_p, bt_p, bt.shape[1],
                                    int(num_pages), ts_p, int(k)))


def dsa_validate_slots(slots, num_pages: int) -> None:
    """Checks host copies of dsa_cache_append slots on the CPU; raises DsaError."""
    s, s_p = _host_i32(slots, "slots")
    _check(lib().dsa_validate_slots(s.shape[0], s_p, int(num_pages)))


def dsa_version() -> str:
    return lib().dsa_version().decode()


def dsa_quantize_q(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """E4M3 codes [rows, heads, dim] (uint8) and power-of-two scales [rows, heads] of q."""
    _expect(q, "q", torch.bfloat16)
    rows, heads, dim = q.shape
    _expect(codes, "codes", torch.uint8, (rows, heads, dim))
    _expect(scales, "scales", torch.float32, (rows, heads))
    _check(lib().dsa_quantize_q(rows, heads, dim, _ptr(q), _ptr(codes), _ptr(scales), _stream(stream)))


def dsa_index_score(cu_q: torch.Tensor, seq_lens: torch.Tensor, q_idx: torch.Tensor,
                    head_w: torch.Tensor, key_pages: torch.Tensor, block_table: torch.Tensor,
                    scores: Optional[torch.Tensor], *, max_seq_len: int, max_q_per_seq: int,
                    key_page_stride: Optional[int] = None, cand_k: int = 0,
                    cand_workspace: Optional[torch.Tensor] = None, key_format: str = "e4m3",
                    mla_query: Optional[tuple] = None, stream=None) -> None:
    """Indexer scores into scores [n_q, score_stride] (fp32); with cand_workspace, also the
    per-chunk top-k candidates for a top-k of cand_k (consumed by dsa_topk with
    from_candidates=True).  scores=None with cand_workspace: candidates only (no scores
    stored; pass rescore=(q_idx, head_w, key_pages) and the same key_format to the final
    top-k pass).  key_format "mxfp4": the key cache holds MXFP4 keys
    (dsa_index_score_mxfp4).  mla_query=(q_mla, codes, scales): the same launch also
    writes dsa_quantize_q(q_mla, codes, scales) (dsa_index_score_quantize_q)."""
    if key_format not in ("e4m3", "mxfp4"):
        raise ValueError(f"key_format must be 'e4m3' or 'mxfp4' (got {key_format!r})")
    num_seqs = seq_lens.shape[0]
    n_q = q_idx.shape[0]
    _expect(cu_q, "cu_q", torch.int32, (num_seqs + 1,))
    _expect(seq_lens, "seq_lens", torch.int32)
    _expect(q_idx, "q_idx", torch.bfloat16, (n_q, IDX_HEADS, IDX_DIM))
    _expect(head_w, "head_w", torch.float32, (n_q, IDX_HEADS))
    _expect(block_table, "block_table", torch.int32)
    if scores is not None:
        _expect(scores, "scores", torch.float32)
        if scores.dim() != 2 or scores.shape[0] != n_q:
            raise ValueError("scores must be [n_q, score_stride]")
    stride = key_page_stride if key_page_stride is not None else key_pages.stride(0) * key_pages.element_size()
    if cand_workspace is not None:
        _expect(cand_workspace, "cand_workspace", torch.uint8)
    if mla_query is not None:
        q_mla, codes, scales = mla_query
        _expect(q_mla, "q_mla", torch.bfloat16, (n_q, MLA_HEADS, LATENT_DIM))
        _expect(codes, "codes", torch.uint8, (n_q, MLA_HEADS, LATENT_DIM))
        _expect(scales, "scales", torch.float32, (n_q, MLA_HEADS))
        _check(lib().dsa_index_score_quantize_q(
            num_seqs, n_q, int(max_seq_len), int(max_q_per_seq), _ptr(cu_q), _ptr(seq_lens),
            _ptr(q_idx), _ptr(head_w), _ptr(key_pages), int(stride), _KEY_FORMATS[key_format],
            _ptr(block_table), block_table.shape[1], _ptr(scores),
            scores.shape[1] if scores is not None else 0, int(cand_k), _ptr(cand_workspace),
            cand_workspace.numel() if cand_workspace is not None else 0, _ptr(q_mla),
            _ptr(codes), _ptr(scales), _stream(stream)))
        return
    fn = lib().dsa_index_score_mxfp4 if key_format == "mxfp4" else lib().dsa_index_score
    _check(fn(num_seqs, n_q, int(max_seq_len), int(max_q_per_seq), _ptr(cu_q),
                                 _ptr(seq_lens), _ptr(q_idx), _ptr(head_w), _ptr(key_pages),
                                 int(stride), _ptr(block_table), block_table.shape[1],
                                 _ptr(scores), scores.shape[1] if scores is not None else 0,
                                 int(cand_k),
                                 _ptr(cand_workspace),
                                 cand_workspace.numel() if cand_workspace is not None else 0,
                                 _stream(stream)))


_KEY_FORMATS = {"e4m3": 0, "mxfp4": 1}


def _rescore_args(rescore, key_format):
    """(q_idx, head_w, key_pages[, key_page_stride]) and the key cache's format -> C
    arguments, or NULLs."""
    if key_format not in _KEY_FORMATS:
        raise ValueError(f"key_format must be 'e4m3' or 'mxfp4' (got {key_format!r})")
    if rescore is None:
        return (None, None, None, 0, 0)
    q_idx, head_w, key_pages = rescore[:3]
    _expect(q_idx, "q_idx", torch.bfloat16)
    _expect(head_w, "head_w", torch.float32)
    stride = (rescore[3] if len(rescore) > 3
              else key_pages.stride(0) * key_pages.element_size())
    return (_ptr(q_idx), _ptr(head_w), _ptr(key_pages), int(stride), _KEY_FORMATS[key_format])


def dsa_topk_workspace_size(n_q: int, max_seq_len: int, k: int) -> int:
    return int(lib().dsa_topk_workspace_size(int(n_q), int(max_seq_len), int(k)))


def dsa_topk_workspace_status(workspace: torch.Tensor, stream=None) -> None:
    """Reads the top-k workspace's layout record (waits for the stream): raises DsaError if no
    call wrote candidates into it, or if a final pass found them written for another
    (k, max_seq_len, n_q) and therefore selected nothing."""
    _check(lib().dsa_topk_workspace_status(_ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                           _stream(stream)))


def dsa_topk(cu_q: torch.Tensor, seq_lens: torch.Tensor, scores: torch.Tensor, k: int,
             block_table: Optional[torch.Tensor], topk_idx: torch.Tensor,
             topk_slot: Optional[torch.Tensor], workspace: torch.Tensor, *, max_seq_len: int,
             from_candidates: bool = False, rescore=None, key_format: str = "e4m3",
             stream=None) -> None:
    """Exact top-k token indices (and physical slots) of every row's visible scores.
    rescore=(q_idx, head_w, key_pages): the indexer stored no scores; scores is scratch
    (key_format: that of the index-key cache, "e4m3" or "mxfp4")."""
    num_seqs = seq_lens.shape[0]
    n_q = scores.shape[0]
    _expect(scores, "scores", torch.float32)
    _expect(topk_idx, "topk_idx", torch.int32, (n_q, k))
    if topk_slot is not None:
        _expect(topk_slot, "topk_slot", torch.int32, (n_q, k))
    _expect(workspace, "workspace", torch.uint8)
    _check(lib().dsa_topk(num_seqs, n_q, int(max_seq_len), _ptr(cu_q), _ptr(seq_lens), _ptr(scores),
                          scores.shape[1], int(k), _ptr(block_table),
                          block_table.shape[1] if block_table is not None else 0,
                          _ptr(topk_idx), _ptr(topk_slot), _ptr(workspace), workspace.numel(),
                          int(bool(from_candidates)), *_rescore_args(rescore, key_format),
                          _stream(stream)))


def dsa_sparse_mla_workspace_size(n_q: int, num_splits: int) -> int:
    return int(lib().dsa_sparse_mla_workspace_size(int(n_q), int(num_splits)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of nbytes (torch's allocator is aligned)."""
    t = torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)
    if t.data_ptr() % 256:
        raise RuntimeError("allocator returned a buffer that is not 256-byte aligned")
    return t


def dsa_sparse_mla_decode(q_mla: Optional[torch.Tensor], latent_pages: torch.Tensor,
                          latent_scale: float, topk_slot: torch.Tensor, softmax_scale: float,
                          num_splits: int, *, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None,
                          o_part: Optional[torch.Tensor] = None,
                          lse_part: Optional[torch.Tensor] = None,
                          q8: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          latent_page_stride: Optional[int] = None, stream=None) -> None:
    """MLA over the selected slots.  Query: q8/q_scale (from dsa_quantize_q) if given, else
    q_mla (bf16).  Output: fp32 split partials (o_part, lse_part) if given, else (out, lse),
    merged inside the call when num_splits > 1."""
    n_q, k = topk_slot.shape
    _expect(topk_slot, "topk_slot", torch.int32, (n_q, k))
    if q8 is not None:
        _expect(q8, "q8", torch.uint8, (n_q, MLA_HEADS, LATENT_DIM))
        _expect(q_scale, "q_scale", torch.float32, (n_q, MLA_HEADS))
    else:
        _expect(q_mla, "q_mla", torch.bfloat16, (n_q, MLA_HEADS, LATENT_DIM))
    if o_part is not None:
        _expect(o_part, "o_part", torch.float32, (num_splits, n_q, MLA_HEADS, V_DIM))
        _expect(lse_part, "lse_part", torch.float32, (num_splits, n_q, MLA_HEADS))
    else:
        _expect(out, "out", torch.bfloat16, (n_q, MLA_HEADS, V_DIM))
        _expect(lse, "lse", torch.float32, (n_q, MLA_HEADS))
        if num_splits > 1 and workspace is None:
            workspace = globals()["workspace"](dsa_sparse_mla_workspace_size(n_q, num_splits),
                                               topk_slot.device)
    if workspace is not None:
        _expect(workspace, "workspace", torch.uint8)
    stride = (latent_page_stride if latent_page_stride is not None
              else latent_pages.stride(0) * latent_pages.element_size())
    _check(lib().dsa_sparse_mla_decode(n_q, _ptr(q_mla), _ptr(q8), _ptr(q_scale),
                                       _ptr(latent_pages), int(stride), float(latent_scale),
                                       _ptr(topk_slot), int(k), float(softmax_scale),
                                       int(num_splits), _ptr(out), _ptr(lse), _ptr(o_part),
                                       _ptr(lse_part), _ptr(workspace),
                                       workspace.numel() if workspace is not None else 0,
                                       _stream(stream)))


def dsa_sparse_mla_decode_noalloc(q_mla: Optional[torch.Tensor], latent_pages: torch.Tensor,
                                  latent_scale: float, topk_slot: torch.Tensor,
                                  softmax_scale: float, num_splits: int, *,
                                  out: Optional[torch.Tensor] = None,
                                  lse: Optional[torch.Tensor] = None,
                                  o_part: Optional[torch.Tensor] = None,
                                  lse_part: Optional[torch.Tensor] = None,
                                  q8: Optional[torch.Tensor] = None,
                                  q_scale: Optional[torch.Tensor] = None,
                                  latent_page_stride: Optional[int] = None, stream=None) -> None:
    """dsa_sparse_mla_decode without a workspace: merged split partials go to the library's
    static device scratch (64 MiB per GPU), so the call allocates nothing."""
    n_q, k = topk_slot.shape
    _expect(topk_slot, "topk_slot", torch.int32, (n_q, k))
    if q8 is not None:
        _expect(q8, "q8", torch.uint8, (n_q, MLA_HEADS, LATENT_DIM))
        _expect(q_scale, "q_scale", torch.float32, (n_q, MLA_HEADS))
    else:
        _expect(q_mla, "q_mla", torch.bfloat16, (n_q, MLA_HEADS, LATENT_DIM))
    if o_part is not None:
        _expect(o_part, "o_part", torch.float32, (num_splits, n_q, MLA_HEADS, V_DIM))
        _expect(lse_part, "lse_part", torch.float32, (num_splits, n_q, MLA_HEADS))
    else:
        _expect(out, "out", torch.bfloat16, (n_q, MLA_HEADS, V_DIM))
        _expect(lse, "lse", torch.float32, (n_q, MLA_HEADS))
    stride = (latent_page_stride if latent_page_stride is not None
              else latent_pages.stride(0) * latent_pages.element_size())
    _check(lib().dsa_sparse_mla_decode_noalloc(n_q, _ptr(q_mla), _ptr(q8), _ptr(q_scale),
                                               _ptr(latent_pages), int(stride),
                                               float(latent_scale), _ptr(topk_slot), int(k),
                                               float(softmax_scale), int(num_splits), _ptr(out),
                                               _ptr(lse), _ptr(o_part), _ptr(lse_part),
                                               _stream(stream)))


def dsa_topk_sparse_mla(cu_q: torch.Tensor, seq_lens: torch.Tensor, scores: torch.Tensor, k: int,
                        block_table: torch.Tensor, cand_workspace: torch.Tensor,
                        q_mla: Optional[torch.Tensor], latent_pages: torch.Tensor,
                        latent_scale: float, softmax_scale: float, num_splits: int, *,
                        max_seq_len: int, out: torch.Tensor, lse: torch.Tensor,
                        topk_idx: Optional[torch.Tensor] = None,
                        topk_slot: Optional[torch.Tensor] = None,
                        q8: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None,
                        latent_page_stride: Optional[int] = None, rescore=None,
                        key_format: str = "e4m3", stream=None) -> None:
    """Final top-k pass and sparse MLA in one launch: every attention workgroup selects its
    row's top k from the candidates dsa_index_score left in cand_workspace (cand_k = k), then
    attends over its split of them.  topk_idx / topk_slot, when given, receive the selection.
    rescore=(q_idx, head_w, key_pages): the indexer stored no scores; scores is scratch
    (key_format: that of the index-key cache)."""
    num_seqs = seq_lens.shape[0]
    n_q = scores.shape[0]
    _expect(scores, "scores", torch.float32)
    _expect(cand_workspace, "cand_workspace", torch.uint8)
    if topk_idx is not None:
        _expect(topk_idx, "topk_idx", torch.int32, (n_q, k))
    if topk_slot is not None:
        _expect(topk_slot, "topk_slot", torch.int32, (n_q, k))
    if q8 is not None:
        _expect(q8, "q8", torch.uint8, (n_q, MLA_HEADS, LATENT_DIM))
        _expect(q_scale, "q_scale", torch.float32, (n_q, MLA_HEADS))
    else:
        _expect(q_mla, "q_mla", torch.bfloat16, (n_q, MLA_HEADS, LATENT_DIM))
    _expect(out, "out", torch.bfloat16, (n_q, MLA_HEADS, V_DIM))
    _expect(lse, "lse", torch.float32, (n_q, MLA_HEADS))
    if num_splits > 1 and workspace is None:
        workspace = globals()["workspace"](dsa_sparse_mla_workspace_size(n_q, num_splits),
                                           scores.device)
    if workspace is not None:
        _expect(workspace, "workspace", torch.uint8)
    stride = (latent_page_stride if latent_page_stride is not None
              else latent_pages.stride(0) * latent_pages.element_size())
    _check(lib().dsa_topk_sparse_mla(
        num_seqs, n_q, int(max_seq_len), _ptr(cu_q), _ptr(seq_lens), _ptr(scores),
        scores.shape[1], int(k), _ptr(block_table), block_table.shape[1], _ptr(cand_workspace),
        cand_workspace.numel(), *_rescore_args(rescore, key_format), _ptr(topk_idx), _ptr(topk_slot),
        _ptr(q_mla), _ptr(q8),
        _ptr(q_scale), _ptr(latent_pages), int(stride), float(latent_scale),
        float(softmax_scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream)))


def dsa_lse_combine(o_part: torch.Tensor, lse_part: torch.Tensor, out: torch.Tensor,
                    lse: torch.Tensor, stream=None) -> None:
    """LSE merge of split partials [S, n_q, 96, 512] / [S, n_q, 96] into bf16 out and lse."""
    S, n_q = o_part.shape[0], o_part.shape[1]
    _expect(o_part, "o_part", torch.float32, (S, n_q, MLA_HEADS, V_DIM))
    _expect(lse_part, "lse_part", torch.float32, (S, n_q, MLA_HEADS))
    _expect(out, "out", torch.bfloat16, (n_q, MLA_HEADS, V_DIM))
    _expect(lse, "lse", torch.float32, (n_q, MLA_HEADS))
    _check(lib().dsa_lse_combine(S, n_q, _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse),
                                 _stream(stream)))


def _cache_append(fn, slots, key, latent, latent_scale, key_pages, latent_pages,
                  key_page_stride, latent_page_stride, stream):
    n = slots.shape[0]
    _expect(slots, "slots", torch.int32, (n,))
    if key is not None:
        _expect(key, "key", torch.bfloat16, (n, IDX_DIM))
    if latent is not None:
        _expect(latent, "latent", torch.bfloat16, (n, LATENT_DIM))
    ks = (key_page_stride if key_page_stride is not None
          else (key_pages.stride(0) * key_pages.element_size() if key_pages is not None else 0))
    ls = (latent_page_stride if latent_page_stride is not None
          else (latent_pages.stride(0) * latent_pages.element_size() if latent_pages is not None else 0))
    _check(fn(int(n), _ptr(slots), _ptr(key), _ptr(latent), float(latent_scale),
              _ptr(key_pages), int(ks), _ptr(latent_pages), int(ls), _stream(stream)))


def dsa_cache_append(slots: torch.Tensor, key: Optional[torch.Tensor],
                     latent: Optional[torch.Tensor], latent_scale: float,
                     key_pages: Optional[torch.Tensor], latent_pages: Optional[torch.Tensor], *,
                     key_page_stride: Optional[int] = None,
                     latent_page_stride: Optional[int] = None, stream=None) -> None:
    """Quantises new tokens (index keys bf16 [n, 128], latents bf16 [n, 576]) into the paged
    caches at their physical slots (int32 [n], -1 = skip); E4M3 index-key pages."""
    _cache_append(lib().dsa_cache_append, slots, key, latent, latent_scale, key_pages,
                  latent_pages, key_page_stride, latent_page_stride, stream)


def dsa_cache_append_mxfp4(slots: torch.Tensor, key: Optional[torch.Tensor],
                           latent: Optional[torch.Tensor], latent_scale: float,
                           key_pages: Optional[torch.Tensor],
                           latent_pages: Optional[torch.Tensor], *,
                           key_page_stride: Optional[int] = None,
                           latent_page_stride: Optional[int] = None, stream=None) -> None:
    """dsa_cache_append for MXFP4 index-key pages (68 bytes per token)."""
    _cache_append(lib().dsa_cache_append_mxfp4, slots, key, latent, latent_scale, key_pages,
                  latent_pages, key_page_stride, latent_page_stride, stream)


class DecodeStep:
    """Device buffers for one pass of the whole path over a fixed batch shape.

    Allocates (through torch) the scores, top-k outputs, workspaces and the prepared MLA
    query once; run() issues the library calls on the current stream.  By default the
    indexer also emits the top-k candidates (fused) and stores no scores (store_scores=False:
    the final pass recomputes the few groups it must re-read), and the final top-k pass runs
    inside the attention kernel (select_in_attention: two launches, plus the split merge);
    otherwise stage 2 is its own call.  The MLA query is quantised inside the attention call
    (query_prep="inline", the default: the kernel stages the bf16 query in LDS while its
    selection runs), by the indexer's launch ("fused": one more workgroup per request there),
    by its own launch ahead of stage 1 ("first"), or on a side stream while stages 1 and 2
    run ("side"; query_on_side_stream=True means the same).
    """

    def __init__(self, n_q: int, max_seq_len: int, k: int, num_splits: int, device="cuda",
                 fused: bool = True, query_on_side_stream: bool = False,
                 select_in_attention: Optional[bool] = None, write_selection: bool = True,
                 store_scores: Optional[bool] = None, key_format: str = "e4m3",
                 query_prep: Optional[str] = None):
        if key_format not in _KEY_FORMATS:
            raise ValueError(f"key_format must be 'e4m3' or 'mxfp4' (got {key_format!r})")
        self.key_format = key_format
        if select_in_attention is None:
            select_in_attention = fused
        if store_scores is None:
            store_scores = not fused
        if not store_scores and not fused:
            raise ValueError("store_scores=False needs the indexer's candidates (fused=True)")
        # without stored scores, the final top-k pass recomputes the groups it re-reads from
        # the indexer's inputs (kept from index()) into self.scores, used as scratch
        self.store_scores = store_scores
        self._rescore = None
        if select_in_attention and not fused:
            raise ValueError("select_in_attention needs the indexer's candidates (fused=True)")
        # with select_in_attention, topk_idx / topk_slot are written only if write_selection
        self.write_selection = write_selection
        self.n_q, self.max_seq_len, self.k, self.num_splits = n_q, max_seq_len, k, num_splits
        self.fused = fused
        self.select_in_attention = select_in_attention
        if query_prep is None:
            query_prep = "side" if query_on_side_stream else "inline"
        if query_prep not in ("fused", "inline", "first", "side"):
            raise ValueError("query_prep must be 'fused', 'inline', 'first' or 'side' "
                             f"(got {query_prep!r})")
        self.query_prep = query_prep
        self.query_on_side_stream = query_prep == "side"
        self.query_prepared = query_prep != "inline"
        dev = torch.device(device)
        self.scores = torch.empty((n_q, max_seq_len), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((n_q, k), dtype=torch.int32, device=dev)
        self.topk_slot = torch.empty((n_q, k), dtype=torch.int32, device=dev)
        self.workspace = workspace(dsa_topk_workspace_size(n_q, max_seq_len, k), dev)
        self.mla_workspace = workspace(dsa_sparse_mla_workspace_size(n_q, num_splits), dev)
        self.q8 = torch.empty((n_q, MLA_HEADS, LATENT_DIM), dtype=torch.uint8, device=dev)
        self.q_scale = torch.empty((n_q, MLA_HEADS), dtype=torch.float32, device=dev)
        self.out = torch.empty((n_q, MLA_HEADS, V_DIM), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((n_q, MLA_HEADS), dtype=torch.float32, device=dev)
        self.side = torch.cuda.Stream(device=dev)  # default priority
        self._ev_start = torch.cuda.Event()
        self._ev_query = torch.cuda.Event()

    def index(self, cu_q, seq_lens, q_idx, head_w, key_pages, block_table, max_q_per_seq,
              stream=None, q_mla=None):
        """Stage 1 (with the fused first top-k pass when self.fused); with query_prep
        "fused", also the MLA query's quantisation (q_mla is then required)."""
        self._rescore = None if self.store_scores else (q_idx, head_w, key_pages)
        mla_query = None
        if self.query_prep == "fused":
            if q_mla is None:
                raise ValueError("query_prep='fused' quantises the MLA query in stage 1: pass q_mla")
            mla_query = (q_mla, self.q8, self.q_scale)
        dsa_index_score(cu_q, seq_lens, q_idx, head_w, key_pages, block_table,
                        self.scores if self.store_scores else None,
                        max_seq_len=self.max_seq_len, max_q_per_seq=max_q_per_seq,
                        cand_k=self.k, cand_workspace=self.workspace if self.fused else None,
                        key_format=self.key_format, mla_query=mla_query, stream=stream)

    def select(self, cu_q, seq_lens, block_table, stream=None):
        """Stage 2."""
        dsa_topk(cu_q, seq_lens, self.scores, self.k, block_table, self.topk_idx, self.topk_slot,
                 self.workspace, max_seq_len=self.max_seq_len, from_candidates=self.fused,
                 rescore=self._rescore, key_format=self.key_format, stream=stream)

    def prepare_query(self, q_mla, stream=None):
        """E4M3 codes and scales of the MLA query (stage 3's own quantisation)."""
        dsa_quantize_q(q_mla, self.q8, self.q_scale, stream=stream)

    def attend(self, q_mla, latent_pages, latent_scale, softmax_scale, stream=None):
        """Stages 3 and 4: on the query prepared by prepare_query when the step quantises it
        beforehand, else on q_mla (quantised inside the call)."""
        if self.query_prepared:
            dsa_sparse_mla_decode(None, latent_pages, latent_scale, self.topk_slot, softmax_scale,
                                  self.num_splits, out=self.out, lse=self.lse, q8=self.q8,
                                  q_scale=self.q_scale, workspace=self.mla_workspace,
                                  stream=stream)
        else:
            dsa_sparse_mla_decode(q_mla, latent_pages, latent_scale, self.topk_slot,
                                  softmax_scale, self.num_splits, out=self.out, lse=self.lse,
                                  workspace=self.mla_workspace, stream=stream)
        return self.out, self.lse

    def select_attend(self, cu_q, seq_lens, block_table, q_mla, latent_pages, latent_scale,
                      softmax_scale, stream=None):
        """Stages 2-4 in one launch (the final top-k pass inside the attention kernel)."""
        prepared = self.query_prepared
        dsa_topk_sparse_mla(cu_q, seq_lens, self.scores, self.k, block_table, self.workspace,
                            None if prepared else q_mla, latent_pages, latent_scale,
                            softmax_scale, self.num_splits, max_seq_len=self.max_seq_len,
                            out=self.out, lse=self.lse,
                            topk_idx=self.topk_idx if self.write_selection else None,
                            topk_slot=self.topk_slot if self.write_selection else None,
                            rescore=self._rescore, key_format=self.key_format,
                            q8=self.q8 if prepared else None,
                            q_scale=self.q_scale if prepared else None,
                            workspace=self.mla_workspace, stream=stream)
        return self.out, self.lse

    def run(self, cu_q, seq_lens, q_idx, head_w, key_pages, block_table, q_mla, latent_pages,
            latent_scale, softmax_scale, max_q_per_seq, stream=None):
        main = torch.cuda.current_stream() if stream is None else stream
        if self.query_prep == "first":
            self.prepare_query(q_mla, stream=main)
        if self.query_on_side_stream:
            self._ev_start.record(main)
            self.side.wait_event(self._ev_start)
            self.prepare_query(q_mla, stream=self.side)
            self._ev_query.record(self.side)
        self.index(cu_q, seq_lens, q_idx, head_w, key_pages, block_table, max_q_per_seq, main,
                   q_mla=q_mla)
        if self.select_in_attention:
            if self.query_on_side_stream:
                main.wait_event(self._ev_query)
            return self.select_attend(cu_q, seq_lens, block_table, q_mla, latent_pages,
                                      latent_scale, softmax_scale, main)
        self.select(cu_q, seq_lens, block_table, main)
        if self.query_on_side_stream:
            main.wait_event(self._ev_query)
        return self.attend(q_mla, latent_pages, latent_scale, softmax_scale, main)
