"""Python binding of libkvq (include/kvq.h): the MI355X decode step for paged,
quantized, query-aware sparse attention.

This module only marshals arguments: torch tensors supply device memory and
the current HIP stream, and every step runs in the HIP kernels of libkvq.so.
There is no CPU or PyTorch fallback; if the library is missing, importing the
entry points raises.

Entry points keep the C names:
  kvq_append_quant, kvq_append_decode, kvq_append_decode_scores, kvq_build_page_meta,
  kvq_page_scores, kvq_topk_pages,
  kvq_sparse_decode_attn, kvq_select_decode_attn, kvq_select_decode_attn_noalloc, kvq_attn_workspace_bytes,
  kvq_default_pages_per_split, kvq_decode_step, kvq_step_workspace_bytes, kvq_step_counter_bytes,
  kvq_build_coarse_meta, kvq_page_scores_masked, kvq_num_selected (as num_selected)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_FP16, KVQ_INT8_TOKEN, KVQ_INT8_GROUP64, KVQ_INT4_TOKEN, KVQ_INT4_GROUP64, KVQ_MIXED_FP16_INT8 = 0, 1, 2, 3, 4, 5
PAGE_SIZE = 16
SELECT_MAX_PAGES = 2048  # KVQ_SELECT_MAX_PAGES: longest row kvq_select_decode_attn takes
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
           3: "workspace missing or too small", 4: "HIP launch failed"}


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} (status {status})")
        self.status = status


class CacheStruct(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_phys_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("kv_params", ctypes.c_void_p), ("page_meta", ctypes.c_void_p), ("num_fp16_pages", ctypes.c_int32)]


class SeqsStruct(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvq.so not found at {LIB_PATH}: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, C, S = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(CacheStruct), ctypes.POINTER(SeqsStruct)
        L.kvq_append_quant.argtypes = [C, S, P, P, I, P, P, P]
        L.kvq_append_decode.argtypes = [C, S, P, P, I, P, P, P]
        L.kvq_append_decode_scores.argtypes = [C, S, P, P, I, P, P, P, I, P, P]
        L.kvq_build_page_meta.argtypes = [C, S, P, I, P]
        L.kvq_page_scores.argtypes = [C, S, P, I, P, P]
        L.kvq_topk_pages.argtypes = [P, S, I, I, I, I, I, P, P, P]
        L.kvq_sparse_decode_attn.argtypes = [C, S, P, I, P, P, I, ctypes.c_float, I, P, P, ctypes.c_size_t, P]
        L.kvq_select_decode_attn.argtypes = [C, S, P, I, P, I, I, I, I, P, P, ctypes.c_float, I, P, P,
                                             ctypes.c_size_t, P]
        L.kvq_select_decode_attn_noalloc.argtypes = [C, S, P, I, P, I, I, I, I, P, P, ctypes.c_float, I, P, P]
        L.kvq_decode_step.argtypes = [C, S, P, P, I, P, P, P, I, P, I, I, I, I, P, P, ctypes.c_float, I, P, P,
                                      ctypes.c_size_t, P]
        L.kvq_build_coarse_meta.argtypes = [C, S, I, P, I, P, P, P, P]
        L.kvq_page_scores_masked.argtypes = [C, S, P, I, I, P, P, I, P, P]
        L.kvq_demote_pages.argtypes = [C, S, I, P, P, P, P]
        L.kvq_step_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.kvq_step_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_step_counter_bytes.argtypes = [I, I]
        L.kvq_step_counter_bytes.restype = ctypes.c_size_t
        for f in ("kvq_append_quant", "kvq_append_decode", "kvq_append_decode_scores", "kvq_build_page_meta",
                  "kvq_page_scores", "kvq_topk_pages", "kvq_sparse_decode_attn", "kvq_select_decode_attn",
                  "kvq_select_decode_attn_noalloc", "kvq_decode_step", "kvq_build_coarse_meta",
                  "kvq_page_scores_masked", "kvq_demote_pages"):
            getattr(L, f).restype = ctypes.c_int
        L.kvq_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
        L.kvq_read_probe.restype = ctypes.c_int
        L.kvq_attn_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.kvq_attn_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_num_selected.argtypes = [I, I, I, I]
        L.kvq_num_selected.restype = I
        L.kvq_default_pages_per_split.argtypes = [I, I, I, I]
        L.kvq_default_pages_per_split.restype = I
        L.kvq_status_string.argtypes = [ctypes.c_int]
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_abi_version.argtypes = []
        L.kvq_abi_version.restype = I
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("libkvq takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libkvq takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvqError(fn, status)


# ----------------------------------------------------------- device views
@dataclass
class PagedCache:
    """One layer's paged cache in device memory (layout of include/kvq.h).
    KVQ_MIXED_FP16_INT8: k_pages / v_pages are one byte array each (the FP16
    pool of num_fp16_pages pages, then the INT8 pool), kv_params the INT8
    pool's."""

    format: int
    num_phys_pages: int
    num_kv_heads: int
    head_dim: int
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    kv_params: torch.Tensor | None
    page_meta: torch.Tensor
    num_fp16_pages: int = 0

    @staticmethod
    def empty(fmt: int, num_phys_pages: int, num_kv_heads: int, head_dim: int, device="cuda",
              num_fp16_pages: int = 0) -> "PagedCache":
        # 4-bit codes: two channels per byte, so a token row is head_dim / 2 bytes
        row = head_dim // 2 if fmt in (KVQ_INT4_TOKEN, KVQ_INT4_GROUP64) else head_dim
        shape = (num_phys_pages, num_kv_heads, PAGE_SIZE, row)
        dt = torch.int16 if fmt == KVQ_FP16 else torch.uint8
        n16 = num_fp16_pages if fmt == KVQ_MIXED_FP16_INT8 else 0
        if fmt == KVQ_MIXED_FP16_INT8:
            if not 0 <= n16 <= num_phys_pages:
                raise ValueError("num_fp16_pages must lie in [0, num_phys_pages]")
            tile = num_kv_heads * PAGE_SIZE * head_dim
            shape = (n16 * tile * 2 + (num_phys_pages - n16) * tile,)
        k = torch.zeros(shape, dtype=dt, device=device)
        v = torch.zeros(shape, dtype=dt, device=device)
        if fmt == KVQ_MIXED_FP16_INT8:
            p = torch.zeros((max(num_phys_pages - n16, 1), num_kv_heads, PAGE_SIZE, 4), dtype=torch.float32,
                            device=device)
        elif fmt in (KVQ_INT8_TOKEN, KVQ_INT4_TOKEN):
            p = torch.zeros((num_phys_pages, num_kv_heads, PAGE_SIZE, 4), dtype=torch.float32, device=device)
        elif fmt in (KVQ_INT8_GROUP64, KVQ_INT4_GROUP64):
            p = torch.zeros((num_phys_pages, num_kv_heads, 4), dtype=torch.float32, device=device)
        else:
            p = None
        meta = torch.zeros((num_phys_pages, num_kv_heads, 2, head_dim), dtype=torch.float32, device=device)
        return PagedCache(fmt, num_phys_pages, num_kv_heads, head_dim, k, v, p, meta, n16)

    def struct(self) -> CacheStruct:
        return CacheStruct(self.format, self.num_phys_pages, PAGE_SIZE, self.num_kv_heads, self.head_dim,
                           _ptr(self.k_pages), _ptr(self.v_pages), _ptr(self.kv_params), _ptr(self.page_meta),
                           self.num_fp16_pages)


@dataclass
class Seqs:
    """Sequence lengths [B] and block table [B][max_pages] (int32, device)."""

    seq_lens: torch.Tensor
    block_table: torch.Tensor

    @property
    def batch(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def struct(self) -> SeqsStruct:
        if self.seq_lens.dtype != torch.int32 or self.block_table.dtype != torch.int32:
            raise TypeError("seq_lens and block_table must be int32")
        return SeqsStruct(self.batch, self.max_pages, _ptr(self.seq_lens), _ptr(self.block_table))


def _half_bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.float16:
        return t.view(torch.int16)
    if t.dtype == torch.int16:
        return t
    raise TypeError("expected fp16 data (torch.float16 or its int16 bits)")


# ------------------------------------------------------------ entry points
def kvq_append_quant(cache: PagedCache, seqs: Seqs, start_pos, new_off, max_new: int, k_new, v_new,
                     stream=None) -> None:
    k = _half_bits(k_new) if k_new is not None else None
    v = _half_bits(v_new) if v_new is not None else None
    _check("kvq_append_quant", lib().kvq_append_quant(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(start_pos), _ptr(new_off),
        int(max_new), _ptr(k), _ptr(v), _stream(stream)))


def kvq_append_decode(cache: PagedCache, seqs: Seqs, start_pos, new_off, max_new: int, k_new, v_new,
                      stream=None) -> None:
    k = _half_bits(k_new) if k_new is not None else None
    v = _half_bits(v_new) if v_new is not None else None
    _check("kvq_append_decode", lib().kvq_append_decode(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(start_pos), _ptr(new_off),
        int(max_new), _ptr(k), _ptr(v), _stream(stream)))


def kvq_append_decode_scores(cache: PagedCache, seqs: Seqs, start_pos, new_off, max_new: int, k_new, v_new, q,
                             scores, stream=None) -> None:
    k = _half_bits(k_new) if k_new is not None else None
    v = _half_bits(v_new) if v_new is not None else None
    qb = _half_bits(q)
    _check("kvq_append_decode_scores", lib().kvq_append_decode_scores(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(start_pos), _ptr(new_off),
        int(max_new), _ptr(k), _ptr(v), _ptr(qb), int(qb.shape[1]), _ptr(scores), _stream(stream)))


def kvq_build_page_meta(cache: PagedCache, seqs: Seqs, page_begin=None, max_span: int = 0, stream=None) -> None:
    _check("kvq_build_page_meta", lib().kvq_build_page_meta(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(page_begin), int(max_span),
        _stream(stream)))


def kvq_demote_pages(cache: PagedCache, seqs: Seqs, seq, page, dst, stream=None) -> None:
    """Move logical page page[i] of sequence seq[i] from the FP16 pool to
    INT8-pool page dst[i] (int32 device tensors of one length); rewrites
    seqs.block_table in place."""
    n = int(seq.numel())
    if int(page.numel()) != n or int(dst.numel()) != n:
        raise ValueError("seq, page and dst must have one length")
    _check("kvq_demote_pages", lib().kvq_demote_pages(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), n, _ptr(seq), _ptr(page), _ptr(dst),
        _stream(stream)))


def kvq_page_scores(cache: PagedCache, seqs: Seqs, q, scores, stream=None) -> None:
    qb = _half_bits(q)
    _check("kvq_page_scores", lib().kvq_page_scores(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(qb), int(qb.shape[1]), _ptr(scores),
        _stream(stream)))


def kvq_build_coarse_meta(cache: PagedCache, seqs: Seqs, group_pages: int, super_begin, coarse_meta, coarse_lens,
                          coarse_table, stream=None, max_span: int = 0) -> None:
    _check("kvq_build_coarse_meta", lib().kvq_build_coarse_meta(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), int(group_pages), _ptr(super_begin),
        int(max_span), _ptr(coarse_meta), _ptr(coarse_lens), _ptr(coarse_table), _stream(stream)))


def kvq_page_scores_masked(cache: PagedCache, seqs: Seqs, q, group_pages: int, sel_super, sel_super_count, scores,
                           stream=None) -> None:
    qb = _half_bits(q)
    _check("kvq_page_scores_masked", lib().kvq_page_scores_masked(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(qb), int(qb.shape[1]), int(group_pages),
        _ptr(sel_super), _ptr(sel_super_count), int(sel_super.shape[-1]), _ptr(scores), _stream(stream)))


def kvq_topk_pages(scores, seqs: Seqs, num_kv_heads: int, ratio_num: int, ratio_den: int, k_fixed: int,
                   sel_pages, sel_count, stream=None) -> None:
    _check("kvq_topk_pages", lib().kvq_topk_pages(
        _ptr(scores), ctypes.byref(seqs.struct()), int(num_kv_heads), int(ratio_num), int(ratio_den),
        int(k_fixed), int(sel_pages.shape[-1]), _ptr(sel_pages), _ptr(sel_count), _stream(stream)))


def kvq_attn_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, max_pages: int, k_cap: int,
                             pages_per_split: int) -> int:
    return int(lib().kvq_attn_workspace_bytes(batch, num_q_heads, head_dim, max_pages, k_cap, pages_per_split))


def kvq_default_pages_per_split(batch: int, num_kv_heads: int, max_pages: int, k_cap: int) -> int:
    return int(lib().kvq_default_pages_per_split(batch, num_kv_heads, max_pages, k_cap))


def kvq_sparse_decode_attn(cache: PagedCache, seqs: Seqs, q, sel_pages, sel_count, out, workspace,
                           sm_scale: float, pages_per_split: int = 0, stream=None) -> None:
    qb = _half_bits(q)
    k_cap = int(sel_pages.shape[-1]) if sel_pages is not None else 0
    _check("kvq_sparse_decode_attn", lib().kvq_sparse_decode_attn(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(qb), int(qb.shape[1]),
        _ptr(sel_pages), _ptr(sel_count), k_cap, float(sm_scale), int(pages_per_split), _ptr(out),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def kvq_select_decode_attn(cache: PagedCache, seqs: Seqs, q, scores, ratio_num: int, ratio_den: int, k_fixed: int,
                           k_cap: int, out, workspace, sm_scale: float, pages_per_split: int = 0, stream=None, *,
                           sel_pages=None, sel_count=None) -> None:
    qb = _half_bits(q)
    _check("kvq_select_decode_attn", lib().kvq_select_decode_attn(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(qb), int(qb.shape[1]), _ptr(scores),
        int(ratio_num), int(ratio_den), int(k_fixed), int(k_cap), _ptr(sel_pages), _ptr(sel_count),
        float(sm_scale), int(pages_per_split), _ptr(out), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _stream(stream)))


def kvq_select_decode_attn_noalloc(cache: PagedCache, seqs: Seqs, q, scores, ratio_num: int, ratio_den: int,
                                   k_fixed: int, k_cap: int, out, sm_scale: float, pages_per_split: int = 0,
                                   stream=None, *, sel_pages=None, sel_count=None) -> None:
    """kvq_select_decode_attn with the library's own scratch in place of a
    workspace (no allocation; calls on one GPU must not overlap)."""
    qb = _half_bits(q)
    _check("kvq_select_decode_attn_noalloc", lib().kvq_select_decode_attn_noalloc(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(qb), int(qb.shape[1]), _ptr(scores),
        int(ratio_num), int(ratio_den), int(k_fixed), int(k_cap), _ptr(sel_pages), _ptr(sel_count),
        float(sm_scale), int(pages_per_split), _ptr(out), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20  # KVQ_NOALLOC_SCRATCH_BYTES
STEP_MAX_SEQS = 512               # KVQ_STEP_MAX_SEQS
STEP_MAX_SPLIT_PAGES = 512        # KVQ_STEP_MAX_SPLIT_PAGES


def kvq_step_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_pages: int,
                             k_cap: int, pages_per_split: int) -> int:
    return int(lib().kvq_step_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_pages, k_cap,
                                              pages_per_split))


def kvq_step_counter_bytes(batch: int, num_kv_heads: int) -> int:
    return int(lib().kvq_step_counter_bytes(batch, num_kv_heads))


def kvq_decode_step(cache: PagedCache, seqs: Seqs, start_pos, new_off, max_new: int, k_new, v_new, q, scores,
                    ratio_num: int, ratio_den: int, k_fixed: int, k_cap: int, out, workspace, sm_scale: float,
                    pages_per_split: int = 0, stream=None, *, sel_pages=None, sel_count=None) -> None:
    """The whole decode step in one launch (append, metadata, scores, top-K,
    attention, combine).  The workspace's leading counter bytes must be zero
    before its first use (allocate it zeroed)."""
    k = _half_bits(k_new) if k_new is not None else None
    v = _half_bits(v_new) if v_new is not None else None
    qb = _half_bits(q)
    _check("kvq_decode_step", lib().kvq_decode_step(
        ctypes.byref(cache.struct()), ctypes.byref(seqs.struct()), _ptr(start_pos), _ptr(new_off), int(max_new),
        _ptr(k), _ptr(v), _ptr(qb), int(qb.shape[1]), _ptr(scores), int(ratio_num), int(ratio_den), int(k_fixed),
        int(k_cap), _ptr(sel_pages), _ptr(sel_count), float(sm_scale), int(pages_per_split), _ptr(out),
        _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream)))


def kvq_read_probe(buf, sink, stream=None) -> None:
    """Measurement helper: one plain streaming read of `buf` (a device tensor)."""
    _check("kvq_read_probe", lib().kvq_read_probe(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(sink),
                                                  _stream(stream)))


def num_selected(P: int, ratio_num: int, ratio_den: int, k_fixed: int) -> int:
    """K for P pages under the library's selection rule (kvq_num_selected);
    sizes sel_pages."""
    return int(lib().kvq_num_selected(int(P), int(ratio_num), int(ratio_den), int(k_fixed)))
