"""Caller-side plumbing around libkvq: device buffers for one decode step and
a cache builder.  Every computation is a libkvq call; this module only
allocates torch tensors, uploads caller data and sequences the calls.

A decode step, as the TinyServe page (lpnh.cn, section 3.1) orders it:
  append the new token (and re-quantize its open group) -> refresh the
  metadata of the pages that changed -> score every page -> top-K ->
  attention over the selected pages (split-K + combine).
DecodeStep.run_with_append does it in three launches: append + metadata +
scores (kvq_append_decode_scores), then top-K inside the attention kernel
(kvq_select_decode_attn), then the split combine; or, with fused_step, in one
persistent launch (kvq_decode_step).
"""
from __future__ import annotations

from typing import Callable

import numpy as np
import torch

from . import (KVQ_INT4_GROUP64, KVQ_INT4_TOKEN, KVQ_INT8_GROUP64, PAGE_SIZE, SELECT_MAX_PAGES, STEP_MAX_SEQS,
               STEP_MAX_SPLIT_PAGES, PagedCache, Seqs,
               kvq_append_decode, kvq_append_decode_scores, kvq_append_quant, kvq_attn_workspace_bytes,
               kvq_build_coarse_meta, kvq_build_page_meta, kvq_decode_step, kvq_default_pages_per_split,
               kvq_page_scores, kvq_page_scores_masked,
               kvq_select_decode_attn, kvq_sparse_decode_attn, kvq_step_workspace_bytes, kvq_topk_pages,
               num_selected)

FUSED_SELECT_MAX_BLOCKS = 512  # one round of attention blocks on 256 CUs (2 per CU)

KVSource = Callable[[int], "tuple[np.ndarray, np.ndarray]"]  # b -> (K [L][H][d], V [L][H][d]) fp16


def _dev_i32(x, device) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(x, np.int32)).to(device)


def append_rows(cache: PagedCache, seqs: Seqs, rows: dict[int, tuple[int, np.ndarray, np.ndarray]],
                device="cuda") -> None:
    """Append rows[b] = (start_pos, K rows, V rows) for the listed sequences
    with one kvq_append_quant call; other sequences receive nothing."""
    B = seqs.batch
    start = np.zeros(B, np.int32)
    cnt = np.zeros(B, np.int64)
    ks, vs = [], []
    for b in range(B):
        if b in rows:
            s, k, v = rows[b]
            start[b] = s
            cnt[b] = k.shape[0]
            ks.append(k)
            vs.append(v)
    off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    if not ks or off[-1] == 0:
        return
    k_new = torch.from_numpy(np.ascontiguousarray(np.concatenate(ks)).view(np.int16)).to(device)
    v_new = torch.from_numpy(np.ascontiguousarray(np.concatenate(vs)).view(np.int16)).to(device)
    kvq_append_quant(cache, seqs, _dev_i32(start, device), _dev_i32(off, device), int(cnt.max()), k_new, v_new)


def build_cache(fmt: int, num_phys_pages: int, num_kv_heads: int, head_dim: int, block_table: np.ndarray,
                seq_lens: np.ndarray, source: KVSource, prefill_lens: np.ndarray | None = None,
                device="cuda", rows_per_call: int = 1 << 20, num_fp16_pages: int = 0) -> tuple[PagedCache, Seqs]:
    """Allocate a cache and prefill sequence b with its first prefill_lens[b]
    tokens (default: all) from source(b), then build every page's metadata.
    Uploads are batched to about rows_per_call tokens per append call.
    num_fp16_pages: the FP16 pool of a mixed-precision cache."""
    cache = PagedCache.empty(fmt, num_phys_pages, num_kv_heads, head_dim, device, num_fp16_pages)
    seqs = Seqs(_dev_i32(seq_lens, device), _dev_i32(block_table, device))
    pre = np.asarray(seq_lens if prefill_lens is None else prefill_lens, np.int64)
    batch: dict[int, tuple[int, np.ndarray, np.ndarray]] = {}
    rows = 0
    for b in range(len(pre)):
        if pre[b] == 0:
            continue
        k, v = source(b)
        batch[b] = (0, k[: pre[b]], v[: pre[b]])
        rows += int(pre[b])
        if rows >= rows_per_call:
            append_rows(cache, seqs, batch, device)
            torch.cuda.current_stream().synchronize()
            batch, rows = {}, 0
    append_rows(cache, seqs, batch, device)
    # metadata over the prefilled tokens, then the real lengths are installed
    pre_seqs = Seqs(_dev_i32(pre, device), seqs.block_table)
    kvq_build_page_meta(cache, pre_seqs)
    torch.cuda.current_stream().synchronize()
    return cache, seqs


class DecodeAppend:
    """Device buffers to append each sequence's newest token at position
    L_b - 1 (per-group formats: re-supply its open 64-token group) and refresh the
    metadata of the pages it touched."""

    def __init__(self, cache: PagedCache, seqs: Seqs, seq_lens: np.ndarray, source_rows: KVSource,
                 device="cuda"):
        self.cache, self.seqs = cache, seqs
        lens = np.asarray(seq_lens, np.int64)
        last = lens - 1
        if cache.format in (KVQ_INT8_GROUP64, KVQ_INT4_GROUP64):
            start = (last // 64) * 64
        else:
            start = last
        ks, vs = [], []
        for b in range(len(lens)):
            k, v = source_rows(b)
            ks.append(k[start[b]: lens[b]])
            vs.append(v[start[b]: lens[b]])
        cnt = lens - start
        self.max_new = int(cnt.max())
        self.start = _dev_i32(start, device)
        self.off = _dev_i32(np.concatenate([[0], np.cumsum(cnt)]), device)
        self.k_new = torch.from_numpy(np.ascontiguousarray(np.concatenate(ks)).view(np.int16)).to(device)
        self.v_new = torch.from_numpy(np.ascontiguousarray(np.concatenate(vs)).view(np.int16)).to(device)
        self.page_begin = _dev_i32(start // PAGE_SIZE, device)
        self.span = int(((lens - 1) // PAGE_SIZE - start // PAGE_SIZE).max()) + 1

    def run(self, stream=None) -> None:
        kvq_append_decode(self.cache, self.seqs, self.start, self.off, self.max_new, self.k_new, self.v_new, stream)

    def run_separate(self, stream=None) -> None:
        """The same step as two calls: kvq_append_quant, then kvq_build_page_meta."""
        kvq_append_quant(self.cache, self.seqs, self.start, self.off, self.max_new, self.k_new, self.v_new, stream)
        kvq_build_page_meta(self.cache, self.seqs, self.page_begin, self.span, stream)


class DecodeStep:
    """Device buffers for score -> top-K -> sparse attention of one step.
    dense=True skips scoring and selection and attends to every page.
    fused_select=True (the default) selects inside the attention kernel
    (kvq_select_decode_attn) when rows have at most SELECT_MAX_PAGES pages and
    the attention grid fits in one round of resident blocks (about 2 per CU,
    FUSED_SELECT_MAX_BLOCKS): every attention block repeats its row's
    selection, which pays off only while all blocks run at once.  Otherwise,
    or with False, it runs kvq_topk_pages, then kvq_sparse_decode_attn.
    Either way sel_pages / sel_count end up holding the selection."""

    def __init__(self, cache: PagedCache, seqs: Seqs, num_q_heads: int, ratio_num: int, ratio_den: int,
                 k_fixed: int, dense: bool = False, pages_per_split: int = 0, device="cuda",
                 fused_select: bool = True, fused_step: bool = False):
        self.cache, self.seqs, self.Hq = cache, seqs, num_q_heads
        self.ratio = (ratio_num, ratio_den, k_fixed)
        self.dense = dense
        B, H, d, maxp = seqs.batch, cache.num_kv_heads, cache.head_dim, seqs.max_pages
        self.k_cap = 0 if dense else num_selected(maxp, ratio_num, ratio_den, k_fixed)
        self.pps = pages_per_split or kvq_default_pages_per_split(B, H, maxp, self.k_cap)
        blocks = B * H * -(-max(self.k_cap, 1) // self.pps)
        self.fused_select = (fused_select and not dense and maxp <= SELECT_MAX_PAGES
                             and blocks <= FUSED_SELECT_MAX_BLOCKS)
        self.scores = torch.empty((B, H, maxp), dtype=torch.float32, device=device)
        self.sel_pages = torch.empty((B, H, max(self.k_cap, 1)), dtype=torch.int32, device=device)
        self.sel_count = torch.empty((B, H), dtype=torch.int32, device=device)
        self.out = torch.empty((B, num_q_heads, d), dtype=torch.float32, device=device)
        nbytes = kvq_attn_workspace_bytes(B, num_q_heads, d, maxp, self.k_cap, self.pps)
        self.workspace = torch.zeros((nbytes + 255) // 4, dtype=torch.float32, device=device)
        self.sm_scale = 1.0 / float(np.sqrt(d))
        # the one-launch step (kvq_decode_step): its workspace starts zeroed
        # (counters) and the step keeps it so
        # (fp16 and INT8 storage only)
        self.fused_step = (fused_step and not dense and maxp <= SELECT_MAX_PAGES and B <= STEP_MAX_SEQS
                           and self.pps <= STEP_MAX_SPLIT_PAGES and cache.format < KVQ_INT4_TOKEN)
        self.step_workspace = None
        if self.fused_step:
            sb = kvq_step_workspace_bytes(B, num_q_heads, H, d, maxp, self.k_cap, self.pps)
            self.step_workspace = torch.zeros((sb + 255) // 4, dtype=torch.float32, device=device)

    def select(self, q, stream=None) -> None:
        kvq_page_scores(self.cache, self.seqs, q, self.scores, stream)
        rn, rd, kf = self.ratio
        kvq_topk_pages(self.scores, self.seqs, self.cache.num_kv_heads, rn, rd, kf, self.sel_pages,
                       self.sel_count, stream)

    def attend(self, q, sel_pages=None, sel_count=None, stream=None) -> torch.Tensor:
        kvq_sparse_decode_attn(self.cache, self.seqs, q, sel_pages, sel_count, self.out, self.workspace,
                               self.sm_scale, self.pps, stream)
        return self.out

    def select_attend(self, q, stream=None) -> torch.Tensor:
        """Top-K of self.scores and attention in one call (kvq_select_decode_attn)."""
        rn, rd, kf = self.ratio
        kvq_select_decode_attn(self.cache, self.seqs, q, self.scores, rn, rd, kf, self.k_cap, self.out,
                               self.workspace, self.sm_scale, self.pps, stream, sel_pages=self.sel_pages,
                               sel_count=self.sel_count)
        return self.out

    def run(self, q, stream=None) -> torch.Tensor:
        if self.dense:
            return self.attend(q, None, None, stream)
        if self.fused_select:
            kvq_page_scores(self.cache, self.seqs, q, self.scores, stream)
            return self.select_attend(q, stream)
        self.select(q, stream)
        return self.attend(q, self.sel_pages, self.sel_count, stream)

    def run_with_append(self, app: "DecodeAppend", q, stream=None) -> torch.Tensor:
        """The whole decode step: append the newest rows (app) and score in
        one kernel, then top-K and attention (fused_step: all of it in one
        launch, kvq_decode_step)."""
        if self.dense:
            app.run(stream)
            return self.attend(q, None, None, stream)
        if self.fused_step:
            rn, rd, kf = self.ratio
            kvq_decode_step(self.cache, self.seqs, app.start, app.off, app.max_new, app.k_new, app.v_new, q,
                            self.scores, rn, rd, kf, self.k_cap, self.out, self.step_workspace, self.sm_scale,
                            self.pps, stream, sel_pages=self.sel_pages, sel_count=self.sel_count)
            return self.out
        kvq_append_decode_scores(self.cache, self.seqs, app.start, app.off, app.max_new, app.k_new, app.v_new, q,
                                 self.scores, stream)
        if self.fused_select:
            return self.select_attend(q, stream)
        rn, rd, kf = self.ratio
        kvq_topk_pages(self.scores, self.seqs, self.cache.num_kv_heads, rn, rd, kf, self.sel_pages,
                       self.sel_count, stream)
        return self.attend(q, self.sel_pages, self.sel_count, stream)


class HierStep:
    """Coarse-then-fine selection (TinyServe page, section 6) in front of the
    attention of a DecodeStep: super-pages of `group` consecutive pages are
    screened by their boxes (kvq_build_coarse_meta, kvq_page_scores on the
    coarse view, kvq_topk_pages keeping `keep` of them per row), then only
    their pages are scored (kvq_page_scores_masked) and the step's top-K and
    attention run on those scores."""

    def __init__(self, step: DecodeStep, group: int, keep: int, device="cuda"):
        self.step, self.group, self.keep = step, group, keep
        cache, seqs = step.cache, step.seqs
        B, H, d, maxp = seqs.batch, cache.num_kv_heads, cache.head_dim, seqs.max_pages
        self.pc_max = -(-maxp // group)
        self.coarse = torch.full((B * self.pc_max, H, 2, d), float("nan"), dtype=torch.float32, device=device)
        self.coarse_lens = torch.zeros(B, dtype=torch.int32, device=device)
        self.coarse_table = torch.zeros((B, self.pc_max), dtype=torch.int32, device=device)
        self.coarse_cache = PagedCache(cache.format, B * self.pc_max, H, d, cache.k_pages, cache.v_pages,
                                       cache.kv_params, self.coarse)
        self.coarse_seqs = Seqs(self.coarse_lens, self.coarse_table)
        self.kc = min(keep, self.pc_max)
        self.coarse_scores = torch.empty((B, H, self.pc_max), dtype=torch.float32, device=device)
        self.sel_super = torch.empty((B, H, self.kc), dtype=torch.int32, device=device)
        self.sel_super_count = torch.empty((B, H), dtype=torch.int32, device=device)

    def build(self, super_begin=None, stream=None, max_span: int = 0) -> None:
        """Boxes of every super-page, or of those from super_begin[b] on (at
        most max_span of them per sequence when max_span > 0)."""
        kvq_build_coarse_meta(self.step.cache, self.step.seqs, self.group, super_begin, self.coarse,
                              self.coarse_lens, self.coarse_table, stream, max_span)

    def screen(self, q, stream=None) -> None:
        """Coarse scores, the kept super-pages, and the masked fine scores."""
        st = self.step
        kvq_page_scores(self.coarse_cache, self.coarse_seqs, q, self.coarse_scores, stream)
        kvq_topk_pages(self.coarse_scores, self.coarse_seqs, st.cache.num_kv_heads, 0, 1, self.kc, self.sel_super,
                       self.sel_super_count, stream)
        kvq_page_scores_masked(st.cache, st.seqs, q, self.group, self.sel_super, self.sel_super_count, st.scores,
                               stream)

    def attend(self, q, stream=None) -> torch.Tensor:
        st = self.step
        if st.fused_select:
            return st.select_attend(q, stream)
        rn, rd, kf = st.ratio
        kvq_topk_pages(st.scores, st.seqs, st.cache.num_kv_heads, rn, rd, kf, st.sel_pages, st.sel_count, stream)
        return st.attend(q, st.sel_pages, st.sel_count, stream)

    def run(self, q, stream=None) -> torch.Tensor:
        self.screen(q, stream)
        return self.attend(q, stream)

    def run_with_append(self, app: "DecodeAppend", super_begin, q, stream=None) -> torch.Tensor:
        """Append the newest rows (and their pages' metadata), refresh the boxes
        of the super-pages they touch (super_begin[b]: the first one), then
        screen, select and attend."""
        app.run(stream)
        # the app.span pages the rows touch lie in at most span // group + 2 super-pages
        self.build(super_begin, stream, app.span // self.group + 2)
        return self.run(q, stream)
