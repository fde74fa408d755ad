"""Seeded synthetic inputs for the paged, quantized, query-aware sparse decode step.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no quantization, no page metadata, no scores, no top-K,
no attention), so the CPU oracle and the HIP path can both consume it without
sharing any code that computes a result.

Every array is a pure function of (config seed, stream id, index): each
sequence's keys and values come from their own numpy PCG64 stream, so a test
can regenerate one sequence of a large workload without drawing the others.

Workload shapes follow the decode workloads named on the pages:
  * GPT2-345M-shaped layer, 16K context (lpnh.cn "TinyServe" page, section 3.2
    latency table);
  * Llama-2-7B-shaped layer, 32 heads x head_dim 128 (intelliparadigm.com
    KV-cache page, section 2.1 memory example; pzsr.cn layout page, section 3);
  * per-prompt outlier key channels 10-20x larger than the rest (pzsr.cn page,
    section 2);
  * 16-token pages (pzsr.cn page, section 2 layout C; TinyServe page, section
    5.1 config), INT8 per-token (pzsr.cn page, section 2) or per-64-token-group
    (uyd888.cn page, chapter 1) storage, 4-bit codes (intelliparadigm.com
    page, section 3.2), or mixed precision (TinyServe page, section 6: pages
    of high importance FP16, the rest INT8; here the first page and the most
    recent hot_recent pages of each sequence are the FP16 ones).
The pages evaluate on trained models and on PG19; no weights or dataset exist
here, so N(0, 1) activations with the stated outlier structure stand in.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

PAGE = 16

FMT_FP16 = 0
FMT_INT8_TOKEN = 1
FMT_INT8_GROUP64 = 2
FMT_INT4_TOKEN = 3
FMT_INT4_GROUP64 = 4
FMT_MIXED = 5
FORMAT_NAMES = {FMT_FP16: "fp16", FMT_INT8_TOKEN: "int8_token", FMT_INT8_GROUP64: "int8_group64",
                FMT_INT4_TOKEN: "int4_token", FMT_INT4_GROUP64: "int4_group64", FMT_MIXED: "mixed_fp16_int8"}

# stream ids: one numpy stream per (stream, index)
_S_LENS, _S_Q, _S_K, _S_V, _S_OUT, _S_TABLE = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-step workload.  Sizes only; arrays come from the methods."""

    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    fmt: int
    # context length per sequence: fixed, or drawn uniformly in [len_lo, len_hi]
    seq_len: int = 0
    len_lo: int = 0
    len_hi: int = 0
    # selection: k_fixed > 0 selects exactly that many pages (capped at the
    # sequence's page count); otherwise the ratio ratio_num / ratio_den applies
    ratio_num: int = 3
    ratio_den: int = 10
    k_fixed: int = 0
    # block table: "identity", "perm" (one global pool, shuffled) or
    # "perm_pool" (a pool of pool_pages shuffled pages, handed out in order)
    table: str = "perm"
    # outlier key channels per (sequence, KV head)
    outlier_channels: int = 0
    outlier_lo: float = 1.0
    outlier_hi: float = 1.0
    # extra physical pages beyond the ones the block table uses (in the INT8
    # pool of a mixed-precision cache)
    spare_pages: int = 0
    # mixed precision: FP16 pages per sequence besides its first page (its
    # last hot_recent pages)
    hot_recent: int = 64

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    # ----------------------------------------------------------------- sizes
    def _rng(self, stream: int, index: int = 0) -> np.random.Generator:
        return np.random.default_rng(np.random.SeedSequence([self.seed, stream, index]))

    def seq_lens(self) -> np.ndarray:
        """int32 [B]: tokens in each sequence's context, the new token included."""
        if self.seq_len > 0:
            return np.full(self.batch, self.seq_len, dtype=np.int32)
        rng = self._rng(_S_LENS)
        return rng.integers(self.len_lo, self.len_hi, size=self.batch, endpoint=True).astype(np.int32)

    def pages_per_seq(self) -> np.ndarray:
        lens = self.seq_lens().astype(np.int64)
        return ((lens + PAGE - 1) // PAGE).astype(np.int32)

    def max_pages(self) -> int:
        return int(self.pages_per_seq().max())

    def hot_pages(self, b: int) -> np.ndarray:
        """bool [P_b]: the pages of sequence b kept in FP16 by a mixed-precision
        cache (its first page and its last hot_recent pages)."""
        P = int(self.pages_per_seq()[b])
        hot = np.zeros(P, dtype=bool)
        if self.fmt == FMT_MIXED and P:
            hot[0] = True
            hot[max(P - self.hot_recent, 0):] = True
        return hot

    def fp16_pool_pages(self) -> int:
        """Physical pages 0 .. n16-1 form the FP16 pool of a mixed-precision
        cache (0 for every other format)."""
        if self.fmt != FMT_MIXED:
            return 0
        return int(sum(int(self.hot_pages(b).sum()) for b in range(self.batch)))

    def block_table(self) -> tuple[np.ndarray, int]:
        """(int32 [B][max_pages], number of physical pages).

        Unused entries hold -1.  Logical page j of sequence b lives in physical
        page table[b, j]; the pages of all sequences are disjoint.
        """
        pages = self.pages_per_seq()
        total = int(pages.sum())
        if self.fmt == FMT_MIXED:   # hot pages from the FP16 pool, the others from the INT8 pool
            n16 = self.fp16_pool_pages()
            ids16, ids8 = np.arange(n16, dtype=np.int32), np.arange(n16, total, dtype=np.int32)
            if self.table == "perm":
                rng = self._rng(_S_TABLE)
                ids16, ids8 = rng.permutation(ids16), rng.permutation(ids8)
            table = np.full((self.batch, self.max_pages()), -1, dtype=np.int32)
            o16 = o8 = 0
            for b, p in enumerate(pages):
                hot = self.hot_pages(b)
                for j in range(int(p)):
                    if hot[j]:
                        table[b, j], o16 = ids16[o16], o16 + 1
                    else:
                        table[b, j], o8 = ids8[o8], o8 + 1
            return table, total + self.spare_pages
        if self.table == "identity":
            phys = np.arange(total, dtype=np.int32)
        elif self.table == "perm":
            phys = self._rng(_S_TABLE).permutation(total).astype(np.int32)
        else:
            raise ValueError(self.table)
        table = np.full((self.batch, self.max_pages()), -1, dtype=np.int32)
        off = 0
        for b, p in enumerate(pages):
            table[b, :p] = phys[off:off + p]
            off += int(p)
        return table, total + self.spare_pages

    # ------------------------------------------------------------ activations
    def query(self) -> np.ndarray:
        """fp16 [B][H_q][d], N(0, 1)."""
        rng = self._rng(_S_Q)
        x = rng.standard_normal((self.batch, self.num_q_heads, self.head_dim), dtype=np.float32)
        return x.astype(np.float16)

    def outliers(self, b: int) -> tuple[np.ndarray, np.ndarray]:
        """(int64 [H_kv][n] channel ids, float32 [H_kv][n] factors) of sequence b."""
        n = self.outlier_channels
        rng = self._rng(_S_OUT, b)
        chans = np.zeros((self.num_kv_heads, n), dtype=np.int64)
        facs = np.ones((self.num_kv_heads, n), dtype=np.float32)
        for h in range(self.num_kv_heads):
            if n:
                chans[h] = np.sort(rng.choice(self.head_dim, size=n, replace=False))
                if self.outlier_lo == self.outlier_hi:
                    facs[h] = np.float32(self.outlier_lo)
                else:
                    facs[h] = rng.uniform(self.outlier_lo, self.outlier_hi, size=n).astype(np.float32)
        return chans, facs

    def keys(self, b: int) -> np.ndarray:
        """fp16 [L_b][H_kv][d]: N(0, 1) with the sequence's outlier channels scaled."""
        L = int(self.seq_lens()[b])
        rng = self._rng(_S_K, b)
        x = rng.standard_normal((L, self.num_kv_heads, self.head_dim), dtype=np.float32)
        chans, facs = self.outliers(b)
        for h in range(self.num_kv_heads):
            for c, f in zip(chans[h], facs[h]):
                x[:, h, c] *= f
        return x.astype(np.float16)

    def values(self, b: int) -> np.ndarray:
        """fp16 [L_b][H_kv][d], N(0, 1)."""
        L = int(self.seq_lens()[b])
        rng = self._rng(_S_V, b)
        return rng.standard_normal((L, self.num_kv_heads, self.head_dim), dtype=np.float32).astype(np.float16)

    # ------------------------------------------------------------ selection
    def selection_args(self) -> tuple[int, int, int]:
        """(ratio_num, ratio_den, k_fixed) handed unchanged to both sides."""
        return self.ratio_num, self.ratio_den, self.k_fixed

    def is_dense(self) -> bool:
        return self.k_fixed == 0 and self.ratio_num >= self.ratio_den

    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def config(n: int) -> Workload:
    """The five decode workloads, numbered 1..5; seed = 1000 + n."""
    if n == 1:
        # tiny single step: identity table, 16 of 64 pages (K = 64 is the dense check)
        return Workload("tiny_b1_h4_d64_L1024_fp16", 1001, 1, 4, 4, 64, FMT_FP16,
                        seq_len=1024, k_fixed=16, table="identity")
    if n == 2:
        # GPT2-345M-shaped layer, 16K context, 4 of 64 key channels x15
        return Workload("gpt2_345m_b1_h16_d64_L16384_fp16", 1002, 1, 16, 16, 64, FMT_FP16,
                        seq_len=16384, outlier_channels=4, outlier_lo=15.0, outlier_hi=15.0)
    if n == 3:
        # Llama-2-7B-shaped layer, dense paged decode over a shuffled 512-page pool
        return Workload("llama2_7b_b4_h32_d128_L2048_fp16_dense", 1003, 4, 32, 32, 128, FMT_FP16,
                        seq_len=2048, ratio_num=1, ratio_den=1)
    if n == 4:
        # Llama-2-7B-shaped layer, 32K context, INT8 per token, 8 of 128 channels x U[10, 20]
        return Workload("llama2_7b_b1_h32_d128_L32768_int8tok", 1004, 1, 32, 32, 128, FMT_INT8_TOKEN,
                        seq_len=32768, outlier_channels=8, outlier_lo=10.0, outlier_hi=20.0)
    if n == 5:
        # GQA ragged batch: 64 sequences of U[1K, 32K] tokens, 32 q heads / 8 KV heads, INT8 per 64-token group
        return Workload("gqa_b64_h32kv8_d128_L1k_32k_int8grp", 1005, 64, 32, 8, 128, FMT_INT8_GROUP64,
                        len_lo=1024, len_hi=32768, outlier_channels=8, outlier_lo=10.0, outlier_hi=20.0)
    raise ValueError(f"no config {n}")


def small(n: int) -> Workload:
    """A cut-down version of config n: same storage, grouping, table and outlier
    structure, at sizes the oracle finishes in well under a second.  Lengths
    are not multiples of 16 or 64, so every stage sees a ragged tail."""
    w = config(n)
    if n == 1:
        return w
    if n == 2:
        return w.with_(name="small_gpt2", num_q_heads=4, num_kv_heads=4, seq_len=1000)
    if n == 3:
        return w.with_(name="small_llama_dense", batch=3, num_q_heads=4, num_kv_heads=4, seq_len=999, spare_pages=5)
    if n == 4:
        return w.with_(name="small_llama_int8tok", num_q_heads=4, num_kv_heads=4, seq_len=2021)
    if n == 5:
        return w.with_(name="small_gqa_int8grp", batch=5, num_q_heads=8, num_kv_heads=2, len_lo=1, len_hi=700)
    raise ValueError(n)
