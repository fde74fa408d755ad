"""CPU oracle for the paged, quantized, query-aware sparse decode step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its Python binding) never does.  The arithmetic lives in plain C
(``kvq_oracle.c``, fp64 accumulation, fp32 quantization without contraction);
this module only allocates numpy arrays and calls it through ctypes.

Every function follows the pages it cites in ``kvq_oracle.c``:
  append      -- paged store and INT8 quantization (pzsr.cn layout page,
                 sections 2-3; uyd888.cn Gemini page, chapter 1)
  page_meta   -- phi(K_j) = per-channel (min, max) in fp32 (TinyServe page,
                 sections 2.1 and 5.2)
  page_scores -- r = sum_i (q_i >= 0 ? q_i M_i : q_i m_i) (TinyServe page,
                 section 2.1), GQA group score = max over the group's heads
  topk        -- top-K pages per (sequence, KV head) (TinyServe page,
                 sections 3.1 and 5.1)
  attention   -- softmax(q k^T / sqrt(d)) v over the selected pages
                 (intelliparadigm.com page, section 2.1; TinyServe page,
                 section 3.1)
  attention_mass -- the share of dense attention weight on the selected
                 pages (selection quality; TinyServe page, section 1 claims
                 the value sits in a minority of the KV cache)
  coarse_meta, mask_scores, hier_select -- coarse-then-fine selection over
                 super-pages of consecutive pages (TinyServe page, section 6)
  demote      -- a mixed-precision cache (TinyServe page, section 6: pages of
                 high importance in FP16, the rest INT8) moves a page from
                 its FP16 pool to its INT8 pool
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")
PAGE = 16

_CFLAGS = ["-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libkvq_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.kvqo_append.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P]
        L.kvqo_append.restype = I
        L.kvqo_page_meta.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P]
        L.kvqo_page_meta.restype = None
        L.kvqo_page_scores.argtypes = [I, I, I, I, I, P, P, P, P, P]
        L.kvqo_page_scores.restype = None
        L.kvqo_num_selected.argtypes = [I, I, I, I]
        L.kvqo_num_selected.restype = I
        L.kvqo_topk.argtypes = [I, I, I, P, P, I, I, I, I, P, P]
        L.kvqo_topk.restype = I
        L.kvqo_attention.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, ctypes.c_double, P]
        L.kvqo_attention.restype = None
        L.kvqo_attention_mass.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, I, ctypes.c_double, P]
        L.kvqo_attention_mass.restype = None
        L.kvqo_decode_step.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, I, I, I, I,
                                       ctypes.c_double, P, P, P, P, I]
        L.kvqo_demote.argtypes = [I, I, I, I, I, I, P, P, I, P, P, P, P, P, P, P]
        L.kvqo_demote.restype = I
        L.kvqo_decode_step.restype = I
        L.kvqo_coarse_meta.argtypes = [I, I, I, I, P, P, I, P, P]
        L.kvqo_coarse_meta.restype = None
        L.kvqo_mask_scores.argtypes = [I, I, I, I, P, P, I, P]
        L.kvqo_mask_scores.restype = None
        L.kvqo_half_to_float.argtypes = [ctypes.c_uint16]
        L.kvqo_half_to_float.restype = ctypes.c_float
        L.kvqo_dequant.argtypes = [ctypes.c_uint8, ctypes.c_float, ctypes.c_float]
        L.kvqo_dequant.restype = ctypes.c_float
        L.kvqo_quant_scale.argtypes = [ctypes.c_float, ctypes.c_float, P, P]
        L.kvqo_quant_scale.restype = None
        L.kvqo_quant_code.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
        L.kvqo_quant_code.restype = ctypes.c_uint8
        L.kvqo_quant_scale_levels.argtypes = [ctypes.c_float, ctypes.c_float, I, P, P]
        L.kvqo_quant_scale_levels.restype = None
        L.kvqo_quant_code_levels.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float, I]
        L.kvqo_quant_code_levels.restype = ctypes.c_uint8
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def _bits(x: np.ndarray) -> np.ndarray:
    """fp16 array -> its uint16 bit pattern (no arithmetic)."""
    return np.ascontiguousarray(x).view(np.uint16) if x.dtype == np.float16 else np.ascontiguousarray(x, np.uint16)


# --------------------------------------------------------------------- cache
class Cache:
    """One layer's paged cache as plain numpy arrays (the layout in kvq_oracle.c).
    MIXED (fmt 5): physical pages 0 .. n16-1 are the FP16 pool and the rest the
    INT8 (per token) pool, k_pages / v_pages one byte array holding both pools
    in that order, params for the INT8 pool only."""

    def __init__(self, fmt: int, num_phys_pages: int, num_kv_heads: int, head_dim: int, n16: int = 0):
        self.fmt, self.P_phys, self.H, self.d = fmt, num_phys_pages, num_kv_heads, head_dim
        self.n16 = n16 if fmt == 5 else 0
        row = head_dim // 2 if fmt in (3, 4) else head_dim   # INT4: two codes per byte
        shape = (num_phys_pages, num_kv_heads, PAGE, row)
        dt = np.uint16 if fmt == 0 else np.uint8
        if fmt == 5:
            assert 0 <= n16 <= num_phys_pages
            tile = num_kv_heads * PAGE * head_dim
            shape = (n16 * tile * 2 + (num_phys_pages - n16) * tile,)
        self.k_pages = np.zeros(shape, dtype=dt)
        self.v_pages = np.zeros(shape, dtype=dt)
        if fmt == 5:
            self.params = np.zeros((max(num_phys_pages - n16, 1), num_kv_heads, PAGE, 4), dtype=np.float32)
        elif fmt in (1, 3):
            self.params = np.zeros((num_phys_pages, num_kv_heads, PAGE, 4), dtype=np.float32)
        elif fmt in (2, 4):
            self.params = np.zeros((num_phys_pages, num_kv_heads, 4), dtype=np.float32)
        else:
            self.params = np.zeros((1,), dtype=np.float32)
        self.meta = np.zeros((num_phys_pages, num_kv_heads, 2, head_dim), dtype=np.float32)


def append(cache: Cache, block_table, start_pos, new_off, k_new, v_new) -> None:
    """Write packed new tokens k_new/v_new [N][H][d] (fp16) into the cache."""
    bt = np.ascontiguousarray(block_table, np.int32)
    sp = np.ascontiguousarray(start_pos, np.int32)
    off = np.ascontiguousarray(new_off, np.int32)
    kb, vb = _bits(k_new), _bits(v_new)
    B = sp.shape[0]
    rc = lib().kvqo_append(cache.fmt, cache.n16, B, cache.H, cache.d, bt.shape[1], _p(bt), _p(sp), _p(off),
                           _p(kb), _p(vb), _p(cache.k_pages), _p(cache.v_pages), _p(cache.params))
    if rc != 0:
        raise ValueError("oracle append: precondition violated")


def page_meta(cache: Cache, block_table, seq_lens, page_begin=None) -> None:
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    pb = None if page_begin is None else np.ascontiguousarray(page_begin, np.int32)
    lib().kvqo_page_meta(cache.fmt, cache.n16, sl.shape[0], cache.H, cache.d, bt.shape[1], _p(bt), _p(sl), _p(pb),
                         _p(cache.k_pages), _p(cache.params), _p(cache.meta))


def page_scores(cache: Cache, block_table, seq_lens, q) -> np.ndarray:
    """float64 [B][H_kv][max_pages]; pages past the sequence's end are -inf."""
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    qb = _bits(q)
    B, Hq, d = qb.shape
    out = np.empty((B, cache.H, bt.shape[1]), dtype=np.float64)
    lib().kvqo_page_scores(B, Hq, cache.H, d, bt.shape[1], _p(bt), _p(sl), _p(qb), _p(cache.meta), _p(out))
    return out


def num_selected(P: int, ratio_num: int, ratio_den: int, k_fixed: int) -> int:
    return lib().kvqo_num_selected(P, ratio_num, ratio_den, k_fixed)


def topk(scores, seq_lens, ratio_num, ratio_den, k_fixed, k_cap) -> tuple[np.ndarray, np.ndarray]:
    """(int32 [B][H][k_cap] ascending page ids padded with -1, int32 [B][H] counts)."""
    sc = np.ascontiguousarray(scores, np.float64)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    B, H, maxp = sc.shape
    sel = np.empty((B, H, k_cap), dtype=np.int32)
    cnt = np.empty((B, H), dtype=np.int32)
    rc = lib().kvqo_topk(B, H, maxp, _p(sl), _p(sc), ratio_num, ratio_den, k_fixed, k_cap, _p(sel), _p(cnt))
    if rc != 0:
        raise ValueError("oracle topk: k_cap too small")
    return sel, cnt


def attention(cache: Cache, block_table, seq_lens, q, sel_pages=None, sel_count=None, sm_scale=None) -> np.ndarray:
    """float64 [B][H_q][d]; sel_pages None attends to every page."""
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    qb = _bits(q)
    B, Hq, d = qb.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    sp = None if sel_pages is None else np.ascontiguousarray(sel_pages, np.int32)
    sc = None if sel_count is None else np.ascontiguousarray(sel_count, np.int32)
    k_cap = 0 if sp is None else sp.shape[2]
    out = np.empty((B, Hq, d), dtype=np.float64)
    lib().kvqo_attention(cache.fmt, cache.n16, B, Hq, cache.H, d, bt.shape[1], _p(bt), _p(sl), _p(qb),
                         _p(cache.k_pages), _p(cache.v_pages), _p(cache.params), _p(sp), _p(sc), k_cap,
                         float(sm_scale), _p(out))
    return out


def attention_mass(cache: Cache, block_table, seq_lens, q, sel_pages, sel_count, sm_scale=None) -> np.ndarray:
    """float64 [B][H_q]: the share of each head's dense softmax weight that
    falls on the tokens of its KV group's selected pages (1 when every page is
    selected; 0 for an empty sequence)."""
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    qb = _bits(q)
    B, Hq, d = qb.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    sp = np.ascontiguousarray(sel_pages, np.int32)
    sc = np.ascontiguousarray(sel_count, np.int32)
    out = np.empty((B, Hq), dtype=np.float64)
    lib().kvqo_attention_mass(cache.fmt, cache.n16, B, Hq, cache.H, d, bt.shape[1], _p(bt), _p(sl), _p(qb),
                              _p(cache.k_pages), _p(cache.params), _p(sp), _p(sc), sp.shape[2],
                              float(sm_scale), _p(out))
    return out


def decode_step(cache: Cache, block_table, seq_lens, q, ratio_num, ratio_den, k_fixed, k_cap,
                sm_scale=None, nthreads=1):
    """(scores, sel_pages, sel_count, out) of one decode step on nthreads host threads."""
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    qb = _bits(q)
    B, Hq, d = qb.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    maxp = bt.shape[1]
    scores = np.empty((B, cache.H, maxp), dtype=np.float64)
    sel = np.empty((B, cache.H, k_cap), dtype=np.int32)
    cnt = np.empty((B, cache.H), dtype=np.int32)
    out = np.empty((B, Hq, d), dtype=np.float64)
    rc = lib().kvqo_decode_step(cache.fmt, cache.n16, B, Hq, cache.H, d, maxp, _p(bt), _p(sl), _p(qb),
                                _p(cache.k_pages), _p(cache.v_pages), _p(cache.params), _p(cache.meta),
                                ratio_num, ratio_den, k_fixed, k_cap, float(sm_scale),
                                _p(scores), _p(sel), _p(cnt), _p(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle decode_step: k_cap too small")
    return scores, sel, cnt, out


# -------------------------------------------------- hierarchical selection
def demote(cache: Cache, block_table: np.ndarray, seq_lens, seq, page, dst) -> None:
    """Move logical page page[i] of sequence seq[i] of a MIXED cache from its
    FP16 page to INT8 page dst[i]: its valid tokens re-quantized per token from
    their fp16 rows, block_table[seq[i]][page[i]] = dst[i] (in place), and the
    page's metadata rebuilt."""
    assert cache.fmt == 5 and block_table.dtype == np.int32 and block_table.flags["C_CONTIGUOUS"]
    sl = np.ascontiguousarray(seq_lens, np.int32)
    sq = np.ascontiguousarray(seq, np.int32)
    pg = np.ascontiguousarray(page, np.int32)
    ds = np.ascontiguousarray(dst, np.int32)
    rc = lib().kvqo_demote(cache.n16, cache.P_phys, sl.shape[0], cache.H, cache.d, block_table.shape[1],
                           _p(block_table), _p(sl), len(sq), _p(sq), _p(pg), _p(ds), _p(cache.k_pages),
                           _p(cache.v_pages), _p(cache.params), _p(cache.meta))
    if rc != 0:
        raise ValueError("demote: an item does not move an FP16 page of its sequence to an INT8 page")


def coarse_meta(cache: Cache, block_table, seq_lens, group: int) -> np.ndarray:
    """float32 [B * pc_max][H][2][d]: each super-page's bounding box, the
    min of its pages' minima and max of their maxima (pc_max =
    ceil(max_pages / group)); super-pages past a sequence stay +inf / -inf."""
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    B, maxp = bt.shape
    pc_max = (maxp + group - 1) // group
    out = np.empty((B * pc_max, cache.H, 2, cache.d), np.float32)
    out[:, :, 0] = np.inf
    out[:, :, 1] = -np.inf
    lib().kvqo_coarse_meta(B, cache.H, cache.d, maxp, _p(bt), _p(sl), group, _p(cache.meta), _p(out))
    return out


def coarse_view(cache: Cache, block_table, seq_lens, group: int):
    """(cache view whose page metadata are the super-pages' boxes, its block
    table b -> b * pc_max + jc, its lengths in 16-token units of super-pages):
    page scores and top-K on this view are the coarse screen."""
    B, maxp = np.asarray(block_table).shape
    pc_max = (maxp + group - 1) // group
    view = Cache(cache.fmt, B * pc_max, cache.H, cache.d)
    view.meta = coarse_meta(cache, block_table, seq_lens, group)
    table = (np.arange(B, dtype=np.int32)[:, None] * pc_max + np.arange(pc_max, dtype=np.int32)[None]).astype(np.int32)
    P = (np.asarray(seq_lens, np.int64) + PAGE - 1) // PAGE
    lens_c = (((P + group - 1) // group) * PAGE).astype(np.int32)
    return view, table, lens_c


def mask_scores(scores, group: int, sel_super, sel_super_count) -> np.ndarray:
    """A copy of the fine scores with every page outside the kept super-pages
    set to -inf."""
    sc = np.array(scores, dtype=np.float64, order="C")
    B, H, maxp = sc.shape
    sel = np.ascontiguousarray(sel_super, np.int32)
    cnt = np.ascontiguousarray(sel_super_count, np.int32)
    lib().kvqo_mask_scores(B, H, maxp, group, _p(sel), _p(cnt), sel.shape[2], _p(sc))
    return sc


def hier_select(cache: Cache, block_table, seq_lens, q, group: int, kc: int, ratio_num: int, ratio_den: int,
                k_fixed: int, k_cap: int):
    """The coarse-then-fine selection ([TS] section 6): coarse scores of the
    super-pages, the top kc of them, the fine scores of their pages (-inf
    elsewhere), then the top-K rule of topk().  Returns (coarse scores,
    coarse selection, coarse counts, masked fine scores, selection, counts)."""
    view, ctable, clens = coarse_view(cache, block_table, seq_lens, group)
    csc = page_scores(view, ctable, clens, q)
    csel, ccnt = topk(csc, clens, 0, 1, kc, kc)
    fine = page_scores(cache, block_table, seq_lens, q)
    masked = mask_scores(fine, group, csel, ccnt)
    sel, cnt = topk(masked, seq_lens, ratio_num, ratio_den, k_fixed, k_cap)
    return csc, csel, ccnt, masked, sel, cnt


# ------------------------------------------------------------ element probes
def half_to_float(bits: int) -> float:
    return float(lib().kvqo_half_to_float(bits))


def dequant(code: int, scale: float, zero: float) -> float:
    return float(lib().kvqo_dequant(code, scale, zero))


def quant_scale(lo: float, hi: float) -> tuple[np.float32, np.float32]:
    s = ctypes.c_float()
    inv = ctypes.c_float()
    lib().kvqo_quant_scale(lo, hi, ctypes.byref(s), ctypes.byref(inv))
    return np.float32(s.value), np.float32(inv.value)


def quant_code(x: float, zero: float, inv: float) -> int:
    return int(lib().kvqo_quant_code(x, zero, inv))


def quant_scale_levels(lo: float, hi: float, levels: int) -> tuple[np.float32, np.float32]:
    s = ctypes.c_float()
    inv = ctypes.c_float()
    lib().kvqo_quant_scale_levels(lo, hi, levels, ctypes.byref(s), ctypes.byref(inv))
    return np.float32(s.value), np.float32(inv.value)


def quant_code_levels(x: float, zero: float, inv: float, levels: int) -> int:
    return int(lib().kvqo_quant_code_levels(x, zero, inv, levels))


# ------------------------------------------------------- whole-workload build
def build_cache(w, upto=None) -> tuple[Cache, np.ndarray]:
    """Build workload w's cache (every sequence, prefill of all its tokens, then
    metadata of every page).  ``upto[b]`` limits sequence b to its first upto[b]
    tokens.  Returns (cache, block_table)."""
    table, n_phys = w.block_table()
    lens = w.seq_lens() if upto is None else np.asarray(upto, np.int32)
    cache = Cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, w.fp16_pool_pages())
    for b in range(w.batch):
        L = int(lens[b])
        k = w.keys(b)[:L]
        v = w.values(b)[:L]
        sp = np.zeros(w.batch, np.int32)
        off = np.zeros(w.batch + 1, np.int32)
        off[b + 1:] = L                      # only sequence b receives rows in this call
        append(cache, table, sp, off, k, v)
    page_meta(cache, table, lens)
    return cache, table
