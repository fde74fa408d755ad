"""GPU parity of every libkvq stage against the CPU oracle, through the C ABI.

Bars (the decode-step contract):
  * INT8 codes, their fp32 (scale, zero) and the fp32 page metadata: bit-exact
    (metadata compares +0 == -0);
  * page scores: |gpu - oracle| <= 1e-4 |oracle|, or, where the sum cancels
    (|oracle| < 1e-2 S), <= 1e-4 S with S = sum_i |q_i c_i| over the terms the
    score picks;
  * top-K fed identical fp32 scores: identical selections (index work);
    fed its own scores: identical except pages whose oracle score lies within
    1e-4 (relative) of the oracle's K-th score;
  * attention: max abs error <= 2e-3 against fp64 (unit-variance V).
Each stage is fed the oracle's inputs for that stage; the end-to-end test runs
the GPU pipeline alone and checks its output against the oracle evaluated on
the selection the GPU made, once that selection passes the near-tie rule.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import PAGE

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-4
ATTN_ATOL = 2e-3


def log(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_quantized_sparse_amd as kvq
    kvq.lib()  # raises if the HIP library is missing


def kvq_mod():
    import paged_quantized_sparse_amd as kvq
    from paged_quantized_sparse_amd import runtime
    return kvq, runtime


# --------------------------------------------------------------- builders
class Built:
    """A workload built on the GPU (prefill of L-1 tokens, then the decode-time
    append of the last token) and by the oracle (one prefill)."""

    def __init__(self, w, with_oracle=True):
        kvq, runtime = kvq_mod()
        self.w = w
        self.table, self.n_phys = w.block_table()
        self.lens = w.seq_lens()
        src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
        log(f"[build] {w.name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
            f"fmt={workloads.FORMAT_NAMES[w.fmt]} pages={self.n_phys}")
        self.cache, self.seqs = runtime.build_cache(w.fmt, self.n_phys, w.num_kv_heads, w.head_dim, self.table,
                                                    self.lens, src, prefill_lens=self.lens - 1,
                                                    num_fp16_pages=w.fp16_pool_pages())
        runtime.DecodeAppend(self.cache, self.seqs, self.lens, src).run()
        torch.cuda.synchronize()
        self.q = w.query()
        self.q_dev = torch.from_numpy(self.q.view(np.int16)).cuda()
        self.ocache = oracle.build_cache(w)[0] if with_oracle else None

    def step(self, **kw):
        _, runtime = kvq_mod()
        w = self.w
        return runtime.DecodeStep(self.cache, self.seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, **kw)


_BUILT = {}


def built(key, w):
    if key not in _BUILT:
        _BUILT[key] = Built(w)
    return _BUILT[key]


SMALL = [1, 2, 3, 4, 5]
FULL = [1, 2, 3, 4]


def workload(kind, n):
    return workloads.small(n) if kind == "small" else workloads.config(n)


CASES = [("small", n) for n in SMALL] + [("full", n) for n in FULL]
IDS = [f"{k}{n}" for k, n in CASES]


# ------------------------------------------------------------ comparisons
def score_tolerance(ocache, table, lens, q, G):
    """Per (b, g, j): max(1e-4 |r|, 1e-4 S) where S = sum_i |q_i c_i| when
    |r| < 1e-2 S (cancellation); c_i is the M_i or m_i term the score picks."""
    B, Hq, d = q.shape
    H = Hq // G
    maxp = table.shape[1]
    S = np.zeros((B, H, maxp))
    qd = q.astype(np.float64)
    for b in range(B):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        meta = ocache.meta[table[b, :P]].astype(np.float64)       # [P][H][2][d]
        for h in range(Hq):
            g = h // G
            c = np.where(qd[b, h] >= 0, meta[:, g, 1], meta[:, g, 0])   # [P][d]
            S[b, g, :P] = np.maximum(S[b, g, :P], np.abs(c * qd[b, h]).sum(1))
    return S


def check_scores(got, want, S):
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(got), np.isneginf(want))
    err = np.abs(got[fin].astype(np.float64) - want[fin])
    r = np.abs(want[fin])
    tol = np.where(r < 1e-2 * S[fin], SCORE_RTOL * S[fin], SCORE_RTOL * r)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} scores off, worst rel {np.max(err / np.maximum(r, 1e-30)):.3g}"


def check_selection_near_ties(sel_gpu, cnt_gpu, oscores, osel, ocnt):
    """Sets equal except pages whose oracle score is within 1e-4 of the K-th."""
    B, H, _ = osel.shape
    n_tie = 0
    for b in range(B):
        for g in range(H):
            K = int(ocnt[b, g])
            assert int(cnt_gpu[b, g]) == K
            a = set(sel_gpu[b, g, :K].tolist())
            o = set(osel[b, g, :K].tolist())
            assert len(a) == K
            assert np.all(np.diff(sel_gpu[b, g, :K]) > 0), "selection not ascending"
            assert np.all(sel_gpu[b, g, K:] == -1)
            diff = a ^ o
            if diff:
                row = oscores[b, g]
                kth = np.sort(row[np.isfinite(row)])[::-1][K - 1]
                for j in diff:
                    assert abs(row[j] - kth) <= SCORE_RTOL * abs(kth), (b, g, j, row[j], kth)
                n_tie += len(diff)
    return n_tie


def to_np(t):
    return t.detach().cpu().numpy()


# ------------------------------------------------------------------ tests
@pytest.mark.parametrize("kind,n", CASES, ids=IDS)
def test_append_codes_params_and_meta_bit_exact(kind, n):
    bt = built((kind, n), workload(kind, n))
    oc = bt.ocache
    k = to_np(bt.cache.k_pages)
    v = to_np(bt.cache.v_pages)
    if bt.w.fmt == workloads.FMT_FP16:
        k, v = k.view(np.uint16), v.view(np.uint16)
    assert np.array_equal(k, oc.k_pages), "K storage differs"
    assert np.array_equal(v, oc.v_pages), "V storage differs"
    if bt.w.fmt != workloads.FMT_FP16:
        p = to_np(bt.cache.kv_params)
        assert np.array_equal(p.view(np.uint32), oc.params.view(np.uint32)), "scale/zero bits differ"
    meta = to_np(bt.cache.page_meta)
    assert np.array_equal(meta, oc.meta), "page metadata differs"   # == treats +0 and -0 alike


@pytest.mark.parametrize("kind,n", CASES, ids=IDS)
def test_page_scores(kind, n):
    kvq, _ = kvq_mod()
    bt = built((kind, n), workload(kind, n))
    st = bt.step()
    kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, st.scores)
    got = to_np(st.scores)
    want = oracle.page_scores(bt.ocache, bt.table, bt.lens, bt.q)
    check_scores(got, want, score_tolerance(bt.ocache, bt.table, bt.lens, bt.q, bt.w.group))


@pytest.mark.parametrize("kind,n", CASES, ids=IDS)
def test_topk_on_identical_scores_is_exact(kind, n):
    kvq, _ = kvq_mod()
    bt = built((kind, n), workload(kind, n))
    w = bt.w
    st = bt.step()   # ratio 1 (the dense configs): K = P, every page in order
    sc32 = oracle.page_scores(bt.ocache, bt.table, bt.lens, bt.q).astype(np.float32)
    st.scores.copy_(torch.from_numpy(sc32))
    kvq.kvq_topk_pages(st.scores, bt.seqs, w.num_kv_heads, w.ratio_num, w.ratio_den, w.k_fixed,
                       st.sel_pages, st.sel_count)
    osel, ocnt = oracle.topk(sc32.astype(np.float64), bt.lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    assert np.array_equal(to_np(st.sel_count), ocnt)
    assert np.array_equal(to_np(st.sel_pages), osel)


def test_topk_ties_plateaus_and_ragged_rows():
    """Constructed equal scores must go to the lowest logical pages; rows of
    different lengths; K = P rows; a row of one page."""
    kvq, _ = kvq_mod()
    rng = np.random.default_rng(21)
    B, H, maxp = 5, 3, 700
    lens = np.array([700 * 16, 699 * 16 + 3, 1, 37 * 16, 300 * 16 - 15], np.int32)
    sc = rng.integers(-3, 4, size=(B, H, maxp)).astype(np.float32)  # heavy ties
    sc[0, 0] = 0.0
    sc[0, 0, ::2] = -0.0                                            # -0 and +0 tie
    sc[1, 2, 100:400] = 7.5
    P = (lens + PAGE - 1) // PAGE
    for b in range(B):
        sc[b, :, P[b]:] = -np.inf
    seqs = kvq.Seqs(torch.from_numpy(lens).cuda(), torch.zeros((B, maxp), dtype=torch.int32, device="cuda"))
    for rn, rd, kf in [(3, 10, 0), (1, 1, 0), (1, 7, 0), (0, 1, 5)]:
        k_cap = kvq.num_selected(maxp, rn, rd, kf)
        sel = torch.empty((B, H, k_cap), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B, H), dtype=torch.int32, device="cuda")
        kvq.kvq_topk_pages(torch.from_numpy(sc).cuda(), seqs, H, rn, rd, kf, sel, cnt)
        osel, ocnt = oracle.topk(sc.astype(np.float64), lens, rn, rd, kf, k_cap)
        assert np.array_equal(to_np(cnt), ocnt)
        assert np.array_equal(to_np(sel), osel), (rn, rd, kf)


@pytest.mark.parametrize("kind,n", CASES, ids=IDS)
def test_attention_on_oracle_selection(kind, n):
    kvq, _ = kvq_mod()
    bt = built((kind, n), workload(kind, n))
    w = bt.w
    st = bt.step()
    if w.is_dense():
        out = st.attend(bt.q_dev)
        want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)
    else:
        osc = oracle.page_scores(bt.ocache, bt.table, bt.lens, bt.q)
        osel, ocnt = oracle.topk(osc, bt.lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
        sel = torch.from_numpy(osel).cuda()
        cnt = torch.from_numpy(ocnt).cuda()
        out = st.attend(bt.q_dev, sel, cnt)
        want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, osel, ocnt)
    err = np.abs(to_np(out).astype(np.float64) - want).max()
    log(f"[attn] {w.name}: max abs err {err:.3g}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("n,fmt", [(2, 0), (4, 1), (5, 2), (5, 3), (5, 5)],
                         ids=["fp16", "int8tok", "int8grp_gqa", "int4tok_gqa", "mixed_gqa"])
def test_attention_on_selection_in_any_order(n, fmt):
    """kvq_sparse_decode_attn takes each row's selected pages in any order:
    the oracle's selection with every row shuffled (seeded) gives, at two split
    sizes, an output within 1e-5 of the ascending selection's (only the order
    of the online softmax's accumulation changes) and within 2e-3 of the
    oracle's attention over that page set."""
    w = workloads.small(n).with_(name=f"small{n}_anyorder_{fmt}", fmt=fmt,
                                 hot_recent=3 if fmt == workloads.FMT_MIXED else 0)
    if workloads.FMT_INT4_TOKEN <= fmt <= workloads.FMT_INT4_GROUP64:
        w = w.with_(head_dim=128)
    bt = Built(w)
    st = bt.step()
    osc = oracle.page_scores(bt.ocache, bt.table, bt.lens, bt.q)
    osel, ocnt = oracle.topk(osc, bt.lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    shuf = osel.copy()
    rng = np.random.default_rng(23)
    for b in range(shuf.shape[0]):
        for g in range(shuf.shape[1]):
            c = int(ocnt[b, g])
            shuf[b, g, :c] = shuf[b, g, rng.permutation(c)]
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, osel, ocnt)
    cnt = torch.from_numpy(ocnt).cuda()
    for pps in (0, 3):
        s = bt.step(pages_per_split=pps, fused_select=False)
        asc = to_np(s.attend(bt.q_dev, torch.from_numpy(osel).cuda(), cnt)).astype(np.float64).copy()
        out = to_np(s.attend(bt.q_dev, torch.from_numpy(shuf).cuda(), cnt)).astype(np.float64)
        assert np.abs(out - asc).max() <= 1e-5, pps
        assert np.abs(out - want).max() <= ATTN_ATOL, pps


@pytest.mark.parametrize("n", [2, 4, 5])
@pytest.mark.parametrize("pps", [1, 3, 4, 16, 64])
def test_attention_independent_of_split_size(n, pps):
    _, runtime = kvq_mod()
    bt = built(("small", n), workloads.small(n))
    w = bt.w
    ref = bt.step()
    ref.run(bt.q_dev)
    base = to_np(ref.out).copy()
    st = bt.step(pages_per_split=pps)
    out = to_np(st.attend(bt.q_dev, ref.sel_pages, ref.sel_count)).astype(np.float64)
    assert np.abs(out - base).max() <= 1e-5
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, to_np(ref.sel_pages), to_np(ref.sel_count))
    assert np.abs(out - want).max() <= ATTN_ATOL
    dense = to_np(bt.step(dense=True, pages_per_split=pps).attend(bt.q_dev)).astype(np.float64)
    assert np.abs(dense - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)).max() <= ATTN_ATOL


def _select_vs_separate(st_sep, st_fus, q_dev, scores=None):
    """Run top-K then attention (st_sep) and the one-call select + attention
    (st_fus) on the same scores; return both outputs and selections."""
    kvq, _ = kvq_mod()
    if scores is not None:
        st_sep.scores.copy_(scores)
    rn, rd, kf = st_sep.ratio
    kvq.kvq_topk_pages(st_sep.scores, st_sep.seqs, st_sep.cache.num_kv_heads, rn, rd, kf, st_sep.sel_pages,
                       st_sep.sel_count)
    out_sep = st_sep.attend(q_dev, st_sep.sel_pages, st_sep.sel_count).clone()
    st_fus.scores.copy_(st_sep.scores)
    st_fus.sel_pages.fill_(-7)
    st_fus.sel_count.fill_(-7)
    out_fus = st_fus.select_attend(q_dev)
    torch.cuda.synchronize()
    return out_sep, out_fus


@pytest.mark.parametrize("kind,n", CASES, ids=IDS)
def test_select_attention_equals_topk_then_attention(kind, n):
    """kvq_select_decode_attn (top-K inside the attention kernel) writes the
    selection kvq_topk_pages writes and, bit for bit, the output of
    kvq_sparse_decode_attn over it, at the default split and at others."""
    kvq, _ = kvq_mod()
    bt = built((kind, n), workload(kind, n))   # ratio 1 runs the selecting path with K = P
    for pps in ([0, 1, 3, 16, 64] if kind == "small" else [0, 16]):
        sep = bt.step(pages_per_split=pps, fused_select=False)
        kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, sep.scores)
        fus = bt.step(pages_per_split=pps)
        out_sep, out_fus = _select_vs_separate(sep, fus, bt.q_dev)
        assert torch.equal(fus.sel_count, sep.sel_count), pps
        assert torch.equal(fus.sel_pages, sep.sel_pages), pps
        assert torch.equal(out_fus, out_sep), pps


@pytest.mark.parametrize("n", [5, 4], ids=["ragged_gqa_short_rows", "rows_of_127_pages"])
def test_select_attention_on_tied_scores(n):
    """Heavily tied scores (small integers, -0 and +0, plateaus): the in-kernel
    selection equals the oracle's top-K exactly and the output equals top-K
    then attention bit for bit -- on a ragged GQA batch of short rows and on
    rows of 127 pages."""
    _, runtime = kvq_mod()
    bt = built(("small", n), workloads.small(n))
    w = bt.w
    B, maxp, H = bt.table.shape[0], bt.table.shape[1], w.num_kv_heads
    rng = np.random.default_rng(33)
    sc = rng.integers(-3, 4, size=(B, H, maxp)).astype(np.float32)
    sc[0, 0] = 0.0
    sc[0, 0, ::2] = -0.0
    sc[1 % B, H - 1, 5:60] = 2.5
    P = (bt.lens + PAGE - 1) // PAGE
    for b in range(B):
        sc[b, :, P[b]:] = -np.inf
    for rn, rd, kf in [(3, 10, 0), (1, 7, 0), (0, 1, 5), (1, 1, 0)]:
        mk = lambda fused: runtime.DecodeStep(bt.cache, bt.seqs, w.num_q_heads, rn, rd, kf,  # noqa: E731
                                              fused_select=fused)
        sep, fus = mk(False), mk(True)
        out_sep, out_fus = _select_vs_separate(sep, fus, bt.q_dev, torch.from_numpy(sc).cuda())
        osel, ocnt = oracle.topk(sc.astype(np.float64), bt.lens, rn, rd, kf, fus.k_cap)
        assert np.array_equal(to_np(fus.sel_count), ocnt), (rn, rd, kf)
        assert np.array_equal(to_np(fus.sel_pages), osel), (rn, rd, kf)
        assert torch.equal(out_fus, out_sep), (rn, rd, kf)


def test_select_attention_rows_at_the_limit():
    """Rows of up to KVQ_SELECT_MAX_PAGES pages (every thread holding all 8 of
    its keys): selection and output equal top-K then attention, at several
    splits, and the selection equals the oracle's top-K of the same scores.
    Longer rows are refused, and the runtime then takes the two-call path."""
    kvq, runtime = kvq_mod()
    w = workloads.small(4).with_(seq_len=kvq.SELECT_MAX_PAGES * PAGE - 3, batch=2)  # last page partial
    bt = Built(w, with_oracle=False)
    assert bt.seqs.max_pages == kvq.SELECT_MAX_PAGES
    for pps in (0, 7, 64):
        sep = bt.step(pages_per_split=pps, fused_select=False)
        kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, sep.scores)
        fus = bt.step(pages_per_split=pps)
        out_sep, out_fus = _select_vs_separate(sep, fus, bt.q_dev)
        osel, ocnt = oracle.topk(to_np(sep.scores).astype(np.float64), bt.lens, w.ratio_num, w.ratio_den,
                                 w.k_fixed, fus.k_cap)
        assert np.array_equal(to_np(fus.sel_count), ocnt), pps
        assert np.array_equal(to_np(fus.sel_pages), osel), pps
        assert torch.equal(out_fus, out_sep), pps
    # one page more per row: refused by the fused call, run in two calls by the runtime
    lens = torch.from_numpy(bt.lens.astype(np.int32)).cuda()
    table = torch.zeros((w.batch, kvq.SELECT_MAX_PAGES + 1), dtype=torch.int32, device="cuda")
    table[:, :-1] = bt.seqs.block_table
    seqs = kvq.Seqs(lens, table)
    st = runtime.DecodeStep(bt.cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, pages_per_split=16)
    assert not st.fused_select
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_select_decode_attn(bt.cache, seqs, bt.q_dev, st.scores, w.ratio_num, w.ratio_den, w.k_fixed,
                                   st.k_cap, st.out, st.workspace, st.sm_scale)
    assert e.value.status == 2
    out = st.run(bt.q_dev).clone()
    fus = bt.step(pages_per_split=16)
    assert fus.fused_select   # 2 x 4 x 39 blocks: one round
    want = fus.run(bt.q_dev)
    torch.cuda.synchronize()
    assert st.k_cap == fus.k_cap
    assert torch.equal(st.sel_pages, fus.sel_pages)   # the extra column is never a live page
    assert torch.equal(out, want)                     # same splits, same pages: same bits


@pytest.mark.parametrize("n", [2, 4, 5])
def test_select_attention_without_selection_outputs(n):
    """sel_pages / sel_count of kvq_select_decode_attn are optional: with both
    NULL the output is the same, bit for bit, as with both given."""
    kvq, _ = kvq_mod()
    bt = built(("small", n), workloads.small(n))
    w = bt.w
    st = bt.step()
    assert st.fused_select
    kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, st.scores)
    st.select_attend(bt.q_dev)
    with_sel = st.out.clone()
    st.out.fill_(7.0)
    kvq.kvq_select_decode_attn(bt.cache, bt.seqs, bt.q_dev, st.scores, w.ratio_num, w.ratio_den, w.k_fixed,
                               st.k_cap, st.out, st.workspace, st.sm_scale, st.pps)
    torch.cuda.synchronize()
    assert torch.equal(st.out, with_sel)


@pytest.mark.parametrize("fused", [True, False])
def test_empty_sequences_in_batch(fused):
    """Sequences of length 0 inside a ragged GQA batch: all their scores are
    -inf, nothing is selected, their output rows are zero, and the other
    sequences still match the oracle."""
    kvq, runtime = kvq_mod()
    w = workloads.small(5)
    bt = built(("small", 5), w)
    lens = bt.lens.copy()
    empty = [1, 3]
    lens[empty] = 0
    seqs = kvq.Seqs(torch.from_numpy(lens.astype(np.int32)).cuda(), bt.seqs.block_table)
    st = runtime.DecodeStep(bt.cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_select=fused)
    out = to_np(st.run(bt.q_dev)).astype(np.float64)
    assert np.isneginf(to_np(st.scores)[empty]).all()
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    assert (gcnt[empty] == 0).all() and (gsel[empty] == -1).all()
    assert (out[empty] == 0).all()
    osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, lens, bt.q, w.ratio_num, w.ratio_den, w.k_fixed,
                                            st.k_cap, nthreads=8)
    check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    want = oracle.attention(bt.ocache, bt.table, lens, bt.q, gsel, gcnt)
    assert np.abs(out - want).max() <= ATTN_ATOL


@pytest.mark.parametrize("n,fmt", [(5, 2), (5, 1), (4, 0), (1, 0)], ids=["gqa_int8grp", "gqa_int8tok", "mha_fp16",
                                                                       "config1"])
def test_one_split_per_row_writes_out_without_combine(n, fmt):
    """When no row has more than one split the split kernel writes out itself:
    the output equals, bit for bit, the split-then-combine result over the same
    single live split (forced by a selection stride of two splits), empty rows
    are zero (out prefilled with NaN), and it matches the oracle."""
    kvq, runtime = kvq_mod()
    w = workloads.small(n).with_(fmt=fmt)
    bt = built(("one_split", n, fmt), w)
    lens = bt.lens.copy()
    if w.batch > 3:
        lens[[1, 3]] = 0
    seqs = kvq.Seqs(torch.from_numpy(lens.astype(np.int32)).cuda(), bt.seqs.block_table)
    osc = oracle.page_scores(bt.ocache, bt.table, lens, bt.q)
    maxp = bt.table.shape[1]
    k_max = kvq.num_selected(maxp, w.ratio_num, w.ratio_den, w.k_fixed)
    pps = max(k_max, 1)
    outs = []
    for k_cap in (k_max, 2 * pps):   # one split per row: no combine; two (the second empty): combine
        osel, ocnt = oracle.topk(osc, lens, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
        out = torch.full((w.batch, w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(kvq.kvq_attn_workspace_bytes(w.batch, w.num_q_heads, w.head_dim, maxp, k_cap, pps) // 4 + 64,
                         dtype=torch.float32, device="cuda")
        kvq.kvq_sparse_decode_attn(bt.cache, seqs, bt.q_dev, torch.from_numpy(osel).cuda(),
                                   torch.from_numpy(ocnt).cuda(), out, ws, w.sm_scale(), pps)
        torch.cuda.synchronize()
        outs.append(to_np(out).astype(np.float64))
    assert np.array_equal(outs[0], outs[1])
    if w.batch > 3:
        assert (outs[0][[1, 3]] == 0).all()
    want = oracle.attention(bt.ocache, bt.table, lens, bt.q, osel, ocnt)
    assert np.abs(outs[0] - want).max() <= ATTN_ATOL


def test_topk_longest_rows():
    """kvq_topk_pages at its longest supported row (12000 pages), on random
    and on tied scores, against the oracle's top-K exactly."""
    kvq, _ = kvq_mod()
    rng = np.random.default_rng(77)
    B, H, maxp = 2, 2, 12000
    lens = np.array([maxp * PAGE, 7777 * PAGE - 5], np.int32)
    sc = rng.standard_normal((B, H, maxp)).astype(np.float32)
    sc[1, 1] = np.round(sc[1, 1] * 4) / 4  # heavy ties
    P = (lens + PAGE - 1) // PAGE
    for b in range(B):
        sc[b, :, P[b]:] = -np.inf
    seqs = kvq.Seqs(torch.from_numpy(lens).cuda(), torch.zeros((B, maxp), dtype=torch.int32, device="cuda"))
    for rn, rd, kf in [(3, 10, 0), (1, 50, 0)]:
        k_cap = kvq.num_selected(maxp, rn, rd, kf)
        sel = torch.empty((B, H, k_cap), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B, H), dtype=torch.int32, device="cuda")
        kvq.kvq_topk_pages(torch.from_numpy(sc).cuda(), seqs, H, rn, rd, kf, sel, cnt)
        osel, ocnt = oracle.topk(sc.astype(np.float64), lens, rn, rd, kf, k_cap)
        assert np.array_equal(to_np(cnt), ocnt), (rn, rd)
        assert np.array_equal(to_np(sel), osel), (rn, rd)


@pytest.mark.parametrize("kind,n", CASES, ids=IDS)
def test_end_to_end_step(kind, n):
    bt = built((kind, n), workload(kind, n))
    w = bt.w
    st = bt.step(dense=w.is_dense())
    out = to_np(st.run(bt.q_dev)).astype(np.float64)
    if w.is_dense():
        want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)
    else:
        osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den,
                                                w.k_fixed, st.k_cap, nthreads=8)
        gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
        ties = check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
        log(f"[step] {w.name}: {ties} near-tie page swaps")
        want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, gsel, gcnt)
    err = np.abs(out - want).max()
    log(f"[step] {w.name}: max abs err {err:.3g}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("fmt", [1, 2])
@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 128), (16, 2, 128), (8, 4, 64), (16, 2, 64)],
                         ids=["g2d128", "g8d128", "g2d64", "g8d64"])
def test_group_sizes_and_head_dims(fmt, hq, hkv, d):
    """Query groups of 2 and 8 heads per KV head, at head_dim 128 and 64, on
    the INT8 caches (the matrix-core form of the attention kernel): attention
    over the oracle's selection, the whole step through both selection paths
    (which agree bit for bit) and the dense path all match the oracle."""
    w = workloads.small(5).with_(name=f"gqa{hq}x{hkv}_d{d}_fmt{fmt}", fmt=fmt, num_q_heads=hq, num_kv_heads=hkv,
                                 head_dim=d)
    bt = built(("gqa", fmt, hq, hkv, d), w)
    st = bt.step()
    osc = oracle.page_scores(bt.ocache, bt.table, bt.lens, bt.q)
    osel, ocnt = oracle.topk(osc, bt.lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    out = to_np(st.attend(bt.q_dev, torch.from_numpy(osel).cuda(), torch.from_numpy(ocnt).cuda()))
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, osel, ocnt)
    err = np.abs(out.astype(np.float64) - want).max()
    log(f"[gqa] {w.name}: attention on the oracle's selection, max abs err {err:.3g}")
    assert err <= ATTN_ATOL
    fus, sep = bt.step(fused_select=True), bt.step(fused_select=False)
    o_fus = fus.run(bt.q_dev).clone()
    o_sep = sep.run(bt.q_dev)
    torch.cuda.synchronize()
    assert torch.equal(fus.sel_pages, sep.sel_pages) and torch.equal(o_fus, o_sep)
    gsel, gcnt = to_np(fus.sel_pages), to_np(fus.sel_count)
    check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, gsel, gcnt)
    assert np.abs(to_np(o_fus).astype(np.float64) - want).max() <= ATTN_ATOL
    dense = to_np(bt.step(dense=True).attend(bt.q_dev)).astype(np.float64)
    assert np.abs(dense - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)).max() <= ATTN_ATOL


@pytest.mark.parametrize("fmt", [1, 2])
def test_scores_ragged_persistent_grid(fmt):
    """A ragged batch large enough that scoring runs as a persistent grid
    balanced over the live items (40 sequences of 1 to 8191 tokens, 8 KV
    heads, groups of 4): every score matches the oracle, pages past each
    length are -inf, and the fused append + scores kernel writes the same
    scores, bit for bit, as the decode-time append followed by
    kvq_page_scores."""
    kvq, runtime = kvq_mod()
    w = workloads.small(5).with_(name=f"ragged40_fmt{fmt}", fmt=fmt, batch=40, num_q_heads=32, num_kv_heads=8,
                                 len_lo=1, len_hi=8191)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    qn = w.query()
    q = torch.from_numpy(qn.view(np.int16)).cuda()
    runs = []
    for fused in (True, False):
        cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                          prefill_lens=lens - 1)
        app = runtime.DecodeAppend(cache, seqs, lens, src)
        st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
        st.scores.fill_(float("nan"))
        if fused:
            kvq.kvq_append_decode_scores(cache, seqs, app.start, app.off, app.max_new, app.k_new, app.v_new, q,
                                         st.scores)
        else:
            app.run()
            kvq.kvq_page_scores(cache, seqs, q, st.scores)
        torch.cuda.synchronize()
        runs.append(to_np(st.scores))
    assert np.array_equal(runs[0], runs[1])
    ocache, _ = oracle.build_cache(w)
    want = oracle.page_scores(ocache, table, lens, qn)
    check_scores(runs[0], want, score_tolerance(ocache, table, lens, qn, w.group))
    log(f"[ragged] {w.name}: {int(np.isfinite(want).sum())} live scores, max_pages {table.shape[1]}")


def test_k_equals_all_pages_matches_dense():
    """Config 1 with K = 64 of 64 pages: the full selection path equals the
    dense path and the oracle's dense attention."""
    w = workloads.config(1).with_(k_fixed=64)
    bt = built(("k64", 1), w)
    st = bt.step()
    sparse = to_np(st.run(bt.q_dev)).copy()
    assert np.array_equal(to_np(st.sel_count), np.full((1, 4), 64))
    dense = to_np(st.attend(bt.q_dev))
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)
    assert np.abs(sparse - want).max() <= ATTN_ATOL
    assert np.abs(sparse - dense).max() <= 1e-6


@pytest.mark.parametrize("n", [4, 5])
def test_deterministic(n):
    """Two runs give bitwise-equal codes, metadata, scores, selections, outputs."""
    w = workloads.small(n)
    a, b = Built(w, with_oracle=False), Built(w, with_oracle=False)
    for x, y in [(a.cache.k_pages, b.cache.k_pages), (a.cache.kv_params, b.cache.kv_params),
                 (a.cache.page_meta, b.cache.page_meta)]:
        assert torch.equal(x, y)
    sa, sb = a.step(), b.step()
    oa, ob = sa.run(a.q_dev), sb.run(b.q_dev)
    torch.cuda.synchronize()
    assert torch.equal(sa.scores, sb.scores) and torch.equal(sa.sel_pages, sb.sel_pages)
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("n", [4, 5])
def test_graph_replay_matches_eager(n):
    """The decode step (append, metadata refresh, scores, top-K, attention)
    captured in a HIP graph and replayed several times, with eager work and
    synchronizations in between, gives the eager result bit for bit, and that
    result matches the oracle."""
    _, runtime = kvq_mod()
    w = workloads.small(n)
    bt = Built(w)
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    app = runtime.DecodeAppend(bt.cache, bt.seqs, bt.lens, src)
    st = bt.step()
    app.run()
    eager = st.run(bt.q_dev).clone()
    eager_sel = st.sel_pages.clone()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            app.run()
            st.run(bt.q_dev)
    torch.cuda.current_stream().wait_stream(cap)
    osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den,
                                            w.k_fixed, st.k_cap)
    check_selection_near_ties(to_np(eager_sel), to_np(st.sel_count), osc, osel, ocnt)
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, to_np(eager_sel), to_np(st.sel_count))
    assert np.abs(to_np(eager).astype(np.float64) - want).max() <= ATTN_ATOL
    for i in range(4):
        st.out.zero_()
        st.sel_pages.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, eager), f"replay {i}"
        assert torch.equal(st.sel_pages, eager_sel), f"replay {i}"
        st.run(bt.q_dev)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_decode_stream_many_steps(fmt, fused):
    """A decode loop: 24 consecutive steps of DecodeStep.run_with_append on a
    ragged batch, each appending every sequence's next token (INT8_GROUP64
    re-supplies its open 64-token group), crossing page and group boundaries,
    with a fresh query per step.  After every step the whole cache (codes,
    scale/zero bits, metadata) equals the oracle's one-shot build of the same
    tokens, the selection passes the near-tie rule and the output is within
    tolerance of the oracle's attention over that selection."""
    _, runtime = kvq_mod()
    T = 24
    w = workloads.small(5).with_(fmt=fmt)
    lens_end = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    L0 = lens_end - T
    assert (L0 >= 1).all()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, L0, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_select=fused)
    rng = np.random.default_rng(4242 + fmt)
    crossed = 0
    for t in range(T):
        lens_t = L0 + t + 1
        crossed += int(((lens_t - 1) % PAGE == 0).sum())
        seqs.seq_lens.copy_(torch.from_numpy(lens_t.astype(np.int32)))
        app = runtime.DecodeAppend(cache, seqs, lens_t, src)
        q = rng.standard_normal((w.batch, w.num_q_heads, w.head_dim)).astype(np.float16)
        out = to_np(st.run_with_append(app, torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
        oc, _ = oracle.build_cache(w, upto=lens_t)
        k, v = to_np(cache.k_pages), to_np(cache.v_pages)
        if fmt == workloads.FMT_FP16:
            k, v = k.view(np.uint16), v.view(np.uint16)
        assert np.array_equal(k, oc.k_pages) and np.array_equal(v, oc.v_pages), f"step {t}: storage"
        if fmt != workloads.FMT_FP16:
            assert np.array_equal(to_np(cache.kv_params).view(np.uint32), oc.params.view(np.uint32)), f"step {t}"
        assert np.array_equal(to_np(cache.page_meta), oc.meta), f"step {t}: metadata"
        osc, osel, ocnt, _ = oracle.decode_step(oc, table, lens_t, q, w.ratio_num, w.ratio_den, w.k_fixed,
                                                st.k_cap, nthreads=8)
        gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
        check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
        want = oracle.attention(oc, table, lens_t, q, gsel, gcnt)
        err = np.abs(out - want).max()
        assert err <= ATTN_ATOL, f"step {t}: max abs err {err:.3g}"
    log(f"[stream] fmt {fmt} fused {fused}: {T} steps, {crossed} new pages opened")
    assert crossed >= w.batch  # every sequence opened at least one page


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("rows", [1, 17, 64])
def test_append_decode_equals_separate_calls_and_oracle(fmt, rows):
    """kvq_append_decode (append + metadata of the touched pages, one kernel)
    gives the same codes, scale/zero bits and metadata as kvq_append_quant
    followed by kvq_build_page_meta, and as the oracle's one-shot build.
    INT8_GROUP64 re-supplies the open group from its 64-aligned start."""
    kvq, runtime = kvq_mod()
    w = workloads.small(5).with_(fmt=fmt, batch=4, len_lo=70, len_hi=300)
    lens = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    start = (lens - 1) // 64 * 64 if fmt == workloads.FMT_INT8_GROUP64 else lens - rows
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    built_caches = []
    for fused in (True, False):
        cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                          prefill_lens=start)
        cnt = lens - start
        k_new = np.concatenate([w.keys(b)[start[b]:lens[b]] for b in range(w.batch)])
        v_new = np.concatenate([w.values(b)[start[b]:lens[b]] for b in range(w.batch)])
        args = (torch.from_numpy(start.astype(np.int32)).cuda(),
                torch.from_numpy(np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)).cuda(), int(cnt.max()),
                torch.from_numpy(k_new.view(np.int16)).cuda(), torch.from_numpy(v_new.view(np.int16)).cuda())
        if fused:
            kvq.kvq_append_decode(cache, seqs, *args)
        else:
            kvq.kvq_append_quant(cache, seqs, *args)
            kvq.kvq_build_page_meta(cache, seqs, torch.from_numpy((start // PAGE).astype(np.int32)).cuda(), 5)
        torch.cuda.synchronize()
        built_caches.append(cache)
    a, b = built_caches
    for x, y in [(a.k_pages, b.k_pages), (a.v_pages, b.v_pages), (a.page_meta, b.page_meta)]:
        assert torch.equal(x, y)
    if fmt != workloads.FMT_FP16:
        assert torch.equal(a.kv_params, b.kv_params)
    oc, _ = oracle.build_cache(w)
    k = to_np(a.k_pages)
    assert np.array_equal(k.view(np.uint16) if fmt == workloads.FMT_FP16 else k, oc.k_pages)
    if fmt != workloads.FMT_FP16:
        assert np.array_equal(to_np(a.kv_params).view(np.uint32), oc.params.view(np.uint32))
    assert np.array_equal(to_np(a.page_meta), oc.meta)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_append_decode_scores_equals_separate_calls(n):
    """kvq_append_decode_scores (append + metadata of the touched pages fused
    into scoring) leaves the same cache and writes the same scores, bit for
    bit, as kvq_append_decode followed by kvq_page_scores; the step built on it
    matches the oracle."""
    kvq, runtime = kvq_mod()
    w = workloads.small(n)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    q = torch.from_numpy(w.query().view(np.int16)).cuda()
    runs = []
    for fused in (True, False):
        cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                          prefill_lens=lens - 1)
        app = runtime.DecodeAppend(cache, seqs, lens, src)
        st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
        if fused:
            kvq.kvq_append_decode_scores(cache, seqs, app.start, app.off, app.max_new, app.k_new, app.v_new, q,
                                         st.scores)
        else:
            app.run()
            kvq.kvq_page_scores(cache, seqs, q, st.scores)
        torch.cuda.synchronize()
        runs.append((cache, st.scores.clone()))
    (ca, sa), (cb, sb) = runs
    assert torch.equal(sa, sb)
    for x, y in [(ca.k_pages, cb.k_pages), (ca.v_pages, cb.v_pages), (ca.page_meta, cb.page_meta)]:
        assert torch.equal(x, y)
    if w.fmt != workloads.FMT_FP16:
        assert torch.equal(ca.kv_params, cb.kv_params)
    # the whole fused step against the oracle
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                      prefill_lens=lens - 1)
    app = runtime.DecodeAppend(cache, seqs, lens, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, dense=w.is_dense())
    out = to_np(st.run_with_append(app, q)).astype(np.float64)
    oc, _ = oracle.build_cache(w)
    if w.is_dense():
        want = oracle.attention(oc, table, lens, w.query())
    else:
        osc, osel, ocnt, _ = oracle.decode_step(oc, table, lens, w.query(), w.ratio_num, w.ratio_den, w.k_fixed,
                                                st.k_cap)
        gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
        check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
        want = oracle.attention(oc, table, lens, w.query(), gsel, gcnt)
    assert np.abs(out - want).max() <= ATTN_ATOL
