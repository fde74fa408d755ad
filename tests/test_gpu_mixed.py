"""GPU parity of the mixed-precision cache (an FP16 pool for the pages of high
importance, an INT8-per-token pool for the rest) against the oracle, through
the C ABI.

Bars as for the single formats: storage bytes, scale/zero bits and metadata
bit-exact (bulk append, decode-time append, append fused into scoring, page
demotion); page scores to 1e-4; top-K exact on identical scores; attention
within 2e-3 of fp64 on the oracle's selection and on the GPU's; the in-kernel
selection bit-equal to top-K then attention.  The attention kernel takes each
split's FP16 pages and INT8 pages in two passes and merges them, so a cache
with its FP16 pool empty must give, bit for bit, the INT8 kernel's output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import FMT_MIXED, PAGE

pytestmark = pytest.mark.gpu

ATTN_ATOL = 2e-3


def log(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_quantized_sparse_amd as kvq
    kvq.lib()


def mods():
    import paged_quantized_sparse_amd as kvq
    from paged_quantized_sparse_amd import runtime
    return kvq, runtime


def to_np(t):
    return t.detach().cpu().numpy()


def mixed(w, hot_recent):
    return w.with_(name=f"{w.name}_mixed{hot_recent}", fmt=FMT_MIXED, hot_recent=hot_recent)


# the small workloads with a few recent pages in FP16, and the 32K layer with
# its first page and last 192 of 2048 pages in FP16
CASES = [("small", 3, 5), ("small", 4, 16), ("small", 5, 5), ("full", 4, 192)]
CASE_IDS = [f"{k}{n}_hot{h}" for k, n, h in CASES]

_BUILT = {}


def built(kind, n, hot):
    from test_gpu_parity import Built
    key = (kind, n, hot)
    if key not in _BUILT:
        w = workloads.small(n) if kind == "small" else workloads.config(n)
        _BUILT[key] = Built(mixed(w, hot))
    return _BUILT[key]


def assert_storage_equal(cache, oc, what):
    assert cache.num_fp16_pages == oc.n16
    assert np.array_equal(to_np(cache.k_pages), oc.k_pages), f"{what}: K storage"
    assert np.array_equal(to_np(cache.v_pages), oc.v_pages), f"{what}: V storage"
    p = to_np(cache.kv_params).view(np.uint32)
    assert np.array_equal(p, oc.params.view(np.uint32)), f"{what}: scale/zero bits"
    assert np.array_equal(to_np(cache.page_meta), oc.meta), f"{what}: metadata"


@pytest.mark.parametrize("kind,n,hot", CASES, ids=CASE_IDS)
def test_mixed_build_bit_exact(kind, n, hot):
    """Prefill of L-1 tokens then the decode-time append of the last one: both
    pools, the INT8 pool's scale/zero bits and all metadata equal the oracle's."""
    bt = built(kind, n, hot)
    assert 0 < bt.cache.num_fp16_pages < bt.cache.num_phys_pages
    assert_storage_equal(bt.cache, bt.ocache, bt.w.name)


@pytest.mark.parametrize("kind,n,hot", CASES, ids=CASE_IDS)
def test_mixed_scores_topk_and_attention(kind, n, hot):
    from test_gpu_parity import check_scores, score_tolerance
    kvq, _ = mods()
    bt = built(kind, n, hot)
    w = bt.w
    st = bt.step()
    kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, st.scores)
    osc = oracle.page_scores(bt.ocache, bt.table, bt.lens, bt.q)
    check_scores(to_np(st.scores), osc, score_tolerance(bt.ocache, bt.table, bt.lens, bt.q, w.group))
    sc32 = osc.astype(np.float32)
    st.scores.copy_(torch.from_numpy(sc32))
    kvq.kvq_topk_pages(st.scores, bt.seqs, w.num_kv_heads, w.ratio_num, w.ratio_den, w.k_fixed, st.sel_pages,
                       st.sel_count)
    osel, ocnt = oracle.topk(sc32.astype(np.float64), bt.lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    assert np.array_equal(to_np(st.sel_count), ocnt) and np.array_equal(to_np(st.sel_pages), osel)
    out = st.attend(bt.q_dev, torch.from_numpy(osel).cuda(), torch.from_numpy(ocnt).cuda())
    err = float(np.abs(to_np(out).astype(np.float64) - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, osel,
                                                                        ocnt)).max())
    dense = to_np(bt.step(dense=True).attend(bt.q_dev)).astype(np.float64)
    derr = float(np.abs(dense - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)).max())
    log(f"[mixed attn] {w.name}: max abs err {err:.3g} (selected), {derr:.3g} (every page)")
    assert err <= ATTN_ATOL and derr <= ATTN_ATOL


@pytest.mark.parametrize("kind,n,hot", CASES, ids=CASE_IDS)
def test_mixed_select_attention_and_step(kind, n, hot):
    """In-kernel selection bit-equal to top-K then attention at several split
    sizes; the whole step from a cache one token short against the oracle."""
    from test_gpu_parity import _select_vs_separate, check_selection_near_ties
    kvq, runtime = mods()
    bt = built(kind, n, hot)
    w = bt.w
    for pps in ([0, 1, 3, 64] if kind == "small" else [0, 16]):
        sep = bt.step(pages_per_split=pps, fused_select=False)
        kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, sep.scores)
        fus = bt.step(pages_per_split=pps)
        out_sep, out_fus = _select_vs_separate(sep, fus, bt.q_dev)
        assert torch.equal(fus.sel_count, sep.sel_count) and torch.equal(fus.sel_pages, sep.sel_pages), pps
        assert torch.equal(out_fus, out_sep), pps
    table, n_phys = w.block_table()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, bt.lens, src,
                                      prefill_lens=bt.lens - 1, num_fp16_pages=w.fp16_pool_pages())
    app = runtime.DecodeAppend(cache, seqs, bt.lens, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_step=True)
    assert not st.fused_step   # the one-launch step takes fp16 and INT8 storage only
    out = to_np(st.run_with_append(app, bt.q_dev)).astype(np.float64)
    torch.cuda.synchronize()
    for x, y in [(cache.k_pages, bt.cache.k_pages), (cache.v_pages, bt.cache.v_pages),
                 (cache.kv_params, bt.cache.kv_params), (cache.page_meta, bt.cache.page_meta)]:
        assert torch.equal(x, y)
    osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den,
                                            w.k_fixed, st.k_cap, nthreads=8)
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    n_tie = check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    err = float(np.abs(out - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, gsel, gcnt)).max())
    log(f"[mixed step] {w.name}: {n_tie} near-tie swaps, max abs err {err:.3g}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("hq,hkv,d", [(4, 4, 128), (8, 4, 128), (8, 2, 128), (16, 2, 128), (8, 2, 64), (4, 4, 64)],
                         ids=["g1d128", "g2d128", "g4d128", "g8d128", "g4d64", "g1d64"])
def test_mixed_group_sizes_and_head_dims(hq, hkv, d):
    """Both passes run on the matrix cores for G >= 2 and on the vector units
    for G = 1: every group size and both head dims, against the oracle."""
    from test_gpu_parity import Built, check_scores, check_selection_near_ties, score_tolerance
    w = mixed(workloads.small(5), 5).with_(name=f"mixed_{hq}x{hkv}_d{d}", num_q_heads=hq, num_kv_heads=hkv,
                                           head_dim=d)
    bt = Built(w)
    assert_storage_equal(bt.cache, bt.ocache, w.name)
    st = bt.step()
    out = to_np(st.run(bt.q_dev)).astype(np.float64)
    torch.cuda.synchronize()
    osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den,
                                            w.k_fixed, st.k_cap, nthreads=8)
    check_scores(to_np(st.scores), osc, score_tolerance(bt.ocache, bt.table, bt.lens, bt.q, w.group))
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    assert np.abs(out - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, gsel, gcnt)).max() <= ATTN_ATOL


@pytest.mark.parametrize("pool", ["all_int8", "all_fp16"])
@pytest.mark.parametrize("fused", [True, False], ids=["select_in_attention", "topk_then_attention"])
def test_mixed_with_one_pool_equals_the_single_format(pool, fused):
    """Every page in the INT8 pool (num_fp16_pages 0) or in the FP16 pool: the
    storage equals an INT8-per-token (fp16) cache's byte for byte, and the
    scores and selection of the step equal that cache's bit for bit.  The
    output too, bit for bit, for the INT8 pool (the other pass contributes
    nothing to the merge); for the FP16 pool of this query group the mixed
    cache's FP16 pass runs on the matrix cores and a plain fp16 cache on the
    vector units, so there the outputs agree to 1e-5."""
    kvq, runtime = mods()
    base = workloads.small(5)
    fmt1 = workloads.FMT_INT8_TOKEN if pool == "all_int8" else workloads.FMT_FP16
    w1 = base.with_(fmt=fmt1)
    table, n_phys = w1.block_table()
    lens = w1.seq_lens()
    src = lambda b: (w1.keys(b), w1.values(b))  # noqa: E731
    n16 = 0 if pool == "all_int8" else n_phys
    c1, s1 = runtime.build_cache(fmt1, n_phys, w1.num_kv_heads, w1.head_dim, table, lens, src)
    cm, sm = runtime.build_cache(FMT_MIXED, n_phys, w1.num_kv_heads, w1.head_dim, table, lens, src,
                                 num_fp16_pages=n16)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(cm.k_pages).view(np.uint8), to_np(c1.k_pages).reshape(-1).view(np.uint8))
    assert np.array_equal(to_np(cm.v_pages).view(np.uint8), to_np(c1.v_pages).reshape(-1).view(np.uint8))
    assert torch.equal(cm.page_meta, c1.page_meta)
    if pool == "all_int8":
        assert torch.equal(cm.kv_params, c1.kv_params)
    q = torch.from_numpy(w1.query().view(np.int16)).cuda()
    outs = []
    for c, s in ((c1, s1), (cm, sm)):
        st = runtime.DecodeStep(c, s, w1.num_q_heads, w1.ratio_num, w1.ratio_den, w1.k_fixed, fused_select=fused)
        outs.append((st.run(q).clone(), st.sel_pages.clone(), st.scores.clone()))
    torch.cuda.synchronize()
    (o1, p1, sc1), (om, pm, scm) = outs
    assert torch.equal(pm, p1)
    if pool == "all_int8":
        assert torch.equal(om, o1)
    else:
        assert (om - o1).abs().max().item() <= 1e-5
    P = (lens + PAGE - 1) // PAGE
    for b in range(len(lens)):
        assert torch.equal(scm[b, :, :P[b]], sc1[b, :, :P[b]])


@pytest.mark.parametrize("fused", [True, False], ids=["select_in_attention", "topk_then_attention"])
def test_mixed_decode_stream(fused):
    """24 decode steps on a ragged GQA batch whose recent pages are FP16: after
    every step both pools, the scale/zero bits and the metadata equal the
    oracle's build, the selection passes the near-tie rule and the output
    matches."""
    from test_gpu_parity import check_selection_near_ties
    _, runtime = mods()
    T = 24
    w = mixed(workloads.small(5), 5)
    lens_end = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    L0 = lens_end - T
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, L0, src,
                                      num_fp16_pages=w.fp16_pool_pages())
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_select=fused)
    rng = np.random.default_rng(4545)
    for t in range(T):
        lens_t = L0 + t + 1
        seqs.seq_lens.copy_(torch.from_numpy(lens_t.astype(np.int32)))
        app = runtime.DecodeAppend(cache, seqs, lens_t, src)
        q = rng.standard_normal((w.batch, w.num_q_heads, w.head_dim)).astype(np.float16)
        out = to_np(st.run_with_append(app, torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
        oc, _ = oracle.build_cache(w, upto=lens_t)
        assert_storage_equal(cache, oc, f"step {t}")
        osc, osel, ocnt, _ = oracle.decode_step(oc, table, lens_t, q, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap,
                                                nthreads=8)
        gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
        check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
        assert np.abs(out - oracle.attention(oc, table, lens_t, q, gsel, gcnt)).max() <= ATTN_ATOL, f"step {t}"


@pytest.mark.parametrize("rows", [1, 17, 64])
def test_mixed_append_paths_agree(rows):
    """kvq_append_decode, kvq_append_quant + kvq_build_page_meta and
    kvq_append_decode_scores leave the same cache (and the same scores), equal
    to the oracle's build; the rows straddle FP16 and INT8 pages."""
    kvq, runtime = mods()
    w = mixed(workloads.small(5).with_(batch=4, len_lo=70, len_hi=300), 2)
    lens = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    start = lens - rows
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    q = torch.from_numpy(w.query().view(np.int16)).cuda()
    caches, scores = [], []
    for mode in ("decode", "separate", "with_scores"):
        cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                          prefill_lens=start, num_fp16_pages=w.fp16_pool_pages())
        cnt = lens - start
        k_new = np.concatenate([w.keys(b)[start[b]:lens[b]] for b in range(w.batch)])
        v_new = np.concatenate([w.values(b)[start[b]:lens[b]] for b in range(w.batch)])
        args = (torch.from_numpy(start.astype(np.int32)).cuda(),
                torch.from_numpy(np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)).cuda(), int(cnt.max()),
                torch.from_numpy(k_new.view(np.int16)).cuda(), torch.from_numpy(v_new.view(np.int16)).cuda())
        st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
        if mode == "decode":
            kvq.kvq_append_decode(cache, seqs, *args)
            kvq.kvq_page_scores(cache, seqs, q, st.scores)
        elif mode == "separate":
            kvq.kvq_append_quant(cache, seqs, *args)
            kvq.kvq_build_page_meta(cache, seqs, torch.from_numpy((start // PAGE).astype(np.int32)).cuda(), 5)
            kvq.kvq_page_scores(cache, seqs, q, st.scores)
        else:
            kvq.kvq_append_decode_scores(cache, seqs, *args, q, st.scores)
        torch.cuda.synchronize()
        caches.append(cache)
        scores.append(st.scores.clone())
    a = caches[0]
    for c in caches[1:]:
        for x, y in [(a.k_pages, c.k_pages), (a.v_pages, c.v_pages), (a.kv_params, c.kv_params),
                     (a.page_meta, c.page_meta)]:
            assert torch.equal(x, y)
    P = (lens + PAGE - 1) // PAGE
    for s in scores[1:]:
        for b in range(w.batch):
            assert torch.equal(s[b, :, :P[b]], scores[0][b, :, :P[b]])
    oc, _ = oracle.build_cache(w)
    assert_storage_equal(a, oc, f"rows {rows}")


def test_demote_pages_matches_oracle():
    """kvq_demote_pages on full and partial pages of several sequences: both
    pools, scale/zero bits, metadata and the block table equal the oracle's
    demotion, and the step after it matches the oracle on the new cache."""
    from test_gpu_parity import check_selection_near_ties
    kvq, runtime = mods()
    w = mixed(workloads.small(5), 5).with_(spare_pages=8)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                      num_fp16_pages=w.fp16_pool_pages())
    oc, _ = oracle.build_cache(w)
    P = w.pages_per_seq()
    # sinks of every non-empty sequence but one, and one partial last page
    picks = [(b, 0) for b in range(1, w.batch) if P[b] > 0]
    last = int(np.argmax(P))
    picks.append((last, int(P[last]) - 1))
    seq = np.array([b for b, _ in picks], np.int32)
    page = np.array([j for _, j in picks], np.int32)
    dst = np.arange(n_phys - len(picks), n_phys, dtype=np.int32)
    assert all(table[b, j] < cache.num_fp16_pages for b, j in picks)
    kvq.kvq_demote_pages(cache, seqs, torch.from_numpy(seq).cuda(), torch.from_numpy(page).cuda(),
                         torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    t2 = table.copy()
    oracle.demote(oc, t2, lens, seq, page, dst)
    assert np.array_equal(to_np(seqs.block_table), t2)
    assert_storage_equal(cache, oc, "after demotion")
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    q = w.query()
    out = to_np(st.run(torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
    torch.cuda.synchronize()
    osc, osel, ocnt, _ = oracle.decode_step(oc, t2, lens, q, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    assert np.abs(out - oracle.attention(oc, t2, lens, q, gsel, gcnt)).max() <= ATTN_ATOL


def test_mixed_steep_softmax():
    """Keys and queries scaled 60x (logits in the thousands) over both pools,
    GQA (the INT8 pass on the matrix cores)."""
    kvq, runtime = mods()
    w = mixed(workloads.small(5), 5).with_(len_lo=200, len_hi=900, seed=2718)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    kv = [((w.keys(b).astype(np.float32) * 60).astype(np.float16), w.values(b)) for b in range(w.batch)]
    q = (w.query().astype(np.float32) * 60).astype(np.float16)
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, lambda b: kv[b],
                                      num_fp16_pages=w.fp16_pool_pages())
    oc = oracle.Cache(FMT_MIXED, n_phys, w.num_kv_heads, w.head_dim, w.fp16_pool_pages())
    for b in range(w.batch):
        off = np.zeros(w.batch + 1, np.int32)
        off[b + 1:] = lens[b]
        oracle.append(oc, table, np.zeros(w.batch, np.int32), off, kv[b][0], kv[b][1])
    oracle.page_meta(oc, table, lens)
    assert_storage_equal(cache, oc, "steep")
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    q_dev = torch.from_numpy(q.view(np.int16)).cuda()
    kvq.kvq_page_scores(cache, seqs, q_dev, st.scores)
    osc = oracle.page_scores(oc, table, lens, q)
    osel, ocnt = oracle.topk(osc, lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    out = to_np(st.attend(q_dev, torch.from_numpy(osel).cuda(), torch.from_numpy(ocnt).cuda()))
    err = float(np.abs(out.astype(np.float64) - oracle.attention(oc, table, lens, q, osel, ocnt)).max())
    log(f"[mixed steep] max abs err {err:.3g}")
    assert err <= ATTN_ATOL
