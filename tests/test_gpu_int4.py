"""GPU parity of the 4-bit formats (per token and per 64-token group, codes
0..15, two per byte) against the oracle, through the C ABI.

The bars are those of the 8-bit formats: codes, the bits of every scale and
zero-point and the page metadata bit-exact (bulk append, decode-time append,
the fused append + scores, and edge rows); page scores to 1e-4; top-K exact on
identical scores, near-tie rule on its own; attention within 2e-3 of fp64 on
the oracle's selection and on the GPU's; the in-kernel selection equal, bit
for bit, to top-K then attention.  4-bit storage is built for head_dim 128;
its attention runs on the vector units for one query head per KV head and on
the matrix cores for query groups (2, 4 and 8 heads), all covered here.  The
one-launch step does not take 4-bit storage and says so.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import FMT_INT4_GROUP64, FMT_INT4_TOKEN, PAGE

pytestmark = pytest.mark.gpu

ATTN_ATOL = 2e-3
FMTS = [FMT_INT4_TOKEN, FMT_INT4_GROUP64]
FMT_IDS = ["int4tok", "int4grp"]


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


# small ragged workloads (head_dim 128) and the 32K-token INT8 layer with 4-bit storage
CASES = [("small", 3), ("small", 4), ("small", 5), ("full", 4)]
CASE_IDS = [f"{k}{n}" for k, n in CASES]

_BUILT = {}


def built(kind, n, fmt):
    from test_gpu_parity import Built
    key = (kind, n, fmt)
    if key not in _BUILT:
        w = workloads.small(n) if kind == "small" else workloads.config(n)
        _BUILT[key] = Built(w.with_(name=f"{w.name}_as_{workloads.FORMAT_NAMES[fmt]}", fmt=fmt))
    return _BUILT[key]


def assert_storage_equal(cache, oc, what):
    assert np.array_equal(to_np(cache.k_pages), oc.k_pages), f"{what}: K codes"
    assert np.array_equal(to_np(cache.v_pages), oc.v_pages), f"{what}: V codes"
    p = to_np(cache.kv_params).view(np.uint32)
    assert np.array_equal(p, oc.params.view(np.uint32)), f"{what}: scale/zero bits"
    assert np.array_equal(to_np(cache.page_meta), oc.meta), f"{what}: metadata"   # == treats +0 and -0 alike


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("kind,n", CASES, ids=CASE_IDS)
def test_int4_build_bit_exact(kind, n, fmt):
    """Prefill of L-1 tokens (bulk append + metadata), then the decode-time
    append of the last token: codes, scale/zero bits and metadata equal the
    oracle's one-shot build."""
    bt = built(kind, n, fmt)
    assert tuple(bt.cache.k_pages.shape[-1:]) == (bt.w.head_dim // 2,)
    assert_storage_equal(bt.cache, bt.ocache, bt.w.name)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("kind,n", CASES, ids=CASE_IDS)
def test_int4_scores_topk_and_attention(kind, n, fmt):
    """Page scores within tolerance; top-K on identical scores exact;
    attention on the oracle's selection (or every page, ratio 1) within 2e-3."""
    from test_gpu_parity import check_scores, score_tolerance
    kvq, _ = mods()
    bt = built(kind, n, fmt)
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
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, osel, ocnt)
    err = float(np.abs(to_np(out).astype(np.float64) - want).max())
    dense = to_np(bt.step(dense=True).attend(bt.q_dev)).astype(np.float64)
    derr = float(np.abs(dense - oracle.attention(bt.ocache, bt.table, bt.lens, bt.q)).max())
    log(f"[int4 attn] {w.name}: max abs err {err:.3g} (selected), {derr:.3g} (every page)")
    assert err <= ATTN_ATOL and derr <= ATTN_ATOL


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("kind,n", CASES, ids=CASE_IDS)
def test_int4_select_attention_and_step(kind, n, fmt):
    """The in-kernel selection equals top-K then attention bit for bit at
    several split sizes; the whole step (append fused into scoring, then the
    selecting attention) passes the near-tie rule and matches the oracle."""
    from test_gpu_parity import _select_vs_separate, check_selection_near_ties
    kvq, runtime = mods()
    bt = built(kind, n, fmt)
    w = bt.w
    for pps in ([0, 1, 3, 64] if kind == "small" else [0, 16]):
        sep = bt.step(pages_per_split=pps, fused_select=False)
        kvq.kvq_page_scores(bt.cache, bt.seqs, bt.q_dev, sep.scores)
        fus = bt.step(pages_per_split=pps)
        out_sep, out_fus = _select_vs_separate(sep, fus, bt.q_dev)
        assert torch.equal(fus.sel_count, sep.sel_count) and torch.equal(fus.sel_pages, sep.sel_pages), pps
        assert torch.equal(out_fus, out_sep), pps
    # the whole step from a cache one token short
    table, n_phys = w.block_table()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(fmt, n_phys, w.num_kv_heads, w.head_dim, table, bt.lens, src,
                                      prefill_lens=bt.lens - 1)
    app = runtime.DecodeAppend(cache, seqs, bt.lens, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_step=True)
    assert not st.fused_step   # 4-bit storage takes the three-launch step
    out = to_np(st.run_with_append(app, bt.q_dev)).astype(np.float64)
    torch.cuda.synchronize()
    for x, y in [(cache.k_pages, bt.cache.k_pages), (cache.v_pages, bt.cache.v_pages),
                 (cache.kv_params, bt.cache.kv_params), (cache.page_meta, bt.cache.page_meta)]:
        assert torch.equal(x, y)
    osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den,
                                            w.k_fixed, st.k_cap, nthreads=8)
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    n_tie = check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, gsel, gcnt)
    err = float(np.abs(out - want).max())
    log(f"[int4 step] {w.name}: {n_tie} near-tie swaps, max abs err {err:.3g}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (16, 2)], ids=["g1", "g2", "g4", "g8"])
def test_int4_group_sizes(fmt, hq, hkv):
    """Every group size (1 on the vector units, 2, 4 and 8 on the matrix
    cores): scores, the selecting step and the output against the oracle."""
    from test_gpu_parity import Built, check_scores, check_selection_near_ties, score_tolerance
    kvq, _ = mods()
    w = workloads.small(5).with_(name=f"int4_f{fmt}_{hq}x{hkv}", fmt=fmt, num_q_heads=hq, num_kv_heads=hkv)
    bt = Built(w)
    st = bt.step()
    out = to_np(st.run(bt.q_dev)).astype(np.float64)
    torch.cuda.synchronize()
    osc, osel, ocnt, _ = oracle.decode_step(bt.ocache, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den,
                                            w.k_fixed, st.k_cap, nthreads=8)
    check_scores(to_np(st.scores), osc, score_tolerance(bt.ocache, bt.table, bt.lens, bt.q, w.group))
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
    want = oracle.attention(bt.ocache, bt.table, bt.lens, bt.q, gsel, gcnt)
    assert np.abs(out - want).max() <= ATTN_ATOL


@pytest.mark.parametrize("decode", [False, True], ids=["bulk", "decode"])
def test_int4_token_edge_rows_bit_exact(decode):
    """4-bit per token on every edge row (constant rows, signed-zero minima,
    subnormals, +-65504, .5 ties): codes, scale/zero bits and metadata equal
    the oracle's, by the bulk and by the decode-time append."""
    from test_gpu_edges import edge_tokens, gpu_cache, oracle_prefill
    H, d, fmt = 2, 128, FMT_INT4_TOKEN
    lens = np.array([45, 23], np.int64)
    kv = [edge_tokens(int(lens[0]), H, d, 0), edge_tokens(int(lens[1]), H, d, 11)]
    P = (lens + PAGE - 1) // PAGE
    n_phys = int(P.sum()) + 1
    table = np.full((2, int(P.max())), -1, np.int32)
    perm = np.random.default_rng(2).permutation(n_phys)
    table[0, :P[0]] = perm[:P[0]]
    table[1, :P[1]] = perm[P[0]:P[0] + P[1]]
    cache, _ = gpu_cache(fmt, n_phys, H, d, table, lens, kv, [17, 5] if decode else [0, 0])
    oc = oracle_prefill(fmt, n_phys, H, d, table, lens, kv)
    assert_storage_equal(cache, oc, f"int4 token decode={decode}")
    assert not np.any(to_np(cache.kv_params).view(np.uint32)[..., 1::2] == 0x80000000), "a -0 zero-point"


@pytest.mark.parametrize("decode", [False, True], ids=["bulk", "decode"])
def test_int4_group_edge_groups_bit_exact(decode):
    """4-bit per 64-token group where each group's min/max is an edge case,
    with a partial trailing group; the decode path re-supplies the open group."""
    from test_gpu_edges import edge_groups, gpu_cache, oracle_prefill
    H, d, fmt = 2, 128, FMT_INT4_GROUP64
    lens = np.array([64 * 20 + 37, 64 * 3 + 1], np.int64)
    kv = [edge_groups(int(lens[0]), H, d), edge_groups(int(lens[1]), H, d)]
    kv[1] = (kv[1][0][:, ::-1].copy(), kv[1][1])
    P = (lens + PAGE - 1) // PAGE
    n_phys = int(P.sum())
    table = np.full((2, int(P.max())), -1, np.int32)
    perm = np.random.default_rng(3).permutation(n_phys)
    table[0, :P[0]] = perm[:P[0]]
    table[1, :P[1]] = perm[P[0]:]
    rows = [int(lens[b] - (lens[b] - 1) // 64 * 64) for b in range(2)] if decode else [0, 0]
    cache, _ = gpu_cache(fmt, n_phys, H, d, table, lens, kv, rows)
    oc = oracle_prefill(fmt, n_phys, H, d, table, lens, kv)
    assert_storage_equal(cache, oc, f"int4 group decode={decode}")


def test_int4_golden_rows_on_the_gpu():
    """The worked 4-bit rows of the golden file, written as one token each by
    the bulk append: the GPU stores exactly the printed bytes, scale and zero."""
    import json
    import os
    kvq, runtime = mods()
    rows = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                       "quant_rows_int4.json")))["rows"]
    for r in rows:
        x = np.zeros(128, np.float16)
        x[:len(r["x"])] = r["x"]
        x[len(r["x"]):] = r["x"][0]   # padding repeats a present value: min and max unchanged
        k = x.reshape(1, 1, 128)
        table = np.array([[0]], np.int32)
        cache, _ = runtime.build_cache(FMT_INT4_TOKEN, 1, 1, 128, table, np.array([1]), lambda b: (k, k))
        torch.cuda.synchronize()
        codes = to_np(cache.k_pages)[0, 0, 0]
        nb = len(r["bytes"])
        assert codes[:nb].tolist() == r["bytes"], r["x"]
        p = to_np(cache.kv_params)[0, 0, 0]
        assert float(p[0]) == r["scale"] and float(p[1]) == r["zero"], r["x"]


@pytest.mark.parametrize("fused", [True, False], ids=["select_in_attention", "topk_then_attention"])
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_int4_decode_stream(fmt, fused):
    """24 consecutive decode steps on a ragged GQA batch, each appending every
    sequence's next token (the group format re-supplies its open group) with a
    fresh query: after every step the cache equals the oracle's build of the
    same tokens, the selection passes the near-tie rule and the output matches."""
    from test_gpu_parity import check_selection_near_ties
    _, runtime = mods()
    T = 24
    w = workloads.small(5).with_(fmt=fmt)
    lens_end = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    L0 = lens_end - T
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(fmt, n_phys, w.num_kv_heads, w.head_dim, table, L0, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_select=fused)
    rng = np.random.default_rng(4343 + fmt)
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
        want = oracle.attention(oc, table, lens_t, q, gsel, gcnt)
        assert np.abs(out - want).max() <= ATTN_ATOL, f"step {t}"


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("rows", [1, 17, 64])
def test_int4_append_decode_equals_separate_calls_and_oracle(fmt, rows):
    """kvq_append_decode equals kvq_append_quant + kvq_build_page_meta and the
    oracle's one-shot build; kvq_append_decode_scores leaves the same cache and
    writes the scores kvq_page_scores writes, bit for bit."""
    kvq, runtime = mods()
    w = workloads.small(5).with_(fmt=fmt, batch=4, len_lo=70, len_hi=300)
    lens = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    start = (lens - 1) // 64 * 64 if fmt == FMT_INT4_GROUP64 else lens - rows
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    q = torch.from_numpy(w.query().view(np.int16)).cuda()
    caches, scores = [], []
    for mode in ("decode", "separate", "with_scores"):
        cache, seqs = runtime.build_cache(fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                          prefill_lens=start)
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
    for b in caches[1:]:
        for x, y in [(a.k_pages, b.k_pages), (a.v_pages, b.v_pages), (a.kv_params, b.kv_params),
                     (a.page_meta, b.page_meta)]:
            assert torch.equal(x, y)
    P = (lens + PAGE - 1) // PAGE
    for s in scores[1:]:
        for b in range(w.batch):
            assert torch.equal(s[b, :, :P[b]], scores[0][b, :, :P[b]])
    oc, _ = oracle.build_cache(w)
    assert_storage_equal(a, oc, f"rows {rows}")


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
def test_int4_steep_softmax(fmt):
    """Keys and queries scaled 60x (logits in the thousands)."""
    from test_gpu_edges import Scaled
    kvq, runtime = mods()
    s = Scaled(fmt, 8, 2, 128, 60.0, 314 + fmt)
    st = runtime.DecodeStep(s.cache, s.seqs, 8, s.w.ratio_num, s.w.ratio_den, s.w.k_fixed)
    kvq.kvq_page_scores(s.cache, s.seqs, s.q_dev, st.scores)
    osc = oracle.page_scores(s.oc, s.table, s.lens, s.q)
    osel, ocnt = oracle.topk(osc, s.lens, s.w.ratio_num, s.w.ratio_den, s.w.k_fixed, st.k_cap)
    out = to_np(st.attend(s.q_dev, torch.from_numpy(osel).cuda(), torch.from_numpy(ocnt).cuda()))
    want = oracle.attention(s.oc, s.table, s.lens, s.q, osel, ocnt)
    err = float(np.abs(out.astype(np.float64) - want).max())
    log(f"[int4 steep] fmt {fmt}: max abs err {err:.3g}")
    assert err <= ATTN_ATOL


def test_int4_hier_step():
    """The coarse-then-fine selection over 4-bit storage (it reads only page
    metadata, so it is format-blind): the output matches the oracle's
    attention over the GPU's selection, which passes the near-tie rule."""
    from test_gpu_parity import check_selection_near_ties
    _, runtime = mods()
    w = workloads.small(5).with_(fmt=FMT_INT4_GROUP64)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    hs = runtime.HierStep(st, 4, 5)
    hs.build()
    q = w.query()
    out = to_np(hs.run(torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
    torch.cuda.synchronize()
    oc, _ = oracle.build_cache(w)
    gcs, gcc = to_np(hs.sel_super), to_np(hs.sel_super_count)
    masked = oracle.mask_scores(oracle.page_scores(oc, table, lens, q), 4, gcs, gcc)
    osel, ocnt = oracle.topk(masked, lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    check_selection_near_ties(gsel, gcnt, masked, osel, ocnt)
    assert np.abs(out - oracle.attention(oc, table, lens, q, gsel, gcnt)).max() <= ATTN_ATOL


def test_int4_rejected_where_not_built():
    """head_dim 64 with 4-bit storage, and the one-launch step on 4-bit
    storage, are refused with KVQ_ERR_UNSUPPORTED before any launch."""
    kvq, runtime = mods()
    w = workloads.small(5).with_(fmt=FMT_INT4_TOKEN)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    cache64 = kvq.PagedCache.empty(FMT_INT4_TOKEN, n_phys, w.num_kv_heads, 64)
    seqs = kvq.Seqs(torch.from_numpy(lens.astype(np.int32)).cuda(), torch.from_numpy(table).cuda())
    scores = torch.empty((w.batch, w.num_kv_heads, table.shape[1]), dtype=torch.float32, device="cuda")
    q = torch.zeros((w.batch, w.num_q_heads, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_page_scores(cache64, seqs, q, scores)
    assert e.value.status == 2
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    ws = torch.zeros(kvq.kvq_step_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                  table.shape[1], st.k_cap, st.pps) // 4 + 64,
                     dtype=torch.float32, device="cuda")
    none = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    off = torch.zeros(w.batch + 1, dtype=torch.int32, device="cuda")
    qd = torch.from_numpy(w.query().view(np.int16)).cuda()
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_step(cache, seqs, none, off, 0, None, None, qd, st.scores, w.ratio_num, w.ratio_den,
                            w.k_fixed, st.k_cap, st.out, ws, st.sm_scale, st.pps)
    assert e.value.status == 2
