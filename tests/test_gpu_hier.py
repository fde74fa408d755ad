"""GPU parity of the coarse-then-fine selection against the oracle, through
the C ABI: super-page boxes (bit-exact), coarse scores (1e-4 relative), the
kept super-pages (exact on identical scores, near-tie rule end to end), the
masked fine scores (-inf pattern exact, kept scores bit-equal to
kvq_page_scores), and the whole step's output (2e-3), also across a decode
stream that refreshes the boxes of the super-pages the new tokens touch."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import PAGE

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


def setup(w, group, keep):
    _, runtime = mods()
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    hs = runtime.HierStep(st, group, keep)
    hs.build()
    torch.cuda.synchronize()
    oc, _ = oracle.build_cache(w)
    return table, lens, cache, seqs, st, hs, oc


CASES = [("small", 2, 8, 3), ("small", 4, 8, 40), ("small", 5, 4, 5), ("small", 5, 1, 9), ("full", 2, 8, 51),
         ("full", 4, 8, 128), ("full", 4, 16, 40)]
IDS = [f"{k}{n}_g{g}_keep{kp}" for k, n, g, kp in CASES]


@pytest.mark.parametrize("kind,n,group,keep", CASES, ids=IDS)
def test_coarse_boxes_scores_and_kept_super_pages(kind, n, group, keep):
    from test_gpu_parity import check_scores, score_tolerance
    kvq, _ = mods()
    w = workloads.small(n) if kind == "small" else workloads.config(n)
    table, lens, cache, seqs, st, hs, oc = setup(w, group, keep)
    view, ctable, clens = oracle.coarse_view(oc, table, lens, group)
    assert np.array_equal(to_np(hs.coarse_lens), clens)
    assert np.array_equal(to_np(hs.coarse_table), ctable)
    got = to_np(hs.coarse)
    Pc = clens // PAGE
    for b in range(w.batch):
        rows = slice(b * hs.pc_max, b * hs.pc_max + int(Pc[b]))
        assert np.array_equal(got[rows], view.meta[rows]), f"boxes of sequence {b}"   # == treats +0 and -0 alike
    q = w.query()
    q_dev = torch.from_numpy(q.view(np.int16)).cuda()
    kvq.kvq_page_scores(hs.coarse_cache, hs.coarse_seqs, q_dev, hs.coarse_scores)
    want = oracle.page_scores(view, ctable, clens, q)
    check_scores(to_np(hs.coarse_scores), want, score_tolerance(view, ctable, clens, q, w.group))
    # kept super-pages on identical scores: exact
    sc32 = want.astype(np.float32)
    hs.coarse_scores.copy_(torch.from_numpy(sc32))
    kvq.kvq_topk_pages(hs.coarse_scores, hs.coarse_seqs, w.num_kv_heads, 0, 1, hs.kc, hs.sel_super,
                       hs.sel_super_count)
    osel, ocnt = oracle.topk(sc32.astype(np.float64), clens, 0, 1, hs.kc, hs.kc)
    assert np.array_equal(to_np(hs.sel_super), osel) and np.array_equal(to_np(hs.sel_super_count), ocnt)
    # masked fine scores on that selection: -inf exactly where the oracle
    # masks, kept pages bit-equal to kvq_page_scores
    kvq.kvq_page_scores(cache, seqs, q_dev, st.scores)
    full = to_np(st.scores).copy()
    st.scores.fill_(float("nan"))
    kvq.kvq_page_scores_masked(cache, seqs, q_dev, group, hs.sel_super, hs.sel_super_count, st.scores)
    masked = to_np(st.scores)
    omask = oracle.mask_scores(np.zeros_like(full, dtype=np.float64), group, osel, ocnt)
    P = (lens + PAGE - 1) // PAGE
    for b in range(w.batch):
        neg = np.isneginf(omask[b]) | (np.arange(seqs.max_pages)[None] >= P[b])
        assert np.array_equal(np.isneginf(masked[b]), neg), f"mask of sequence {b}"
        assert np.array_equal(masked[b][~neg], full[b][~neg])
    log(f"[hier] {w.name} group {group} keep {keep}: kept {int(ocnt.sum())} super-pages of {int(Pc.sum()) * w.num_kv_heads}")


@pytest.mark.parametrize("kind,n,group,keep", CASES, ids=IDS)
def test_hier_step_end_to_end(kind, n, group, keep):
    """The whole coarse-then-fine step: the kept super-pages pass the
    near-tie rule on the oracle's coarse scores; the oracle's fine scores
    masked by the GPU's kept super-pages give a top-K the GPU's selection
    matches up to near-ties; the output matches the oracle's attention over
    the GPU's selection."""
    from test_gpu_parity import check_selection_near_ties
    w = workloads.small(n) if kind == "small" else workloads.config(n)
    table, lens, cache, seqs, st, hs, oc = setup(w, group, keep)
    q = w.query()
    out = to_np(hs.run(torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
    torch.cuda.synchronize()
    csc, csel, ccnt, *_ = oracle.hier_select(oc, table, lens, q, group, hs.kc, w.ratio_num, w.ratio_den, w.k_fixed,
                                             st.k_cap)
    _, _, clens = oracle.coarse_view(oc, table, lens, group)
    gcs, gcc = to_np(hs.sel_super), to_np(hs.sel_super_count)
    n_tie = check_selection_near_ties(gcs, gcc, csc, csel, ccnt)
    masked = oracle.mask_scores(oracle.page_scores(oc, table, lens, q), group, gcs, gcc)
    osel, ocnt = oracle.topk(masked, lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    n_tie += check_selection_near_ties(gsel, gcnt, masked, osel, ocnt)
    want = oracle.attention(oc, table, lens, q, gsel, gcnt)
    err = float(np.abs(out - want).max())
    log(f"[hier step] {w.name} group {group} keep {keep}: {n_tie} near-tie swaps, max abs err {err:.3g}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_hier_decode_stream(fmt):
    """12 decode steps, each appending every sequence's next token and
    refreshing the boxes of the super-pages it touches: boxes equal the
    oracle's after every step, and the step matches the oracle."""
    from test_gpu_parity import check_selection_near_ties
    _, runtime = mods()
    T, group, keep = 12, 4, 4
    w = workloads.small(5).with_(fmt=fmt)
    lens_end = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    L0 = lens_end - T
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, L0, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    hs = runtime.HierStep(st, group, keep)
    hs.build()
    rng = np.random.default_rng(99 + fmt)
    for t in range(T):
        lens_t = L0 + t + 1
        seqs.seq_lens.copy_(torch.from_numpy(lens_t.astype(np.int32)))
        app = runtime.DecodeAppend(cache, seqs, lens_t, src)
        super_begin = torch.from_numpy(((app.page_begin.cpu().numpy()) // group).astype(np.int32)).cuda()
        q = rng.standard_normal((w.batch, w.num_q_heads, w.head_dim)).astype(np.float16)
        out = to_np(hs.run_with_append(app, super_begin, torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
        oc, _ = oracle.build_cache(w, upto=lens_t)
        view, ctable, clens = oracle.coarse_view(oc, table, lens_t, group)
        got = to_np(hs.coarse)
        Pc = clens // PAGE
        for b in range(w.batch):
            rows = slice(b * hs.pc_max, b * hs.pc_max + int(Pc[b]))
            assert np.array_equal(got[rows], view.meta[rows]), f"step {t}: boxes of sequence {b}"
        gcs, gcc = to_np(hs.sel_super), to_np(hs.sel_super_count)
        masked = oracle.mask_scores(oracle.page_scores(oc, table, lens_t, q), group, gcs, gcc)
        osel, ocnt = oracle.topk(masked, lens_t, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
        gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
        check_selection_near_ties(gsel, gcnt, masked, osel, ocnt)
        want = oracle.attention(oc, table, lens_t, q, gsel, gcnt)
        assert np.abs(out - want).max() <= ATTN_ATOL, f"step {t}"
