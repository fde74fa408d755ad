"""The one-launch decode step (kvq_decode_step) against the three-launch step
(kvq_append_decode_scores, kvq_select_decode_attn and its combine) and the
oracle, through the C ABI.

The fused kernel computes every score, selection and split with the same
arithmetic in the same order as the separate kernels, so the two paths must
agree bit for bit: codes, scale/zero and metadata after the append, every
page's score, the selection, and the output.  Its per-row counters must be
back at zero after every launch (checked by launching repeatedly on one
workspace, inside and outside a HIP graph), and its wait bound must never
trigger (the error word stays 0).
"""
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


def build(w, lens=None):
    _, runtime = mods()
    table, n_phys = w.block_table()
    lens = w.seq_lens() if lens is None else lens
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                      prefill_lens=np.maximum(lens.astype(np.int64) - 1, 0))
    app = runtime.DecodeAppend(cache, seqs, lens, src)
    return table, lens, cache, seqs, app


def error_word(st):
    return int(st.step_workspace.view(torch.int32)[1].item())


def compare_paths(w, pps=0, reps=3):
    """Build w twice; run the three-launch step on one and the fused step on
    the other (reps times); everything must agree bit for bit."""
    kvq, runtime = mods()
    q = torch.from_numpy(w.query().view(np.int16)).cuda()
    t1, lens, c1, s1, a1 = build(w)
    _, _, c2, s2, a2 = build(w)
    ref = runtime.DecodeStep(c1, s1, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, pages_per_split=pps)
    fus = runtime.DecodeStep(c2, s2, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, pages_per_split=pps,
                             fused_step=True)
    assert fus.fused_step and fus.pps == ref.pps
    out_ref = ref.run_with_append(a1, q).clone()
    outs = []
    for _ in range(reps):
        fus.sel_pages.fill_(-7)
        fus.out.fill_(float("nan"))
        outs.append(fus.run_with_append(a2, q).clone())
    torch.cuda.synchronize()
    assert error_word(fus) == 0
    ctr = to_np(fus.step_workspace.view(torch.int32)[: kvq.kvq_step_counter_bytes(s2.batch, w.num_kv_heads) // 4])
    assert ctr[0] == 0 and (ctr[2:] == 0).all(), "counters not reset"
    for x, y in [(c1.k_pages, c2.k_pages), (c1.v_pages, c2.v_pages), (c1.page_meta, c2.page_meta)]:
        assert torch.equal(x, y)
    if w.fmt != workloads.FMT_FP16:
        assert torch.equal(c1.kv_params, c2.kv_params)
    P = (lens + PAGE - 1) // PAGE
    sa, sb = to_np(ref.scores), to_np(fus.scores)
    for b in range(len(lens)):
        assert np.array_equal(sa[b, :, :P[b]], sb[b, :, :P[b]]), f"scores of sequence {b}"
    assert torch.equal(ref.sel_count, fus.sel_count) and torch.equal(ref.sel_pages, fus.sel_pages)
    for o in outs:
        assert torch.equal(o, out_ref)
    return t1, lens, c2, fus, out_ref


@pytest.mark.parametrize("kind,n", [("small", 1), ("small", 2), ("small", 4), ("small", 5), ("full", 1), ("full", 2),
                                    ("full", 4), ("full", 5)],
                         ids=["small1", "small2", "small4", "small5", "full1", "full2", "full4", "full5"])
def test_fused_step_equals_three_launches(kind, n):
    w = workloads.small(n) if kind == "small" else workloads.config(n)
    table, lens, cache, st, out = compare_paths(w)
    if kind == "small":
        oc, _ = oracle.build_cache(w)
        want = oracle.attention(oc, table, lens, w.query(), to_np(st.sel_pages), to_np(st.sel_count))
        err = float(np.abs(to_np(out).astype(np.float64) - want).max())
        log(f"[fused] {w.name}: max abs err {err:.3g}")
        assert err <= ATTN_ATOL


@pytest.mark.parametrize("pps", [1, 7, 64])
def test_fused_step_split_sizes_and_dense_ratio(pps):
    """Several split sizes on the ragged GQA batch, and ratio 1 (K = P)."""
    compare_paths(workloads.small(5), pps=pps, reps=2)
    compare_paths(workloads.small(3).with_(ratio_num=1, ratio_den=1), pps=pps, reps=2)


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (16, 2, 64), (4, 4, 64)], ids=["g4d128", "g8d64", "g1d64"])
def test_fused_step_formats_groups_dims(fmt, hq, hkv, d):
    w = workloads.small(5).with_(name=f"fused_f{fmt}_{hq}x{hkv}_d{d}", fmt=fmt, num_q_heads=hq, num_kv_heads=hkv,
                                 head_dim=d)
    compare_paths(w, reps=2)


def test_fused_step_empty_sequences():
    """Zero-length sequences inside the batch: their rows select nothing and
    their outputs are zero; the other rows equal the three-launch step."""
    kvq, runtime = mods()
    w = workloads.small(5)
    lens = w.seq_lens().copy()
    empty = [1, 3]
    q = torch.from_numpy(w.query().view(np.int16)).cuda()
    table, _, c1, s1, _ = build(w)
    lens0 = lens.copy()
    lens0[empty] = 0
    seqs = kvq.Seqs(torch.from_numpy(lens0.astype(np.int32)).cuda(), s1.block_table)
    ref = runtime.DecodeStep(c1, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    fus = runtime.DecodeStep(c1, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_step=True)
    none = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    off = torch.zeros(w.batch + 1, dtype=torch.int32, device="cuda")
    kvq.kvq_page_scores(c1, seqs, q, ref.scores)
    o_ref = ref.select_attend(q).clone()
    fus.out.fill_(float("nan"))
    kvq.kvq_decode_step(c1, seqs, none, off, 0, None, None, q, fus.scores, w.ratio_num, w.ratio_den, w.k_fixed,
                        fus.k_cap, fus.out, fus.step_workspace, fus.sm_scale, fus.pps, sel_pages=fus.sel_pages,
                        sel_count=fus.sel_count)
    torch.cuda.synchronize()
    assert error_word(fus) == 0
    assert (to_np(fus.out)[empty] == 0).all() and (to_np(fus.sel_count)[empty] == 0).all()
    assert torch.equal(fus.out, o_ref) and torch.equal(fus.sel_pages, ref.sel_pages)


def test_fused_step_graph_replays():
    """The fused step captured in a HIP graph and replayed with eager work in
    between equals its eager result every time (its counters are reset by the
    launch itself, so replays need no memset)."""
    _, runtime = mods()
    w = workloads.small(4)
    q = torch.from_numpy(w.query().view(np.int16)).cuda()
    _, _, cache, seqs, app = build(w)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_step=True)
    eager = st.run_with_append(app, q).clone()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            st.run_with_append(app, q)
    torch.cuda.current_stream().wait_stream(cap)
    for i in range(5):
        st.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, eager), f"replay {i}"
        st.run_with_append(app, q)
        torch.cuda.synchronize()
    assert error_word(st) == 0


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_fused_step_decode_stream(fmt):
    """24 consecutive fused steps on a ragged batch, each appending every
    sequence's next token with a fresh query: after every step the cache
    equals the oracle's build of the same tokens, the selection passes the
    near-tie rule and the output matches the oracle."""
    from test_gpu_parity import check_selection_near_ties
    _, runtime = mods()
    T = 24
    w = workloads.small(5).with_(fmt=fmt)
    lens_end = w.seq_lens().astype(np.int64)
    table, n_phys = w.block_table()
    L0 = lens_end - T
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, L0, src)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, fused_step=True)
    rng = np.random.default_rng(777 + fmt)
    for t in range(T):
        lens_t = L0 + t + 1
        seqs.seq_lens.copy_(torch.from_numpy(lens_t.astype(np.int32)))
        app = runtime.DecodeAppend(cache, seqs, lens_t, src)
        q = rng.standard_normal((w.batch, w.num_q_heads, w.head_dim)).astype(np.float16)
        out = to_np(st.run_with_append(app, torch.from_numpy(q.view(np.int16)).cuda())).astype(np.float64)
        oc, _ = oracle.build_cache(w, upto=lens_t)
        k = to_np(cache.k_pages)
        if fmt == workloads.FMT_FP16:
            k = k.view(np.uint16)
        assert np.array_equal(k, oc.k_pages), f"step {t}"
        if fmt != workloads.FMT_FP16:
            assert np.array_equal(to_np(cache.kv_params).view(np.uint32), oc.params.view(np.uint32)), f"step {t}"
        assert np.array_equal(to_np(cache.page_meta), oc.meta), f"step {t}"
        osc, osel, ocnt, _ = oracle.decode_step(oc, table, lens_t, q, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap,
                                                nthreads=8)
        gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
        check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
        want = oracle.attention(oc, table, lens_t, q, gsel, gcnt)
        assert np.abs(out - want).max() <= ATTN_ATOL, f"step {t}"
    assert error_word(st) == 0
