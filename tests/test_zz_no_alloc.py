"""kvq_select_decode_attn_noalloc (the variant that takes no workspace and
allocates nothing: its per-split partials live in the library's own device
scratch) against kvq_select_decode_attn with a caller's workspace, through the
C ABI: two calls in a row, the second on a smaller batch, each bit-identical
to the workspace call and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

ATTN_ATOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_quantized_sparse_amd as kvq
    kvq.lib()


def _case(w):
    import paged_quantized_sparse_amd as kvq
    from paged_quantized_sparse_amd import runtime
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src)
    q = w.query()
    q_dev = torch.from_numpy(q.view(np.int16)).cuda()
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
    kvq.kvq_page_scores(cache, seqs, q_dev, st.scores)
    return kvq, table, lens, cache, seqs, q, q_dev, st


def _noalloc_vs_workspace(w):
    kvq, table, lens, cache, seqs, q, q_dev, st = _case(w)
    need = kvq.kvq_attn_workspace_bytes(seqs.batch, w.num_q_heads, w.head_dim, seqs.max_pages, st.k_cap, st.pps)
    assert 0 < need <= kvq.NOALLOC_SCRATCH_BYTES
    ref = st.select_attend(q_dev).clone()
    ref_sel, ref_cnt = st.sel_pages.clone(), st.sel_count.clone()
    out = torch.full_like(st.out, float("nan"))
    sel = torch.full_like(st.sel_pages, -7)
    cnt = torch.full_like(st.sel_count, -7)
    rn, rd, kf = st.ratio
    kvq.kvq_select_decode_attn_noalloc(cache, seqs, q_dev, st.scores, rn, rd, kf, st.k_cap, out, st.sm_scale,
                                       st.pps, sel_pages=sel, sel_count=cnt)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref_sel) and torch.equal(cnt, ref_cnt)
    assert torch.equal(out, ref)
    oc, _ = oracle.build_cache(w)
    want = oracle.attention(oc, table, lens, q, sel.cpu().numpy(), cnt.cpu().numpy())
    err = float(np.abs(out.cpu().numpy().astype(np.float64) - want).max())
    print(f"[noalloc] {w.name}: {need} scratch bytes, max abs err {err:.3g}", flush=True)
    assert err <= ATTN_ATOL
    return need


def test_noalloc_two_calls_second_smaller():
    big = workloads.small(4).with_(name="noalloc_big", num_q_heads=16, num_kv_heads=16, seq_len=20000)
    small = workloads.small(5)
    n1 = _noalloc_vs_workspace(big)
    n2 = _noalloc_vs_workspace(small)
    assert n2 < n1


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import paged_quantized_sparse_amd as kvq
    w = workloads.small(4)
    kvq_, table, lens, cache, seqs, q, q_dev, st = _case(w)
    B = 2048   # a batch whose partials need far more than the scratch holds
    big_lens = torch.ones(B, dtype=torch.int32, device="cuda")
    big_table = torch.zeros((B, seqs.max_pages), dtype=torch.int32, device="cuda")
    big = kvq.Seqs(big_lens, big_table)
    need = kvq.kvq_attn_workspace_bytes(B, w.num_q_heads, w.head_dim, seqs.max_pages, st.k_cap, 1)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    scores = torch.zeros((B, w.num_kv_heads, seqs.max_pages), dtype=torch.float32, device="cuda")
    out = torch.zeros((B, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    rn, rd, kf = st.ratio
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_select_decode_attn_noalloc(cache, big, torch.zeros((B, w.num_q_heads, w.head_dim),
                                                                   dtype=torch.int16, device="cuda"),
                                           scores, rn, rd, kf, st.k_cap, out, st.sm_scale, 1)
    assert e.value.status == 3
