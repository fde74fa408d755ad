"""Randomized shapes through the whole step, against the oracle, through the C ABI.

Each case draws (seeded) a storage format, head_dim, query-group size, batch,
ragged lengths (1 token to ~90 pages, never multiples of 16 or 64 on purpose),
a selection rule (ratio or fixed K, sometimes every page), a split size, and
either the in-kernel or the two-call selection, then checks:
  * the cache after prefill + decode-time append equals the oracle's build
    (storage bytes, scale/zero bits, metadata);
  * the selection passes the near-tie rule and the output is within 2e-3 of
    the oracle's attention over it;
  * the same step at another split size gives the same selection and an output
    within 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import PAGE

pytestmark = pytest.mark.gpu

ATTN_ATOL = 2e-3
N_CASES = 24


def log(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_quantized_sparse_amd as kvq
    kvq.lib()


def draw(i):
    rng = np.random.default_rng(90210 + i)
    fmt = int(rng.choice([0, 1, 2, 3, 4, 5]))
    d = 128 if fmt in (3, 4) else int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 7))
    lo = int(rng.integers(1, 400))
    hi = lo + int(rng.integers(0, 1100))
    kind = int(rng.choice([0, 0, 0, 1, 1, 2]))  # ratio, fixed K, every page
    rn, rd, kf = ((int(rng.integers(1, 6)), 10, 0) if kind == 0 else
                  (0, 1, int(rng.integers(1, 40))) if kind == 1 else (1, 1, 0))
    w = workloads.small(5).with_(name=f"rand{i}_f{fmt}_d{d}_g{G}x{hkv}_b{B}", seed=5000 + i, fmt=fmt, head_dim=d,
                                 num_q_heads=G * hkv, num_kv_heads=hkv, batch=B, len_lo=lo, len_hi=hi,
                                 ratio_num=rn, ratio_den=rd, k_fixed=kf, hot_recent=int(rng.integers(1, 8)),
                                 outlier_channels=int(rng.choice([0, d // 16])))
    pps = [0, 1, 5, 16, 64][int(rng.integers(0, 5))]
    fused = bool(rng.integers(0, 2))
    return w, pps, fused


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_step(i):
    from test_gpu_parity import Built, check_selection_near_ties
    w, pps, fused = draw(i)
    log(f"[rand] case {i}: {w.name} lens U[{w.len_lo}, {w.len_hi}] rule {w.ratio_num}/{w.ratio_den} k={w.k_fixed} "
        f"pps {pps} in-kernel selection {fused}")
    bt = Built(w)
    oc = bt.ocache
    k = bt.cache.k_pages.cpu().numpy()
    assert np.array_equal(k.view(np.uint16) if w.fmt == workloads.FMT_FP16 else k, oc.k_pages)
    if w.fmt != workloads.FMT_FP16:
        assert np.array_equal(bt.cache.kv_params.cpu().numpy().view(np.uint32), oc.params.view(np.uint32))
    assert np.array_equal(bt.cache.page_meta.cpu().numpy(), oc.meta)
    st = bt.step(pages_per_split=pps, fused_select=fused, dense=w.is_dense())
    out = st.run(bt.q_dev).cpu().numpy().astype(np.float64)
    if w.is_dense():
        want = oracle.attention(oc, bt.table, bt.lens, bt.q)
    else:
        osc, osel, ocnt, _ = oracle.decode_step(oc, bt.table, bt.lens, bt.q, w.ratio_num, w.ratio_den, w.k_fixed,
                                                st.k_cap, nthreads=8)
        gsel, gcnt = st.sel_pages.cpu().numpy(), st.sel_count.cpu().numpy()
        check_selection_near_ties(gsel, gcnt, osc, osel, ocnt)
        want = oracle.attention(oc, bt.table, bt.lens, bt.q, gsel, gcnt)
    err = float(np.abs(out - want).max())
    assert err <= ATTN_ATOL, f"max abs err {err}"
    other = bt.step(pages_per_split=7 if pps != 7 else 3, fused_select=fused, dense=w.is_dense())
    out2 = other.run(bt.q_dev).cpu().numpy().astype(np.float64)
    if not w.is_dense():
        assert torch.equal(other.sel_pages, st.sel_pages)
    assert np.abs(out2 - out).max() <= 1e-5
    P = (bt.lens + PAGE - 1) // PAGE
    log(f"[rand] case {i}: {int(P.sum())} pages, max abs err {err:.3g}")
