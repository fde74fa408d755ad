"""GPU parity on the method's edge cases, through the C ABI, against the oracle.

Quantization is graded bit for bit (codes and the bits of every scale and
zero-point), so the GPU sees here the rows where a kernel could plausibly take
another branch than the oracle: constant rows (scale 1, all codes 0), values
that land exactly on .5 after scaling (round half to even), rows whose minimum
is a zero of either sign, fp16 subnormals and the fp16 extremes +-65504.  Both
write paths run: the bulk append (kvq_append_quant + kvq_build_page_meta) and
the decode-time append of the newest rows (kvq_append_decode).

Attention is checked where the softmax is steep (keys and queries scaled up
60x, logits in the thousands) on the vector and the matrix-core forms, where a
lazy running max or a cancelling dequantization could lose accuracy.

Also: a split longer than 256 pages (a wave with more than 64 pages) through
both selection paths, a workspace filled with NaN and -inf before the call,
config 3 through the selecting pipeline with K = P, and every sequence of
config 5 at full size in the benchmark's launch configuration.
"""
import functools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import PAGE

pytestmark = pytest.mark.gpu

ATTN_ATOL = 2e-3
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


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


def dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


def f16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float16).view(np.int16)).cuda()


# ------------------------------------------------------------ edge rows
def edge_rows(d: int) -> list[np.ndarray]:
    """fp16 rows of d values, each one quantization edge case."""
    rows = []
    for r in json.load(open(os.path.join(GOLDEN, "quant_rows.json")))["rows"]:
        rows.append(np.resize(np.array(r["x"], np.float16), d))        # exact .5 ties, constant row
    pz, nz = np.float16(0.0), np.float16(-0.0)
    rows.append(np.full(d, 0.7, np.float16))                            # constant
    rows.append(np.full(d, nz, np.float16))                             # constant -0
    rows.append(np.full(d, pz, np.float16))                             # constant +0
    r = np.resize(np.array([pz, nz, 1.0, 2.5, 3.0], np.float16), d)     # min: +0 first, -0 present
    rows.append(r)
    r = np.resize(np.array([nz, pz, 7.0, 0.25], np.float16), d)         # min: -0 first, +0 present
    rows.append(r)
    r = np.resize(np.array([nz, 5.0, 9.0], np.float16), d)              # min -0 only
    rows.append(r)
    sub = (np.arange(d, dtype=np.int64) % 1024).astype(np.uint16).view(np.float16)  # subnormals and 0
    rows.append(sub.copy())
    rows.append((-sub).astype(np.float16))
    rows.append(np.resize(np.array([np.float16(2.0 ** -24), np.float16(3 * 2.0 ** -24)], np.float16), d))
    big = np.resize(np.array([-65504.0, 65504.0, 0.0, 1.0, -3.5, 65472.0], np.float16), d)
    rows.append(big)
    rows.append(np.full(d, 65504.0, np.float16))
    rows.append(np.full(d, -65504.0, np.float16))
    rows.append(np.resize(np.array([-65504.0, -65472.0, -65440.0], np.float16), d))
    rng = np.random.default_rng(5)
    rows.append(rng.standard_normal(d).astype(np.float16))
    return rows


def edge_tokens(n_tokens: int, H: int, d: int, salt: int):
    """K and V [n][H][d] fp16 filled with the edge rows, K and V apart."""
    rows = edge_rows(d)
    n = len(rows)
    k = np.empty((n_tokens, H, d), np.float16)
    v = np.empty((n_tokens, H, d), np.float16)
    for t in range(n_tokens):
        for h in range(H):
            k[t, h] = rows[(t * H + h + salt) % n]
            v[t, h] = rows[(t * H + h + 3 * salt + 5) % n]
    return k, v


def edge_groups(n_tokens: int, H: int, d: int):
    """K and V [n][H][d] for per-64-token-group storage: each group of 64
    tokens is built from one edge row, so the group's own min/max is the
    edge case (constant groups, signed-zero minima, subnormals, extremes)."""
    rows = edge_rows(d)
    n = len(rows)
    k = np.empty((n_tokens, H, d), np.float16)
    v = np.empty((n_tokens, H, d), np.float16)
    for t in range(n_tokens):
        g = t // 64
        for h in range(H):
            base_k = rows[(g * H + h) % n]
            base_v = rows[(g * H + h + 7) % n]
            k[t, h] = np.roll(base_k, t % 5)
            v[t, h] = np.roll(base_v, t % 3)
    return k, v


def oracle_prefill(fmt, n_phys, H, d, table, lens, kv):
    oc = oracle.Cache(fmt, n_phys, H, d)
    B = len(lens)
    for b in range(B):
        L = int(lens[b])
        sp = np.zeros(B, np.int32)
        off = np.zeros(B + 1, np.int32)
        off[b + 1:] = L
        oracle.append(oc, table, sp, off, kv[b][0][:L], kv[b][1][:L])
    oracle.page_meta(oc, table, lens)
    return oc


def gpu_cache(fmt, n_phys, H, d, table, lens, kv, decode_rows):
    """Prefill sequence b with its first lens[b] - decode_rows[b] tokens by
    kvq_append_quant + kvq_build_page_meta, then append the rest with
    kvq_append_decode (0 rows: prefill only)."""
    kvq, runtime = mods()
    src = lambda b: kv[b]  # noqa: E731
    lens = np.asarray(lens, np.int64)
    pre = lens - np.asarray(decode_rows, np.int64)
    cache, seqs = runtime.build_cache(fmt, n_phys, H, d, table, lens, src, prefill_lens=pre)
    if np.any(pre < lens):
        start = pre
        cnt = lens - start
        k_new = np.concatenate([kv[b][0][start[b]:lens[b]] for b in range(len(lens))])
        v_new = np.concatenate([kv[b][1][start[b]:lens[b]] for b in range(len(lens))])
        kvq.kvq_append_decode(cache, seqs, dev_i32(start), dev_i32(np.concatenate([[0], np.cumsum(cnt)])),
                              int(cnt.max()), f16_bits(k_new), f16_bits(v_new))
    torch.cuda.synchronize()
    return cache, seqs


def assert_cache_equal(cache, oc, fmt, what):
    k, v = to_np(cache.k_pages), to_np(cache.v_pages)
    if fmt == workloads.FMT_FP16:
        k, v = k.view(np.uint16), v.view(np.uint16)
    assert np.array_equal(k, oc.k_pages), f"{what}: K codes"
    assert np.array_equal(v, oc.v_pages), f"{what}: V codes"
    if fmt != workloads.FMT_FP16:
        p = to_np(cache.kv_params).view(np.uint32)
        assert np.array_equal(p, oc.params.view(np.uint32)), f"{what}: scale/zero bits"
        zeros = p[..., 1::2]
        assert not np.any(zeros == 0x80000000), f"{what}: a -0 zero-point"
    meta = to_np(cache.page_meta)
    assert np.array_equal(meta, oc.meta), f"{what}: metadata"     # == treats +0 and -0 alike


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("decode", [False, True], ids=["bulk", "decode"])
def test_int8_token_edge_rows_bit_exact(d, decode):
    """INT8 per token on every edge row, K and V: codes, scale/zero bits and
    metadata equal the oracle's, by the bulk append and by the decode-time
    append of the newest rows."""
    H, fmt = 2, workloads.FMT_INT8_TOKEN
    lens = np.array([45, 23], np.int64)
    kv = [edge_tokens(int(lens[0]), H, d, 0), edge_tokens(int(lens[1]), H, d, 11)]
    P = (lens + PAGE - 1) // PAGE
    n_phys = int(P.sum()) + 1
    table = np.full((2, int(P.max())), -1, np.int32)
    perm = np.random.default_rng(2).permutation(n_phys)
    table[0, :P[0]] = perm[:P[0]]
    table[1, :P[1]] = perm[P[0]:P[0] + P[1]]
    rows = [17, 5] if decode else [0, 0]
    cache, _ = gpu_cache(fmt, n_phys, H, d, table, lens, kv, rows)
    oc = oracle_prefill(fmt, n_phys, H, d, table, lens, kv)
    assert_cache_equal(cache, oc, fmt, f"token d={d} decode={decode}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("decode", [False, True], ids=["bulk", "decode"])
def test_int8_group_edge_groups_bit_exact(d, decode):
    """INT8 per 64-token group where each group's min/max is an edge case
    (constant groups, signed-zero minima, subnormals, +-65504), with a partial
    trailing group: codes, scale/zero bits and metadata equal the oracle's.
    The decode path re-supplies the open group from its aligned start."""
    H, fmt = 2, workloads.FMT_INT8_GROUP64
    lens = np.array([64 * 20 + 37, 64 * 3 + 1], np.int64)
    kv = [edge_groups(int(lens[0]), H, d), edge_groups(int(lens[1]), H, d)]
    kv[1] = (kv[1][0][:, ::-1].copy(), kv[1][1])
    P = (lens + PAGE - 1) // PAGE
    n_phys = int(P.sum())
    table = np.full((2, int(P.max())), -1, np.int32)
    perm = np.random.default_rng(3).permutation(n_phys)
    table[0, :P[0]] = perm[:P[0]]
    table[1, :P[1]] = perm[P[0]:]
    rows = [int(lens[0] - (lens[0] - 1) // 64 * 64), int(lens[1] - (lens[1] - 1) // 64 * 64)] if decode else [0, 0]
    cache, _ = gpu_cache(fmt, n_phys, H, d, table, lens, kv, rows)
    oc = oracle_prefill(fmt, n_phys, H, d, table, lens, kv)
    assert_cache_equal(cache, oc, fmt, f"group d={d} decode={decode}")


@pytest.mark.parametrize("decode", [False, True], ids=["bulk", "decode"])
def test_fp16_edge_rows_copied_and_bounded(decode):
    """fp16 storage copies the edge rows bit for bit (signed zeros and
    subnormals included) and their metadata equals the oracle's."""
    H, d, fmt = 2, 64, workloads.FMT_FP16
    lens = np.array([41], np.int64)
    kv = [edge_tokens(41, H, d, 3)]
    n_phys = 3
    table = np.array([[2, 0, 1]], np.int32)
    cache, _ = gpu_cache(fmt, n_phys, H, d, table, lens, kv, [9] if decode else [0])
    oc = oracle_prefill(fmt, n_phys, H, d, table, lens, kv)
    assert_cache_equal(cache, oc, fmt, f"fp16 decode={decode}")


# ------------------------------------------------- steep softmax (large logits)
class Scaled:
    """A small ragged batch with keys and queries scaled by `scale` (fp32,
    then cast to fp16), built on the GPU and by the oracle."""

    def __init__(self, fmt, hq, hkv, d, scale, seed):
        _, runtime = mods()
        self.w = workloads.small(5).with_(name=f"steep_f{fmt}_g{hq // hkv}_d{d}", seed=seed, fmt=fmt,
                                          num_q_heads=hq, num_kv_heads=hkv, head_dim=d, len_lo=200,
                                          len_hi=900)
        w = self.w
        self.table, self.n_phys = w.block_table()
        self.lens = w.seq_lens()
        self.kv = [((w.keys(b).astype(np.float32) * scale).astype(np.float16), w.values(b))
                   for b in range(w.batch)]
        self.q = (w.query().astype(np.float32) * scale).astype(np.float16)
        src = lambda b: self.kv[b]  # noqa: E731
        self.cache, self.seqs = runtime.build_cache(fmt, self.n_phys, hkv, d, self.table, self.lens, src)
        self.q_dev = f16_bits(self.q)
        self.oc = oracle_prefill(fmt, self.n_phys, hkv, d, self.table, self.lens, self.kv)


@pytest.mark.parametrize("fmt,hq,hkv,d", [(0, 4, 4, 128), (0, 8, 2, 64), (1, 4, 4, 128), (1, 8, 2, 128),
                                          (2, 8, 2, 128), (2, 4, 4, 64)],
                         ids=["fp16_mha", "fp16_gqa", "int8tok_mha", "int8tok_mfma", "int8grp_mfma",
                              "int8grp_mha"])
def test_attention_steep_softmax(fmt, hq, hkv, d):
    """Keys and queries scaled 60x (logits in the thousands, so the running
    max moves by far more than the lazy rescale threshold): attention over the
    oracle's selection, the whole step, and the dense path match the oracle."""
    kvq, runtime = mods()
    s = Scaled(fmt, hq, hkv, d, 60.0, 7000 + 10 * fmt + hq)
    w = s.w
    st = runtime.DecodeStep(s.cache, s.seqs, hq, w.ratio_num, w.ratio_den, w.k_fixed)
    osc = oracle.page_scores(s.oc, s.table, s.lens, s.q)
    osel, ocnt = oracle.topk(osc, s.lens, w.ratio_num, w.ratio_den, w.k_fixed, st.k_cap)
    out = to_np(st.attend(s.q_dev, torch.from_numpy(osel).cuda(), torch.from_numpy(ocnt).cuda())).astype(np.float64)
    want = oracle.attention(s.oc, s.table, s.lens, s.q, osel, ocnt)
    lg_max = 0.0
    for b in range(w.batch):
        kdec = s.kv[b][0].astype(np.float64)
        lg_max = max(lg_max, float(np.abs(np.einsum("thd,hd->th", kdec[:, :, :],
                                                    s.q[b, ::hq // hkv].astype(np.float64))).max() / np.sqrt(d)))
    err = np.abs(out - want).max()
    log(f"[steep] {w.name}: |logit| up to {lg_max:.0f}, max abs err {err:.3g} (oracle selection)")
    assert lg_max > 500
    assert np.all(np.isfinite(out)) and err <= ATTN_ATOL
    full = to_np(st.run(s.q_dev)).astype(np.float64)
    gsel, gcnt = to_np(st.sel_pages), to_np(st.sel_count)
    want2 = oracle.attention(s.oc, s.table, s.lens, s.q, gsel, gcnt)
    assert np.abs(full - want2).max() <= ATTN_ATOL
    dense = to_np(runtime.DecodeStep(s.cache, s.seqs, hq, 1, 1, 0, dense=True).attend(s.q_dev)).astype(np.float64)
    err_d = np.abs(dense - oracle.attention(s.oc, s.table, s.lens, s.q)).max()
    log(f"[steep] {w.name}: dense max abs err {err_d:.3g}")
    assert err_d <= ATTN_ATOL


# --------------------------------------------- long splits, dirty workspace
@pytest.mark.parametrize("fmt,hq,hkv", [(1, 4, 4), (2, 8, 2), (0, 4, 4)], ids=["int8tok", "int8grp_gqa", "fp16"])
def test_split_longer_than_256_pages(fmt, hq, hkv):
    """pages_per_split 300 on rows of 2048 pages with half of them selected
    (4 splits, waves of 75 pages, so a wave reads its pages beyond the first
    64 from the selection): the in-kernel selection equals kvq_topk_pages and
    the outputs of the two paths agree bit for bit and with the oracle."""
    kvq, runtime = mods()
    w = workloads.small(4).with_(name=f"long_split_f{fmt}", fmt=fmt, num_q_heads=hq, num_kv_heads=hkv,
                                 seq_len=2048 * PAGE - 5, batch=2, ratio_num=1, ratio_den=2,
                                 outlier_channels=0)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, hkv, w.head_dim, table, lens, src)
    q = w.query()
    q_dev = f16_bits(q)
    sep = runtime.DecodeStep(cache, seqs, hq, 1, 2, 0, pages_per_split=300, fused_select=False)
    fus = runtime.DecodeStep(cache, seqs, hq, 1, 2, 0, pages_per_split=300)
    assert fus.fused_select and sep.k_cap == 1024
    out_sep = sep.run(q_dev).clone()
    fus.sel_pages.fill_(-7)
    out_fus = fus.run(q_dev)
    torch.cuda.synchronize()
    assert torch.equal(fus.sel_pages, sep.sel_pages)
    assert torch.equal(out_fus, out_sep)
    oc, _ = oracle.build_cache(w)
    want = oracle.attention(oc, table, lens, q, to_np(sep.sel_pages), to_np(sep.sel_count))
    err = np.abs(to_np(out_fus).astype(np.float64) - want).max()
    log(f"[long split] {w.name}: max abs err {err:.3g}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("fused", [True, False])
def test_workspace_contents_do_not_matter(fused):
    """A ragged GQA batch (rows with fewer splits than the widest row) with
    the workspace filled with NaN, then with -inf, before each call: the
    output is the same and matches the oracle."""
    kvq, runtime = mods()
    w = workloads.small(5)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src)
    q = w.query()
    q_dev = f16_bits(q)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, pages_per_split=3,
                            fused_select=fused)
    outs = []
    for fill in (float("nan"), float("-inf"), 0.0):
        st.workspace.fill_(fill)
        outs.append(st.run(q_dev).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[2])
    oc, _ = oracle.build_cache(w)
    want = oracle.attention(oc, table, lens, q, to_np(st.sel_pages), to_np(st.sel_count))
    assert np.abs(to_np(outs[0]).astype(np.float64) - want).max() <= ATTN_ATOL


# ----------------------------------------------- config 3 through selection
@pytest.mark.parametrize("fused", [True, False])
def test_config3_selecting_pipeline_with_k_equal_p(fused):
    """Config 3 (4 x 2048 tokens, 32 heads, fp16) run once through scoring,
    top-K with K = P and attention: every page is selected, in order, and the
    output matches the oracle's dense attention and the GPU's dense path."""
    kvq, runtime = mods()
    w = workloads.config(3)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    src = lambda b: (w.keys(b), w.values(b))  # noqa: E731
    cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                      prefill_lens=lens - 1)
    app = runtime.DecodeAppend(cache, seqs, lens, src)
    q = w.query()
    q_dev = f16_bits(q)
    st = runtime.DecodeStep(cache, seqs, w.num_q_heads, 1, 1, 0, fused_select=fused)
    assert st.fused_select == fused
    out = to_np(st.run_with_append(app, q_dev)).astype(np.float64)
    P = (lens + PAGE - 1) // PAGE
    cnt, sel = to_np(st.sel_count), to_np(st.sel_pages)
    assert (cnt == P[:, None]).all()
    assert (sel == np.arange(int(P.max()))[None, None, :]).all()
    dense = to_np(runtime.DecodeStep(cache, seqs, w.num_q_heads, 1, 1, 0, dense=True).attend(q_dev))
    oc, _ = oracle.build_cache(w)
    want = oracle.attention(oc, table, lens, q)
    err = np.abs(out - want).max()
    log(f"[cfg3 K=P] fused={fused}: max abs err {err:.3g}")
    assert err <= ATTN_ATOL
    assert np.abs(out - dense).max() <= 1e-5


# ----------------------------------------- config 5, every sequence, full size
_C5 = {}


def c5_state():
    """Config 5 built as the benchmark builds it (prefill of L - 1 tokens),
    then one whole step in its launch configuration: the decode-time append
    fused into scoring, top-K, attention, combine."""
    if "st" not in _C5:
        _, runtime = mods()
        w = workloads.config(5)
        table, n_phys = w.block_table()
        lens = w.seq_lens()
        src = functools.lru_cache(maxsize=None)(lambda b: (w.keys(b), w.values(b)))
        log(f"[cfg5] building {w.name}: {int(lens.sum())} tokens")
        cache, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                          prefill_lens=lens - 1)
        app = runtime.DecodeAppend(cache, seqs, lens, src)
        q = w.query()
        st = runtime.DecodeStep(cache, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed)
        out = to_np(st.run_with_append(app, f16_bits(q))).astype(np.float64)
        torch.cuda.synchronize()
        _C5.update(w=w, table=table, lens=lens, q=q, st=st, out=out, scores=to_np(st.scores),
                   sel=to_np(st.sel_pages), cnt=to_np(st.sel_count), k=to_np(cache.k_pages),
                   v=to_np(cache.v_pages), params=to_np(cache.kv_params), meta=to_np(cache.page_meta), errs={})
    return _C5


@pytest.mark.timeout(900)
@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_config5_every_sequence(part):
    """Config 5 at full size: for sequences 16*part .. 16*part+15, the codes,
    scale/zero bits and metadata of every page, every page score, the
    selection (near-tie rule) and the output of every head against the
    oracle run on that sequence alone."""
    from test_gpu_parity import check_scores, check_selection_near_ties, score_tolerance
    c = c5_state()
    w, lens, st = c["w"], c["lens"], c["st"]
    for b in range(16 * part, 16 * part + 16):
        L = int(lens[b])
        P = (L + PAGE - 1) // PAGE
        ocache = oracle.Cache(w.fmt, P, w.num_kv_heads, w.head_dim)
        tab = np.arange(P, dtype=np.int32)[None]
        oracle.append(ocache, tab, [0], [0, L], w.keys(b), w.values(b))
        oracle.page_meta(ocache, tab, [L])
        phys = c["table"][b, :P]
        assert np.array_equal(c["k"][phys], ocache.k_pages), f"K codes of sequence {b}"
        assert np.array_equal(c["v"][phys], ocache.v_pages), f"V codes of sequence {b}"
        assert np.array_equal(c["params"][phys].view(np.uint32), ocache.params.view(np.uint32)), b
        assert np.array_equal(c["meta"][phys], ocache.meta), b
        qb = c["q"][b:b + 1]
        osc, osel, ocnt, _ = oracle.decode_step(ocache, tab, [L], qb, w.ratio_num, w.ratio_den, w.k_fixed,
                                                st.k_cap, nthreads=16)
        S = score_tolerance(ocache, tab, np.array([L]), qb, w.group)
        check_scores(c["scores"][b:b + 1, :, :P], osc[:, :, :P], S[:, :, :P])
        assert np.isneginf(c["scores"][b, :, P:]).all()
        check_selection_near_ties(c["sel"][b:b + 1], c["cnt"][b:b + 1], osc, osel, ocnt)
        want = oracle.attention(ocache, tab, [L], qb, c["sel"][b:b + 1], c["cnt"][b:b + 1])
        err = float(np.abs(c["out"][b] - want[0]).max())
        c["errs"][b] = err
        log(f"[cfg5] sequence {b} L={L}: max abs err {err:.3g}")
        assert err <= ATTN_ATOL, f"sequence {b} L={L}: max abs err {err:.3g}"
    log(f"[cfg5] sequences {16 * part}..{16 * part + 15}: max abs err "
        f"{max(c['errs'][b] for b in range(16 * part, 16 * part + 16)):.3g}")


# ------------------------------------------------------ rows past max_new
@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4, 5],
                         ids=["fp16", "int8tok", "int8grp", "int4tok", "int4grp", "mixed"])
def test_bulk_append_writes_no_row_past_max_new(fmt):
    """kvq_append_quant writes rows 0 .. max_new-1 of each sequence and no row
    past them: sequence 0 supplies 100 rows but max_new is 70, so its rows
    70 .. 99 are left as they were (a byte pattern laid down first), and every
    byte of the caches equals the oracle appending the same 70 (and 30) rows
    into caches that hold the same pattern.  Per-token formats start mid-page;
    per-group formats start on a group (64 tokens)."""
    kvq, _ = mods()
    H, d = 2, 128
    group = fmt in (workloads.FMT_INT8_GROUP64, workloads.FMT_INT4_GROUP64)
    start = np.array([64 if group else 21, 5 if not group else 0], np.int64)
    rows = np.array([100, 30], np.int64)
    max_new = 70
    P = (start + rows + PAGE - 1) // PAGE
    n_phys = int(P.sum()) + 2
    table = np.full((2, int(P.max())), -1, np.int32)
    perm = np.random.default_rng(4).permutation(n_phys)
    table[0, :P[0]] = perm[:P[0]]
    table[1, :P[1]] = perm[P[0]:P[0] + P[1]]
    rng = np.random.default_rng(17)
    k_all = [rng.standard_normal((int(r), H, d)).astype(np.float16) for r in rows]
    v_all = [rng.standard_normal((int(r), H, d)).astype(np.float16) for r in rows]
    n16 = n_phys // 2 if fmt == workloads.FMT_MIXED else 0
    cache = kvq.PagedCache.empty(fmt, n_phys, H, d, num_fp16_pages=n16)
    oc = oracle.Cache(fmt, n_phys, H, d, n16)
    for t in (cache.k_pages, cache.v_pages):
        t.view(torch.uint8).fill_(0xAB)
    oc.k_pages.view(np.uint8)[...] = 0xAB
    oc.v_pages.view(np.uint8)[...] = 0xAB
    if cache.kv_params is not None:
        cache.kv_params.view(torch.int32).fill_(0x7FC0ABAB)
        oc.params.view(np.uint32)[...] = 0x7FC0ABAB
    seqs = kvq.Seqs(dev_i32(start + rows), dev_i32(table))
    k_new = np.concatenate(k_all)
    v_new = np.concatenate(v_all)
    off = np.concatenate([[0], np.cumsum(rows)])
    kvq.kvq_append_quant(cache, seqs, dev_i32(start), dev_i32(off), max_new, f16_bits(k_new), f16_bits(v_new))
    torch.cuda.synchronize()
    # the oracle appends what max_new lets through: 70 rows of sequence 0, all 30 of sequence 1
    kept = np.minimum(rows, max_new)
    ok = np.concatenate([k_all[0][:kept[0]], k_all[1][:kept[1]]])
    ov = np.concatenate([v_all[0][:kept[0]], v_all[1][:kept[1]]])
    oracle.append(oc, table, start.astype(np.int32), np.concatenate([[0], np.cumsum(kept)]).astype(np.int32), ok, ov)
    k, v = to_np(cache.k_pages), to_np(cache.v_pages)
    assert np.array_equal(k.view(np.uint8), oc.k_pages.view(np.uint8)), "K bytes"
    assert np.array_equal(v.view(np.uint8), oc.v_pages.view(np.uint8)), "V bytes"
    if cache.kv_params is not None:
        assert np.array_equal(to_np(cache.kv_params).view(np.uint32), oc.params.view(np.uint32)), "scale/zero bits"
