"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas retyped.

Each test names the mistake it is there to catch.  Independent references are
numpy routines on the unpaged arrays (fp16 casts, min/max, sort, dense
softmax attention), hand-derived fixtures under tests/golden/, closed forms,
and invariants (the no-underestimate property of the TinyServe page, section
2.1; the scale/2 error bound of min/max quantization)."""
import copy
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from workloads import PAGE

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ helpers
def np_dequant(codes, scale, zero):
    """code*scale + zero rounded once to fp32.  code*scale is exact in fp64
    (8 x 24 bits); the sum is checked exact against extended precision, so the
    single fp64 -> fp32 rounding equals a fused multiply-add."""
    c = codes.astype(np.float64)
    s = np.asarray(scale, np.float32).astype(np.float64)
    z = np.asarray(zero, np.float32).astype(np.float64)
    r64 = c * s + z
    rl = c.astype(np.longdouble) * s.astype(np.longdouble) + z.astype(np.longdouble)
    assert np.all(rl == r64.astype(np.longdouble)), "fp64 sum not exact; reference would double-round"
    return r64.astype(np.float32)


def gather_tokens(arr, table_row, L):
    """[P_phys][H][16][...] paged array -> [L][H][...] logical order."""
    t = np.arange(L)
    return arr[table_row[t // PAGE], :, t % PAGE]


def decoded_keys_values(w, cache, table, b):
    """(K, V) fp32 [L][H][d] of sequence b as stored, decoded by numpy."""
    L = int(w.seq_lens()[b])
    kc = gather_tokens(cache.k_pages, table[b], L)
    vc = gather_tokens(cache.v_pages, table[b], L)
    if w.fmt == workloads.FMT_FP16:
        return kc.view(np.float16).astype(np.float32), vc.view(np.float16).astype(np.float32)
    t = np.arange(L)
    if w.fmt == workloads.FMT_INT8_TOKEN:
        p = cache.params[table[b][t // PAGE], :, t % PAGE]          # [L][H][4]
    else:
        p = cache.params[table[b][t // PAGE]]                        # [L][H][4]
    K = np_dequant(kc, p[..., 0:1], p[..., 1:2])
    V = np_dequant(vc, p[..., 2:3], p[..., 3:4])
    return K, V


def dense_attention(q, K, V, scale):
    """numpy fp64 softmax(q K^T * scale) V for one head: q [d], K/V [n][d]."""
    lg = K.astype(np.float64) @ q.astype(np.float64) * scale
    w = np.exp(lg - lg.max())
    return (w[:, None] * V.astype(np.float64)).sum(0) / w.sum()


def one_token_cache(fmt, x_k, x_v=None):
    """Cache with one sequence of len(x_k) tokens, 1 KV head, d = row length."""
    x_k = np.asarray(x_k, np.float16)
    L, d = x_k.shape
    x_v = x_k if x_v is None else np.asarray(x_v, np.float16)
    P = (L + PAGE - 1) // PAGE
    cache = oracle.Cache(fmt, P, 1, d)
    table = np.arange(P, dtype=np.int32)[None]
    oracle.append(cache, table, [0], [0, L], x_k[:, None, :], x_v[:, None, :])
    return cache, table


# ------------------------------------------------------------ fp16 decoding
def test_half_decode_matches_numpy_for_every_bit_pattern():
    """Catches a wrong exponent bias, subnormal or sign handling."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.half_to_float(int(b)) for b in bits[::7]], dtype=np.float32)
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), r[~nan].view(np.uint32))


# ---------------------------------------------------------- quantization
def test_quant_golden_rows():
    """Hand-worked rows pin scale, zero, round-half-even and clamping."""
    for row in gold("quant_rows.json")["rows"]:
        x = np.array([row["x"]], np.float16)
        cache, table = one_token_cache(workloads.FMT_INT8_TOKEN, x)
        codes = cache.k_pages[0, 0, 0, :x.shape[1]]
        assert codes.tolist() == row["codes"], row["derivation"]
        s, z = cache.params[0, 0, 0, 0], cache.params[0, 0, 0, 1]
        assert s == np.float32(row["scale"]) and z == np.float32(row["zero"])
        dec = np_dequant(codes, s, z)
        assert dec.tolist() == [float(v) for v in row["decoded"]]


def test_quant_zero_point_of_a_signed_zero_minimum_is_plus_zero():
    """A row whose minimum is zero stores the zero-point +0 whichever sign the
    first zero had (the reading that makes the stored bits independent of
    reduction order); codes and decoded values are those of the number 0."""
    nz, pz = np.float16(-0.0), np.float16(0.0)
    for row in ([nz, pz, 1.0, 3.0], [pz, nz, 1.0, 3.0], [nz, 2.0], [nz, nz, nz], [pz, pz]):
        x = np.array([row], np.float16)
        cache, _ = one_token_cache(workloads.FMT_INT8_TOKEN, x)
        z = cache.params[0, 0, 0, 1]
        assert z.view(np.uint32) == 0, row
        codes = cache.k_pages[0, 0, 0, :x.shape[1]]
        assert all(int(c) == 0 for c, v in zip(codes, row) if v == 0)
        assert np_dequant(codes[:1], cache.params[0, 0, 0, 0], z)[0].view(np.uint32) == 0


def _random_rows(rng, n, d):
    x = rng.standard_normal((n, d)).astype(np.float32)
    x[: n // 3] *= 30.0                                      # wide rows
    x[n // 3: n // 2, : d // 8] *= 15.0                      # outlier channels
    x[-3:] = 0.75                                            # constant rows
    return x.astype(np.float16)


@pytest.mark.parametrize("d", [64, 128])
def test_quant_error_within_half_scale_and_nearest_code(d):
    """|x - decode(code)| <= scale/2 (+fp32 slack), the code is the nearest of
    its neighbours, min -> code 0 decoding to min exactly, max -> 255.
    Catches floor-instead-of-round, a wrong scale or zero, missing clamp."""
    rng = np.random.default_rng(7)
    x = _random_rows(rng, 300, d)
    cache, table = one_token_cache(workloads.FMT_INT8_TOKEN, x)
    L = x.shape[0]
    t = np.arange(L)
    codes = cache.k_pages[t // PAGE, 0, t % PAGE].astype(np.int64)      # [L][d]
    p = cache.params[t // PAGE, 0, t % PAGE]                             # [L][4]
    s, z = p[:, 0], p[:, 1]
    xf = x.astype(np.float32)
    lo, hi = xf.min(1), xf.max(1)
    assert np.array_equal(z, lo), "zero-point must be the row minimum"
    const = hi == lo
    assert np.all(s[const] == 1.0) and np.all(codes[const] == 0)
    rng_ = (hi - lo).astype(np.float64)
    assert np.allclose(s[~const].astype(np.float64), rng_[~const] / 255.0, rtol=2 ** -22, atol=0)
    dec = np_dequant(codes, s[:, None], z[:, None]).astype(np.float64)
    err = np.abs(xf.astype(np.float64) - dec)
    ulp = np.spacing(np.maximum(np.abs(lo), np.abs(hi)).astype(np.float32)).astype(np.float64)
    slack = 2 * ulp + 255 * s.astype(np.float64) * 2 ** -22
    assert np.all(err <= s[:, None] / 2 + slack[:, None])
    # nearest code: neighbours are no closer
    for dc in (-1, 1):
        nb = np.clip(codes + dc, 0, 255)
        dn = np.abs(xf - np_dequant(nb, s[:, None], z[:, None])).astype(np.float64)
        assert np.all(err <= dn + slack[:, None])
    amin = xf.argmin(1)
    amax = xf.argmax(1)
    assert np.all(codes[t, amin] == 0)
    assert np.all(dec[t, amin] == lo)
    assert np.all(codes[~const][:, None].squeeze(1)[np.arange((~const).sum()), amax[~const]] == 255)


def test_value_rows_quantized_separately_with_same_scheme():
    """K and V rows each get their own (scale, zero); catches V reusing K's."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((20, 64)).astype(np.float16)
    v = (rng.standard_normal((20, 64)) * 7 + 3).astype(np.float16)
    cache, _ = one_token_cache(workloads.FMT_INT8_TOKEN, k, v)
    t = np.arange(20)
    p = cache.params[t // PAGE, 0, t % PAGE]
    assert np.array_equal(p[:, 3], v.astype(np.float32).min(1))
    assert np.array_equal(p[:, 1], k.astype(np.float32).min(1))


def test_group64_scope_alignment_and_partial_tail():
    """Per-group quantization: 64-token groups aligned to logical positions 64g
    (uyd888.cn Gemini page, chapter 1), all channels of a KV head share one
    (scale, zero); a trailing partial group uses only its valid tokens.
    Catches per-page or per-token scope and misaligned groups."""
    rng = np.random.default_rng(11)
    L, H, d = 150, 2, 64
    k = rng.standard_normal((L, H, d)).astype(np.float32)
    k[64:128] *= 40.0                     # second group is much wider
    k[140, 1, 5] = -90.0                  # tail group, head 1 only
    v = rng.standard_normal((L, H, d)).astype(np.float32)
    k16, v16 = k.astype(np.float16), v.astype(np.float16)
    P = (L + PAGE - 1) // PAGE
    table = np.random.default_rng(5).permutation(P + 3)[:P].astype(np.int32)[None]
    cache = oracle.Cache(workloads.FMT_INT8_GROUP64, P + 3, H, d)
    oracle.append(cache, table, [0], [0, L], k16, v16)
    kf = k16.astype(np.float32)
    for g0 in range(0, L, 64):
        g1 = min(g0 + 64, L)
        for h in range(H):
            lo = kf[g0:g1, h].min()
            for j in range(g0 // PAGE, (g1 + PAGE - 1) // PAGE):
                assert cache.params[table[0, j], h, 1] == lo, (g0, h, j)
    # tokens of group 0 are not affected by group 1's range: their codes span 0..255
    c0 = cache.k_pages[table[0, :4], 0]
    assert c0.min() == 0 and c0.max() == 255
    # decoded values within scale/2 of the inputs everywhere
    w = workloads.small(5).with_(batch=1, num_kv_heads=H, num_q_heads=H, head_dim=d, seq_len=L)
    K, _ = decoded_keys_values(w, cache, table, 0)
    t = np.arange(L)
    s = cache.params[table[0][t // PAGE], :, 0]
    assert np.all(np.abs(K - kf) <= s[:, :, None] / 2 + 1e-5 * np.abs(kf).max())


def test_group64_rejects_unaligned_start():
    cache = oracle.Cache(workloads.FMT_INT8_GROUP64, 8, 1, 64)
    x = np.zeros((3, 1, 64), np.float16)
    with pytest.raises(ValueError):
        oracle.append(cache, np.arange(8, dtype=np.int32)[None], [16], [0, 3], x, x)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_paged_placement_through_shuffled_table(n):
    """Token t lands in physical page table[b][t/16], slot t%16 (pzsr.cn page,
    section 3).  Checked by gathering with numpy: fp16 storage returns the input
    bits exactly; INT8 storage decodes to within scale/2.  Slots past a
    sequence's end stay untouched.  Catches transposed page/slot indexing."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    used = np.zeros(cache.P_phys, bool)
    for b in range(w.batch):
        L = int(lens[b])
        kin = w.keys(b).astype(np.float32)
        vin = w.values(b).astype(np.float32)
        if w.fmt == workloads.FMT_FP16:
            kc = gather_tokens(cache.k_pages, table[b], L)
            assert np.array_equal(kc, w.keys(b).view(np.uint16))
            assert np.array_equal(gather_tokens(cache.v_pages, table[b], L), w.values(b).view(np.uint16))
        else:
            K, V = decoded_keys_values(w, cache, table, b)
            t = np.arange(L)
            if w.fmt == workloads.FMT_INT8_TOKEN:
                p = cache.params[table[b][t // PAGE], :, t % PAGE]
            else:
                p = cache.params[table[b][t // PAGE]]
            tol_k = p[..., 0:1] / 2 + 1e-6 * np.abs(kin).max()
            tol_v = p[..., 2:3] / 2 + 1e-6 * np.abs(vin).max()
            assert np.all(np.abs(K - kin) <= tol_k)
            assert np.all(np.abs(V - vin) <= tol_v)
        P = (L + PAGE - 1) // PAGE
        used[table[b, :P]] = True
        tail = L % PAGE
        if tail:
            assert not cache.k_pages[table[b, P - 1], :, tail:].any()
    assert not cache.k_pages[~used].any()


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_incremental_append_equals_prefill(fmt):
    """Appending in decode-sized steps gives the same cache as one prefill.
    Per-group storage re-supplies the open group from its first token."""
    w = workloads.small(5).with_(fmt=fmt, batch=3, len_lo=60, len_hi=200)
    full, table = oracle.build_cache(w)
    lens = w.seq_lens()
    inc = oracle.Cache(w.fmt, full.P_phys, w.num_kv_heads, w.head_dim)
    cur = np.minimum(lens, 37)
    ks = [w.keys(b) for b in range(w.batch)]
    vs = [w.values(b) for b in range(w.batch)]
    # prefill of the first 37 tokens
    off = np.concatenate([[0], np.cumsum(cur)]).astype(np.int32)
    oracle.append(inc, table, np.zeros(w.batch, np.int32), off,
                  np.concatenate([ks[b][:cur[b]] for b in range(w.batch)]),
                  np.concatenate([vs[b][:cur[b]] for b in range(w.batch)]))
    while np.any(cur < lens):
        nxt = np.minimum(cur + 1, lens)
        start = (cur // 64) * 64 if fmt == 2 else cur
        start = np.where(nxt > cur, start, cur)
        rows_k = [ks[b][start[b]:nxt[b]] for b in range(w.batch)]
        rows_v = [vs[b][start[b]:nxt[b]] for b in range(w.batch)]
        cnt = np.array([len(r) for r in rows_k])
        off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
        oracle.append(inc, table, start.astype(np.int32), off, np.concatenate(rows_k), np.concatenate(rows_v))
        cur = nxt
    assert np.array_equal(inc.k_pages, full.k_pages)
    assert np.array_equal(inc.v_pages, full.v_pages)
    assert np.array_equal(inc.params, full.params)


# -------------------------------------------------------------- metadata
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_meta_is_min_max_of_decoded_keys(n):
    """phi(K_j) = per-channel (min, max) over the page's valid keys, as
    decoded (TinyServe page, section 2.1), brute force with numpy.
    Catches swapped rows, reading padding slots, wrong token ranges."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    for b in range(w.batch):
        K, _ = decoded_keys_values(w, cache, table, b)
        L = int(lens[b])
        for j in range((L + PAGE - 1) // PAGE):
            blk = K[j * PAGE: min((j + 1) * PAGE, L)]
            m = cache.meta[table[b, j], :, 0]
            M = cache.meta[table[b, j], :, 1]
            assert np.array_equal(m, blk.min(0)) and np.array_equal(M, blk.max(0))


def test_meta_ignores_padding_slots_and_honours_page_begin():
    """Garbage in the unused slots of a partial last page must not leak into
    phi; page_begin restricts the rebuild to the tail pages."""
    w = workloads.small(4).with_(seq_len=40)
    cache, table = oracle.build_cache(w)
    ref = cache.meta.copy()
    last = table[0, 2]
    cache.k_pages[last, :, 8:] = 255                     # slots 40..47 are padding
    cache.params[last, :, 8:, 0] = 1e6
    cache.meta[:] = 0
    oracle.page_meta(cache, table, w.seq_lens(), page_begin=np.array([2], np.int32))
    assert np.array_equal(cache.meta[last], ref[last])
    assert not cache.meta[table[0, :2]].any()


# ---------------------------------------------------------------- scores
def test_score_golden():
    g = gold("page_score_hand.json")
    cache = oracle.Cache(workloads.FMT_FP16, 1, 1, 4)
    table = np.zeros((1, 1), np.int32)
    keys = np.array(g["keys"], np.float16)[:, None, :]
    oracle.append(cache, table, [0], [0, 2], keys, keys)
    oracle.page_meta(cache, table, [2])
    assert cache.meta[0, 0, 0].tolist() == g["min"] and cache.meta[0, 0, 1].tolist() == g["max"]
    s = oracle.page_scores(cache, table, [2], np.array(g["q"], np.float16)[None, None])
    assert s[0, 0, 0] == g["score"]


@pytest.mark.parametrize("n", [2, 4, 5])
def test_score_never_underestimates(n):
    """r >= max over the page of q.k for every page and query head (TinyServe
    page, section 2.1).  Catches swapped min/max or a flipped sign test."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    q = w.query().astype(np.float64)
    sc = oracle.page_scores(cache, table, w.seq_lens(), w.query())
    lens = w.seq_lens()
    G = w.group
    for b in range(w.batch):
        K, _ = decoded_keys_values(w, cache, table, b)
        L = int(lens[b])
        P = (L + PAGE - 1) // PAGE
        assert np.all(np.isneginf(sc[b, :, P:]))
        for h in range(w.num_q_heads):
            g = h // G
            dots = K[:, g].astype(np.float64) @ q[b, h]              # [L]
            for j in range(P):
                mx = dots[j * PAGE: min((j + 1) * PAGE, L)].max()
                mm = cache.meta[table[b, j], g].astype(np.float64)
                slack = 1e-12 * (np.abs(q[b, h]) * np.abs(mm).max(0)).sum()
                assert sc[b, g, j] >= mx - slack


def test_score_exact_cases():
    """A 1-token page, or a page of identical keys, scores exactly q.k; an
    all-non-negative q scores q.M, an all-negative q scores q.m.
    Catches a dropped or duplicated term."""
    rng = np.random.default_rng(2)
    d = 64
    k = rng.standard_normal((17, d)).astype(np.float16)      # page 1 holds a single token
    k[:16] = k[3]                                            # page 0: 16 identical keys
    cache, table = one_token_cache(workloads.FMT_FP16, k)
    oracle.page_meta(cache, table, [17])
    q = rng.standard_normal(d).astype(np.float16)
    s = oracle.page_scores(cache, table, [17], q[None, None])[0, 0]
    kd = k.astype(np.float64)
    qd = q.astype(np.float64)
    assert s[0] == pytest.approx(kd[3] @ qd, rel=1e-13, abs=1e-13)
    assert s[1] == pytest.approx(kd[16] @ qd, rel=1e-13, abs=1e-13)
    k2 = rng.standard_normal((16, d)).astype(np.float16)
    cache2, table2 = one_token_cache(workloads.FMT_FP16, k2)
    oracle.page_meta(cache2, table2, [16])
    qp = np.abs(q)
    qn = -np.abs(q)
    sp = oracle.page_scores(cache2, table2, [16], qp[None, None])[0, 0, 0]
    sn = oracle.page_scores(cache2, table2, [16], qn[None, None])[0, 0, 0]
    k2d = k2.astype(np.float64)
    assert sp == pytest.approx(qp.astype(np.float64) @ k2d.max(0), rel=1e-13)
    assert sn == pytest.approx(qn.astype(np.float64) @ k2d.min(0), rel=1e-13)


def test_gqa_group_score_is_max_over_member_heads():
    """KV head g serves query heads g*G .. g*G+G-1 and scores with the max of
    their r.  Catches h % H_kv mapping and sum/first-head aggregation."""
    w = workloads.small(5).with_(batch=2, len_lo=100, len_hi=130)
    cache, table = oracle.build_cache(w)
    q = w.query()
    G = w.group
    sc = oracle.page_scores(cache, table, w.seq_lens(), q)
    for h in range(w.num_q_heads):
        solo = np.zeros_like(q)
        solo[:, h] = q[:, h]
        # a query of zeros scores 0; every other head is silenced
        per = oracle.page_scores(cache, table, w.seq_lens(), solo)
        g = h // G
        for b in range(w.batch):
            P = (int(w.seq_lens()[b]) + PAGE - 1) // PAGE
            assert np.all(per[b, g, :P] <= sc[b, g, :P])
    # the group score equals the max of the single-head scores
    singles = []
    for hh in range(G):
        qq = np.zeros_like(q)
        for g in range(w.num_kv_heads):
            qq[:, g * G:(g + 1) * G] = q[:, g * G + hh: g * G + hh + 1]
        singles.append(oracle.page_scores(cache, table, w.seq_lens(), qq))
    assert np.array_equal(np.maximum.reduce(singles), sc)


# ------------------------------------------------------------------ top-K
def test_num_selected_golden():
    g = gold("num_selected.json")
    rn, rd = g["ratio"]
    for P, K in g["cases"]:
        assert oracle.num_selected(P, rn, rd, 0) == K, (P, K)
    for P, kf, K in g["fixed"]["cases"]:
        assert oracle.num_selected(P, rn, rd, kf) == K
    assert oracle.num_selected(37, 1, 1, 0) == 37


def test_topk_matches_full_sort_with_ties():
    """Against numpy lexsort by (-score, page): largest K, ties to the lower
    logical index, emitted ascending, -1 padded."""
    rng = np.random.default_rng(4)
    B, H, maxp = 3, 4, 300
    lens = np.array([300 * 16, 77 * 16 - 5, 1], np.int32)
    sc = rng.standard_normal((B, H, maxp))
    sc[:, :, 50:120] = 0.5                                   # a plateau of equal scores
    sc[1, 2, :] = 1.0                                        # an all-equal row
    k_cap = 128
    sel, cnt = oracle.topk(sc, lens, 3, 10, 0, k_cap)
    for b in range(B):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        K = oracle.num_selected(P, 3, 10, 0)
        for h in range(H):
            order = np.lexsort((np.arange(P), -sc[b, h, :P]))
            want = np.sort(order[:K])
            assert cnt[b, h] == K
            assert np.array_equal(sel[b, h, :K], want)
            assert np.all(sel[b, h, K:] == -1)
    assert np.array_equal(sel[1, 2, :cnt[1, 2]], np.arange(cnt[1, 2]))


def test_topk_all_pages_when_k_equals_p():
    rng = np.random.default_rng(8)
    sc = rng.standard_normal((2, 3, 40))
    lens = np.array([40 * 16, 13 * 16 + 1], np.int32)
    sel, cnt = oracle.topk(sc, lens, 1, 1, 0, 40)
    assert cnt.tolist() == [[40] * 3, [14] * 3]
    assert np.array_equal(sel[0, 0], np.arange(40))
    assert np.array_equal(sel[1, 1, :14], np.arange(14))


# -------------------------------------------------------------- attention
def test_attention_golden():
    g = gold("attention_hand.json")
    cache, table = one_token_cache(workloads.FMT_FP16, g["keys"], g["values"])
    out = oracle.attention(cache, table, [2], np.array(g["q"], np.float16)[None, None])
    assert np.allclose(out[0, 0], g["out"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_dense_selection_equals_textbook_attention(n):
    """K = P reduces to softmax(q K^T / sqrt(d)) V (intelliparadigm.com page,
    section 2.1), computed by numpy in fp64 on the unpaged arrays.  Catches a
    missing 1/sqrt(d), a dropped max-shift or normalizer, a wrong head map."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    q = w.query()
    maxp = table.shape[1]
    sc, sel, cnt, out = oracle.decode_step(cache, table, lens, q, 1, 1, 0, maxp)
    out_null = oracle.attention(cache, table, lens, q)
    assert np.array_equal(out, out_null)
    for b in range(w.batch):
        K, V = decoded_keys_values(w, cache, table, b)
        for h in range(w.num_q_heads):
            g = h // w.group
            ref = dense_attention(q[b, h], K[:, g], V[:, g], 1 / math.sqrt(w.head_dim))
            assert np.allclose(out[b, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 4, 5])
def test_sparse_attention_equals_dense_over_selected_tokens(n):
    """With a selection, attention covers exactly the valid tokens of the
    selected pages (TinyServe page, section 3.1 phase 3), partial last page
    included."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    q = w.query()
    k_cap = table.shape[1]
    sc, sel, cnt, out = oracle.decode_step(cache, table, lens, q, 3, 10, 0, k_cap)
    for b in range(w.batch):
        K, V = decoded_keys_values(w, cache, table, b)
        L = int(lens[b])
        for h in range(w.num_q_heads):
            g = h // w.group
            pages = sel[b, g, :cnt[b, g]]
            toks = np.concatenate([np.arange(j * PAGE, min((j + 1) * PAGE, L)) for j in pages])
            ref = dense_attention(q[b, h], K[toks, g], V[toks, g], 1 / math.sqrt(w.head_dim))
            assert np.allclose(out[b, h], ref, rtol=0, atol=1e-12)


def test_attention_special_cases():
    """L = 1 returns v; q = 0 gives equal logits and the mean of V."""
    rng = np.random.default_rng(12)
    k = rng.standard_normal((1, 64)).astype(np.float16)
    v = rng.standard_normal((1, 64)).astype(np.float16)
    cache, table = one_token_cache(workloads.FMT_FP16, k, v)
    out = oracle.attention(cache, table, [1], rng.standard_normal((1, 1, 64)).astype(np.float16))
    assert np.array_equal(out[0, 0], v[0].astype(np.float64))
    k = rng.standard_normal((37, 64)).astype(np.float16)
    v = rng.standard_normal((37, 64)).astype(np.float16)
    cache, table = one_token_cache(workloads.FMT_FP16, k, v)
    out = oracle.attention(cache, table, [37], np.zeros((1, 1, 64), np.float16))
    assert np.allclose(out[0, 0], v.astype(np.float64).mean(0), rtol=0, atol=1e-14)


def test_block_table_permutation_does_not_change_results():
    """Same logical contents through identity and shuffled tables."""
    w = workloads.small(4)
    c1, t1 = oracle.build_cache(w.with_(table="identity"))
    c2, t2 = oracle.build_cache(w)
    assert not np.array_equal(t1, t2)
    q = w.query()
    lens = w.seq_lens()
    r1 = oracle.decode_step(c1, t1, lens, q, 3, 10, 0, 64)
    r2 = oracle.decode_step(c2, t2, lens, q, 3, 10, 0, 64)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


def test_decode_step_threads_agree_and_compose():
    """The threaded step equals the single-threaded one and the separate stages."""
    w = workloads.small(5)
    cache, table = oracle.build_cache(w)
    lens, q = w.seq_lens(), w.query()
    a = oracle.decode_step(cache, table, lens, q, 3, 10, 0, 64, nthreads=1)
    b = oracle.decode_step(cache, table, lens, q, 3, 10, 0, 64, nthreads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    sc = oracle.page_scores(cache, table, lens, q)
    sel, cnt = oracle.topk(sc, lens, 3, 10, 0, 64)
    out = oracle.attention(cache, table, lens, q, sel, cnt)
    assert np.array_equal(sc, a[0]) and np.array_equal(sel, a[1]) and np.array_equal(out, a[3])


def test_attention_large_logits_stay_finite():
    """Logits near 1000 overflow exp() unless the softmax is shifted by its
    max; the result must still equal the (shift-invariant) textbook value."""
    rng = np.random.default_rng(13)
    k = (rng.standard_normal((40, 64)) * 60).astype(np.float16)
    v = rng.standard_normal((40, 64)).astype(np.float16)
    q = (rng.standard_normal(64) * 60).astype(np.float16)
    cache, table = one_token_cache(workloads.FMT_FP16, k, v)
    out = oracle.attention(cache, table, [40], q[None, None])
    lg = k.astype(np.float64) @ q.astype(np.float64) / 8.0
    assert lg.max() > 800
    ref = dense_attention(q, k, v, 1 / 8.0)
    assert np.all(np.isfinite(out)) and np.allclose(out[0, 0], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------- selection quality
def _complement(sel, cnt, lens, k_cap):
    """Every valid page not in the selection, ascending, with its count."""
    B, H, _ = sel.shape
    out = np.full((B, H, k_cap), -1, np.int32)
    c = np.zeros((B, H), np.int32)
    for b in range(B):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        for g in range(H):
            rest = sorted(set(range(P)) - set(sel[b, g, :cnt[b, g]].tolist()))
            out[b, g, :len(rest)] = rest
            c[b, g] = len(rest)
    return out, c


@pytest.mark.parametrize("n", [2, 4, 5])
def test_attention_mass_pins(n):
    """The share of dense attention weight on the selected pages: numpy's own
    softmax over the unpaged tokens agrees; every page selected gives exactly
    1; a selection and its complement sum to 1; and the top-K sets are nested,
    so the share never drops as K grows."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    q = w.query()
    k_cap = table.shape[1]
    sc, sel, cnt, _ = oracle.decode_step(cache, table, lens, q, 3, 10, 0, k_cap)
    # a selection whose count differs between the KV heads of a sequence (each
    # row keeps a prefix of its top-K), so a row's own count must be used
    cnt_v = np.maximum(cnt - np.arange(w.num_kv_heads)[None, :], np.minimum(cnt, 1)).astype(np.int32)
    sel_v = sel.copy()
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            sel_v[b, g, cnt_v[b, g]:] = -1
    mv = oracle.attention_mass(cache, table, lens, q, sel_v, cnt_v)
    for b in range(w.batch):
        K, _ = decoded_keys_values(w, cache, table, b)
        L = int(lens[b])
        for h in range(w.num_q_heads):
            g = h // w.group
            lg = K[:, g].astype(np.float64) @ q[b, h].astype(np.float64) / math.sqrt(w.head_dim)
            p = np.exp(lg - lg.max())
            mask = np.isin(np.arange(L) // PAGE, sel_v[b, g, :cnt_v[b, g]])
            assert abs(mv[b, h] - p[mask].sum() / p.sum()) <= 1e-12
    m = oracle.attention_mass(cache, table, lens, q, sel, cnt)
    _, sel_all, cnt_all, _ = oracle.decode_step(cache, table, lens, q, 1, 1, 0, k_cap)
    assert np.all(oracle.attention_mass(cache, table, lens, q, sel_all, cnt_all) == 1.0)
    sel_c, cnt_c = _complement(sel, cnt, lens, k_cap)
    assert np.allclose(m + oracle.attention_mass(cache, table, lens, q, sel_c, cnt_c), 1.0, rtol=0, atol=1e-12)
    prev = None
    for k in (1, 2, 4, 8, 16):
        _, s_k, c_k, _ = oracle.decode_step(cache, table, lens, q, 1, 1, k, k_cap)
        mk = oracle.attention_mass(cache, table, lens, q, s_k, c_k)
        if prev is not None:
            assert np.all(mk >= prev - 1e-12)
        prev = mk


def test_attention_mass_dominant_token():
    """One key far along q in page 1 of 3: the closed-form softmax shares of
    page 1 alone and of pages 0 and 2."""
    d = 16
    x = np.zeros((48, d), np.float32)
    x[20, 0] = 40.0
    cache, table = one_token_cache(workloads.FMT_FP16, x)
    q = np.zeros((1, 1, d), np.float16)
    q[0, 0, 0] = 1.0
    lens = np.array([48], np.int32)
    one = oracle.attention_mass(cache, table, lens, q, np.array([[[1, -1, -1]]], np.int32), np.array([[1]], np.int32))
    two = oracle.attention_mass(cache, table, lens, q, np.array([[[0, 2, -1]]], np.int32), np.array([[2]], np.int32))
    # logit 40 / sqrt(16) = 10 for token 20, 0 for the other 47 (15 of them in page 1)
    total = math.exp(10.0) + 47.0
    assert abs(one[0, 0] - (math.exp(10.0) + 15.0) / total) <= 1e-12
    assert abs(two[0, 0] - 32.0 / total) <= 1e-12


def test_selection_quality_report():
    """Selection quality on the synthetic workloads (parity unpinned: the
    pages print no values for it; reported, not graded): the mean share of
    dense attention weight on the top-K pages by score, and on K pages drawn
    at random, at several selection ratios."""
    rng = np.random.default_rng(2024)
    for w in [workloads.small(2), workloads.small(4), workloads.small(5), workloads.config(2), workloads.config(4)]:
        cache, table = oracle.build_cache(w)
        lens = w.seq_lens()
        q = w.query()
        k_cap = table.shape[1]
        row = []
        for num, den in ((1, 10), (2, 10), (3, 10), (5, 10)):
            _, sel, cnt, _ = oracle.decode_step(cache, table, lens, q, num, den, 0, k_cap, nthreads=8)
            top = oracle.attention_mass(cache, table, lens, q, sel, cnt)
            rnd_sel = np.full_like(sel, -1)
            for b in range(w.batch):
                P = (int(lens[b]) + PAGE - 1) // PAGE
                for g in range(w.num_kv_heads):
                    c = int(cnt[b, g])
                    rnd_sel[b, g, :c] = np.sort(rng.choice(P, c, replace=False))
            rnd = oracle.attention_mass(cache, table, lens, q, rnd_sel, cnt)
            live = lens > 0
            row.append(f"rho {num}/{den}: top-K {top[live].mean():.3f}, random {rnd[live].mean():.3f}")
            assert np.all((top >= 0) & (top <= 1 + 1e-12))
        print(f"[quality] {w.name}: " + "; ".join(row))


def test_selection_variants_report():
    """Selection variants on the GQA workload, by the same measure (parity
    unpinned; reported, not graded): the group score as the max of its query
    heads' page scores (the method here) or their sum, and the top-K with the
    first and the last page of each sequence forced in (K stays the same).
    A head's own page scores come from the oracle with that head's query
    copied over its whole group, so the group max is that head's score."""
    w = workloads.small(5).with_(batch=16, len_lo=600, len_hi=4000)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    q = w.query()
    k_cap = table.shape[1]
    G, H = w.group, w.num_kv_heads
    per_head = []
    for hh in range(G):
        qh = q.copy()
        for g in range(H):
            qh[:, g * G:(g + 1) * G] = q[:, g * G + hh][:, None]
        per_head.append(oracle.page_scores(cache, table, lens, qh))
    r_max = oracle.page_scores(cache, table, lens, q)
    assert np.array_equal(r_max, np.maximum.reduce(per_head))   # the group score is the max over its heads
    r_sum = np.sum(per_head, axis=0)
    r_sum[np.isneginf(r_max)] = -np.inf
    out = []
    for num, den in ((1, 10), (3, 10)):
        sel_m, cnt = oracle.topk(r_max, lens, num, den, 0, k_cap)
        sel_s, cnt_s = oracle.topk(r_sum, lens, num, den, 0, k_cap)
        assert np.array_equal(cnt, cnt_s)
        # forced first and last pages: the top K-2 others plus those two
        sel_f = np.full_like(sel_m, -1)
        for b in range(w.batch):
            P = (int(lens[b]) + PAGE - 1) // PAGE
            for g in range(H):
                K = int(cnt[b, g])
                row = r_max[b, g, :P].copy()
                forced = sorted({0, P - 1})[:K]
                row[forced] = -np.inf
                rest = np.lexsort((np.arange(P), -row))[:K - len(forced)]
                sel_f[b, g, :K] = np.sort(np.concatenate([forced, rest]))
        m = [oracle.attention_mass(cache, table, lens, q, s, cnt).mean() for s in (sel_m, sel_s, sel_f)]
        out.append(f"rho {num}/{den}: max {m[0]:.3f}, sum {m[1]:.3f}, max + first/last page {m[2]:.3f}")
    print(f"[variants] {w.name} B=16 L 600-4000: " + "; ".join(out))


def _decoded_keys_upto(w, cache, table, b, L):
    """Decoded keys fp32 [L][H][d] of sequence b's first L tokens as stored."""
    t = np.arange(L)
    kc = cache.k_pages[table[b][t // PAGE], :, t % PAGE]
    if w.fmt == workloads.FMT_FP16:
        return kc.view(np.float16).astype(np.float32)
    p = (cache.params[table[b][t // PAGE], :, t % PAGE] if w.fmt == workloads.FMT_INT8_TOKEN
         else cache.params[table[b][t // PAGE]])
    return np_dequant(kc, p[..., 0:1], p[..., 1:2])


def test_lazy_metadata_refresh_report():
    """A decode stream of 24 steps, one token appended per sequence per step and
    a fresh query each step, with page metadata refreshed every step (as built)
    or every 4th step (the lazy refresh TinyServe section 5.2 suggests).  Counts
    the (sequence, KV head, page) scores that fall below the page's true
    max q.k (the no-underestimate property, TinyServe section 2.1) and the
    selections that differ from the exact-metadata ones.  Exact refresh never
    underestimates (asserted); the lazy figures are reported, not graded."""
    w = workloads.small(4).with_(batch=6, seq_len=0, len_lo=300, len_hi=900)
    T = 24
    lens_end = w.seq_lens().astype(np.int64)
    table, _ = w.block_table()
    L0 = lens_end - T
    rng = np.random.default_rng(77)
    G, H, d = w.group, w.num_kv_heads, w.head_dim
    results = {}
    for every in (1, 4):
        cache, _ = oracle.build_cache(w, upto=L0)
        under = pages = changed = 0
        worst = 0.0
        for t in range(T):
            L = L0 + t + 1
            ks = np.concatenate([w.keys(b)[L[b] - 1:L[b]] for b in range(w.batch)])
            vs = np.concatenate([w.values(b)[L[b] - 1:L[b]] for b in range(w.batch)])
            oracle.append(cache, table, (L - 1).astype(np.int32), np.arange(w.batch + 1, dtype=np.int32), ks, vs)
            if (t + 1) % every == 0:
                oracle.page_meta(cache, table, L.astype(np.int32))
            q = rng.standard_normal((w.batch, w.num_q_heads, d)).astype(np.float16)
            r = oracle.page_scores(cache, table, L, q)
            exact_cache = cache
            if every != 1:  # the exact metadata of the same cache, for the selection comparison
                exact_cache = copy.deepcopy(cache)
                oracle.page_meta(exact_cache, table, L.astype(np.int32))
            r_exact = oracle.page_scores(exact_cache, table, L, q)
            k_cap = table.shape[1]
            s_lazy, c = oracle.topk(r, L, 3, 10, 0, k_cap)
            s_exact, _ = oracle.topk(r_exact, L, 3, 10, 0, k_cap)
            changed += int((s_lazy != s_exact).any(axis=-1).sum())
            for b in range(w.batch):
                K = _decoded_keys_upto(w, cache, table, b, int(L[b])).astype(np.float64)
                P = (int(L[b]) + PAGE - 1) // PAGE
                for g in range(H):
                    qq = q[b, g * G:(g + 1) * G].astype(np.float64)          # [G][d]
                    dots = (K[:, g] @ qq.T).max(axis=1)                      # [L]: max over the group's heads
                    true = np.array([dots[j * PAGE:min((j + 1) * PAGE, int(L[b]))].max() for j in range(P)])
                    gap = true - r[b, g, :P]
                    tol = 1e-9 * (1.0 + np.abs(true))
                    under += int((gap > tol).sum())
                    worst = max(worst, float(gap.max()))
                    pages += P
        results[every] = (under, pages, changed, worst)
    assert results[1][0] == 0 and results[1][2] == 0
    u, p, ch, worst = results[4]
    print(f"[lazy] {w.name}, 6 sequences, 24 steps: refresh every 4th step -> {u} of {p} page scores "
          f"underestimate (worst by {worst:.3g}), {ch} of {T * w.batch * H} selections differ from exact metadata")


# ------------------------------------------------- hierarchical selection
def _unpack4(packed):
    """[..][d/2] bytes -> [..][d] codes: channel 2i is the low nibble of byte i."""
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def _decoded_keys(cache, table, lens, b, g, values=False):
    """float64 [L][d]: sequence b's keys (or values) for KV head g as decoded,
    straight from the storage arrays (fp16 bits, or code * scale + zero
    rounded once)."""
    L = int(lens[b])
    t = np.arange(L)
    phys = table[b, t // PAGE]
    pages = cache.v_pages if values else cache.k_pages
    if cache.fmt == workloads.FMT_FP16:
        return pages[phys, g, t % PAGE].view(np.float16).astype(np.float64)
    codes = pages[phys, g, t % PAGE]
    if cache.fmt in (workloads.FMT_INT4_TOKEN, workloads.FMT_INT4_GROUP64):
        codes = _unpack4(codes)
    sz = (2, 3) if values else (0, 1)
    if cache.fmt in (workloads.FMT_INT8_TOKEN, workloads.FMT_INT4_TOKEN):
        p = cache.params[phys, g, t % PAGE]
    else:
        p = cache.params[phys, g]
    return np_dequant(codes, p[:, sz[0]:sz[0] + 1], p[:, sz[1]:sz[1] + 1]).astype(np.float64)


@pytest.mark.parametrize("n,group", [(4, 8), (5, 4), (2, 16), (5, 1)])
def test_coarse_boxes_are_the_min_max_of_their_tokens(n, group):
    """A super-page's box equals the min / max of the decoded keys of all its
    tokens (brute force over the storage), and past the sequence nothing is
    written."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    cm = oracle.coarse_meta(cache, table, lens, group)
    pc_max = (table.shape[1] + group - 1) // group
    for b in range(w.batch):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        for g in range(w.num_kv_heads):
            k = _decoded_keys(cache, table, lens, b, g)
            for jc in range(pc_max):
                box = cm[b * pc_max + jc, g].astype(np.float64)
                t0, t1 = jc * group * PAGE, min((jc + 1) * group * PAGE, int(lens[b]))
                if jc * group >= P:
                    assert np.all(np.isinf(box)), (b, g, jc)
                    continue
                assert np.array_equal(box[0], k[t0:t1].min(0)) and np.array_equal(box[1], k[t0:t1].max(0))


@pytest.mark.parametrize("n,group", [(4, 8), (5, 4), (2, 8)])
def test_coarse_score_bounds_every_member_page(n, group):
    """The coarse score of a super-page is at least the fine score of every
    page in it (its box contains theirs), so it never underestimates q.k of
    any of its tokens either."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens, q = w.seq_lens(), w.query()
    view, ct, cl = oracle.coarse_view(cache, table, lens, group)
    csc = oracle.page_scores(view, ct, cl, q)
    fine = oracle.page_scores(cache, table, lens, q)
    for b in range(w.batch):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        for j in range(P):
            r = fine[b, :, j]
            R = csc[b, :, j // group]
            assert np.all(R >= r - 1e-9 * np.maximum(1.0, np.abs(r))), (b, j)


@pytest.mark.parametrize("n", [2, 4, 5])
def test_hier_select_reduces_to_flat_top_k(n):
    """Keeping every super-page, or super-pages of one page with at least K
    kept, gives exactly the flat top-K selection; in general the selection
    lies inside the kept super-pages once they hold at least K pages."""
    w = workloads.small(n)
    cache, table = oracle.build_cache(w)
    lens, q = w.seq_lens(), w.query()
    k_cap = table.shape[1]
    flat_sc = oracle.page_scores(cache, table, lens, q)
    fsel, fcnt = oracle.topk(flat_sc, lens, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
    for group in (4, 8):
        pc_max = (k_cap + group - 1) // group
        *_, sel, cnt = oracle.hier_select(cache, table, lens, q, group, pc_max, w.ratio_num, w.ratio_den, w.k_fixed,
                                          k_cap)
        assert np.array_equal(sel, fsel) and np.array_equal(cnt, fcnt)
    *_, sel, cnt = oracle.hier_select(cache, table, lens, q, 1, k_cap, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
    assert np.array_equal(sel, fsel) and np.array_equal(cnt, fcnt)
    group, kc = 4, 3
    csc, csel, ccnt, masked, sel, cnt = oracle.hier_select(cache, table, lens, q, group, kc, w.ratio_num, w.ratio_den,
                                                           w.k_fixed, k_cap)
    for b in range(w.batch):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        for g in range(w.num_kv_heads):
            kept = set(csel[b, g, :ccnt[b, g]].tolist())
            cand = [j for j in range(P) if j // group in kept]
            assert ccnt[b, g] == min(kc, (P + group - 1) // group)
            assert np.all(np.isneginf(masked[b, g, [j for j in range(P) if j not in cand]]))
            assert np.array_equal(masked[b, g, cand], flat_sc[b, g, cand])
            chosen = sel[b, g, :cnt[b, g]].tolist()
            if len(cand) >= cnt[b, g]:
                assert set(chosen) <= set(cand)
            # the kept super-pages are the kc best coarse scores
            order = sorted(range((P + group - 1) // group), key=lambda jc: (-csc[b, g, jc], jc))
            assert kept == set(order[:kc])


def test_hier_select_recall_report():
    """Coarse-then-fine selection on the synthetic workloads (parity
    unpinned, reported): the share of the flat top-K pages it keeps, the
    share of dense attention weight on its pages beside flat top-K's, and
    the metadata it reads (coarse boxes + the kept super-pages' pages) as a
    share of all pages' metadata, for super-pages of 8 pages keeping 20-60%
    of them."""
    for w in [workloads.config(2), workloads.config(4), workloads.small(5).with_(batch=16, len_lo=600, len_hi=4000)]:
        cache, table = oracle.build_cache(w)
        lens, q = w.seq_lens(), w.query()
        k_cap = table.shape[1]
        flat = oracle.page_scores(cache, table, lens, q)
        fsel, fcnt = oracle.topk(flat, lens, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
        flat_mass = oracle.attention_mass(cache, table, lens, q, fsel, fcnt)
        group = 8
        P = (lens.astype(np.int64) + PAGE - 1) // PAGE
        Pc = (P + group - 1) // group
        row = [f"flat mass {flat_mass.mean():.3f}"]
        for frac in (0.2, 0.4, 0.6):
            kc = int(np.ceil(frac * Pc.max()))
            *_, sel, cnt = oracle.hier_select(cache, table, lens, q, group, kc, w.ratio_num, w.ratio_den, w.k_fixed,
                                              k_cap)
            hit = tot = 0
            for b in range(w.batch):
                for g in range(w.num_kv_heads):
                    K = int(fcnt[b, g])
                    hit += len(set(sel[b, g, :K].tolist()) & set(fsel[b, g, :K].tolist()))
                    tot += K
            mass = oracle.attention_mass(cache, table, lens, q, sel, cnt)
            read = (Pc.sum() + np.minimum(kc, Pc).sum() * group) / P.sum()
            row.append(f"keep {frac:.0%}: recall {hit / tot:.3f}, mass {mass.mean():.3f}, metadata {read:.2f}")
        print(f"[hier] {w.name}: " + "; ".join(row))



# ------------------------------------------------------------ 4-bit codes
def test_quant4_golden_rows():
    """Hand-worked 4-bit rows pin the scale (range / 15), zero, round half to
    even, clamping, and the nibble order of the packed bytes."""
    for row in gold("quant_rows_int4.json")["rows"]:
        x = np.array([row["x"]], np.float16)
        cache, table = one_token_cache(workloads.FMT_INT4_TOKEN, x)
        packed = cache.k_pages[0, 0, 0, :x.shape[1] // 2]
        assert packed.tolist() == row["bytes"], row["derivation"]
        assert _unpack4(packed).tolist() == row["codes"]
        s, z = cache.params[0, 0, 0, 0], cache.params[0, 0, 0, 1]
        assert s == np.float32(row["scale"]) and z == np.float32(row["zero"])
        assert np_dequant(_unpack4(packed), s, z).tolist() == [float(v) for v in row["decoded"]]


@pytest.mark.parametrize("d", [64, 128])
def test_quant4_error_within_half_scale_and_nearest_code(d):
    """|x - decode(code)| <= scale/2 (+fp32 slack) with scale = range / 15,
    the code is the nearest of its neighbours, min -> 0 decoding to min
    exactly, max -> 15."""
    rng = np.random.default_rng(17)
    x = _random_rows(rng, 200, d)
    cache, table = one_token_cache(workloads.FMT_INT4_TOKEN, x)
    L = x.shape[0]
    t = np.arange(L)
    codes = _unpack4(cache.k_pages[t // PAGE, 0, t % PAGE]).astype(np.int64)
    p = cache.params[t // PAGE, 0, t % PAGE]
    s, z = p[:, 0], p[:, 1]
    xf = x.astype(np.float32)
    lo, hi = xf.min(1), xf.max(1)
    assert np.array_equal(z, lo)
    const = hi == lo
    assert np.allclose(s[~const].astype(np.float64), (hi - lo)[~const].astype(np.float64) / 15.0, rtol=2 ** -22)
    dec = np_dequant(codes, s[:, None], z[:, None]).astype(np.float64)
    err = np.abs(xf.astype(np.float64) - dec)
    ulp = np.spacing(np.maximum(np.abs(lo), np.abs(hi)).astype(np.float32)).astype(np.float64)
    slack = 2 * ulp + 15 * s.astype(np.float64) * 2 ** -22
    assert np.all(err <= s[:, None] / 2 + slack[:, None])
    for dc in (-1, 1):
        nb = np.clip(codes + dc, 0, 15)
        dn = np.abs(xf - np_dequant(nb, s[:, None], z[:, None])).astype(np.float64)
        assert np.all(err <= dn + slack[:, None])
    assert np.all(codes.max(1)[~const] == 15) and np.all(codes.min(1) == 0)


@pytest.mark.parametrize("fmt", [workloads.FMT_INT4_TOKEN, workloads.FMT_INT4_GROUP64])
def test_int4_cache_metadata_scores_and_dense_attention(fmt):
    """On 4-bit caches: metadata is the brute-force min/max of the decoded
    keys; every page score bounds its tokens' q.k; per-group storage shares
    one (scale, zero) over each 64-token group; K = P equals numpy's dense
    softmax attention over the decoded keys and values."""
    w = workloads.small(5).with_(fmt=fmt)
    cache, table = oracle.build_cache(w)
    lens, q = w.seq_lens(), w.query()
    sc = oracle.page_scores(cache, table, lens, q)
    out = oracle.attention(cache, table, lens, q)
    G = w.group
    for b in range(w.batch):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        for g in range(w.num_kv_heads):
            k = _decoded_keys(cache, table, lens, b, g)
            v = _decoded_keys(cache, table, lens, b, g, values=True)
            for j in range(P):
                kj = k[16 * j:16 * (j + 1)]
                m = cache.meta[table[b, j], g].astype(np.float64)
                assert np.array_equal(m[0], kj.min(0)) and np.array_equal(m[1], kj.max(0))
                for hh in range(G):
                    qh = q[b, g * G + hh].astype(np.float64)
                    assert sc[b, g, j] >= (kj @ qh).max() - 1e-9 * (1 + np.abs(sc[b, g, j]))
            if fmt == workloads.FMT_INT4_GROUP64 and len(k):
                t = np.arange(int(lens[b]))
                pr = cache.params[table[b, t // PAGE], g]
                for g0 in range(0, int(lens[b]), 64):
                    assert (pr[g0:g0 + 64] == pr[g0]).all()
            for hh in range(G):
                qh = q[b, g * G + hh].astype(np.float64)
                if len(k):
                    lg = k @ qh / np.sqrt(w.head_dim)
                    p_ = np.exp(lg - lg.max())
                    ref = p_ @ v / p_.sum()
                    assert np.allclose(out[b, g * G + hh], ref, rtol=0, atol=1e-12)


# ------------------------------------------------- mixed-precision pages
def _pools(cache, values=False):
    """(FP16 pool [n16][H][16][d] fp16 bits, INT8 pool [P-n16][H][16][d]) of a
    MIXED cache, as views of its one byte array."""
    raw = cache.v_pages if values else cache.k_pages
    tile = cache.H * PAGE * cache.d
    p16 = raw[: cache.n16 * tile * 2].view(np.uint16).reshape(cache.n16, cache.H, PAGE, cache.d)
    p8 = raw[cache.n16 * tile * 2:].reshape(cache.P_phys - cache.n16, cache.H, PAGE, cache.d)
    return p16, p8


def _decoded_mixed(cache, table, lens, b, g, values=False):
    """float64 [L][d]: a MIXED cache's keys (values) for (b, g), page by page
    from the pool the block table points into."""
    p16, p8 = _pools(cache, values)
    sz = (2, 3) if values else (0, 1)
    rows = []
    for t in range(int(lens[b])):
        phys, slot = int(table[b, t // PAGE]), t % PAGE
        if phys < cache.n16:
            rows.append(p16[phys, g, slot].view(np.float16).astype(np.float64))
        else:
            p = cache.params[phys - cache.n16, g, slot]
            rows.append(np_dequant(p8[phys - cache.n16, g, slot], p[sz[0]], p[sz[1]]).astype(np.float64))
    return np.array(rows).reshape(int(lens[b]), cache.d)


def test_mixed_is_the_splice_of_fp16_and_int8_caches():
    """A mixed-precision cache holds, page for page, exactly what an fp16 cache
    (for its FP16-pool pages) or an INT8-per-token cache (for the others) of
    the same tokens holds: codes, scale/zero bits and metadata."""
    w = workloads.small(5).with_(fmt=workloads.FMT_MIXED, hot_recent=5)
    cm, table = oracle.build_cache(w)
    assert 0 < cm.n16 < cm.P_phys
    c16, t16 = oracle.build_cache(w.with_(fmt=workloads.FMT_FP16))
    c8, t8 = oracle.build_cache(w.with_(fmt=workloads.FMT_INT8_TOKEN))
    p16, p8 = _pools(cm)
    v16, v8 = _pools(cm, values=True)
    P = w.pages_per_seq()
    n_hot = 0
    for b in range(w.batch):
        hot = w.hot_pages(b)
        for j in range(int(P[b])):
            phys = int(table[b, j])
            assert (phys < cm.n16) == bool(hot[j])
            if phys < cm.n16:
                n_hot += 1
                assert np.array_equal(p16[phys], c16.k_pages[t16[b, j]])
                assert np.array_equal(v16[phys], c16.v_pages[t16[b, j]])
                assert np.array_equal(cm.meta[phys], c16.meta[t16[b, j]])
            else:
                i = phys - cm.n16
                assert np.array_equal(p8[i], c8.k_pages[t8[b, j]]) and np.array_equal(v8[i], c8.v_pages[t8[b, j]])
                assert np.array_equal(cm.params[i].view(np.uint32), c8.params[t8[b, j]].view(np.uint32))
                assert np.array_equal(cm.meta[phys], c8.meta[t8[b, j]])
    assert 0 < n_hot < int(P.sum())


def test_mixed_with_one_pool_reduces_to_that_format():
    """n16 = 0 (every page INT8) stores the bytes, scale/zero and metadata of
    an INT8-per-token cache; n16 = P (every page FP16) those of an fp16 cache;
    attention agrees with theirs exactly."""
    w = workloads.small(4).with_(seq_len=300)
    table, n_phys = w.with_(fmt=workloads.FMT_INT8_TOKEN).block_table()
    lens, q = w.seq_lens(), w.query()
    for fmt, n16 in [(workloads.FMT_INT8_TOKEN, 0), (workloads.FMT_FP16, n_phys)]:
        ref = oracle.Cache(fmt, n_phys, w.num_kv_heads, w.head_dim)
        mix = oracle.Cache(workloads.FMT_MIXED, n_phys, w.num_kv_heads, w.head_dim, n16)
        for c in (ref, mix):
            for b in range(w.batch):
                off = np.zeros(w.batch + 1, np.int32)
                off[b + 1:] = lens[b]
                oracle.append(c, table, np.zeros(w.batch, np.int32), off, w.keys(b), w.values(b))
            oracle.page_meta(c, table, lens)
        assert np.array_equal(mix.k_pages.view(np.uint8), ref.k_pages.reshape(-1).view(np.uint8))
        assert np.array_equal(mix.v_pages.view(np.uint8), ref.v_pages.reshape(-1).view(np.uint8))
        if fmt == workloads.FMT_INT8_TOKEN:
            assert np.array_equal(mix.params.view(np.uint32), ref.params.view(np.uint32))
        assert np.array_equal(mix.meta, ref.meta)
        assert np.array_equal(oracle.attention(mix, table, lens, q), oracle.attention(ref, table, lens, q))


def test_mixed_metadata_scores_and_attention_by_brute_force():
    """On a mixed cache: each page's metadata is the min/max of its decoded
    keys taken from its own pool, its score bounds every token's q.k, and
    attention over every page equals numpy's dense softmax over those
    decoded keys and values; over a selection, numpy's softmax restricted to
    the selected pages' tokens."""
    w = workloads.small(5).with_(fmt=workloads.FMT_MIXED, hot_recent=5)
    cache, table = oracle.build_cache(w)
    lens, q = w.seq_lens(), w.query()
    sc = oracle.page_scores(cache, table, lens, q)
    out = oracle.attention(cache, table, lens, q)
    k_cap = table.shape[1]
    sel, cnt = oracle.topk(sc, lens, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
    out_sel = oracle.attention(cache, table, lens, q, sel, cnt)
    G = w.group
    for b in range(w.batch):
        P = (int(lens[b]) + PAGE - 1) // PAGE
        for g in range(w.num_kv_heads):
            k = _decoded_mixed(cache, table, lens, b, g)
            v = _decoded_mixed(cache, table, lens, b, g, values=True)
            for j in range(P):
                kj = k[16 * j:16 * (j + 1)]
                m = cache.meta[table[b, j], g].astype(np.float64)
                assert np.array_equal(m[0], kj.min(0)) and np.array_equal(m[1], kj.max(0))
                for hh in range(G):
                    qh = q[b, g * G + hh].astype(np.float64)
                    assert sc[b, g, j] >= (kj @ qh).max() - 1e-9 * (1 + np.abs(sc[b, g, j]))
            keep = np.zeros(int(lens[b]), bool)
            for j in sel[b, g, :cnt[b, g]]:
                keep[16 * j:16 * (j + 1)] = True
            for hh in range(G):
                qh = q[b, g * G + hh].astype(np.float64)
                if not len(k):
                    continue
                for o, mask in ((out, np.ones_like(keep)), (out_sel, keep)):
                    lg = k[mask] @ qh / np.sqrt(w.head_dim)
                    p_ = np.exp(lg - lg.max())
                    assert np.allclose(o[b, g * G + hh], p_ @ v[mask] / p_.sum(), rtol=0, atol=1e-12)


def test_demote_equals_building_the_page_in_int8():
    """Demoting FP16 pages of a mixed cache to spare INT8 pages leaves the cache
    a build with those pages in the INT8 pool from the start would give
    (codes, scale/zero bits, metadata), points the block table at the new
    pages, and rejects a page that is not in the FP16 pool."""
    w = workloads.small(5).with_(fmt=workloads.FMT_MIXED, hot_recent=5, spare_pages=6)
    cache, table = oracle.build_cache(w)
    lens = w.seq_lens()
    P = w.pages_per_seq()
    # the first page of three sequences and the last page of one (partial)
    picks = [(b, 0) for b in range(3) if P[b] > 0] + [(3, int(P[3]) - 1)]
    seq = [b for b, _ in picks]
    page = [j for _, j in picks]
    dst = list(range(cache.P_phys - len(picks), cache.P_phys))
    t2 = table.copy()
    before16 = _pools(cache)[0].copy()
    oracle.demote(cache, t2, lens, seq, page, dst)
    for (b, j), dd in zip(picks, dst):
        assert t2[b, j] == dd
    assert np.array_equal(np.delete(t2.reshape(-1), [b * t2.shape[1] + j for b, j in picks]),
                          np.delete(table.reshape(-1), [b * table.shape[1] + j for b, j in picks]))
    # the same tokens built with those pages in the INT8 pool from the start
    ref = oracle.Cache(workloads.FMT_MIXED, cache.P_phys, w.num_kv_heads, w.head_dim, cache.n16)
    for b in range(w.batch):
        off = np.zeros(w.batch + 1, np.int32)
        off[b + 1:] = lens[b]
        oracle.append(ref, t2, np.zeros(w.batch, np.int32), off, w.keys(b), w.values(b))
    oracle.page_meta(ref, t2, lens)
    r8 = _pools(ref)[1]
    c16, c8 = _pools(cache)
    for dd in dst:
        i = dd - cache.n16
        assert np.array_equal(c8[i], r8[i]) and np.array_equal(_pools(cache, True)[1][i], _pools(ref, True)[1][i])
        assert np.array_equal(cache.params[i].view(np.uint32), ref.params[i].view(np.uint32))
        assert np.array_equal(cache.meta[dd], ref.meta[dd])
    assert np.array_equal(c16, before16)   # the FP16 pool (the old pages too) is left as it was
    q = w.query()
    assert np.array_equal(oracle.attention(cache, t2, lens, q), oracle.attention(ref, t2, lens, q))
    with pytest.raises(ValueError):   # that page is in the INT8 pool now
        oracle.demote(cache, t2, lens, [seq[0]], [page[0]], [dst[0]])
