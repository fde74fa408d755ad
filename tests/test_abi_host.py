"""Host-only checks of libkvq's C ABI: the library loads, exports every
function include/kvq.h declares, sizes workspaces, and rejects bad arguments
with the documented status before touching the GPU.  No kernel runs here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
LIB = os.path.join(ROOT, "paged_quantized_sparse_amd", "libkvq.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvq_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libkvq.so not built")
    import paged_quantized_sparse_amd as kvq
    return kvq.lib()


def test_header_declares_the_five_decode_step_calls():
    names = declared_functions()
    for f in ("kvq_append_quant", "kvq_build_page_meta", "kvq_page_scores", "kvq_topk_pages",
              "kvq_sparse_decode_attn"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for f in names:
        assert hasattr(lib, f), f
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    assert set(names) <= exported


def test_library_never_allocates_or_synchronizes():
    """The ABI promises no allocation and no synchronization: the library
    imports no HIP allocator, free or device/stream synchronize."""
    if not os.path.exists(LIB):
        pytest.skip("libkvq.so not built")
    out = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True, check=True).stdout
    banned = re.compile(r"\b(hipMalloc\w*|hipFree\w*|hipHostMalloc|hipDeviceSynchronize|hipStreamSynchronize|"
                        r"hipMemcpy\b|hipMemset\b|hipExtMallocWithFlags|hipMallocAsync)\b")
    assert not banned.findall(out), banned.findall(out)


def test_version_and_status_strings(lib):
    assert lib.kvq_abi_version() == 8
    assert "#define KVQ_ABI_VERSION 8" in open(HEADER).read()
    for s, word in [(0, b"ok"), (1, b"invalid"), (2, b"unsupported"), (3, b"workspace"), (4, b"HIP"), (99, b"unknown")]:
        assert word in lib.kvq_status_string(s)


def test_workspace_bytes(lib):
    # B * Hq * ceil(cap / pps) * (d + 2) * 4
    assert lib.kvq_attn_workspace_bytes(1, 32, 128, 2048, 615, 16) == 1 * 32 * 39 * 130 * 4
    assert lib.kvq_attn_workspace_bytes(4, 32, 128, 128, 0, 8) == 4 * 32 * 16 * 130 * 4
    assert lib.kvq_attn_workspace_bytes(0, 32, 128, 128, 0, 8) == 0
    assert lib.kvq_attn_workspace_bytes(1, 32, 128, 128, 0, 0) == 0
    pps = lib.kvq_default_pages_per_split(1, 32, 2048, 615)
    assert pps == 40   # ceil(32 * 615 / 512) = 39, rounded up to a multiple of 4
    assert lib.kvq_default_pages_per_split(1, 4, 64, 16) == 24      # the minimum: one split of K = 16
    assert lib.kvq_default_pages_per_split(1, 16, 1024, 308) == 24   # 16 rows of 308 pages
    assert lib.kvq_default_pages_per_split(64, 8, 2048, 615) == 128


def _structs(fmt=1, page=16, d=128, H=4, B=1, maxp=8, meta=True):
    import paged_quantized_sparse_amd as kvq
    c = kvq.CacheStruct(fmt, 64, page, H, d, FAKE, FAKE, FAKE, FAKE if meta else None)
    s = kvq.SeqsStruct(B, maxp, FAKE, FAKE)
    return c, s


def _attn(lib, c, s, hq=4, sel=FAKE, cnt=FAKE, k_cap=3, pps=8, ws=FAKE, ws_bytes=1 << 30, q=FAKE, scale=0.1):
    return lib.kvq_sparse_decode_attn(ctypes.byref(c), ctypes.byref(s), q, hq, sel, cnt, k_cap, scale, pps, FAKE,
                                      ws, ws_bytes, None)


def test_attention_argument_errors(lib):
    c, s = _structs()
    assert lib.kvq_sparse_decode_attn(None, ctypes.byref(s), FAKE, 4, None, None, 0, 0.1, 8, FAKE, FAKE, 1 << 20,
                                      None) == INVALID
    assert _attn(lib, c, s, hq=6) == INVALID                 # H_q not a multiple of H_kv
    assert _attn(lib, c, s, hq=12) == UNSUPPORTED            # group size 3
    assert _attn(lib, c, s, hq=64) == UNSUPPORTED            # group size 16: past the supported 1, 2, 4, 8
    assert _attn(lib, c, s, cnt=None) == INVALID             # selection without counts
    assert _attn(lib, c, s, k_cap=0) == INVALID
    assert _attn(lib, c, s, pps=5000) == INVALID
    assert _attn(lib, c, s, q=FAKE + 2) == INVALID           # misaligned query
    assert _attn(lib, c, s, ws=None) == WORKSPACE
    assert _attn(lib, c, s, ws_bytes=16) == WORKSPACE
    assert _attn(lib, c, s, scale=float("nan")) == INVALID
    c2, s2 = _structs(page=8)
    assert _attn(lib, c2, s2) == UNSUPPORTED
    c3, s3 = _structs(d=96)
    assert _attn(lib, c3, s3) == UNSUPPORTED
    c4, s4 = _structs(fmt=7)
    assert _attn(lib, c4, s4) == UNSUPPORTED
    for fmt in (3, 4):   # 4-bit storage is built for head_dim 128 only
        c6, s6 = _structs(fmt=fmt, d=64)
        assert _attn(lib, c6, s6) == UNSUPPORTED
    c5, s5 = _structs(B=0)
    assert _attn(lib, c5, s5) == INVALID


def test_stage_argument_errors(lib):
    c, s = _structs()
    # append: null offsets, negative max_new, missing rows
    assert lib.kvq_append_quant(ctypes.byref(c), ctypes.byref(s), None, FAKE, 1, FAKE, FAKE, None) == INVALID
    assert lib.kvq_append_quant(ctypes.byref(c), ctypes.byref(s), FAKE, FAKE, -1, FAKE, FAKE, None) == INVALID
    assert lib.kvq_append_quant(ctypes.byref(c), ctypes.byref(s), FAKE, FAKE, 4, None, FAKE, None) == INVALID
    c_nop, _ = _structs()
    c_nop.kv_params = None
    assert lib.kvq_append_quant(ctypes.byref(c_nop), ctypes.byref(s), FAKE, FAKE, 1, FAKE, FAKE, None) == INVALID
    # metadata needs the metadata array
    cm, sm = _structs(meta=False)
    assert lib.kvq_build_page_meta(ctypes.byref(cm), ctypes.byref(sm), None, 0, None) == INVALID
    assert lib.kvq_build_page_meta(ctypes.byref(c), ctypes.byref(s), None, -1, None) == INVALID
    # scores
    assert lib.kvq_page_scores(ctypes.byref(c), ctypes.byref(s), FAKE, 5, FAKE, None) == INVALID
    assert lib.kvq_page_scores(ctypes.byref(c), ctypes.byref(s), None, 4, FAKE, None) == INVALID
    # top-K: k_cap below K(max_pages), bad ratio, over-long rows
    assert lib.kvq_topk_pages(FAKE, ctypes.byref(s), 4, 3, 10, 0, 2, FAKE, FAKE, None) == INVALID   # K(8) = 3
    assert lib.kvq_topk_pages(FAKE, ctypes.byref(s), 4, 0, 10, 0, 8, FAKE, FAKE, None) == INVALID
    assert lib.kvq_topk_pages(FAKE, ctypes.byref(s), 4, 3, 10, -1, 8, FAKE, FAKE, None) == INVALID
    _, s_long = _structs(maxp=20000)
    assert lib.kvq_topk_pages(FAKE, ctypes.byref(s_long), 4, 3, 10, 0, 8000, FAKE, FAKE, None) == UNSUPPORTED


def test_mixed_precision_argument_errors(lib):
    """A mixed-precision cache needs 0 <= num_fp16_pages <= P_phys; demotion
    takes only that format, a non-negative count and its three arrays; a
    count of 0 enqueues nothing."""
    for n16 in (-1, 65):   # P_phys is 64
        c, s = _structs(fmt=5)
        c.num_fp16_pages = n16
        assert lib.kvq_build_page_meta(ctypes.byref(c), ctypes.byref(s), None, 0, None) == INVALID
        assert lib.kvq_demote_pages(ctypes.byref(c), ctypes.byref(s), 1, FAKE, FAKE, FAKE, None) == INVALID
    c, s = _structs(fmt=1)
    assert lib.kvq_demote_pages(ctypes.byref(c), ctypes.byref(s), 1, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    c, s = _structs(fmt=5)
    c.num_fp16_pages = 16
    assert lib.kvq_demote_pages(ctypes.byref(c), ctypes.byref(s), -1, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.kvq_demote_pages(ctypes.byref(c), ctypes.byref(s), 2, FAKE, None, FAKE, None) == INVALID
    assert lib.kvq_demote_pages(ctypes.byref(c), ctypes.byref(s), 0, None, None, None, None) == 0
    # the one-launch step takes fp16 and INT8 storage only
    for fmt in (3, 5):
        c, s = _structs(fmt=fmt)
        assert lib.kvq_decode_step(ctypes.byref(c), ctypes.byref(s), FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, FAKE,
                                   3, 10, 0, 8, FAKE, FAKE, 0.1, 0, FAKE, None, 1 << 30, None) == UNSUPPORTED


def test_coarse_then_fine_argument_errors(lib):
    """Super-page boxes need 1 <= group_pages <= 64, a non-negative span and
    their three arrays; the masked scorer needs its selection and a valid
    query-head count."""
    c, s = _structs()
    build = lib.kvq_build_coarse_meta
    assert build(ctypes.byref(c), ctypes.byref(s), 0, None, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert build(ctypes.byref(c), ctypes.byref(s), 65, None, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert build(ctypes.byref(c), ctypes.byref(s), 8, FAKE, -1, FAKE, FAKE, FAKE, None) == INVALID
    assert build(ctypes.byref(c), ctypes.byref(s), 8, None, 0, None, FAKE, FAKE, None) == INVALID
    cm, sm = _structs(meta=False)
    assert build(ctypes.byref(cm), ctypes.byref(sm), 8, None, 0, FAKE, FAKE, FAKE, None) == INVALID
    masked = lib.kvq_page_scores_masked
    assert masked(ctypes.byref(c), ctypes.byref(s), FAKE, 5, 8, FAKE, FAKE, 4, FAKE, None) == INVALID


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import paged_quantized_sparse_amd as kvq
    monkeypatch.setattr(kvq, "_lib", None)
    monkeypatch.setattr(kvq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="libkvq.so not found"):
        kvq.lib()


def _sel_attn(lib, c, s, hq=4, scores=FAKE, rn=3, rd=10, kf=0, k_cap=3, sel=None, cnt=None, pps=8, ws=FAKE,
              ws_bytes=1 << 30, q=FAKE, scale=0.1):
    return lib.kvq_select_decode_attn(ctypes.byref(c), ctypes.byref(s), q, hq, scores, rn, rd, kf, k_cap, sel, cnt,
                                      scale, pps, FAKE, ws, ws_bytes, None)


def test_select_attention_argument_errors(lib):
    c, s = _structs()                                        # max_pages 8: K(8) = 3 at 3/10
    assert _sel_attn(lib, c, s, scores=None) == INVALID
    assert _sel_attn(lib, c, s, k_cap=2) == INVALID          # below K(max_pages)
    assert _sel_attn(lib, c, s, rn=0) == INVALID
    assert _sel_attn(lib, c, s, kf=-1) == INVALID
    assert _sel_attn(lib, c, s, sel=FAKE) == INVALID         # selection copy without its counts
    assert _sel_attn(lib, c, s, hq=12) == UNSUPPORTED        # group size 3
    assert _sel_attn(lib, c, s, pps=5000) == INVALID
    assert _sel_attn(lib, c, s, q=FAKE + 2) == INVALID
    assert _sel_attn(lib, c, s, ws=None) == WORKSPACE
    assert _sel_attn(lib, c, s, ws_bytes=16) == WORKSPACE
    _, s_long = _structs(maxp=2049)
    assert _sel_attn(lib, c, s_long, k_cap=2049) == UNSUPPORTED  # rows over KVQ_SELECT_MAX_PAGES


def test_select_limit_matches_header():
    import paged_quantized_sparse_amd as kvq
    assert f"#define KVQ_SELECT_MAX_PAGES {kvq.SELECT_MAX_PAGES} " in open(HEADER).read()


def test_bench_refuses_more_than_one_gpu():
    """The decode step runs on one GPU; bench.py says so for --gpus N > 1
    before it touches a device."""
    r = subprocess.run(["python", os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_num_selected_rule_matches_oracle(lib):
    """The library's K rule (kvq_num_selected, which also sizes k_cap in the
    binding) equals the oracle's on every row length up to 2048 pages and on
    the fixed-K and ratio-1 cases; degenerate rows select nothing."""
    import oracle
    for P in range(0, 2049):
        for rn, rd, kf in ((3, 10, 0), (1, 1, 0), (1, 7, 0), (0, 1, 16), (0, 1, 5000)):
            assert lib.kvq_num_selected(P, rn, rd, kf) == oracle.num_selected(P, rn, rd, kf), (P, rn, rd, kf)
    assert lib.kvq_num_selected(2048, 3, 10, 0) == 615
    assert lib.kvq_num_selected(1024, 3, 10, 0) == 308
    assert lib.kvq_num_selected(-5, 3, 10, 0) == 0


def test_noalloc_attention_rejects_sizes_beyond_its_scratch(lib):
    """kvq_select_decode_attn_noalloc checks its arguments like the workspace
    call and refuses sizes whose partials exceed KVQ_NOALLOC_SCRATCH_BYTES
    before any device work; the limit in the header is the binding's."""
    import paged_quantized_sparse_amd as kvq
    assert f"#define KVQ_NOALLOC_SCRATCH_BYTES ({kvq.NOALLOC_SCRATCH_BYTES >> 20}u << 20)" in open(HEADER).read()

    def call(c, s, hq=4, k_cap=3, pps=8, q=FAKE):
        return lib.kvq_select_decode_attn_noalloc(ctypes.byref(c), ctypes.byref(s), q, hq, FAKE, 3, 10, 0, k_cap,
                                                  None, None, 0.1, pps, FAKE, None)
    c, s = _structs()
    assert call(c, s, k_cap=2) == INVALID
    assert call(c, s, hq=12) == UNSUPPORTED
    assert call(c, s, q=FAKE + 2) == INVALID
    _, big = _structs(B=60000, maxp=2048)                     # 60000 x 4 heads x 2048 pages: far beyond 16 MiB
    assert call(c, big, k_cap=2048, pps=1) == WORKSPACE
