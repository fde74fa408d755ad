"""Decode-step benchmark: paged, INT8, query-aware sparse attention at 32K context.

One step = the whole hot path for one layer of the Llama-2-7B-shaped workload
(1 sequence, 32 heads, head_dim 128, 32768 tokens in 16-token pages, INT8 per
token, selection ratio 0.3 -> 615 of 2048 pages per head):
  append the newest token (quantize into its page) and refresh that page's
  metadata, fused into scoring all pages -> top-K inside the split-K
  attention kernel -> split combine.
Steps rotate over `--layers` independent copies of the layer cache (distinct
device buffers), so a step never finds the previous step's working set in the
256 MB Infinity Cache, as in a real decode pass over many layers.

Prints one JSON line:
  * achieved GB/s of the whole step (metadata of every page + the selected KV
    tiles with their scale/zero, i.e. the bytes the method must read) and
    microseconds per step, with its p10/p50/p90 over rotations;
  * `roofline`: the attention call exactly as the step runs it (selection
    inside the split-K kernel, then the split combine), HIP events on its
    launch stream around HIP-graph replays, against the 8 TB/s HBM peak;
  * secondary figures, each timed the same way (graph replays, HIP events):
    the attention over a given selection (no in-kernel selection), the fused
    append + scores kernel, the decode-time append alone, the one-time cache
    build (quantize + metadata of the whole prefill), and what a plain
    streaming-read kernel reaches over 2 GiB on this GPU;
  * the CPU oracle timed on the host on the same workload (all threads this
    process may use, up to 16, and one thread), the oracle's own cache build,
    and parity statistics of this run's step against the oracle.
"""
from __future__ import annotations

import argparse
import functools
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(w, k_per_row, n_fp16_tiles=0):
    """(metadata bytes of every page, selected KV bytes): each (page, KV head)
    counted once; a quantized tile carries its codes (a byte per channel, or
    half a byte for 4-bit codes) and its fp32 scale/zero.  A mixed-precision
    cache's selected tiles are INT8 per token except n_fp16_tiles fp16 ones."""
    import workloads
    d = w.head_dim
    pages = w.pages_per_seq().astype(np.int64)
    meta = int(pages.sum()) * w.num_kv_heads * 8 * d
    int4 = w.fmt in (workloads.FMT_INT4_TOKEN, workloads.FMT_INT4_GROUP64)
    codes = 2 * 16 * (d // 2 if int4 else d)
    fp16_tile = 2 * 16 * d * 2
    if w.fmt == workloads.FMT_FP16:
        tile = fp16_tile
    elif w.fmt in (workloads.FMT_INT8_TOKEN, workloads.FMT_INT4_TOKEN, workloads.FMT_MIXED):
        tile = codes + 16 * 16
    else:
        tile = codes + 16
    n = int(np.asarray(k_per_row, np.int64).sum())
    return meta, (n - n_fp16_tiles) * tile + n_fp16_tiles * fp16_tile


def fp16_tiles(w, table, sel, cnt):
    """Selected (page, KV head) tiles of a mixed-precision cache that lie in its
    FP16 pool (sel None: every page)."""
    n16 = w.fp16_pool_pages()
    if not n16:
        return 0
    P = w.pages_per_seq()
    tot = 0
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            pages = np.arange(P[b]) if sel is None else sel[b, g, :cnt[b, g]]
            tot += int((table[b, pages] < n16).sum())
    return tot


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "decode_attn_cfg4_traffic.json")


def measured_traffic():
    """HBM bytes per call of the step's attention (selecting split kernel +
    combine) from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE record, or
    None once its sources changed."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        h = hashlib.sha256()
        for p in rec["sources"]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec["read_bytes"]) + int(rec["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, seconds: float, threads: int, built):
    """The oracle's decode step (scores -> top-K -> attention) on host threads;
    (median seconds, runs, last result)."""
    import oracle
    cache, table = built
    lens, q = w.seq_lens(), w.query()
    k_cap = oracle.num_selected(int(table.shape[1]), w.ratio_num, w.ratio_den, w.k_fixed)
    times = []
    res = None
    t_end = time.perf_counter() + seconds
    while True:
        t0 = time.perf_counter()
        res = oracle.decode_step(cache, table, lens, q, w.ratio_num, w.ratio_den, w.k_fixed, k_cap, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() > t_end or len(times) >= 20:
            break
    return float(np.median(times)), len(times), res


def parity_stats(w, built, oracle_step, gpu):
    """This run's step against the oracle on the same inputs: cache codes and
    metadata, scores, selection (near-tie rule) and output."""
    import oracle
    cache, table = built
    lens, q = w.seq_lens(), w.query()
    osc, osel, ocnt, oout = oracle_step
    st = {}
    k = gpu["k_pages"]
    st["k_codes_bit_exact"] = bool(np.array_equal(k.view(np.uint16) if k.dtype == np.int16 else k, cache.k_pages))
    st["metadata_exact"] = bool(np.array_equal(gpu["meta"], cache.meta))
    fin = np.isfinite(osc)
    st["scores_max_rel_err"] = float(np.max(np.abs(gpu["scores"][fin] - osc[fin]) / np.maximum(np.abs(osc[fin]),
                                                                                               1e-30)))
    sel, cnt = gpu["sel"], gpu["cnt"]
    rows = same = swaps = 0
    for b in range(sel.shape[0]):
        for g in range(sel.shape[1]):
            K = int(ocnt[b, g])
            rows += 1
            d = set(sel[b, g, :K].tolist()) ^ set(osel[b, g, :K].tolist())
            same += not d and int(cnt[b, g]) == K
            swaps += len(d) // 2
    st["selection_rows_identical"] = f"{same}/{rows}"
    st["near_tie_page_swaps"] = swaps
    want = oracle.attention(cache, table, lens, q, sel, cnt)
    st["out_max_abs_err"] = float(np.abs(gpu["out"].astype(np.float64) - want).max())
    st["out_max_abs_err_vs_oracle_step"] = float(np.abs(gpu["out"].astype(np.float64) - oout).max())
    st["tolerance"] = 2e-3
    return st


def hier_parity_stats(w, built, hs, gpu):
    """The coarse-then-fine step against the oracle: kept super-pages (equal
    to the oracle's on its own coarse scores, up to near-ties), the fine
    selection (near-tie rule on the oracle's masked scores), the output (the
    oracle's attention over the GPU's selection), and the recall of the flat
    top-K (share of its pages the coarse-then-fine selection keeps)."""
    import oracle
    cache, table = built
    lens, q = w.seq_lens(), w.query()
    k_cap = oracle.num_selected(int(table.shape[1]), w.ratio_num, w.ratio_den, w.k_fixed)
    csc, csel, ccnt, _, _, _ = oracle.hier_select(cache, table, lens, q, hs.group, hs.kc, w.ratio_num, w.ratio_den,
                                                  w.k_fixed, k_cap)
    st = {}
    gcs, gcc = gpu["coarse_sel"], gpu["coarse_cnt"]
    rows = same = 0
    for b in range(gcs.shape[0]):
        for g in range(gcs.shape[1]):
            rows += 1
            K = int(ccnt[b, g])
            same += int(gcc[b, g]) == K and np.array_equal(gcs[b, g, :K], csel[b, g, :K])
    st["kept_super_page_rows_identical"] = f"{same}/{rows}"
    fine = oracle.page_scores(cache, table, lens, q)
    masked = oracle.mask_scores(fine, hs.group, gcs, gcc)
    osel, ocnt = oracle.topk(masked, lens, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
    sel, cnt = gpu["sel"], gpu["cnt"]
    same = swaps = 0
    for b in range(sel.shape[0]):
        for g in range(sel.shape[1]):
            K = int(ocnt[b, g])
            d = set(sel[b, g, :K].tolist()) ^ set(osel[b, g, :K].tolist())
            same += not d and int(cnt[b, g]) == K
            swaps += len(d) // 2
    st["selection_rows_identical"] = f"{same}/{rows}"
    st["near_tie_page_swaps"] = swaps
    want = oracle.attention(cache, table, lens, q, sel, cnt)
    st["out_max_abs_err"] = float(np.abs(gpu["out"].astype(np.float64) - want).max())
    fsel, fcnt = oracle.topk(fine, lens, w.ratio_num, w.ratio_den, w.k_fixed, k_cap)
    hit = tot = 0
    for b in range(sel.shape[0]):
        for g in range(sel.shape[1]):
            K = int(fcnt[b, g])
            hit += len(set(fsel[b, g, :K].tolist()) & set(sel[b, g, :int(cnt[b, g])].tolist()))
            tot += K
    st["recall_of_flat_topk"] = round(hit / max(tot, 1), 4)
    st["tolerance"] = 2e-3
    return st


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=4, help="workload number 1-5 (default 4: 32K INT8 sparse)")
    ap.add_argument("--layers", type=int, default=8, help="independent layer caches rotated per step")
    ap.add_argument("--eager", action="store_true", help="launch every kernel from the host (no HIP graph)")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--one-launch", action="store_true",
                    help="run the step as one persistent launch (kvq_decode_step) instead of three")
    ap.add_argument("--hier", default="",
                    help="coarse-then-fine selection GROUP:KEEP (super-pages of GROUP pages, KEEP = share of "
                         "super-pages kept per row), e.g. 8:0.5")
    ap.add_argument("--storage", default="",
                    help="store the workload's cache in another format: fp16, int8_token, int8_group64, "
                         "int4_token or int4_group64 (4-bit: head_dim 128)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle legs (CPU baseline and parity)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB 10 times (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this decode-step path runs on one GPU; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 10}))
        return 0

    import workloads
    import paged_quantized_sparse_amd as kvq
    from paged_quantized_sparse_amd import runtime

    kvq.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = workloads.config(args.config)
    if args.storage:
        fmt = {v: k for k, v in workloads.FORMAT_NAMES.items()}.get(args.storage)
        if fmt is None:
            print(f"bench.py: unknown storage {args.storage!r}", file=sys.stderr)
            return 2
        if fmt != w.fmt:
            w = w.with_(name=f"{w.name}_as_{args.storage}", fmt=fmt)
    table, n_phys = w.block_table()
    lens = w.seq_lens()
    # each sequence's rows are drawn once: the prefill and the decode-time
    # append both read them (the 64-sequence ragged batch draws ~1.2M tokens
    # per pass)
    src = functools.lru_cache(maxsize=None)(lambda b: (w.keys(b), w.values(b)))
    print(f"[bench] building {w.name} ...", file=sys.stderr, flush=True)
    base, seqs = runtime.build_cache(w.fmt, n_phys, w.num_kv_heads, w.head_dim, table, lens, src,
                                     prefill_lens=lens - 1, device=dev, num_fp16_pages=w.fp16_pool_pages())
    stream = torch.cuda.current_stream()

    def events():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # ---- the one-time cache build (quantize + metadata of the prefill),
    # rows already resident in HBM; run again on the built cache, which it
    # rewrites with the same values
    pre = lens.astype(np.int64) - 1
    k_all = torch.from_numpy(np.ascontiguousarray(np.concatenate([src(b)[0][:pre[b]] for b in range(w.batch)]))
                             .view(np.int16)).to(dev)
    v_all = torch.from_numpy(np.ascontiguousarray(np.concatenate([src(b)[1][:pre[b]] for b in range(w.batch)]))
                             .view(np.int16)).to(dev)
    zeros_b = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    off_all = torch.from_numpy(np.concatenate([[0], np.cumsum(pre)]).astype(np.int32)).to(dev)
    pre_seqs = kvq.Seqs(torch.from_numpy(pre.astype(np.int32)).to(dev), seqs.block_table)
    build_us = []
    for _ in range(3):
        e0, e1 = events()
        e0.record(stream)
        kvq.kvq_append_quant(base, seqs, zeros_b, off_all, int(pre.max()), k_all, v_all)
        kvq.kvq_build_page_meta(base, pre_seqs)
        e1.record(stream)
        torch.cuda.synchronize()
        build_us.append(e0.elapsed_time(e1) * 1e3)
    del k_all, v_all
    cache_build_us = float(np.median(build_us))

    layers = [base]
    for _ in range(args.layers - 1):
        layers.append(kvq.PagedCache(base.format, base.num_phys_pages, base.num_kv_heads, base.head_dim,
                                     base.k_pages.clone(), base.v_pages.clone(),
                                     None if base.kv_params is None else base.kv_params.clone(),
                                     base.page_meta.clone(), base.num_fp16_pages))
    q = torch.from_numpy(w.query().view(np.int16)).to(dev)
    dense = w.is_dense()
    appends = [runtime.DecodeAppend(c, seqs, lens, src, device=dev) for c in layers]
    steps = [runtime.DecodeStep(c, seqs, w.num_q_heads, w.ratio_num, w.ratio_den, w.k_fixed, dense=dense,
                                pages_per_split=args.pages_per_split, device=dev,
                                fused_step=args.one_launch) for c in layers]
    NL = len(layers)
    hiers = None
    if args.hier:
        group, keep_frac = args.hier.split(":")
        group = int(group)
        pc_max = -(-seqs.max_pages // group)
        kc = max(1, int(np.ceil(float(keep_frac) * pc_max)))
        hiers = [runtime.HierStep(st, group, kc, device=dev) for st in steps]
        super_begin = [(a.page_begin // group).contiguous() for a in appends]
        for h in hiers:
            h.build()
    torch.cuda.synchronize()

    def one_step(i):
        if hiers is not None:
            hiers[i % NL].run_with_append(appends[i % NL], super_begin[i % NL], q)
        else:
            steps[i % NL].run_with_append(appends[i % NL], q)

    # warm-up (eager), which also fills every layer's selection
    for i in range(max(args.warmup, NL)):
        one_step(i)
    torch.cuda.synchronize()

    def rotation_graph(body):
        """One HIP graph running body(li) for every layer li in turn."""
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for li in range(NL):
                    body(li)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        return g

    def per_call_us(g, replays):
        """Microseconds per body call: HIP events on the launch stream around
        `replays` back-to-back replays of a rotation graph."""
        e0, e1 = events()
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * NL)

    # HIP graphs: one per layer, and one holding a whole rotation over the
    # layers (a multi-layer decode pass is captured once and replayed)
    graphs = rotation = None
    if not args.eager:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graphs = []
        with torch.cuda.stream(cap):
            for li in range(NL):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    one_step(li)
                graphs.append(g)
        stream.wait_stream(cap)
        rotation = rotation_graph(one_step)
        rotation.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` decode steps
    n_rot, rest = divmod(args.steps, NL)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs is not None:
        for _ in range(n_rot):
            rotation.replay()
        for i in range(rest):
            graphs[i].replay()
    else:
        for i in range(args.steps):
            one_step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3

    # ---- per-step spread (outside the timed region): HIP events around each
    # replay of the rotation graph, or around each eager rotation
    per_step_us = []
    ev = [events() for _ in range(50)]
    for r in range(50):
        ev[r][0].record(stream)
        if rotation is not None:
            rotation.replay()
        else:
            for i in range(NL):
                one_step(i)
        ev[r][1].record(stream)
    torch.cuda.synchronize()
    for r in range(50):
        per_step_us.append(ev[r][0].elapsed_time(ev[r][1]) * 1e3 / NL)
    p10, p50, p90 = (float(np.percentile(per_step_us, x)) for x in (10, 50, 90))

    # ---- each call of the step on its own, in rotation graphs
    replays = max(10, args.steps // NL)
    st0 = steps[0]
    rn, rd, kf = w.ratio_num, w.ratio_den, w.k_fixed

    def step_attention(li):  # the attention call as run_with_append runs it
        st = steps[li]
        if dense:
            st.attend(q, None, None)
        elif st.fused_select:
            st.select_attend(q)
        else:
            kvq.kvq_topk_pages(st.scores, st.seqs, w.num_kv_heads, rn, rd, kf, st.sel_pages, st.sel_count)
            st.attend(q, st.sel_pages, st.sel_count)

    def given_attention(li):  # attention over the step's selection, no selection in the kernel
        st = steps[li]
        st.attend(q, None if dense else st.sel_pages, None if dense else st.sel_count)

    def append_scores(li):
        st, app = steps[li], appends[li]
        kvq.kvq_append_decode_scores(st.cache, st.seqs, app.start, app.off, app.max_new, app.k_new, app.v_new, q,
                                     st.scores)

    attn_step_us = per_call_us(rotation_graph(step_attention), replays)
    attn_given_us = per_call_us(rotation_graph(given_attention), replays)
    append_us = per_call_us(rotation_graph(lambda li: appends[li].run()), replays)
    scores_us = None if dense else per_call_us(rotation_graph(append_scores), replays)
    # leave every layer as the step leaves it
    if rotation is not None:
        rotation.replay()
    torch.cuda.synchronize()

    counts = st0.sel_count.cpu().numpy() if not dense else np.tile(w.pages_per_seq()[:, None], (1, w.num_kv_heads))
    n16_tiles = fp16_tiles(w, table, None if dense else st0.sel_pages.cpu().numpy(), counts)
    meta_b, kv_b = algorithmic_bytes(w, counts, n16_tiles)
    if hiers is not None:  # boxes of every super-page, then the kept super-pages' pages
        h0 = hiers[0]
        P = w.pages_per_seq().astype(np.int64)
        Pc = -(-P // h0.group)
        kept = h0.sel_super.cpu().numpy()
        kcnt = h0.sel_super_count.cpu().numpy()
        fine_pages = 0
        for b in range(w.batch):
            for g in range(w.num_kv_heads):
                for jc in kept[b, g, :kcnt[b, g]]:
                    fine_pages += max(0, min(int(P[b]), (int(jc) + 1) * h0.group) - int(jc) * h0.group)
        meta_b = (int(Pc.sum()) * w.num_kv_heads + fine_pages) * 8 * w.head_dim
    step_bytes = (0 if dense else meta_b) + kv_b
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    attn_gbs = kv_b / (attn_step_us * 1e-6) / 1e9

    # the attainable streaming read on this GPU: a plain read kernel over 2 GiB
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    kvq.kvq_read_probe(big, sink)
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record(stream)
    for _ in range(5):
        kvq.kvq_read_probe(big, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    read_gbs = 5 * big.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big

    # layer 0's step once more, eagerly, for the parity statistics
    one_step(0)
    torch.cuda.synchronize()
    gpu = {"out": st0.out.cpu().numpy(), "sel": st0.sel_pages.cpu().numpy(), "cnt": st0.sel_count.cpu().numpy(),
           "scores": st0.scores.cpu().numpy().astype(np.float64), "k_pages": base.k_pages.cpu().numpy(),
           "meta": base.page_meta.cpu().numpy()}

    cpu = cpu1 = parity = None
    oracle_build_s = None
    threads = host_threads()
    if hiers is not None:
        gpu["coarse_sel"] = hiers[0].sel_super.cpu().numpy()
        gpu["coarse_cnt"] = hiers[0].sel_super_count.cpu().numpy()
    if not args.no_cpu:
        import oracle
        print("[bench] building the oracle's cache ...", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        built = oracle.build_cache(w)
        oracle_build_s = time.perf_counter() - t0
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        # the oracle's flat step (every page scored), priced at its own bytes
        flat_bytes = step_bytes
        t_cpu, reps, res = cpu_baseline(w, args.cpu_seconds, threads, built)
        if hiers is not None:
            flat_bytes = sum(algorithmic_bytes(w, res[2], fp16_tiles(w, table, res[1], res[2])))
        cpu = {"value": round(flat_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"full decode step (scores, top-K, attention) of this workload on {threads} threads "
                         f"({cpu_model()}), median of {reps} runs, {t_cpu * 1e3:.1f} ms each"
                         + ("; the flat selection (every page scored)" if hiers is not None else ""),
               "us_per_step": round(t_cpu * 1e6, 1)}
        t1, reps1, _ = cpu_baseline(w, args.cpu_seconds / 2, 1, built)
        cpu1 = {"value": round(flat_bytes / t1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the same step on one thread, median of {reps1} runs", "us_per_step": round(t1 * 1e6, 1)}
        if hiers is not None:
            parity = hier_parity_stats(w, built, hiers[0], gpu)
        elif not dense:
            parity = parity_stats(w, built, res, gpu)
        else:
            want = oracle.attention(built[0], built[1], lens, w.query())
            parity = {"out_max_abs_err": float(np.abs(gpu["out"].astype(np.float64) - want).max()), "tolerance": 2e-3}

    ratio = f"{w.ratio_num}/{w.ratio_den}" if not w.k_fixed else f"k={w.k_fixed}"
    kernel = ("kvq_sparse_decode_attn over every page (split kernel + combine)" if dense else
              "kvq_select_decode_attn as the step runs it (top-K inside the split kernel + combine)"
              if st0.fused_select else "kvq_topk_pages + kvq_sparse_decode_attn as the step runs them")
    rec = {
        "metric": "achieved HBM GB/s (% of peak) + us/decode-step, 32K ctx INT8 sparse",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "context": int(lens.max()), "page": 16,
                   "storage": workloads.FORMAT_NAMES[w.fmt], "selection": ratio,
                   "selected_pages_per_head": int(counts.max()), "layers_rotated": NL,
                   "launch": "eager" if graphs is None else "hip_graph",
                   "pages_per_split": st0.pps, "select_in_attention_kernel": bool(st0.fused_select),
                   "one_launch_step": bool(st0.fused_step),
                   "coarse_then_fine": None if hiers is None else {"group_pages": hiers[0].group,
                                                                   "kept_per_row": hiers[0].kc}},
        "bytes_per_step": {"metadata": meta_b if not dense else 0, "selected_kv": kv_b,
                           **({"selected_fp16_tiles": n16_tiles, "fp16_pool_pages": w.fp16_pool_pages()}
                              if w.fmt == workloads.FMT_MIXED else {})},
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.config == 4 and not args.pages_per_split else None,
                     "algorithmic_bytes": kv_b, "us_per_launch": round(attn_step_us, 2)},
        "us_per_step_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],
        "attention_given_selection_us": round(attn_given_us, 2),
        "attention_given_selection_gbs": round(kv_b / (attn_given_us * 1e-6) / 1e9, 1),
        "append_scores_us": None if scores_us is None else round(scores_us, 2),
        "append_scores_gbs": None if scores_us is None else round(meta_b / (scores_us * 1e-6) / 1e9, 1),
        "append_decode_us": round(append_us, 2),
        "cache_build_us": round(cache_build_us, 1),
        "oracle_cache_build_s": None if oracle_build_s is None else round(oracle_build_s, 3),
        "read_probe_2gib_gbs": round(read_gbs, 1),
        "attention_vs_read_probe": round(attn_gbs / read_gbs, 4),
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
