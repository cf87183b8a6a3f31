#!/usr/bin/env python3
"""Benchmark of the sparse-attention decode pass on one MI355X.

One step = one pass of the whole hot path over one batch: indexer scores ->
top-k -> one sparse-MLA call per layer (the layers share the top-k, as in
IndexShare). Inputs are seeded synthetic data already resident in HBM.

Timing: W untimed warm-up steps, then K timed steps. Before every timed step a
1 GiB buffer is read (outside the timed interval) so the 256 MB Infinity Cache
and the L2s hold none of the step's inputs; reading (not writing) leaves the
caches clean, so no write-back of the eviction traffic lands inside the timed
step. Each step is timed
with HIP events on the stream the kernels run on, with one extra event between
consecutive library calls on separate (eager) steps to time each kernel. With
--graph the timed steps are replayed from a captured HIP graph (checked
bit-exact against the eager step); by default they are eager stream launches.
The whole timed loop is bracketed by device synchronizations; ms_per_step is
the median step (p10 and p90 beside it).

Prints one JSON line: throughput in query tokens/s, the dominant kernel's
achieved algorithmic bandwidth against the HBM peak, and the CPU oracle's
rate on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, vendor figure (no sparsity)
WORKLOAD_DEFAULT = "decode_b32_l8k"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOAD_DEFAULT)
    ap.add_argument("--no-flush", action="store_true", help="skip the cache eviction between steps")
    ap.add_argument("--mla-per-layer", action="store_true",
                    help="with several IndexShare layers: one dsa_sparse_mla_fwd call per layer "
                         "instead of one dsa_sparse_mla_fwd_layers call for all of them")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=False,
                    help="replay the step as a captured HIP graph instead of eager launches")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline sample (0 = skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, copy 256 MiB device to device once (the "
                         "reference for scaling rocprofv3 byte counters)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs of this script "
                         "(FETCH_SIZE, WRITE_SIZE) into profiles/traffic_<workload>.json")
    ap.add_argument("--page-budget", type=int, default=0, metavar="KP",
                    help="select the KP best pages (of the workload's page size) per row "
                         "instead of the top-k tokens, and attend to their positions")
    ap.add_argument("--commands", nargs="*", default=[],
                    help="with --traffic-summary: the commands that made the runs")
    ap.add_argument("--mla-routes", choices=["topk", "locality"],
                    help="no step: time dsa_sparse_mla_fwd and dsa_sparse_mla_fwd_qblocked on "
                         "the same selections (the library's top-k of the workload's scores, "
                         "or locality-shaped lists) and print one JSON line comparing them")
    ap.add_argument("--fused-topk", action="store_true",
                    help="score and select in one dsa_indexer_topk launch (one query row per "
                         "sequence, rows of up to 16K positions) instead of two calls")
    ap.add_argument("--group-route", action="store_true",
                    help="no step: time the components of a two-pass exact token selection "
                         "(16-key group maxima, their top-k, a per-row re-score of the chosen "
                         "groups, a final top-k) beside the two-call route, one JSON line")
    ap.add_argument("--mla-heads", type=int, default=0,
                    help="with --mla-routes: MLA heads per query (a head-sharded share of the "
                         "workload's 64), default the workload's")
    return ap.parse_args()


# --------------------------------------------------------------------------
# algorithmic bytes (compulsory traffic through the three calls)
# --------------------------------------------------------------------------


def algorithmic_bytes(inp, k_sel=None, page=0, fused=False) -> dict:
    """Compulsory bytes and MFMA flops of one step. With ``page`` > 0 the selection is a
    page budget of k_sel / page pages: page maxima written and read (4 + 4 B per page),
    pages and positions written, and every legal position of the kept pages attended."""
    wl = inp.wl
    k_sel = wl.topk if k_sel is None else k_sel
    lens, qls = inp.seq_lens_host, inp.q_lens_host
    T = inp.total_q
    key_b = {"bf16": 2 * wl.idx_dim, "f32": 4 * wl.idx_dim, "fp8": wl.idx_dim + 4}[wl.idx_k_dtype]
    q_b = {"bf16": 2, "f32": 4}[wl.idx_q_dtype]
    valid = sum(sum(L - q + i + 1 for i in range(q)) for L, q in zip(lens, qls))  # (row, s) pairs
    if page:
        kp = k_sel // page
        # legal positions of the kp pages kept: all pages if the row has at most kp,
        # else kp pages of which the last may be partial (bounded by kp full pages)
        sel = sum(sum(min(kp * page, L - q + i + 1) for i in range(q)) for L, q in zip(lens, qls))
        n_pages = sum(sum((L - q + i) // page + 1 for i in range(q)) for L, q in zip(lens, qls))
    else:
        sel = sum(sum(min(wl.topk, L - q + i + 1) for i in range(q)) for L, q in zip(lens, qls))
    pages = sum((L + wl.page_size - 1) // wl.page_size for L in lens)
    e = {"bf16": 2, "f32": 4}[wl.mla_dtype]
    row_b = (wl.d_latent + wl.d_rope) * e
    indexer = (sum(lens) * key_b + T * wl.idx_heads * (wl.idx_dim * q_b + 4) + 4 * valid
               + 4 * pages)
    if page and fused:  # page maxima come out of the indexer: no token score in memory
        indexer = indexer - 4 * valid + 4 * n_pages
        topk = 4 * n_pages + 4 * T * (k_sel // page) + 4 * T * k_sel
    elif page:
        topk = 4 * valid + 8 * n_pages + 4 * T * (k_sel // page) + 4 * T * k_sel
    else:
        topk = 4 * valid + 4 * T * wl.topk
    mla_one = (sel * row_b + T * wl.mla_heads * (wl.d_latent + wl.d_rope) * e
               + T * k_sel * 4 + T * wl.mla_heads * (wl.d_latent + 1) * 4)
    flops_idx = 2 * wl.idx_heads * wl.idx_dim * valid
    flops_mla = 2 * wl.mla_heads * (2 * wl.d_latent + wl.d_rope) * sel
    return {"indexer": indexer, "topk": topk, "mla_per_layer": mla_one,
            "total": indexer + topk + wl.n_layers * mla_one,
            "flops_indexer": flops_idx, "flops_mla_per_layer": flops_mla,
            "valid_pairs": valid, "selected_rows": sel}


# --------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# --------------------------------------------------------------------------


def cpu_baseline(inp, budget_s: float, kp: int = 0):
    from oracle import dsa_oracle as O
    from workloads import host_view

    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = None
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                          "MKL_NUM_THREADS")}
    host = host_view(inp, lazy=True)
    rng = np.random.default_rng(0)
    order = rng.permutation(inp.total_q)
    done, t0 = 0, time.perf_counter()
    stage = {"indexer": 0.0, "selection": 0.0, "mla": 0.0}  # seconds per stage, summed
    for r in order:
        a = time.perf_counter()
        s = O.indexer_scores(host, [int(r)])
        b = time.perf_counter()
        idx = (O.page_budget_select(s, inp.wl.page_size, kp)[1] if kp
               else O.topk(s, inp.wl.topk))
        c = time.perf_counter()
        for l in range(inp.wl.n_layers):
            O.sparse_mla(host, l, idx)
        d = time.perf_counter()
        stage["indexer"] += b - a
        stage["selection"] += c - b
        stage["mla"] += d - c
        done += 1
        if d - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query tokens/s", "cores": int(threads), "kind": "oracle",
            "stage_ms_per_row": {k: 1e3 * v / max(done, 1) for k, v in stage.items()},
            "cores_detail": {"os_cpu_count": os.cpu_count(), "affinity": affinity,
                             "blas_threads": int(threads), "env": env,
                             "note": "the oracle's numpy BLAS threads are the cores it uses"},
            "sample": f"{done} of {inp.total_q} query rows (random, seed 0), full pass per row "
                      f"(indexer over all causal keys, "
                      + (f"{kp}-page budget" if kp else f"top-{inp.wl.topk}")
                      + f", {inp.wl.n_layers} MLA "
                      f"layer(s)), numpy float64, {dt:.1f} s"}


# --------------------------------------------------------------------------
# traffic from committed rocprofv3 counter summaries
# --------------------------------------------------------------------------


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_decode_lightning_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


# Kernels behind each library call (substrings of the kernel symbols); a call's
# traffic is the sum over its kernels per call.
STAGE_KERNELS = {
    "indexer": ["indexer_"],
    "topk": ["topk_"],
    "sparse_mla": ["sparse_mla_", "mla_combine_kernel"],
}
COPY_PROBE_BYTES = 256 << 20


READ_PEAK_BYTES = 2 << 30  # the read-stream peak is measured over 2 GiB (>= 1 GiB)


def read_stream_gbs(nbytes: int, flush, stream, reps: int = 5) -> float:
    """Median rate of the library's read-stream probe (dsa_bench_read, libdsa_bench.so:
    16-byte non-temporal loads, grid-stride, every byte read once) over nbytes, each run
    after reading the 1 GiB eviction buffer, timed with HIP events on `stream`."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_decode_lightning_amd",
                                   "libdsa_bench.so"))
    lib.dsa_bench_read.restype = ctypes.c_int
    lib.dsa_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.dsa_bench_read_blocks.restype = ctypes.c_uint32
    buf = torch.ones(max(16, nbytes) // 16 * 16, dtype=torch.uint8, device=flush.device)
    sink = torch.empty(int(lib.dsa_bench_read_blocks()), dtype=torch.int32, device=flush.device)
    ms = []
    for _ in range(reps):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib.dsa_bench_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), stream.cuda_stream)
        b.record(stream)
        if rc != 0:
            raise RuntimeError(f"dsa_bench_read failed ({rc})")
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    n = buf.numel()
    del buf, sink
    return n / (float(np.median(ms)) * 1e-3) / 1e9


def committed_traffic(workload: str, stage: str):
    """HBM bytes per call of a stage, from rocprofv3 FETCH_SIZE/WRITE_SIZE counters taken on
    the current kernel sources and scaled by a plain copy of known size; None otherwise."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != kernel_source_hash():
        return None
    st = d.get("stages", {}).get(stage)
    return None if st is None else st.get("bytes_per_call")


def _pmc_rows(run_dir: str, counter: str):
    """(kernel name, value in bytes) per dispatch from a rocprofv3 --pmc csv run directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        if r.get("Counter_Name") != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        name = r["Kernel_Name"]
        per.setdefault(key, [name, 0.0])[1] += float(r["Counter_Value"]) * 1024.0  # KiB
    # in dispatch order
    order = sorted(per, key=lambda k: (0, int(k)) if str(k).isdigit() else (1, str(k)))
    return [per[k] for k in order]


def traffic_summary(fetch_dir: str, write_dir: str, workload: str, calls_per_stage: dict,
                    commands: list):
    """Write profiles/traffic_<workload>.json from two counter runs of
    `bench.py --copy-probe` (one FETCH_SIZE, one WRITE_SIZE)."""
    fetch, write = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")

    def probe(rows):  # the largest plain copy is the probe
        copies = [v for n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        return max(copies) if copies else None

    def read_probe(rows):  # the read-stream probe over COPY_PROBE_BYTES: the run's last one
        reads = [v for n, v in rows if "read_stream_kernel" in n]
        return reads[-1] if reads else None

    pf, pw, pr = probe(fetch), probe(write), read_probe(fetch)
    # reads are scaled by what FETCH_SIZE gives for a plain read of known size
    # (the kernels' traffic is reads like it); the copy's reading is kept for
    # comparison. Writes are scaled by the copy's WRITE_SIZE.
    f_scale = COPY_PROBE_BYTES / pr if pr else (COPY_PROBE_BYTES / pf if pf else 1.0)
    w_scale = COPY_PROBE_BYTES / pw if pw else 1.0
    kernels = {}
    for rows, field, scale in ((fetch, "fetch", f_scale), (write, "write", w_scale)):
        for name, v in rows:
            if not any(sub in name for subs in STAGE_KERNELS.values() for sub in subs):
                continue
            short = name.replace("void ", "").replace("(anonymous namespace)::", "")
            short = short.split("(")[0].split("::")[-1]
            k = kernels.setdefault(short, {"fetch": [], "write": []})
            k[field].append(v * scale)
    out_k = {}
    for short, k in kernels.items():
        f = float(np.median(k["fetch"])) if k["fetch"] else 0.0
        w = float(np.median(k["write"])) if k["write"] else 0.0
        out_k[short] = {"fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
                        "bytes_per_launch": f + w, "launches": len(k["fetch"])}
    stages = {}
    for stage, subs in STAGE_KERNELS.items():
        ks = [n for n in out_k if any(sub in n for sub in subs)]
        if ks:
            stages[stage] = {"kernels": ks,
                             "bytes_per_call": sum(out_k[n]["bytes_per_launch"] for n in ks)}
    d = {"workload": workload, "source_hash": kernel_source_hash(),
         "copy_probe_bytes": COPY_PROBE_BYTES,
         "copy_probe_measured": {"fetch": pf, "write": pw},
         "read_probe_measured": {"fetch": pr},
         "scale": {"fetch": f_scale, "write": w_scale,
                   "fetch_source": "read probe" if pr else "copy",
                   "fetch_from_copy": COPY_PROBE_BYTES / pf if pf else None},
         "kernels": out_k, "stages": stages, "commands": commands,
         "note": ("FETCH_SIZE / WRITE_SIZE in KiB per dispatch (x1024), median over the "
                  "dispatches of each kernel; FETCH_SIZE scaled by copy_probe_bytes / its "
                  "reading for one plain read of copy_probe_bytes (dsa_bench_read), "
                  "WRITE_SIZE by copy_probe_bytes / its reading for one device-to-device "
                  "copy of copy_probe_bytes")}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    json.dump(d, open(path, "w"), indent=1)
    print(json.dumps({k: v["bytes_per_call"] for k, v in stages.items()}))


# --------------------------------------------------------------------------
# the cache append that precedes the path (measured on its own, not in `value`)
# --------------------------------------------------------------------------


def time_kv_append(dsa, inp, wl, kvs, keys, stream, flush, args, reps=10):
    """Append one new token per query row (its own position t_r) to every layer's latent
    cache and to the indexer-key cache; HIP events around each append after a cache
    eviction. Runs after the timed steps: it overwrites those rows of the caches."""
    dev = inp.block_table.device
    bt = inp.block_table.cpu().numpy()
    P = wl.page_size
    slots = []
    for b, (L, q) in enumerate(zip(inp.seq_lens_host, inp.q_lens_host)):
        for i in range(q):
            t = L - q + i
            slots.append(int(bt[b, t // P]) * P + t % P)
    T = len(slots)
    slot_t = torch.tensor(slots, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev).manual_seed(11)
    row = wl.d_latent + wl.d_rope
    lat_dt = torch.bfloat16 if wl.mla_dtype == "bf16" else torch.float32
    key_src_dt = torch.float32 if wl.idx_k_dtype == "f32" else torch.bfloat16
    lat_new = [torch.randn((T, row), generator=g, device=dev).to(lat_dt) for _ in kvs]
    key_new = torch.randn((T, wl.idx_dim), generator=g, device=dev).to(key_src_dt)

    def append():
        for l, kv in enumerate(kvs):
            if l == 0:
                dsa.kv_append(slot_t, lat_new[0], kv, key_new, keys)
            else:
                dsa.kv_append(slot_t, lat_new[l], kv)

    append()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if not args.no_flush:
            flush.sum()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        append()
        b_.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b_))
    ms = float(np.median(ts))
    e = 2 if wl.mla_dtype == "bf16" else 4
    key_in = wl.idx_dim * (4 if wl.idx_k_dtype == "f32" else 2)
    key_out = {"bf16": 2 * wl.idx_dim, "f32": 4 * wl.idx_dim, "fp8": wl.idx_dim + 4}[wl.idx_k_dtype]
    per_token = len(kvs) * (2 * row * e) + key_in + key_out + 4 * len(kvs)
    return {"tokens": T, "calls": len(kvs), "us": ms * 1e3, "bytes": T * per_token,
            "gbs": T * per_token / (ms * 1e-3) / 1e9,
            "note": "one new token per query row into every layer's latent cache and the "
                    "indexer-key cache (fp8 keys quantised per token); median of "
                    f"{reps} evicted runs; not part of value"}


# --------------------------------------------------------------------------
# per-query vs query-blocked sparse MLA on one set of selections
# --------------------------------------------------------------------------

# Locality-shaped selections: a block of 64 consecutive queries draws its rows
# from a shared set of pages whose size is 2.16 times one query's selection,
# the union-to-selection ratio of the pages' own example ("Making GLM-5.2
# Sparse on TPUs", section "Reuse pages across queries": 64 queries of 32
# pages each with a union of about 69 pages).
LOCALITY_BLOCK = 64
LOCALITY_UNION_RATIO = 2.16


def group_route(args, dsa, wl, dev):
    """Components of an exact token route that never writes [T, L] scores.

    The k-th largest maximum of 16-key groups bounds the row's k-th score from
    below, so only the k groups with the largest maxima can hold top-k tokens.
    Proxies: pass 1 is the page-max indexer (page maxima instead of group
    maxima); the group top-k and the final top-k are the top-k call on rows of
    L/16 and 16k random scores; pass 2 is the indexer on 16k keys per query row
    (each row re-scores its own groups), and on 16k keys shared by a
    sequence's queries (the bound if they chose the same groups).
    """
    from workloads import make_inputs

    stream = torch.cuda.current_stream(dev)
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev)

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return round(float(np.median(ts)), 1)

    def setup(w):
        inp = make_inputs(w, device="cuda", poison=False)
        batch = dsa.Batch(inp.block_table, inp.seq_lens, inp.cu_q, inp.total_q,
                          inp.max_seq_len, inp.max_q)
        return inp, batch, dsa.PagedCache(inp.k_cache, inp.k_scale)

    k = wl.topk
    res = {}
    inp, batch, keys = setup(wl)
    T, L, nq = inp.total_q, inp.max_seq_len, inp.max_q
    sc = torch.empty((T, L), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = torch.empty(max(dsa.topk_workspace_size(T, L, k), 16), dtype=torch.uint8, device=dev)
    res["indexer_us"] = timed(lambda: dsa.indexer_scores(batch, inp.q_idx, inp.w, keys, scores=sc))
    res["topk_us"] = timed(lambda: dsa.topk(batch, sc, k, indices=idx, workspace=ws))
    pg = torch.empty((T, -(-L // wl.page_size)), dtype=torch.float32, device=dev)
    res["pass1_page_max_indexer_us"] = timed(
        lambda: dsa.indexer_page_scores(batch, inp.q_idx, inp.w, keys, wl.page_size, out=pg))
    del inp, batch, keys, sc
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    for name, n in (("group_topk_us", L // 16), ("final_topk_us", 16 * k)):
        inp, batch, keys = setup(wl.replace(batch=T, q_per_seq=1, lens=n))
        s2 = torch.randn((T, n), generator=gen, device=dev)
        i2 = torch.empty((T, k), dtype=torch.int32, device=dev)
        w2 = torch.empty(max(dsa.topk_workspace_size(T, n, k), 16), dtype=torch.uint8, device=dev)
        res[name] = timed(lambda: dsa.topk(batch, s2, k, indices=i2, workspace=w2))
        if name == "final_topk_us":
            res["pass2_per_row_us"] = timed(
                lambda: dsa.indexer_scores(batch, inp.q_idx, inp.w, keys, scores=s2))
        del inp, batch, keys
        torch.cuda.empty_cache()
    inp, batch, keys = setup(wl.replace(batch=T // nq, q_per_seq=nq, lens=16 * k))
    s4 = torch.empty((T, 16 * k), dtype=torch.float32, device=dev)
    res["pass2_shared_us"] = timed(lambda: dsa.indexer_scores(batch, inp.q_idx, inp.w, keys, scores=s4))
    res["two_call_us"] = round(res["indexer_us"] + res["topk_us"], 1)
    res["group_route_us"] = [round(res["pass1_page_max_indexer_us"] + res["group_topk_us"]
                                   + res[p] + res["final_topk_us"], 1)
                             for p in ("pass2_shared_us", "pass2_per_row_us")]
    print(json.dumps({"workload": wl.name, "rows": T, "L": L, "k": k, **res}))


def mla_routes(args, dsa, wl, dev):
    from workloads import locality_indices, make_inputs, small_variant

    if args.mla_heads:
        wl = small_variant(wl, mla_heads=args.mla_heads)
    inp = make_inputs(wl, device="cuda")
    T = inp.total_q
    batch = dsa.Batch(inp.block_table, inp.seq_lens, inp.cu_q, T, inp.max_seq_len, inp.max_q)
    stream = torch.cuda.current_stream(dev)
    if args.mla_routes == "topk":
        keys = dsa.PagedCache(inp.k_cache, inp.k_scale)
        scores = dsa.indexer_scores(batch, inp.q_idx, inp.w, keys)
        indices = dsa.topk(batch, scores, wl.topk)
        del scores
        recipe = "the library's top-k of the workload's indexer scores"
    else:
        hot = int(round(LOCALITY_UNION_RATIO * wl.topk / wl.page_size))
        indices = locality_indices(inp.seq_lens_host, inp.q_lens_host, wl.topk, wl.page_size,
                                   block=LOCALITY_BLOCK, hot_pages=hot, seed=wl.seed).to(dev)
        recipe = (f"blocks of {LOCALITY_BLOCK} queries drawing from {hot} shared pages "
                  f"({LOCALITY_UNION_RATIO} x one query's {wl.topk} positions)")
    torch.cuda.synchronize()
    # union statistics of the blocks the blocked call forms (a block whose rows
    # span sequences takes every entry as its own slot)
    qb = 8 if wl.mla_heads == 8 else 4
    a = indices.cpu().numpy()
    seq_of = np.repeat(np.arange(wl.batch), inp.q_lens_host)
    union = sel = 0
    for m in range(0, T, qb):
        v = a[m:m + qb]
        v = v[v >= 0]
        one_seq = len(set(seq_of[m:m + qb].tolist())) == 1
        union += int(np.unique(v).size) if one_seq else int(v.size)
        sel += int(v.size)
    n_blocks = (T + qb - 1) // qb
    kv = dsa.PagedCache(inp.kv_cache[0])
    q = inp.q_mla[0]
    out_u = torch.empty((T, wl.mla_heads, wl.d_latent), dtype=torch.float32, device=dev)
    lse_u = torch.empty((T, wl.mla_heads), dtype=torch.float32, device=dev)
    out_b, lse_b = torch.empty_like(out_u), torch.empty_like(lse_u)
    ws_u = torch.empty(max(16, dsa.sparse_mla_workspace_size(T, wl.mla_heads, wl.d_latent,
                                                             wl.topk)), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(max(16, dsa.sparse_mla_qblocked_workspace_size(T, wl.mla_heads, wl.topk)),
                       dtype=torch.uint8, device=dev)
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev)

    def per_query():
        dsa.sparse_mla_fwd(batch, q, kv, indices, wl.d_latent, wl.scale, out=out_u, lse=lse_u,
                           workspace=ws_u)

    def blocked():
        dsa.sparse_mla_fwd_qblocked(batch, q, kv, indices, wl.d_latent, wl.scale, out=out_b,
                                    lse=lse_b, workspace=ws_b)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ts = []
        for _ in range(args.steps):
            if not args.no_flush:
                flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    ms_u = timed(per_query)
    ms_b = timed(blocked)
    # a head-sharded share against the 64-head kernel of the per-query call, its
    # queries zero-padded to 64 heads (what that kernel would cost such a share)
    ms_pad = None
    if wl.mla_heads < 64 and wl.mla_dtype == "bf16" and wl.d_latent == 512 and wl.d_rope == 64:
        q64 = torch.zeros((T, 64, q.shape[2]), dtype=q.dtype, device=dev)
        q64[:, :wl.mla_heads] = q
        out64 = torch.empty((T, 64, wl.d_latent), dtype=torch.float32, device=dev)
        lse64 = torch.empty((T, 64), dtype=torch.float32, device=dev)
        ws64 = torch.empty(max(16, dsa.sparse_mla_workspace_size(T, 64, wl.d_latent, wl.topk)),
                           dtype=torch.uint8, device=dev)

        def padded():
            dsa.sparse_mla_fwd(batch, q64, kv, indices, wl.d_latent, wl.scale, out=out64,
                               lse=lse64, workspace=ws64)

        ms_pad = timed(padded)
        del q64, out64, lse64, ws64
    rms = float(out_u.double().pow(2).mean().sqrt())
    diff = float((out_b - out_u).abs().max())
    if not diff <= 1e-2 * rms:
        raise RuntimeError(f"blocked and per-query MLA disagree: {diff} vs rms {rms}")
    line = {"mode": "mla_routes", "workload": wl.name, "selection": args.mla_routes,
            "selection_recipe": recipe, "n_queries": T, "mla_heads": wl.mla_heads,
            "topk": wl.topk, "page_size": wl.page_size, "query_block": qb,
            "union_rows_per_block": union / n_blocks, "selected_rows_per_block": sel / n_blocks,
            "row_load_reduction": sel / max(1, union),
            "per_query_ms": ms_u, "blocked_ms": ms_b, "blocked_speedup": ms_u / ms_b,
            "per_query_padded_to_64_heads_ms": ms_pad,
            "blocked_speedup_vs_padded": None if ms_pad is None else ms_pad / ms_b,
            "max_abs_diff_over_rms": diff / rms, "steps": args.steps, "warmup": args.warmup,
            "timing": "median of HIP-event-timed calls, each after the 1 GiB cache eviction"}
    print(json.dumps(line), flush=True)


# --------------------------------------------------------------------------


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload, {},
                        args.commands)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the decode path "
              "shards by sequence with no exchange, see the design notes", file=sys.stderr)
        sys.exit(2)
    import sparse_attention_decode_lightning_amd as dsa
    from workloads import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    if args.mla_routes:
        mla_routes(args, dsa, wl, dev)
        return
    if args.group_route:
        group_route(args, dsa, wl, dev)
        return
    inp = make_inputs(wl, device="cuda")
    T = inp.total_q
    batch = dsa.Batch(inp.block_table, inp.seq_lens, inp.cu_q, T, inp.max_seq_len, inp.max_q)
    keys = dsa.PagedCache(inp.k_cache, inp.k_scale)
    kvs = [dsa.PagedCache(c) for c in inp.kv_cache]
    scores = torch.empty((T, inp.max_seq_len), dtype=torch.float32, device=dev)
    page = wl.page_size
    kp = args.page_budget
    k_sel = kp * page if kp else wl.topk  # positions attention reads per row
    indices = torch.empty((T, k_sel), dtype=torch.int32, device=dev)
    if kp:
        n_pages = -(-inp.max_seq_len // page)
        page_sc = torch.empty((T, n_pages), dtype=torch.float32, device=dev)
        pages_sel = torch.empty((T, kp), dtype=torch.int32, device=dev)
        pk_bytes = dsa.page_topk_workspace_size(T, inp.max_seq_len, page, kp)
        pk_ws = torch.empty(max(pk_bytes, 16), dtype=torch.uint8, device=dev) if pk_bytes else None
    outs = [torch.empty((T, wl.mla_heads, wl.d_latent), dtype=torch.float32, device=dev)
            for _ in range(wl.n_layers)]
    lses = [torch.empty((T, wl.mla_heads), dtype=torch.float32, device=dev)
            for _ in range(wl.n_layers)]
    layered = wl.n_layers > 1 and not args.mla_per_layer
    ws_bytes = (dsa.sparse_mla_layers_workspace_size(wl.n_layers, T, wl.mla_heads, wl.d_latent,
                                                     k_sel) if layered else
                dsa.sparse_mla_workspace_size(T, wl.mla_heads, wl.d_latent, k_sel))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    tk_bytes = dsa.topk_workspace_size(T, inp.max_seq_len, wl.topk)
    tk_ws = torch.empty(max(tk_bytes, 16), dtype=torch.uint8, device=dev) if tk_bytes else None
    flush = torch.ones(1 << 27, dtype=torch.int64, device=dev)  # 1 GiB, evicted by reading
    stream = torch.cuda.current_stream(dev)
    # page budget: page maxima straight from the indexer where it streams the keys,
    # else token scores then their page maxima
    fused = False
    if kp:
        try:
            dsa.indexer_page_scores(batch, inp.q_idx, inp.w, keys, page, out=page_sc)
            fused = True
        except dsa.DSAError:
            fused = False
    fused_topk = bool(args.fused_topk) and not kp
    if fused_topk:
        tk_state = torch.zeros(max(dsa.indexer_topk_state_size(T), 16), dtype=torch.uint8,
                               device=dev)
    sel_names = ((["page_topk"] if fused else ["page_scores", "page_topk"]) if kp else
                 ([] if fused_topk else ["topk"]))
    mla_calls = 1 if layered else wl.n_layers
    n_ev = 2 + len(sel_names) + mla_calls

    def step(evs=None):
        e = 0
        if evs is not None:
            evs[e].record(stream)
        if fused:
            dsa.indexer_page_scores(batch, inp.q_idx, inp.w, keys, page, out=page_sc)
        elif fused_topk:
            dsa.indexer_topk(batch, inp.q_idx, inp.w, keys, wl.topk, scores=scores,
                             indices=indices, state=tk_state)
        else:
            dsa.indexer_scores(batch, inp.q_idx, inp.w, keys, scores=scores)
        e += 1
        if evs is not None:
            evs[e].record(stream)
        if kp and not fused:
            dsa.page_scores(batch, scores, page, out=page_sc)
            e += 1
            if evs is not None:
                evs[e].record(stream)
        if kp:
            dsa.page_topk(batch, page_sc, page, kp, pages=pages_sel, indices=indices,
                          workspace=pk_ws)
        elif not fused_topk:
            dsa.topk(batch, scores, wl.topk, indices=indices, workspace=tk_ws)
        if not fused_topk:
            e += 1
            if evs is not None:
                evs[e].record(stream)
        if layered:
            dsa.sparse_mla_fwd_layers(batch, inp.q_mla, kvs, indices, wl.d_latent, wl.scale,
                                      outs=outs, lses=lses, workspace=ws)
            e += 1
            if evs is not None:
                evs[e].record(stream)
            return
        for l in range(wl.n_layers):
            dsa.sparse_mla_fwd(batch, inp.q_mla[l], kvs[l], indices, wl.d_latent, wl.scale,
                               out=outs[l], lse=lses[l], workspace=ws)
            e += 1
            if evs is not None:
                evs[e].record(stream)

    def evict():
        if not args.no_flush:
            flush.sum()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref_out = outs[-1].clone()
    ref_idx = indices.clone()

    replay = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(3):
            outs[-1].zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not (torch.equal(outs[-1], ref_out) and torch.equal(indices, ref_idx)):
                raise RuntimeError("graph replay does not reproduce the eager step")
        replay = graph.replay

    # per-stage breakdown: eager launches, an event between consecutive calls
    n_stage = min(args.steps, 10)
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n_stage)]
    for i in range(n_stage):
        evict()
        step(evsets[i])
    torch.cuda.synchronize()
    per = np.array([[evs[j].elapsed_time(evs[j + 1]) for j in range(n_ev - 1)]
                    for evs in evsets])  # ms, [steps, stages]
    stage_ms = per.mean(axis=0)

    # timed steps: start/end events only
    tev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evict()
        tev[i][0].record(stream)
        replay()
        tev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in tev])
    ms = float(np.median(step_ms))

    # warm back-to-back figure (no eviction), for context
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        replay()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps

    ab = algorithmic_bytes(inp, k_sel=k_sel, page=page if kp else 0, fused=fused)
    names = ["indexer_topk" if fused_topk else "indexer"] + sel_names + (
        [f"mla_{wl.n_layers}_layers"] if layered else
                                       [f"mla_l{l}" for l in range(wl.n_layers)])
    n_sel = len(sel_names)
    mla_ms = float(np.sum(stage_ms[1 + n_sel:]))
    sel_ms = float(np.sum(stage_ms[1:1 + n_sel]))
    kern = {"indexer": (float(stage_ms[0]), ab["indexer"] + (ab["topk"] if fused_topk else 0),
                        "dsa_indexer_topk" if fused_topk else "dsa_indexer_scores",
                        ab["flops_indexer"]),
            "topk": (sel_ms, ab["topk"], "dsa_page_topk" if kp else "dsa_topk", 0),
            # one call: one layer, or every layer through dsa_sparse_mla_fwd_layers
            "sparse_mla": (mla_ms / mla_calls, ab["mla_per_layer"] * (wl.n_layers // mla_calls),
                           "dsa_sparse_mla_fwd_layers" if layered else "dsa_sparse_mla_fwd",
                           ab["flops_mla_per_layer"] * (wl.n_layers // mla_calls))}
    dom = max(kern, key=lambda k: kern[k][0] * (mla_calls if k == "sparse_mla" else 1))
    d_ms, d_bytes, d_sym, d_flops = kern[dom]
    # the dominant call against the roofline it is closer to: HBM bytes or bf16 MFMA flops
    hbm_gbs = d_bytes / (d_ms * 1e-3) / 1e9
    mfma_tfs = d_flops / (d_ms * 1e-3) / 1e12
    mfma_bound = wl.mla_dtype == "bf16" and mfma_tfs / MFMA_BF16_PEAK_TFS > hbm_gbs / HBM_PEAK_GBS
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": mfma_tfs, "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": mfma_tfs / MFMA_BF16_PEAK_TFS,
                "algorithmic_flops_per_launch": d_flops}
    else:
        roof = {"bound": "hbm", "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm_gbs / HBM_PEAK_GBS}
    # the measured read-stream peak (a plain streaming read of 2 GiB after the same
    # eviction), the second denominator; and the same probe over the dominant call's
    # own byte count, the rate a perfect cold streaming kernel of that size reaches
    read_peak = read_stream_gbs(READ_PEAK_BYTES, flush, stream)
    read_same = read_stream_gbs(int(d_bytes), flush, stream)
    if not mfma_bound:
        roof.update(read_peak_gbs=read_peak, frac_of_read_peak=hbm_gbs / read_peak,
                    read_same_bytes_gbs=read_same, frac_of_read_same_bytes=hbm_gbs / read_same)
    step_gbs = ab["total"] / (ms * 1e-3) / 1e9
    roof["step"] = {"algorithmic_bytes": ab["total"], "achieved_gbs": step_gbs,
                    "frac": step_gbs / HBM_PEAK_GBS, "frac_of_read_peak": step_gbs / read_peak,
                    "note": "the whole step (every call) at its median duration"}
    roof["read_peak"] = {"gbs": read_peak, "bytes": READ_PEAK_BYTES,
                         "probe": "dsa_bench_read (libdsa_bench.so), median of 5 runs, each "
                                  "after the 1 GiB eviction read"}
    line = {
        "metric": "sparse-decode query tokens/s at B=32,L=8K,topk=2048; achieved HBM GB/s",
        "value": T / (ms * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.mla_dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) caches and queries, random paged block table)",
        "config": {"workload": wl.name, "description": wl.description, "batch": wl.batch,
                   "total_q": T, "max_seq_len": inp.max_seq_len, "topk": wl.topk,
                   "page_size": wl.page_size, "mla_layers": wl.n_layers,
                   "selection": (f"page budget: {kp} pages of {page} positions"
                                 + (", page maxima from the indexer" if fused else "") if kp
                                 else f"token top-{wl.topk}"
                                 + (", fused into the indexer launch" if fused_topk else "")),
                   "parallelism": "single GPU"},
        "achieved_hbm_gbs": ab["total"] / (ms * 1e-3) / 1e9,
        "algorithmic_bytes_per_step": ab["total"],
        # the fused lower bound: the same step without the token scores' 8 B per
        # valid (row, position) pair written by the indexer and read by the top-k
        "algorithmic_bytes_per_step_without_score_round_trip":
            None if kp else ab["total"] - 8 * ab["valid_pairs"],
        "stage_ms": {n: float(v) for n, v in zip(names, stage_ms)},
        "ms_per_step_stat": "median",
        "ms_per_step_mean": float(np.mean(step_ms)),
        "ms_per_step_p10_p90": [float(np.percentile(step_ms, 10)),
                                float(np.percentile(step_ms, 90))],
        "ms_per_step_warm_no_flush": warm_ms,
        "timing": ("HIP events around each step" +
                   ("" if args.no_flush else " after a 1 GiB read that evicts the caches") +
                   ("; HIP graph replay of the captured step" if args.graph
                    else "; plain stream launches")),
        "roofline": dict(roof, kernel=d_sym, kernels=STAGE_KERNELS[dom],
                         traffic=None if kp else committed_traffic(wl.name, dom),
                         algorithmic_bytes_per_launch=d_bytes, avg_launch_ms=d_ms),
        "wall_s_timed_loop": wall,
    }
    line["kv_append"] = time_kv_append(dsa, inp, wl, kvs, keys, stream, flush, args)
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        read_stream_gbs(COPY_PROBE_BYTES, flush, stream, reps=1)  # FETCH_SIZE calibration
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, kp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
