"""Throughput of the fused ANS decode + virtual-detector queries on one MI355X.

Workload (default): 1024 x 1024 scans x 192 x 192 uint16 Poisson counts
(bright-field disk r = 30, mean 5 inside / 0.1 outside, smoothly drifting
centre: 38.65 G counts, 77.3 GB raw), held as the paired-count tANS resident
in HBM (about 4 GB). One step runs every query of the hot path once on it:
masked_sum (BF disk, block stride 1 and 4), dense DF (warm total cache), CoM
over the full detector and over the BF disk, and an 8 x 8-scan region read.

Prints one JSON line: value = counts per second over the step (the logical
counts each query reads, summed; the region counts its 64 requested scans),
plus encoded-byte GB/s, a roofline entry for the dominant kernel and the CPU
oracle timed on a bounded sample.

The dominant kernel (the full-detector CoM decode) is bound by vector ALU
issue, not by HBM: the coded streams hold about 0.1 encoded bytes per count,
so even a handful of VALU instructions per count keep the HBM traffic far
below 8 TB/s. Its roofline therefore counts algorithmic integer operations
per decoded count (alg_ops_per_count below) against the chip's VALU issue
rate of 256 CUs x 64 lanes x 2.4 GHz. HBM bytes per launch come from
FETCH_SIZE/WRITE_SIZE counters recorded under profiles/ for the current kernel
source (null otherwise).

--all-workloads instead prints one JSON line per workload with every query
timed alone (the per-workload table of the design notes), the 64-position
sweep and the device encoder; the scaled (float32) variant of the sentinel
workload, whose uint16 codes are escape-heavy, has a line of its own, and so
has that workload's geometry filled with uniform 16-bit values (every stream
stored RAW: the queries there are bound by HBM, not by the decode).

--only-query times one query alone (--scaled: on the float32 variant; --raw:
on the uniform 16-bit values) for
profiling runs, and --summarize turns rocprofv3 output directories of
--only-step or --only-query runs into the markdown tables kept under profiles/.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# vector ALU issue peak: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz, in T lane-ops/s
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# algorithmic integer operations per decoded count of the moments decode
#  byte-rANS: split x>>12, slot address, multiply-add, renorm test, renorm select (5)
#             + M0, Mr, Mc accumulations (3)
#  paired tANS, per pair: table address, code-length extract, bit take, reservoir
#             shift, next-state add (5) and the two window values (2); per count
#             3.5, + M0, Mr, Mc accumulations (3)
ALG_OPS_MOMENTS = {0: 8.0, 1: 6.5}
KERNEL_NAME = {0: "k_reduce_rans<uint16, Moments>", 1: "k_reduce_paired<uint16, Moments>"}
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = {0: "k_reduce_rans_moments_u16_128x128x192x192_traffic.md",
                1: "k_reduce_paired_moments_u16_1024x1024x192x192_traffic.md"}
SQ_FILE = {0: "bench_128x128x192x192_u16_sq_counters.md",
           1: "k_reduce_paired_u16_1024x1024x192x192_sq_counters.md"}
# a wave64 VALU instruction occupies a 16-lane SIMD for 4 clocks; 1024 SIMDs at 2.4 GHz
SIMD_CLOCKS_PER_VALU = 4
SIMD_CLOCKS_PER_S = 256 * 4 * 2.4e9
KERNEL_SOURCE = os.path.join(ROOT, "stem_compressed_count_amd", "csrc", "kernels.hip")
BLOCK = 512


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="scan1024_u16_paired")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time the step only (no per-query table, no next rows, no CPU baseline): profiling runs")
    ap.add_argument("--blob-cache", default=None,
                    help="path of an encoded container to reuse between runs of one session (written if missing)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="one JSON line per workload: every query timed alone, the sweep and the device encoder")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (the FETCH_SIZE/WRITE_SIZE calibration kernel)")
    ap.add_argument("--scaled", action="store_true",
                    help="with --only-query: the workload's float32 intensities (a scaled resident)")
    ap.add_argument("--raw", action="store_true",
                    help="with --only-query: uniform 16-bit values on the workload's geometry (every stream RAW)")
    ap.add_argument("--only-query", choices=QUERY_NAMES, default=None,
                    help="time one query alone, warm, --steps times after --warmup (profiling runs)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR", default=None,
                    help="print markdown tables of rocprofv3 output directories (kernel trace or counters)")
    ap.add_argument("--label", default="step",
                    help="with --summarize: 'step' for --only-step runs, else the query of an --only-query run")
    ap.add_argument("--calibration", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="with --summarize: FETCH_SIZE and WRITE_SIZE runs of --copy-probe")
    return ap.parse_args()


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_field(name, field):
    """An integer recorded in a profile summary for the current kernel source, else None."""
    try:
        with open(os.path.join(PROFILES, name)) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith(("source_sha256:", field + ":")))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != kernel_source_hash() or field not in fields:
        return None
    return int(fields[field].strip())


def copy_ceiling(torch, reps=10):
    """Device-to-device copy of 1 GiB (read + write): the measured HBM ceiling, in GB/s."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbps = 2 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def region_blocks(scan_cols, n_scans):
    """Blocks holding a scan of the step's 8 x 8 rectangle (rows 0-7, columns 0-7)."""
    return sorted({(r * scan_cols + c) // BLOCK for r in range(8) for c in range(8) if r * scan_cols + c < n_scans})


def step_counts(n_scans, scan_cols, stride_scans, bf, df_mask, valid, P):
    """Logical counts the step's queries read over the first n_scans scans: every
    selected (scan, pixel) of each query; the region counts its requested scans."""
    v = np.ones(P, bool) if valid is None else valid.astype(bool)
    nbf = int((bf.astype(bool) & v).sum())
    ncomp = int((~df_mask.astype(bool) & v).sum())
    nvalid = int(v.sum())
    region = sum(1 for r in range(8) for c in range(8) if r * scan_cols + c < n_scans) * nvalid
    return n_scans * nbf + stride_scans * nbf + n_scans * ncomp + n_scans * nvalid + n_scans * nbf + region


def visited_scans(n_scans, stride):
    return sum(min(BLOCK, n_scans - b * BLOCK) for b in range(0, (n_scans + BLOCK - 1) // BLOCK, stride))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_step(oracle, dec, w, bf, df_mask, valid, region_rows):
    """The step's queries on decoded counts (the oracle as it stands)."""
    oracle.masked_sum(dec, bf, valid)
    oracle.masked_sum(dec, bf, valid, stride=4)
    oracle.dense_df(dec, df_mask, valid)
    oracle.com(dec, w.det_rows, w.det_cols, None, valid)
    oracle.com(dec, w.det_rows, w.det_cols, bf, valid)
    if region_rows is not None:
        oracle.region(dec, w.scan_cols, region_rows[0], region_rows[1], 0, 8, valid)


def cpu_baseline(w, bf, df_mask, valid):
    """The oracle (plain C, as it stands) on bounded samples of the same workload.

    Single thread: the first 32 blocks, one oracle decode of their container,
    then the step's queries on the decoded counts. All cores: one run of four blocks per core of the affinity set, each
    encoded as a container of its own and handled by its own thread (the
    oracle's C calls release the interpreter lock and share no state); runs of
    four blocks keep the stride-4 query on the same blocks."""
    import concurrent.futures

    import oracle
    import stem_compressed_count_amd as qsc
    import synth

    run = 4 * BLOCK
    rows_per_run = run // w.scan_cols if run % w.scan_cols == 0 else None
    n1 = min(w.S, 32 * BLOCK)
    n1 -= n1 % w.scan_cols
    rows1 = n1 // w.scan_cols
    counts = synth.counts(w, 0, n1)
    blob = qsc.encode(counts, rows1, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout).tobytes()
    payload = int(oracle.header(blob)["payload_bytes"])
    oracle.masked_sum(counts[:1], bf)  # loads the library before timing
    t0 = time.perf_counter()
    dec = oracle.decode(blob)
    oracle_step(oracle, dec, w, bf, df_mask, valid, (0, min(8, rows1)))
    dt = time.perf_counter() - t0
    done = step_counts(n1, w.scan_cols, visited_scans(n1, 4), bf, df_mask, valid, w.P)
    line = {"value": round(done / dt, 1), "unit": "counts/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n1} scans ({(n1 + BLOCK - 1) // BLOCK} blocks) of the same workload: one oracle "
                      f"decode, then the step's queries on the decoded counts; {dt:.2f} s single-threaded",
            "payload_GBps": round(payload / dt / 1e9, 4), "cpu": cpu_model()}
    del dec, counts
    cores = len(os.sched_getaffinity(0))
    if rows_per_run is None or w.S < run:
        return line
    n_runs = min(cores, w.S // run)
    blobs = []
    for i in range(n_runs):
        c = synth.counts(w, i * run, run)
        blobs.append(qsc.encode(c, rows_per_run, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout).tobytes())
    pay_all = sum(int(oracle.header(b)["payload_bytes"]) for b in blobs)

    def work(i):
        dec = oracle.decode(blobs[i])
        a, b = max(0, i * rows_per_run), min(8, (i + 1) * rows_per_run)  # the step's region rows this run holds
        oracle_step(oracle, dec, w, bf, df_mask, valid, (a - i * rows_per_run, b - i * rows_per_run) if a < b else None)

    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(n_runs) as ex:
        list(ex.map(work, range(n_runs)))
    dt_all = time.perf_counter() - t0
    n_all = n_runs * run
    done_all = step_counts(n_all, w.scan_cols, visited_scans(n_all, 4), bf, df_mask, valid, w.P)
    line["all_cores"] = {"value": round(done_all / dt_all, 1), "unit": "counts/s", "cores": n_runs, "kind": "oracle",
                         "sample": f"the first {n_all} scans as {n_runs} containers of 4 blocks, one thread each "
                                   f"({n_runs} threads on {cores} cores of the affinity set); {dt_all:.2f} s",
                         "payload_GBps": round(pay_all / dt_all / 1e9, 4)}
    return line


def raw_values(w, s0, n):
    """Uniform 16-bit values for scans [s0, s0 + n) of w's geometry (seeded per chunk start): incompressible
    data that the encoder stores as RAW streams, the path bound by HBM."""
    return np.random.default_rng([w.seed, s0]).integers(0, 65536, size=(n, w.P), dtype=np.uint16)


def build_blob(qsc, synth, w, cache=None, scaled=False, raw=False):
    """The workload's container, from the host encoder (generated and added 16 blocks at a time);
    scaled: from the float32 intensities; raw: from uniform 16-bit values (neither cached)."""
    if raw:
        enc = qsc.Encoder(w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, dtype=2, layout=0)
        for s0 in range(0, w.S, BLOCK * 16):
            enc.add(raw_values(w, s0, min(BLOCK * 16, w.S - s0)))
        blob = enc.blob()
        enc.close()
        return blob
    if scaled:
        enc = qsc.Encoder(w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, dtype=2, layout=0, scaled=True)
        for s0 in range(0, w.S, BLOCK * 16):
            enc.add(synth.scaled(w, s0, min(BLOCK * 16, w.S - s0)))
        blob = enc.blob()
        enc.close()
        return blob
    if cache and os.path.exists(cache):
        blob = np.fromfile(cache, dtype=np.uint8)
        h = blob[:256]
        geo = h[48:68].view(np.uint32)
        if tuple(int(x) for x in geo) == (w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, w.dtype) \
                and int(h[44:48].view(np.uint32)[0]) == w.layout:
            log(f"container {w.name} read from {cache}")
            return blob
    enc = qsc.Encoder(w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, dtype=w.dtype, layout=w.layout)
    chunk = BLOCK * 16
    t0 = last = time.perf_counter()
    for s0 in range(0, w.S, chunk):
        enc.add(synth.counts(w, s0, min(chunk, w.S - s0)))
        if time.perf_counter() - last > 15:
            last = time.perf_counter()
            log(f"encoding {w.name}: {s0 + chunk} of {w.S} scans, {last - t0:.0f} s")
    blob = enc.blob()
    enc.close()
    if cache:
        blob.tofile(cache)
    return blob


def timed(torch, stream, fn, reps, flush=None):
    """Median and p95 ms of reps calls of fn, each bracketed by HIP events on stream."""
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ts.append((a, b))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ts])
    return float(np.median(ms)), float(np.percentile(ms, 95))


QUERY_NAMES = ["masked_sum_bf_k1", "masked_sum_bf_k4", "dense_df_warm", "com_full", "com_bf", "decode_region_8x8",
               "masked_sum_full"]


def query_fns(torch, res, w, d_bf, d_df, valid):
    """The queries of the step, plus the full-detector sum, as calls queued without waiting."""
    dev = d_bf.device
    out = torch.empty(w.S, dtype=res.sum_dtype, device=dev)
    row, col = torch.empty(w.S, dtype=torch.float32, device=dev), torch.empty(w.S, dtype=torch.float32, device=dev)
    reg = torch.empty(64 * w.P, dtype=torch.int16 if w.dtype == 2 else torch.uint8, device=dev)
    rr, rc = min(8, w.scan_rows), min(8, w.scan_cols)
    full = torch.as_tensor(np.ones(w.P, np.uint8) if valid is None else valid, device=dev)
    return {
        "masked_sum_bf_k1": lambda: res.masked_sum(d_bf, 1, out=out, wait=False),
        "masked_sum_bf_k4": lambda: res.masked_sum(d_bf, 4, out=out, wait=False),
        "dense_df_warm": lambda: res.dense_df(d_df, out=out, wait=False),
        "com_full": lambda: res.com(None, out_row=row, out_col=col, wait=False),
        "com_bf": lambda: res.com(d_bf, out_row=row, out_col=col, wait=False),
        "decode_region_8x8": lambda: res.decode_region(0, rr, 0, rc, out=reg[:rr * rc * w.P], wait=False),
        "masked_sum_full": lambda: res.masked_sum(full, 1, out=out, wait=False),
    }


def query_table(torch, res, w, d_bf, d_df, valid, reps=20, flushed=True, full_sum=False):
    """Each query of the step alone: median and p95 of reps runs, warm, and with a
    1 GiB scratch write before every run so the 256 MB MALL and the L2s hold nothing
    of the resident (flushed)."""
    dev = d_bf.device
    stream = torch.cuda.current_stream()
    queries = query_fns(torch, res, w, d_bf, d_df, valid)
    if not full_sum:
        del queries["masked_sum_full"]
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if flushed else None
    table = {}
    for name, q in queries.items():
        q()
        torch.cuda.synchronize()
        m, p = timed(torch, stream, q, reps)
        row_stats = {"warm_median_ms": round(m, 4), "warm_p95_ms": round(p, 4)}
        if flushed:
            m, p = timed(torch, stream, q, reps, scratch)
            row_stats.update({"flushed_median_ms": round(m, 4), "flushed_p95_ms": round(p, 4)})
        table[name] = row_stats
    res.finish()
    del scratch
    torch.cuda.empty_cache()
    return table


def sweep_rows(torch, qsc, synth, res, w, blob, valid, out):
    """The moving-mask sweep (64 positions of a BF r = 53 disk) three ways: a full
    decode per mask, one decode then 63 deltas, and the polar index."""
    dev = out.device
    stream = torch.cuda.current_stream()
    sweep = [torch.as_tensor(m, device=dev) for m in synth.sweep_masks(w)]
    souts = [torch.empty_like(out) for _ in range(2)]

    def once(run):
        run()  # warm
        torch.cuda.synchronize()
        m, _ = timed(torch, stream, run, 1)
        return m

    def sweep_decode(r):
        def run():
            for m in sweep:
                r.masked_sum(m, 1, out=souts[0], wait=False)
        return run

    def sweep_delta():
        res.masked_sum(sweep[0], 1, out=souts[0], wait=False)
        for j in range(1, len(sweep)):
            res.masked_sum_delta(sweep[j - 1], souts[(j - 1) % 2], sweep[j], 1, out=souts[j % 2], wait=False)

    sw_decode = once(sweep_decode(res))
    sw_delta = once(sweep_delta)
    res.finish()
    exact = bool(torch.equal(souts[(len(sweep) - 1) % 2], res.masked_sum(sweep[-1], 1)))
    ires = qsc.Resident(blob, valid=valid)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ires.index_build()
    torch.cuda.synchronize()
    build_ms = (time.perf_counter() - t0) * 1e3
    sw_index = once(sweep_decode(ires))
    ires.finish()
    ix_bytes = int(ires.info.index_bytes)
    ires.close()
    torch.cuda.empty_cache()
    return {"positions": len(sweep), "decode_ms": round(sw_decode, 3), "delta_ms": round(sw_delta, 3),
            "index_ms": round(sw_index, 3), "index_build_ms": round(build_ms, 2), "index_bytes": ix_bytes,
            "delta_exact": exact,
            "what": "64-position moving BF disk (r = 53): a full decode per mask, one decode then deltas, "
                    "or the polar index"}


def encode_device_row(torch, qsc, synth, w, blob, max_blocks=64):
    """The device encoder on the first blocks of the workload (all of it when small):
    values uploaded once, then encoded from device memory (host-timed, synchronised,
    workspace allocation included); the container must equal the host encoder's."""
    n_blocks = min(max_blocks, (w.S + BLOCK - 1) // BLOCK)
    n = min(w.S, n_blocks * BLOCK)
    n -= n % w.scan_cols
    rows = n // w.scan_cols
    counts = synth.counts(w, 0, n)
    host = qsc.encode(counts, rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
    raw = torch.from_numpy(counts.view(np.int16) if w.dtype == 2 else counts).to("cuda:0")
    del counts
    dblob = qsc.encode_device(raw, rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
    identical = bool(np.array_equal(dblob.cpu().numpy(), host))
    del dblob
    ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dblob = qsc.encode_device(raw, rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t0) * 1e3)
        del dblob
    del raw
    torch.cuda.empty_cache()
    return {"ms": round(min(ms), 3), "values_per_s": round(n * w.P / (min(ms) * 1e-3), 1),
            "scans": n, "identical_to_host_encoder": identical,
            "what": f"the first {n} scans encoded on the GPU from native counts in device memory "
                    f"(host-timed, synchronised, workspace included)"}


def feed_rows(torch, res, w, max_blocks=64):
    """The reconstruction feed: whole blocks decoded back to frames, native counts and
    float32 square-root amplitude (the paired-resident page's feed table)."""
    stream = torch.cuda.current_stream()
    nb = min(max_blocks, res.info.n_blocks)
    counts = min(w.S, nb * BLOCK) * w.P
    feed = {"blocks": nb}
    for kind in ("native", "amplitude"):
        fbuf = res.decode_blocks(0, nb, kind, wait=True)
        m, _ = timed(torch, stream, lambda: res.decode_blocks(0, nb, kind, out=fbuf.view(-1), wait=False), 5)
        res.finish()
        feed[kind] = {"ms": round(m, 4), "counts_per_s": round(counts / (m * 1e-3), 1),
                      "out_GBps": round(fbuf.numel() * fbuf.element_size() / (m * 1e-3) / 1e9, 1)}
        # the same blocks through the block feed: items of one and of eight
        # blocks, two buffers, decoded ahead on the library's stream while the
        # consumer stream waits for each item in turn
        for per, key in ((1, "feed"), (8, "feed8")):
            def iterate():
                for _frames, _s0 in res.feed(0, nb, per, kind, 2):
                    pass
            iterate()
            torch.cuda.synchronize()
            m, _ = timed(torch, stream, iterate, 3)
            feed[kind][key + "_ms"] = round(m, 4)
            feed[kind][key + "_counts_per_s"] = round(counts / (m * 1e-3), 1)
        del fbuf
        torch.cuda.empty_cache()
    feed["what"] = (f"the first {nb} blocks decoded to frames (not in the step): one decode_blocks call, "
                    f"and the block feed (items of one and of eight blocks, depth 2)")
    return feed


def all_workloads(torch, qsc, synth):
    """One JSON line per workload: each query alone, plus the sweep (512^2 u8) and the device encoder."""
    for name, w in synth.WORKLOADS.items():
        t0 = time.perf_counter()
        blob = build_blob(qsc, synth, w)
        setup = time.perf_counter() - t0
        valid = synth.valid_pixels(w)
        masks = synth.query_masks(w)
        bf = masks["bf"]
        df_mask = masks.get("df", (1 - bf).astype(np.uint8))
        dev = torch.device("cuda:0")
        res = qsc.Resident(blob, valid=valid)
        d_bf, d_df = torch.as_tensor(bf, device=dev), torch.as_tensor(df_mask, device=dev)
        line = {"workload": name, "resident_bytes": int(res.info.resident_bytes),
                "counts": w.S * w.P, "setup_s": round(setup, 1),
                "queries": query_table(torch, res, w, d_bf, d_df, valid, flushed=False, full_sum=True)}
        if "adf" in masks:
            d_adf = torch.as_tensor(masks["adf"], device=dev)
            out = torch.empty(w.S, dtype=res.sum_dtype, device=dev)
            res.masked_sum(d_adf, 1, out=out)
            m, p = timed(torch, torch.cuda.current_stream(), lambda: res.masked_sum(d_adf, 1, out=out, wait=False), 20)
            line["queries"]["masked_sum_adf_k1"] = {"warm_median_ms": round(m, 4), "warm_p95_ms": round(p, 4)}
        if name == "scan512_u8_lowdose":
            line["mask_sweep"] = sweep_rows(torch, qsc, synth, res, w, blob, valid,
                                            torch.empty(w.S, dtype=res.sum_dtype, device=dev))
        if w.dtype == 2 or w.layout == 1 or name == "scan512_u8_lowdose":
            line["encode_device"] = encode_device_row(torch, qsc, synth, w, blob,
                                                      max_blocks=128 if w.layout == 0 else 64)
        res.finish()
        res.close()
        del blob
        torch.cuda.empty_cache()
        print(json.dumps(line), flush=True)
    # the scaled variant: calibrated float32 intensities held as uint16 codes, most
    # of them above 254 (escape-heavy byte-rANS streams, RAW ones in the BF disk)
    w = synth.WORKLOADS["scan256_u16_sentinel"]
    t0 = time.perf_counter()
    blob = build_blob(qsc, synth, w, scaled=True)
    setup = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    res = qsc.Resident(blob)
    masks = synth.query_masks(w)
    d_bf = torch.as_tensor(masks["bf"], device=dev)
    d_df = torch.as_tensor(masks.get("df", (1 - masks["bf"]).astype(np.uint8)), device=dev)
    line = {"workload": w.name + " (scaled float32)", "resident_bytes": int(res.info.resident_bytes),
            "counts": w.S * w.P, "setup_s": round(setup, 1),
            "queries": query_table(torch, res, w, d_bf, d_df, None, flushed=False, full_sum=True)}
    res.close()
    del blob
    torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)
    # uniform 16-bit values on the same geometry: every stream RAW, 2 bytes per
    # count, the one case where HBM rather than the decode bounds the queries
    t0 = time.perf_counter()
    blob = build_blob(qsc, synth, w, raw=True)
    setup = time.perf_counter() - t0
    res = qsc.Resident(blob)
    line = {"workload": w.name + " geometry, uniform 16-bit values (RAW)", "resident_bytes": int(res.info.resident_bytes),
            "counts": w.S * w.P, "setup_s": round(setup, 1),
            "queries": query_table(torch, res, w, d_bf, d_df, None, flushed=False, full_sum=True)}
    nbytes, _ = res.query_bytes(np.ones(w.P, np.uint8), 1)
    ms = line["queries"]["masked_sum_full"]["warm_median_ms"]
    line["full_sum_encoded_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    line["full_sum_hbm_frac"] = round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    res.close()
    del blob
    torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


def only_query(torch, qsc, synth, args):
    """One query alone, warm: --warmup untimed runs, then --steps runs each bracketed by HIP events."""
    w = synth.WORKLOADS[args.workload]
    if (args.scaled or args.raw) and w.dtype != 2:
        raise SystemExit("--scaled and --raw need a uint16 workload")
    t0 = time.perf_counter()
    blob = build_blob(qsc, synth, w, None if (args.scaled or args.raw) else args.blob_cache, scaled=args.scaled,
                      raw=args.raw)
    kind = " (scaled)" if args.scaled else (" (uniform, RAW)" if args.raw else "")
    log(f"container {w.name}{kind}: {blob.size} bytes, {time.perf_counter() - t0:.1f} s")
    valid = None if (args.scaled or args.raw) else synth.valid_pixels(w)
    dev = torch.device("cuda:0")
    res = qsc.Resident(blob, valid=valid)
    masks = synth.query_masks(w)
    bf = masks["bf"]
    df_mask = masks.get("df", (1 - bf).astype(np.uint8))
    q = query_fns(torch, res, w, torch.as_tensor(bf, device=dev), torch.as_tensor(df_mask, device=dev), valid)
    fn = q[args.only_query]
    for _ in range(args.warmup):
        fn()
    res.finish()
    torch.cuda.synchronize()
    m, p = timed(torch, torch.cuda.current_stream(), fn, args.steps)
    res.finish()
    full = np.ones(w.P, np.uint8) if valid is None else valid
    sel = {"masked_sum_bf_k1": (bf, 1), "masked_sum_bf_k4": (bf, 4), "com_full": (full, 1), "com_bf": (bf, 1),
           "dense_df_warm": ((1 - df_mask).astype(np.uint8), 1), "masked_sum_full": (full, 1)}.get(args.only_query)
    line = {"workload": w.name + (" (scaled float32)" if args.scaled else (" (uniform 16-bit, RAW)" if args.raw else "")),
            "query": args.only_query,
            "steps": args.steps, "warmup": args.warmup, "warm_median_ms": round(m, 4), "warm_p95_ms": round(p, 4)}
    if sel is not None:
        nbytes, ncounts = res.query_bytes(*sel)
        line.update({"encoded_bytes_per_launch": int(nbytes), "counts_per_launch": int(ncounts),
                     "counts_per_s": round(ncounts / (m * 1e-3), 1), "encoded_GBps": round(nbytes / (m * 1e-3) / 1e9, 2),
                     "encoded_hbm_frac": round(nbytes / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
    res.close()
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------------ rocprofv3 summaries
STEP_QUERIES = ["masked_sum BF k=1", "masked_sum BF k=4", "dense_df warm", "com full detector", "com BF",
                "decode_region 8x8"]
COLD_QUERIES = ["dense_df cold (total)", "dense_df cold (complement)"]


OP_NAMES = ["Sum", "Moments", "Region", "Dp", "Index", "Amp", "Frames", "Split"]


def short_kernel(name):
    name = re.sub(r"\(qsc::Op\)(\d)", lambda m: OP_NAMES[int(m.group(1))], name)
    m = re.search(r"(k_\w+)(<[^()]*>)?", name)
    return name[:60] if not m else m.group(1) + (m.group(2) or "")


def dispatch_labels(kernel_by_dispatch, label):
    """Query of each decode dispatch (k_reduce_*): an --only-step run issues the cold
    dense DF (two), then six per step; an --only-query run issues its one query."""
    split = {d for d, k in kernel_by_dispatch.items() if "k_reduce" in k and "(qsc::Op)7" in k}
    red = [d for d in sorted(kernel_by_dispatch) if "k_reduce" in kernel_by_dispatch[d] and d not in split]
    seq = COLD_QUERIES + STEP_QUERIES * (len(red) // len(STEP_QUERIES) + 1) if label == "step" else [label] * len(red)
    labels = dict(zip(red, seq))
    labels.update({d: "split points (resident creation)" for d in split})
    return labels


def read_csv(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        return None
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def copy_scale(d, counter):
    """Bytes per KiB that a counter reads on the 1 GiB copy probe (1 GiB read, 1 GiB written)."""
    rows = read_csv(d, "counter_collection.csv")
    per = collections.defaultdict(float)
    for r in rows:
        if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    kib = statistics.median(per.values())
    return (1 << 30) / kib, kib


def summarize(dirs, label, calibration):
    """Markdown tables of rocprofv3 runs, and the fields bench.py reads back from them."""
    main_query = "com full detector" if label == "step" else label
    fields = {}
    for d in dirs:
        trace = read_csv(d, "kernel_trace.csv")
        if trace:
            kernels = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in trace}
            labels = dispatch_labels(kernels, label)
            groups = collections.defaultdict(list)
            for r in trace:
                k = int(r["Dispatch_Id"])
                groups[(short_kernel(r["Kernel_Name"]), labels.get(k, "-"))].append(
                    ((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, r))
            print(f"Kernel trace ({d}):\n")
            print("| kernel | query | dispatches | average us | median us | VGPR | SGPR | LDS B | scratch | WG | grid |")
            print("|---|---|---|---|---|---|---|---|---|---|---|")
            for (k, lab), v in sorted(groups.items(), key=lambda kv: -sum(x[0] for x in kv[1])):
                ds = [x[0] for x in v]
                r = v[0][1]
                print(f"| {k} | {lab} | {len(ds)} | {statistics.mean(ds):.1f} | {statistics.median(ds):.1f} | "
                      f"{r.get('VGPR_Count', '')} | {r.get('SGPR_Count', '')} | {r.get('LDS_Block_Size', '')} | "
                      f"{r.get('Scratch_Size', '')} | {r.get('Workgroup_Size_X', '')} | {r.get('Grid_Size_X', '')} |")
            print()
            continue
        rows = read_csv(d, "counter_collection.csv")
        if not rows:
            raise SystemExit(f"no kernel trace or counter collection under {d}")
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        kernels = {}
        for r in rows:
            k = int(r["Dispatch_Id"])
            per[k][r["Counter_Name"]] += float(r["Counter_Value"])
            kernels[k] = r["Kernel_Name"]
        labels = dispatch_labels(kernels, label)
        names = sorted({c for k in per for c in per[k]})
        scale = {}
        if calibration:
            for c, cd in zip(("FETCH_SIZE", "WRITE_SIZE"), calibration):
                if c in names:
                    scale[c] = copy_scale(cd, c)
        groups = collections.defaultdict(list)
        decode = any("k_reduce" in n for n in kernels.values())  # else a copy probe: list every kernel
        for k in sorted(per):
            if "k_reduce" in kernels[k] or not decode:
                groups[(short_kernel(kernels[k]), labels.get(k, "-"))].append(per[k])
        cols = names + (["SQ_WAIT_ANY / SQ_WAVE_CYCLES"] if {"SQ_WAIT_ANY", "SQ_WAVE_CYCLES"} <= set(names) else [])
        cols += [f"{c} scaled MB" for c in names if c in scale]
        print(f"Counters ({d}), median per dispatch:\n")
        for c, (f, kib) in scale.items():
            print(f"- {c}: the copy probe reads {kib:.1f} KiB per 1 GiB copy, so 1 KiB counts as {f / 1024:.4f} KiB")
        print("\n| kernel | query | dispatches | " + " | ".join(cols) + " |")
        print("|---|---|---|" + "---|" * len(cols))
        for (k, lab), v in groups.items():
            med = {n: statistics.median(x.get(n, 0.0) for x in v) for n in names}
            vals = [f"{med[n]:.4g}" for n in names]
            if "SQ_WAIT_ANY / SQ_WAVE_CYCLES" in cols:
                vals.append(f"{med['SQ_WAIT_ANY'] / med['SQ_WAVE_CYCLES']:.3f}")
            vals += [f"{med[c] * scale[c][0] / 1e6:.2f}" for c in names if c in scale]
            print(f"| {k} | {lab} | {len(v)} | " + " | ".join(vals) + " |")
            if lab == main_query:
                if "SQ_INSTS_VALU" in med:
                    fields["valu_insts_per_launch"] = int(round(med["SQ_INSTS_VALU"]))
                for c in ("FETCH_SIZE", "WRITE_SIZE"):
                    if c in scale:
                        fields[c] = med[c] * scale[c][0]
        print()
    print(f"Fields for the {main_query} launch, read back by bench.py:\n")
    print(f"source_sha256: {kernel_source_hash()}")
    if "valu_insts_per_launch" in fields:
        print(f"valu_insts_per_launch: {fields['valu_insts_per_launch']}")
    if "FETCH_SIZE" in fields and "WRITE_SIZE" in fields:
        print(f"traffic_bytes: {int(round(fields['FETCH_SIZE'] + fields['WRITE_SIZE']))}")


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.label, args.calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every query runs on a single device's resident "
              "(the sharded design is described, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import stem_compressed_count_amd as qsc
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.copy_probe:
        print(json.dumps({"copy_GBps": round(copy_ceiling(torch), 1), "bytes_per_copy": 2 << 30}), flush=True)
        return
    if args.all_workloads:
        all_workloads(torch, qsc, synth)
        return
    if args.only_query:
        only_query(torch, qsc, synth, args)
        return
    copy_gbps = copy_ceiling(torch)
    w = synth.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    blob = build_blob(qsc, synth, w, args.blob_cache)
    t_setup = time.perf_counter() - t0
    log(f"container {w.name}: {blob.size} bytes, {t_setup:.1f} s")
    valid = synth.valid_pixels(w)
    masks = synth.query_masks(w)
    bf = masks["bf"]
    df_mask = masks.get("df", (1 - bf).astype(np.uint8))
    res = qsc.Resident(blob, valid=valid)
    stream = torch.cuda.current_stream()
    d_bf = torch.as_tensor(bf, device=dev)
    d_df = torch.as_tensor(df_mask, device=dev)
    out = torch.empty(w.S, dtype=res.sum_dtype, device=dev)
    out4 = torch.empty_like(out)
    outdf = torch.empty_like(out)
    row = torch.empty(w.S, dtype=torch.float32, device=dev)
    col = torch.empty_like(row)
    rowb = torch.empty_like(row)
    colb = torch.empty_like(row)
    reg = torch.empty(64 * w.P, dtype=torch.int16 if w.dtype == 2 else torch.uint8, device=dev)

    # cold: the first dense DF builds the full-detector total cache
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    res.dense_df(d_df, out=outdf, wait=True)
    cold_ms = (time.perf_counter() - c0) * 1e3

    ev = {}

    def step(timed_com):
        res.masked_sum(d_bf, 1, out=out, wait=False)
        res.masked_sum(d_bf, 4, out=out4, wait=False)
        res.dense_df(d_df, out=outdf, wait=False)
        if timed_com:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        res.com(None, out_row=row, out_col=col, wait=False)
        if timed_com:
            b.record(stream)
            ev.setdefault("com_full", []).append((a, b))
        res.com(d_bf, out_row=rowb, out_col=colb, wait=False)
        res.decode_region(0, 8, 0, 8, out=reg, wait=False)

    for _ in range(args.warmup):
        step(False)
    res.finish()
    torch.cuda.synchronize()
    log("timing the step")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step(True)
    e1.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    res.finish()
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / args.steps

    # logical counts and encoded bytes each query of the step reads
    P = w.P
    full = np.ones(P, np.uint8) if valid is None else valid
    by_bf, _ = res.query_bytes(bf, 1)
    by_bf4, _ = res.query_bytes(bf, 4)
    by_df, _ = res.query_bytes((1 - df_mask).astype(np.uint8), 1)
    by_full, cn_full = res.query_bytes(full, 1)
    n_reg_blocks = len(region_blocks(w.scan_cols, w.S))
    step_cnt = step_counts(w.S, w.scan_cols, visited_scans(w.S, 4), bf, df_mask, valid, P)
    step_bytes = by_bf + by_bf4 + by_df + by_full + by_bf + by_full * n_reg_blocks / res.info.n_blocks
    value = step_cnt / (ms_per_step * 1e-3)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    com_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["com_full"]]))
    com_gbps = by_full / (com_ms * 1e-3) / 1e9
    alg = ALG_OPS_MOMENTS[w.layout]
    tops = cn_full * alg / (com_ms * 1e-3) / 1e12
    traffic = recorded_field(TRAFFIC_FILE[w.layout], "traffic_bytes")
    roofline = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 3), "unit": "TOP/s",
                "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": KERNEL_NAME[w.layout] + " (full-detector CoM: zero + decode/reduce + finalize)",
                "launch_ms": round(com_ms, 4), "counts_per_launch": int(cn_full),
                "alg_ops_per_count": alg,
                "counts_per_s": round(cn_full / (com_ms * 1e-3), 1),
                "encoded_bytes_per_launch": int(by_full), "encoded_GBps": round(com_gbps, 2),
                "encoded_hbm_frac": round(com_gbps / HBM_PEAK_GBPS, 4),
                "kernel_source_sha256": kernel_source_hash()}
    # what the chip actually issues for it (SQ_INSTS_VALU recorded under profiles/): VALU
    # instructions per decoded count, and the share of SIMD clocks they occupy
    valu = recorded_field(SQ_FILE[w.layout], "valu_insts_per_launch")
    roofline["issued_valu_per_count"] = None if valu is None else round(valu * 64 / cn_full, 2)
    roofline["valu_issue_frac"] = (None if valu is None else
                                   round(valu * SIMD_CLOCKS_PER_VALU / (com_ms * 1e-3 * SIMD_CLOCKS_PER_S), 4))

    layout_name = "byte-rANS" if w.layout == 0 else "paired tANS"
    line = {
        "metric": "decode+masked_sum counts/s and encoded-byte GB/s (fraction of HBM peak)",
        "value": round(value, 1), "unit": "counts/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u16" if w.dtype == 2 else "u8", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.scan_rows}x{w.scan_cols} scans x {w.det_rows}x{w.det_cols} "
                               f"{'uint16' if w.dtype == 2 else 'uint8'} Poisson, {layout_name} resident",
                   "step": "masked_sum BF (stride 1, 4) + dense_df (warm) + com full + com BF + 8x8 region",
                   "resident_bytes": int(res.info.resident_bytes), "payload_bytes": int(res.info.payload_bytes)},
        "encoded_GBps": round(gbps, 2), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "copy_GBps": round(copy_gbps, 1), "copy_frac": round(gbps / copy_gbps, 4),
        "step_counts": int(step_cnt), "step_encoded_bytes": int(step_bytes),
        "host_ms_per_step": round(host_s * 1e3 / args.steps, 4), "cold_dense_df_ms": round(cold_ms, 3),
        "setup_s": round(t_setup, 2),
        "roofline": roofline,
    }
    if not args.only_step:
        log("per-query table")
        line["queries"] = query_table(torch, res, w, d_bf, d_df, valid)
        log("next rows")
        dsum = torch.empty(w.P, dtype=torch.int64, device=dev)
        dmean = torch.empty(w.P, dtype=torch.float32, device=dev)
        res.sum_dp(None, 1, out_sum=dsum, out_mean=dmean, wait=True)
        dp_ms, _ = timed(torch, stream, lambda: res.sum_dp(None, 1, out_sum=dsum, out_mean=dmean, wait=False), 10)
        res.finish()
        nvalid = int(full.astype(bool).sum())
        line["next_rows"] = {
            "sum_dp": {"ms": round(dp_ms, 4), "counts_per_s": round(w.S * nvalid / (dp_ms * 1e-3), 1),
                       "what": "sum + mean diffraction pattern over every scan (not in the step)"},
            "decode_blocks": feed_rows(torch, res, w),
            "mask_sweep": sweep_rows(torch, qsc, synth, res, w, blob, valid, out),
            "encode_device": encode_device_row(torch, qsc, synth, w, blob),
        }
    res.close()
    del blob
    if not (args.no_cpu_baseline or args.only_step):
        log("oracle baseline")
        line["cpu_baseline"] = cpu_baseline(w, bf, df_mask, valid)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
