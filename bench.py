"""Throughput of the fused ANS decode + virtual-detector queries on one MI355X.

Workload: 128 x 128 scans x 192 x 192 uint16 Poisson counts (bright-field
disk r = 30, mean 5 inside / 0.1 outside, smoothly drifting centre), byte-rANS
resident in HBM. One step runs every query of the hot path once on it:
masked_sum (BF disk, block stride 1 and 4), dense DF (warm total cache), CoM
over the full detector and over the BF disk, and an 8 x 8-scan region read.

Prints one JSON line: value = decoded counts per second over the step (the
logical counts each query reads, summed), plus encoded-byte GB/s, a roofline
entry for the dominant kernel and the CPU oracle timed on a bounded sample.

The dominant kernel (the full-detector CoM decode) is bound by vector ALU
issue, not by HBM: the entropy-coded streams hold about 0.15 encoded bytes per
count, so even 10 VALU instructions per count keep the HBM traffic far below
8 TB/s. Its roofline therefore counts algorithmic integer operations:
ALG_OPS_MOMENTS per decoded count (the decode step's state split, table
address, multiply-add, renormalisation test and select, plus the three moment
accumulations), against the chip's VALU issue rate of 256 CUs x 64 lanes x
2.4 GHz. HBM bytes per launch come from FETCH_SIZE/WRITE_SIZE counters
recorded under profiles/ for the current kernel source (null otherwise).
"""
import hashlib
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# vector ALU issue peak: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz, in T lane-ops/s
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# algorithmic integer operations per decoded count of the byte-rANS moments decode:
# split x>>12, slot address, multiply-add, renorm test, renorm select (5) + M0, Mr, Mc adds (3)
ALG_OPS_MOMENTS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_reduce_rans_moments_u16_128x128x192x192_traffic.md")
SQ_FILE = os.path.join(ROOT, "profiles", "bench_128x128x192x192_u16_sq_counters.md")
# a wave64 VALU instruction occupies a 16-lane SIMD for 4 clocks; 1024 SIMDs at 2.4 GHz
SIMD_CLOCKS_PER_VALU = 4
SIMD_CLOCKS_PER_S = 256 * 4 * 2.4e9
KERNEL_SOURCE = os.path.join(ROOT, "stem_compressed_count_amd", "csrc", "kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="scan128_u16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=32)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (the FETCH_SIZE/WRITE_SIZE calibration kernel)")
    return ap.parse_args()


def kernel_source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_field(path, name):
    """An integer recorded in a profile summary for the current kernel source, else None."""
    try:
        with open(path) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith(("source_sha256:", name + ":")))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != kernel_source_hash() or name not in fields:
        return None
    return int(fields[name].strip())


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel (FETCH_SIZE + WRITE_SIZE, copy-calibrated)."""
    return recorded_field(TRAFFIC_FILE, "traffic_bytes")


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


def step_counts(n_scans, scan_cols, stride_scans, bf, df_mask, valid, P):
    """Logical counts the step's queries read over the first n_scans scans."""
    v = np.ones(P, bool) if valid is None else valid.astype(bool)
    nbf = int((bf.astype(bool) & v).sum())
    ncomp = int((~df_mask.astype(bool) & v).sum())
    nvalid = int(v.sum())
    blocks = sorted({(r * scan_cols + c) // 512 for r in range(8) for c in range(8)})
    region = sum(min(512, n_scans - b * 512) for b in blocks) * nvalid
    return n_scans * nbf + stride_scans * nbf + n_scans * ncomp + n_scans * nvalid + n_scans * nbf + region


def visited_scans(n_scans, stride):
    return sum(min(512, n_scans - b * 512) for b in range(0, (n_scans + 511) // 512, stride))


def cpu_baseline(w, masks, df_mask, sample_blocks):
    """The oracle (single-threaded C, as it stands) on the first blocks of the same workload."""
    import oracle
    import stem_compressed_count_amd as qsc
    import synth

    n = min(w.S, 512 * sample_blocks)
    rows = n // w.scan_cols
    n = rows * w.scan_cols
    counts = synth.counts(w, 0, n)
    blob = qsc.encode(counts, rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout).tobytes()
    valid = synth.valid_pixels(w)
    bf = masks["bf"]
    t0 = time.perf_counter()
    dec = oracle.decode(blob)
    oracle.masked_sum(dec, bf, valid)
    oracle.masked_sum(dec, bf, valid, stride=4)
    oracle.dense_df(dec, df_mask, valid)
    oracle.com(dec, w.det_rows, w.det_cols, None, valid)
    oracle.com(dec, w.det_rows, w.det_cols, bf, valid)
    oracle.region(dec, w.scan_cols, 0, 8, 0, 8, valid)
    dt = time.perf_counter() - t0
    done = step_counts(n, w.scan_cols, visited_scans(n, 4), bf, df_mask, valid, w.P)
    # the oracle decodes every stream of the sample once: its encoded-byte rate is the payload over the time
    payload = int(oracle.header(blob)["payload_bytes"])
    line = {"value": round(done / dt, 1), "unit": "counts/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} scans ({(n + 511) // 512} blocks) of the same workload: one oracle decode, "
                      f"then the step's queries on the decoded counts; {dt:.2f} s single-threaded",
            "payload_GBps": round(payload / dt / 1e9, 3), "cpu": cpu_model()}
    del dec
    par = cpu_baseline_threads(w, counts, n, bf, df_mask, valid)
    if par is not None:
        s = par.pop("s")
        par["value"] = round(done / s, 1)
        par["payload_GBps"] = round(payload / s / 1e9, 3)
        line["all_cores"] = par
    return line


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_threads(w, counts, n, bf, df_mask, valid):
    """The same sample and queries, cut into runs of four blocks, each encoded as a
    container of its own and handled by its own thread on the host's cores (the
    oracle's C calls release the interpreter lock; it has no shared state).
    Runs of four blocks keep the stride-4 query on the same blocks."""
    import concurrent.futures
    import oracle
    import stem_compressed_count_amd as qsc

    run = 4 * 512
    if run % w.scan_cols or n % run:
        return None
    rows = run // w.scan_cols
    blobs = [qsc.encode(counts[s0:s0 + run], rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout).tobytes()
             for s0 in range(0, n, run)]

    def work(i):
        dec = oracle.decode(blobs[i])
        oracle.masked_sum(dec, bf, valid)
        oracle.masked_sum(dec, bf, valid, stride=4)
        oracle.dense_df(dec, df_mask, valid)
        oracle.com(dec, w.det_rows, w.det_cols, None, valid)
        oracle.com(dec, w.det_rows, w.det_cols, bf, valid)
        a, b = max(0, i * rows), min(8, (i + 1) * rows)  # the step's region, rows 0-7, where this run holds them
        if a < b:
            oracle.region(dec, w.scan_cols, a - i * rows, b - i * rows, 0, 8, valid)

    cores = min(len(os.sched_getaffinity(0)), len(blobs))
    oracle.masked_sum(counts[:1], bf)  # loads the library before the threads start
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(cores) as ex:
        list(ex.map(work, range(len(blobs))))
    dt = time.perf_counter() - t0
    return {"s": dt, "unit": "counts/s", "cores": cores, "kind": "oracle",
            "sample": f"the same {n} scans as {len(blobs)} containers of 4 blocks, one thread each "
                      f"({cores} at a time); {dt:.2f} s"}


def main():
    args = parse()
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
    copy_gbps = copy_ceiling(torch)
    w = synth.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    enc = qsc.Encoder(w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, dtype=w.dtype, layout=w.layout)
    chunk = 512 * 16
    for s0 in range(0, w.S, chunk):
        enc.add(synth.counts(w, s0, min(chunk, w.S - s0)))
    blob = enc.blob()
    enc.close()
    t_setup = time.perf_counter() - t0
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

    def step(timed):
        res.masked_sum(d_bf, 1, out=out, wait=False)
        res.masked_sum(d_bf, 4, out=out4, wait=False)
        res.dense_df(d_df, out=outdf, wait=False)
        if timed:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
        res.com(None, out_row=row, out_col=col, wait=False)
        if timed:
            b.record(stream)
            ev.setdefault("com_full", []).append((a, b))
        res.com(d_bf, out_row=rowb, out_col=colb, wait=False)
        res.decode_region(0, 8, 0, 8, out=reg, wait=False)

    for _ in range(args.warmup):
        step(False)
    res.finish()
    torch.cuda.synchronize()
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

    # each query of the step alone: median and p95 of 20 runs, warm, and with a
    # 1 GiB scratch write before every run so the 256 MB MALL and the L2s hold
    # nothing of the resident (flushed)
    queries = {
        "masked_sum_bf_k1": lambda: res.masked_sum(d_bf, 1, out=out, wait=False),
        "masked_sum_bf_k4": lambda: res.masked_sum(d_bf, 4, out=out4, wait=False),
        "dense_df_warm": lambda: res.dense_df(d_df, out=outdf, wait=False),
        "com_full": lambda: res.com(None, out_row=row, out_col=col, wait=False),
        "com_bf": lambda: res.com(d_bf, out_row=rowb, out_col=colb, wait=False),
        "decode_region_8x8": lambda: res.decode_region(0, 8, 0, 8, out=reg, wait=False),
    }
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    per_query = {}
    for name, q in queries.items():
        row_stats = {}
        for flushed in (False, True):
            ts = []
            for _ in range(20):
                if flushed:
                    scratch.fill_(1)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                q()
                b.record(stream)
                ts.append((a, b))
            torch.cuda.synchronize()
            ms = np.array([a.elapsed_time(b) for a, b in ts])
            key = "flushed" if flushed else "warm"
            row_stats[key + "_median_ms"] = round(float(np.median(ms)), 4)
            row_stats[key + "_p95_ms"] = round(float(np.percentile(ms, 95)), 4)
        per_query[name] = row_stats
    res.finish()
    del scratch
    torch.cuda.empty_cache()

    # logical counts and encoded bytes each query of the step reads
    P = w.P
    full = np.ones(P, np.uint8) if valid is None else valid
    by_bf, _ = res.query_bytes(bf, 1)
    by_bf4, _ = res.query_bytes(bf, 4)
    by_df, _ = res.query_bytes((1 - df_mask).astype(np.uint8), 1)
    by_full, cn_full = res.query_bytes(full, 1)
    n_reg_blocks = len({(r * w.scan_cols + c) // 512 for r in range(8) for c in range(8)})
    step_cnt = step_counts(w.S, w.scan_cols, visited_scans(w.S, 4), bf, df_mask, valid, P)
    step_bytes = by_bf + by_bf4 + by_df + by_full + by_bf + by_full * n_reg_blocks / res.info.n_blocks
    value = step_cnt / (ms_per_step * 1e-3)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    # widened rows, timed on the same resident (not part of the step): the sum and
    # mean diffraction pattern over every scan
    dsum = torch.empty(w.P, dtype=torch.int64, device=dev)
    dmean = torch.empty(w.P, dtype=torch.float32, device=dev)
    for _ in range(3):
        res.sum_dp(None, 1, out_sum=dsum, out_mean=dmean, wait=False)
    dp_ev = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        res.sum_dp(None, 1, out_sum=dsum, out_mean=dmean, wait=False)
        b.record(stream)
        dp_ev.append((a, b))
    torch.cuda.synchronize()
    res.finish()
    dp_ms = float(np.median([a.elapsed_time(b) for a, b in dp_ev]))
    dp_counts = w.S * int((np.ones(w.P, bool) if valid is None else valid.astype(bool)).sum())

    # the reconstruction feed: every block decoded back to frames, native counts
    # and float32 square-root amplitude (the paired-resident page's feed table)
    feed = {}
    for kind in ("native", "amplitude"):
        fbuf = res.decode_blocks(0, res.info.n_blocks, kind, wait=True)
        f_ev = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            res.decode_blocks(0, res.info.n_blocks, kind, out=fbuf.view(-1), wait=False)
            b.record(stream)
            f_ev.append((a, b))
        torch.cuda.synchronize()
        res.finish()
        f_ms = float(np.median([a.elapsed_time(b) for a, b in f_ev]))
        feed[kind] = {"ms": round(f_ms, 4), "counts_per_s": round(w.S * w.P / (f_ms * 1e-3), 1),
                      "out_GBps": round(fbuf.numel() * fbuf.element_size() / (f_ms * 1e-3) / 1e9, 1)}
        del fbuf
        torch.cuda.empty_cache()

    # the moving-mask sweep (64 positions of a BF disk), three ways: a full
    # decode per mask, one decode then 63 deltas, and the polar index
    sweep = [torch.as_tensor(m, device=dev) for m in synth.sweep_masks(w)]
    souts = [torch.empty_like(out) for _ in range(2)]

    def timed_sweep(run):
        run()  # warm
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def sweep_decode(r):
        def run():
            for m in sweep:
                r.masked_sum(m, 1, out=souts[0], wait=False)
        return run

    def sweep_delta():
        res.masked_sum(sweep[0], 1, out=souts[0], wait=False)
        for j in range(1, len(sweep)):
            res.masked_sum_delta(sweep[j - 1], souts[(j - 1) % 2], sweep[j], 1, out=souts[j % 2], wait=False)

    sw_decode = timed_sweep(sweep_decode(res))
    sw_delta = timed_sweep(sweep_delta)
    res.finish()
    sweep_exact = bool(torch.equal(souts[(len(sweep) - 1) % 2], res.masked_sum(sweep[-1], 1)))
    ires = qsc.Resident(blob, valid=valid)
    t0 = time.perf_counter()
    ires.index_build()
    ix_build_ms = (time.perf_counter() - t0) * 1e3
    sw_index = timed_sweep(sweep_decode(ires))
    ires.finish()
    ix_bytes = int(ires.info.index_bytes)
    ires.close()

    # the device encoder: the whole workload from native counts in HBM
    raw = torch.from_numpy(synth.counts(w).view(np.int16) if w.dtype == 2 else synth.counts(w)).to(dev)
    dblob = qsc.encode_device(raw, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
    enc_identical = bool(np.array_equal(dblob.cpu().numpy(), blob))
    del dblob
    enc_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dblob = qsc.encode_device(raw, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
        torch.cuda.synchronize()
        enc_ms.append((time.perf_counter() - t0) * 1e3)
        del dblob
    del raw
    torch.cuda.empty_cache()

    com_ms = float(np.mean([a.elapsed_time(b) for a, b in ev["com_full"]]))
    com_gbps = by_full / (com_ms * 1e-3) / 1e9
    tops = cn_full * ALG_OPS_MOMENTS / (com_ms * 1e-3) / 1e12
    traffic = recorded_traffic()
    roofline = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 3), "unit": "TOP/s",
                "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": traffic,
                "kernel": "k_reduce_rans<uint16, Moments> (full-detector CoM: zero + decode/reduce + finalize)",
                "launch_ms": round(com_ms, 4), "counts_per_launch": int(cn_full),
                "alg_ops_per_count": ALG_OPS_MOMENTS,
                "counts_per_s": round(cn_full / (com_ms * 1e-3), 1),
                "encoded_bytes_per_launch": int(by_full), "encoded_GBps": round(com_gbps, 2),
                "encoded_hbm_frac": round(com_gbps / HBM_PEAK_GBPS, 4),
                "kernel_source_sha256": kernel_source_hash()}
    # what the chip actually issues for it (SQ_INSTS_VALU recorded under profiles/): VALU
    # instructions per decoded count, and the share of SIMD clocks they occupy
    valu = recorded_field(SQ_FILE, "valu_insts_per_launch")
    roofline["issued_valu_per_count"] = None if valu is None else round(valu * 64 / cn_full, 2)
    roofline["valu_issue_frac"] = (None if valu is None else
                                   round(valu * SIMD_CLOCKS_PER_VALU / (com_ms * 1e-3 * SIMD_CLOCKS_PER_S), 4))

    line = {
        "metric": "decode+masked_sum counts/s and encoded-byte GB/s (fraction of HBM peak)",
        "value": round(value, 1), "unit": "counts/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u16" if w.dtype == 2 else "u8", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.scan_rows}x{w.scan_cols} scans x {w.det_rows}x{w.det_cols} "
                               f"{'uint16' if w.dtype == 2 else 'uint8'} Poisson, "
                               f"{'byte-rANS' if w.layout == 0 else 'paired tANS'} resident",
                   "step": "masked_sum BF (stride 1, 4) + dense_df (warm) + com full + com BF + 8x8 region",
                   "resident_bytes": int(res.info.resident_bytes), "payload_bytes": int(res.info.payload_bytes)},
        "encoded_GBps": round(gbps, 2), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "copy_GBps": round(copy_gbps, 1), "copy_frac": round(gbps / copy_gbps, 4),
        "step_counts": int(step_cnt), "step_encoded_bytes": int(step_bytes),
        "host_ms_per_step": round(host_s * 1e3 / args.steps, 4), "cold_dense_df_ms": round(cold_ms, 3),
        "setup_s": round(t_setup, 2),
        "roofline": roofline,
        "queries": per_query,
        "next_rows": {"sum_dp": {"ms": round(dp_ms, 4), "counts_per_s": round(dp_counts / (dp_ms * 1e-3), 1),
                                 "what": "sum + mean diffraction pattern over every scan (not in the step)"},
                      "decode_blocks": dict(feed, what="every block decoded to frames (not in the step)"),
                      "mask_sweep": {"positions": len(sweep), "decode_ms": round(sw_decode, 3),
                                     "delta_ms": round(sw_delta, 3), "index_ms": round(sw_index, 3),
                                     "index_build_ms": round(ix_build_ms, 2), "index_bytes": ix_bytes,
                                     "delta_exact": sweep_exact,
                                     "what": "64-position moving BF disk (r = 53): a full decode per mask, "
                                             "one decode then deltas, or the polar index"},
                      "encode_device": {"ms": round(min(enc_ms), 3),
                                        "values_per_s": round(w.S * w.P / (min(enc_ms) * 1e-3), 1),
                                        "identical_to_host_encoder": enc_identical,
                                        "what": "the whole workload encoded on the GPU from native counts in "
                                                "device memory (host-timed, synchronised, workspace included)"}},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, masks, df_mask, args.cpu_sample_blocks)
    res.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
