"""GPU parity at the workloads' full sizes, on sampled scans.

Each resident holds every scan of its workload and is queried through the same
entry points the benchmark times. The oracle recomputes the products for
sampled scans one at a time from the generator's counts (for the scaled
variant, from its own calibration of the sampled regions). Properties that hold
at any size are checked on every scan:
- dense DF plus the masked sum of its complement equals the full total;
- a stride-k output equals the stride-1 output on visited blocks and is zero
  elsewhere;
- the diffraction pattern summed over pixels equals the full-detector virtual
  image summed over the same scans (the pattern itself is checked on sampled
  pixels, whose values over every scan are kept while encoding);
- on the low-dose workload, the 64-position sweep answered by deltas and by
  the polar index equals the per-mask decodes on every scan.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BLOCK = 512


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def q():
    import stem_compressed_count_amd as m
    return m


def u(t):
    return q().as_unsigned(t).astype(np.uint64)


def encode_full(w, scaled=False, keep=None):
    """The whole workload, generated and encoded in order, 16 blocks at a time.

    keep: pixel indices whose values over every scan are returned as well
    (counts, or for a scaled workload the oracle's codes, with the oracle's
    calibration of each region), for sampled diffraction-pattern checks.
    """
    enc = q().Encoder(w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, dtype=w.dtype, layout=w.layout,
                      scaled=scaled)
    cols, cal = [], []
    try:
        step = 16 * BLOCK
        for s0 in range(0, w.S, step):
            n = min(step, w.S - s0)
            x = synth.scaled(w, s0, n) if scaled else synth.counts(w, s0, n)
            enc.add(x)
            if keep is None:
                continue
            if not scaled:
                cols.append(x[:, keep])
                continue
            for b0 in range(0, n, BLOCK):
                sc, off, codes = oracle.calibrate(x[b0:b0 + BLOCK])
                cal.append((sc, off))
                cols.append(codes.reshape(-1, w.P)[:, keep])
        blob = enc.blob()
    finally:
        enc.close()
    if keep is None:
        return blob
    return blob, np.concatenate(cols), (np.array(cal) if scaled else None)


def sample_scans(w, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, BLOCK - 1, BLOCK, w.S // 2, w.S - BLOCK, w.S - 1]
    return sorted(set(fixed) | set(int(s) for s in rng.choice(w.S, size=n, replace=False)))


def rows(w, scans):
    return np.concatenate([synth.counts(w, s, 1) for s in scans])


def rect_counts(w, r0, r1, c0, c1):
    """Counts of a scan rectangle as its own (r1-r0) x (c1-c0) scan grid."""
    return np.concatenate([synth.counts(w, r * w.scan_cols + c0, c1 - c0) for r in range(r0, r1)])


def check_stride(full, strided, k):
    blocks = np.arange(full.size) // BLOCK
    visited = blocks % k == 0
    assert np.array_equal(strided[visited], full[visited])
    assert not strided[~visited].any()


def check_com_rows(res, w, mask, valid, scans, sampled):
    row, col = res.com(mask)
    orow, ocol, _ = oracle.com(sampled, w.det_rows, w.det_cols, mask=mask, valid=valid)
    g = np.stack([row.cpu().numpy()[scans], col.cpu().numpy()[scans]])
    o = np.stack([orow, ocol])
    rel = np.abs(g.astype(np.float64) - o) / np.maximum(np.abs(o).astype(np.float64), 1.0)
    assert rel.max() <= 1e-5
    assert np.array_equal(g, o)


def check_rects(res, w, valid, rects):
    for (r0, r1, c0, c1) in rects:
        got = q().as_unsigned(res.decode_region(r0, r1, c0, c1))
        sub = rect_counts(w, r0, r1, c0, c1)
        want = oracle.region(sub, c1 - c0, 0, r1 - r0, 0, c1 - c0, valid)
        assert np.array_equal(got, want), (r0, r1, c0, c1)


def check_dp_sampled(res, w, keep, cols, valid, calib=None, strides=(1, 4)):
    """Sum and mean diffraction pattern on the kept pixels, plus a property on
    every pixel: the sum over pixels equals the full-detector virtual image
    summed over the same scans."""
    vk = None if valid is None else valid[keep]
    scan_mask = (np.random.default_rng(w.S).random(w.S) < 0.25).astype(np.uint8)
    for m in (None, scan_mask):
        for k in strides:
            s, mean = res.sum_dp(m, k)
            s = u(s)
            ws, wm = oracle.sum_dp(cols, m, vk, k, calib)
            assert np.array_equal(s[keep], ws), k
            assert np.array_equal(mean.cpu().numpy()[keep], wm), k
            if calib is None:
                vi = u(res.masked_sum(np.ones(w.P, np.uint8), block_stride=k))
                sel = np.ones(w.S, bool) if m is None else m != 0
                assert int(s.sum()) == int(vi[sel].sum()), k


def check_frames_ends(res, w, valid):
    """The first and the last block decoded to frames, native and amplitude."""
    nb = res.info.n_blocks
    for first in (0, nb - 1):
        s0, s1 = first * BLOCK, min(w.S, (first + 1) * BLOCK)
        counts = synth.counts(w, s0, s1 - s0)
        for kind in ("native", "amplitude"):
            got = res.decode_blocks(first, 1, kind)
            got = q().as_unsigned(got) if kind == "native" else got.cpu().numpy()
            assert np.array_equal(got, oracle.frames(counts, 0, 1, valid, kind)), (first, kind)


def keep_pixels(w, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, w.P // 2 + w.det_cols // 2, w.P - 1]  # a corner, the disk centre, the last pixel
    return np.array(sorted(set(fixed) | set(int(p) for p in rng.choice(w.P, size=n, replace=False))))


def rects_for(w, seed):
    rng = np.random.default_rng(seed)
    out = [(0, 8, 0, 8), (1, 9, w.scan_cols // 2 - 4, w.scan_cols // 2 + 4),
           (w.scan_rows - 8, w.scan_rows, w.scan_cols - 8, w.scan_cols)]
    for _ in range(3):
        r0 = int(rng.integers(0, w.scan_rows - 8))
        c0 = int(rng.integers(0, w.scan_cols - 8))
        out.append((r0, r0 + 8, c0, c0 + 8))
    return out


def test_u16_256x256_with_sentinels_full_size():
    w = synth.WORKLOADS["scan256_u16_sentinel"]
    valid = synth.valid_pixels(w)
    masks = synth.query_masks(w)
    bf, df = masks["bf"], masks["df"]
    full = np.ones(w.P, np.uint8)
    scans = sample_scans(w, 40, 31)
    sampled = rows(w, scans)
    keep = keep_pixels(w, 12, 34)
    blob, cols, _ = encode_full(w, keep=keep)
    with q().Resident(blob, valid=valid) as res:
        s1 = u(res.masked_sum(bf))
        assert np.array_equal(s1[scans], oracle.masked_sum(sampled, bf, valid))
        check_stride(s1, u(res.masked_sum(bf, block_stride=4)), 4)
        total = u(res.masked_sum(full))
        assert np.array_equal(total[scans], oracle.masked_sum(sampled, full, valid))
        for _ in range(2):  # cold, then warm from the cached total
            d = u(res.dense_df(df))
            assert np.array_equal(d[scans], oracle.dense_df(sampled, df, valid))
            assert np.array_equal(d + s1, total)
        check_com_rows(res, w, None, valid, scans, sampled)
        check_com_rows(res, w, bf, valid, scans, sampled)
        check_rects(res, w, valid, rects_for(w, 32))
        check_dp_sampled(res, w, keep, cols, valid)
        check_frames_ends(res, w, valid)
        res.finish()


def test_scaled_u16_256x256_full_size():
    w = synth.WORKLOADS["scan256_u16_sentinel"]
    bf = synth.query_masks(w)["bf"]
    rects = rects_for(w, 33)
    keep = keep_pixels(w, 8, 35)
    blob, cols, cal = encode_full(w, scaled=True, keep=keep)
    with q().Resident(blob) as res:
        check_dp_sampled(res, w, keep, cols, None, calib=cal, strides=(1, 3))
        sums = u(res.masked_sum(bf))
        region_cache = {}

        def region_codes(b):
            if b not in region_cache:
                n = min(BLOCK, w.S - b * BLOCK)
                region_cache[b] = oracle.calibrate(synth.scaled(w, b * BLOCK, n))
            return region_cache[b]

        for (r0, r1, c0, c1) in rects:
            got_f = res.decode_region(r0, r1, c0, c1, calibrated=True).cpu().numpy()
            got_c = q().as_unsigned(res.decode_region(r0, r1, c0, c1))
            want_f, want_c = [], []
            for r in range(r0, r1):
                for c in range(c0, c1):
                    s = r * w.scan_cols + c
                    sc, off, codes = region_codes(s // BLOCK)
                    code = codes.reshape(-1, w.P)[s % BLOCK]
                    want_c.append(code)
                    want_f.append(oracle.reconstruct(code, sc, off))
            assert np.array_equal(got_c, np.stack(want_c)), (r0, r1, c0, c1)
            assert np.array_equal(got_f, np.stack(want_f)), (r0, r1, c0, c1)
        # integer products of a scaled resident are exact sums of its codes; the
        # whole detector (mostly escape-heavy streams) takes the staged decode
        full = np.ones(w.P, np.uint8)
        fsum = u(res.masked_sum(full))
        frow, fcol = (t.cpu().numpy() for t in res.com())
        for b in sorted(region_cache)[:4]:
            codes = region_cache[b][2].reshape(-1, w.P)
            s0, n = b * BLOCK, codes.shape[0]
            assert np.array_equal(sums[s0:s0 + n], oracle.masked_sum(codes, bf))
            assert np.array_equal(fsum[s0:s0 + n], oracle.masked_sum(codes, full))
            orow, ocol, _ = oracle.com(codes, w.det_rows, w.det_cols)
            assert np.array_equal(frow[s0:s0 + n], orow) and np.array_equal(fcol[s0:s0 + n], ocol), b
        res.finish()


def test_u8_512x512_low_dose_full_size():
    w = synth.WORKLOADS["scan512_u8_lowdose"]
    masks = synth.query_masks(w)
    sweep = synth.sweep_masks(w)
    scans = sample_scans(w, 32, 41)
    sampled = rows(w, scans)
    keep = keep_pixels(w, 12, 43)
    blob, cols, _ = encode_full(w, keep=keep)
    with q().Resident(blob) as res:
        check_dp_sampled(res, w, keep, cols, None)
        for name, m in masks.items():
            s1 = u(res.masked_sum(m))
            assert np.array_equal(s1[scans], oracle.masked_sum(sampled, m)), name
            check_stride(s1, u(res.masked_sum(m, block_stride=4)), 4)
        outs = [u(res.masked_sum(m)) for m in sweep]  # the full 64-position sweep
        for i in (0, 21, 42, 63):
            assert np.array_equal(outs[i][scans], oracle.masked_sum(sampled, sweep[i])), i
        check_com_rows(res, w, None, None, scans, sampled)
        check_rects(res, w, None, rects_for(w, 42)[:3])
        check_frames_ends(res, w, None)
        # the sweep as one decode and 63 deltas equals the per-mask decodes on every scan
        prev = res.masked_sum(sweep[0])
        for i in range(1, len(sweep)):
            prev = res.masked_sum_delta(sweep[i - 1], prev, sweep[i])
            if i % 9 == 0 or i == len(sweep) - 1:
                assert np.array_equal(u(prev), outs[i]), i
        # and through the polar index
        res.index_build((96, 96))
        for i in (0, 5, 21, 42, 63):
            assert np.array_equal(u(res.masked_sum(sweep[i])), outs[i]), i
        res.finish()


def test_paired_u16_1024x1024_full_size():
    w = synth.WORKLOADS["scan1024_u16_paired"]
    masks = synth.query_masks(w)
    bf, df = masks["bf"], masks["df"]
    scans = sample_scans(w, 24, 51)
    sampled = rows(w, scans)
    keep = keep_pixels(w, 12, 53)
    blob, cols, _ = encode_full(w, keep=keep)
    with q().Resident(blob) as res:
        assert res.info.geom.layout == 1
        check_dp_sampled(res, w, keep, cols, None)
        s1 = u(res.masked_sum(bf))
        assert np.array_equal(s1[scans], oracle.masked_sum(sampled, bf))
        check_stride(s1, u(res.masked_sum(bf, block_stride=4)), 4)
        d = u(res.dense_df(df))
        assert np.array_equal(d[scans], oracle.dense_df(sampled, df))
        total = u(res.masked_sum(np.ones(w.P, np.uint8)))
        assert np.array_equal(d + s1, total)
        check_com_rows(res, w, bf, None, scans, sampled)
        check_com_rows(res, w, None, None, scans, sampled)  # the whole detector
        check_rects(res, w, None, rects_for(w, 52)[:3])
        check_frames_ends(res, w, None)
        res.finish()
