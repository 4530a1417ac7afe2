"""GPU parity: every query of the HIP path against the CPU oracle.

Integer products (masked sums, dense DF, region reads, exact moments) must be
bit-exact. CoM must be within 1e-5 relative (the optimization matrix page's
real-crop agreement gate); it is also checked bit for bit, because both sides
divide the same exact moments once in float64. Inputs are the seeded synthetic
workloads; reduced scan counts keep the oracle fast while still spanning many
workgroup tiles, several 512-scan blocks and a ragged final block.
"""
import functools
import struct

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def q():
    import stem_compressed_count_amd as m
    return m


@functools.lru_cache(maxsize=8)
def case(name, sr=None, sc=None, layout=None):
    w = synth.WORKLOADS[name]
    if sr is not None:
        w = w.with_scans(sr, sc)
    lay = w.layout if layout is None else layout
    counts = synth.counts(w)
    blob = q().encode(counts, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=lay)
    return w, counts, synth.valid_pixels(w), blob


def u(t):
    return q().as_unsigned(t).astype(np.uint64)


def check_com(res, counts, w, mask, valid):
    row, col = res.com(mask)
    orow, ocol, m0 = oracle.com(counts, w.det_rows, w.det_cols, mask=mask, valid=valid)
    grow, gcol = row.cpu().numpy(), col.cpu().numpy()
    for g, o in ((grow, orow), (gcol, ocol)):
        rel = np.abs(g.astype(np.float64) - o) / np.maximum(np.abs(o).astype(np.float64), 1.0)
        assert rel.max() <= 1e-5
        assert np.array_equal(g, o)


def check_all_products(w, counts, valid, blob, masks, df_mask, rects, strides=(1,)):
    with q().Resident(blob, valid=valid) as res:
        for name, m in masks.items():
            for k in strides:
                got = u(res.masked_sum(m, block_stride=k))
                assert np.array_equal(got, oracle.masked_sum(counts, m, valid, stride=k)), (name, k)
        if df_mask is not None:
            for _ in range(2):  # cold (builds the total cache), then warm
                got = u(res.dense_df(df_mask))
                assert np.array_equal(got, oracle.dense_df(counts, df_mask, valid))
        check_com(res, counts, w, None, valid)
        for m in masks.values():
            check_com(res, counts, w, m, valid)
        for (r0, r1, c0, c1) in rects:
            got = q().as_unsigned(res.decode_region(r0, r1, c0, c1))
            assert np.array_equal(got, oracle.region(counts, w.scan_cols, r0, r1, c0, c1, valid)), (r0, r1, c0, c1)
        check_dp(res, counts, valid, strides)
        check_frames(res, counts, valid)
        res.finish()


def check_frames(res, counts, valid, calib=None):
    """Whole-block frames: the first block, the last (possibly partial) one and a run of two."""
    nb = (counts.shape[0] + 511) // 512
    ranges = [(0, 1), (nb - 1, 1)] + ([(1, 2)] if nb > 2 else [])
    kinds = ("native", "amplitude") + (("calibrated",) if calib is not None else ())
    for first, n in ranges:
        for kind in kinds:
            got = res.decode_blocks(first, n, kind)
            got = q().as_unsigned(got) if kind == "native" else got.cpu().numpy()
            want = oracle.frames(counts, first, n, valid, kind, calib)
            assert np.array_equal(got, want), (first, n, kind)


def check_dp(res, counts, valid, strides=(1,), calib=None):
    """Sum and mean diffraction pattern: every scan, a random scan selection, each stride."""
    S = counts.shape[0]
    rng = np.random.default_rng(S)
    for scan_mask in (None, (rng.random(S) < 0.3).astype(np.uint8)):
        for k in strides:
            s, m = res.sum_dp(scan_mask, k)
            ws, wm = oracle.sum_dp(counts, scan_mask, valid, k, calib)
            assert np.array_equal(u(s), ws), k
            assert np.array_equal(m.cpu().numpy(), wm), k


def random_rects(w, n, seed, size=8):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        h = int(rng.integers(1, size + 1))
        wd = int(rng.integers(1, size + 1))
        r0 = int(rng.integers(0, w.scan_rows - h + 1))
        c0 = int(rng.integers(0, w.scan_cols - wd + 1))
        out.append((r0, r0 + h, c0, c0 + wd))
    return out


def test_tiny_full_size():
    w, counts, valid, blob = case("tiny_u8")
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, masks, masks["adf"],
                       [(0, 16, 0, 16), (0, 1, 0, 1), (15, 16, 15, 16), (3, 11, 2, 10)] + random_rects(w, 4, 1))


def test_u16_128x128_full_size():
    w, counts, valid, blob = case("scan128_u16")
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, {"bf": masks["bf"]}, masks["df"],
                       [(0, 8, 0, 8), (60, 68, 124, 128)], strides=(1, 3, 4))


def test_u16_sentinels_and_valid_pixels():
    w, counts, valid, blob = case("scan256_u16_sentinel", 40, 256)  # 10240 scans: 20 blocks
    assert valid is not None and valid.sum() < w.P
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, {"bf": masks["bf"], "full": np.ones(w.P, np.uint8)}, masks["df"],
                       [(0, 8, 0, 8), (1, 9, 124, 132), (32, 40, 248, 256)] + random_rects(w, 6, 3))


def test_scaled_region_reads():
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(10, 256)  # 2560 scans: 5 regions
    x = synth.scaled(w)
    blob = q().encode(x, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, scaled=True)
    codes = oracle.decode(blob.tobytes())
    cal = oracle.calibration(blob.tobytes())
    with q().Resident(blob) as res:
        for (r0, r1, c0, c1) in [(0, 8, 0, 8), (1, 9, 124, 132), (0, 10, 250, 256)] + random_rects(w, 4, 5):
            got = res.decode_region(r0, r1, c0, c1, calibrated=True).cpu().numpy()
            want = []
            for r in range(r0, r1):
                for c in range(c0, c1):
                    s = r * w.scan_cols + c
                    sc, off = cal[s // 512]
                    want.append(oracle.reconstruct(codes[s], sc, off))
            assert np.array_equal(got, np.stack(want)), (r0, r1, c0, c1)
            raw = q().as_unsigned(res.decode_region(r0, r1, c0, c1))
            assert np.array_equal(raw, oracle.region(codes, w.scan_cols, r0, r1, c0, c1))
        # integer products of a scaled resident are exact sums of the codes
        bf = synth.query_masks(w)["bf"]
        assert np.array_equal(u(res.masked_sum(bf)), oracle.masked_sum(codes, bf))
        # the mean diffraction pattern of a scaled resident is that of its calibrated intensities
        check_dp(res, codes, None, (1, 2), calib=cal)
        check_frames(res, codes, None, calib=cal)


def test_u8_low_dose():
    w, counts, valid, blob = case("scan512_u8_lowdose", 48, 512)  # 24576 scans: 48 blocks
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, masks, masks["bf"], [(0, 8, 0, 8), (47, 48, 500, 512)],
                       strides=(1, 4))


@pytest.mark.parametrize("name", ["scan512_u8_lowdose", "scan128_u16"])
def test_dim_waves_on_a_ragged_final_block(name):
    """1147 scans (37 x 31): two complete blocks and a final one of 123 scans,
    seven 16-scan chunks and a tail of 11 scans decoded one at a time. Most
    waves hold dim streams (mean 0.02 or 0.1 outside the disk), which refill
    on demand, and the disk's waves keep the two-step cadence; the switch
    between the chunks and the tail must keep every lane supplied. Every
    product against the oracle at strides 1 and 3, and the polar index's sums
    (the index build decodes the same way)."""
    w, counts, valid, blob = case(name, 37, 31)
    assert w.S % 512 == 123
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, masks, masks["df"] if "df" in masks else masks["bf"],
                       [(0, 8, 0, 8), (33, 37, 20, 31)] + random_rects(w, 3, 11), strides=(1, 3))
    full = np.ones(w.P, np.uint8)
    with q().Resident(blob, valid=valid) as res:
        res.index_build()
        for m in (full, masks["bf"]):
            for k in (1, 3):
                assert np.array_equal(u(res.masked_sum(m, block_stride=k)), oracle.masked_sum(counts, m, valid, stride=k))
        res.finish()


def test_u8_moving_mask_sweep():
    w, counts, valid, blob = case("scan512_u8_lowdose", 16, 512)
    sweep = synth.sweep_masks(w)
    with q().Resident(blob) as res:
        for i, m in enumerate(sweep[::5]):
            assert np.array_equal(u(res.masked_sum(m)), oracle.masked_sum(counts, m)), i


def test_paired_layout():
    w, counts, valid, blob = case("scan1024_u16_paired", 24, 1024)  # 24576 scans: 48 blocks
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, {"bf": masks["bf"]}, masks["df"],
                       [(0, 8, 0, 8), (23, 24, 1016, 1024)] + random_rects(w, 3, 7), strides=(1, 4))


def test_paired_generator_byte_rans_too():
    w, counts, valid, blob = case("scan1024_u16_paired", 8, 1024, 0)
    masks = synth.query_masks(w)
    check_all_products(w, counts, valid, blob, {"bf": masks["bf"]}, masks["df"], [(0, 8, 0, 8)], strides=(1, 4))


@pytest.mark.parametrize("dtype", [np.uint16, np.uint8])
def test_paired_moments_of_row_waves_with_escapes(dtype):
    """Full-detector CoM on a paired resident whose waves each lie inside one
    192-pixel detector row (the packed moment accumulators): bright columns
    coded with the lambda = 20 model (window 13..27, so counts below 13 escape
    below the window base and are negative relative to it), counts far above
    the window, saturated pixels, and a masked CoM with some waves spanning
    two rows. Bit-exact against the oracle."""
    rng = np.random.default_rng(88)
    R, C, S = 12, 192, 1024
    P = R * C
    maxv = np.iinfo(dtype).max
    c = rng.poisson(0.3, size=(S, P)).astype(np.int64)
    bright = rng.choice(P, 400, replace=False)
    c[:, bright] = rng.poisson(20.0, size=(S, 400))
    c[:, bright[:40]] = rng.integers(0, 40, size=(S, 40))          # wide spread around the window
    spikes = rng.choice(S * P, 3000, replace=False)
    c.reshape(-1)[spikes] = rng.choice([300 % (maxv + 1), maxv, 16, 200], size=3000)
    c[:, 5 * C + 17] = maxv                                         # a saturated pixel
    c = np.minimum(c, maxv).astype(dtype)
    blob = q().encode(c, 2, 512, R, C, layout=1)
    masks = [None, synth.disk_mask(R, C, 6, 96, 5), (rng.random(P) < 0.7).astype(np.uint8)]
    with q().Resident(blob) as res:
        for m in masks:
            check_com(res, c, synth.Workload("rows", 2, 512, R, C, 2, 0, 0, 0, 0, 0, 0, 0, 0, 1), m, None)
            mm = np.ones(P, np.uint8) if m is None else m
            assert np.array_equal(u(res.masked_sum(mm)), oracle.masked_sum(c, mm))
        res.finish()


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
def test_paired_moments_packed_per_slot_at_the_bound(dtype):
    """Full-detector CoM on an 8 x 192 paired resident (1536 pixels: two streams
    per lane, so every second wave's two 64-pixel slots lie in different rows
    and keep one packed word each). Every count is uniform in 10..40, so the
    chosen model's window (15 values) holds many counts at 13-14 and the rest
    escape and are clamped to 15 in the packed word: each slot's word reaches
    its bound of 64 lanes x 15 x 63 columns. Bit-exact against the oracle, with
    a mask that shifts the slots off the 64-pixel grid as well."""
    rng = np.random.default_rng(4242)
    R, C, S = 8, 192, 1024
    P = R * C
    c = rng.integers(10, 41, size=(S, P)).astype(dtype)
    c[:, 3 * C + 64: 3 * C + 128] = 14  # a whole slot at one value: CONST streams beside PAIRED ones
    blob = q().encode(c, 2, 512, R, C, layout=1)
    shifted = np.ones(P, np.uint8)
    shifted[0] = 0
    w = synth.Workload("bound", 2, 512, R, C, 2, 0, 0, 0, 0, 0, 0, 0, 0, 1)
    with q().Resident(blob) as res:
        for m in (None, shifted):
            check_com(res, c, w, m, None)
            mm = np.ones(P, np.uint8) if m is None else m
            assert np.array_equal(u(res.masked_sum(mm)), oracle.masked_sum(c, mm))
        res.finish()


@pytest.mark.parametrize("R,C", [(1024, 64), (64, 1024)])
def test_paired_moments_packed_at_the_largest_coordinates(R, C):
    """Full-detector CoM on 65,536-pixel paired residents at the detector-side
    limit of 1024. With 1024 rows of 64 pixels every two-slot wave keeps one
    packed word per slot with rows up to 1023; with 64 rows of 1024 pixels
    every wave lies in one row and keeps one packed word with columns up to
    1023. Counts are uniform in 10..40, so the streams take the highest-mean
    models (window bases up to 13) and most counts escape: each wave's
    per-scan moments, formed in 32 bits before the 64-bit partials, are at
    their largest. Bit-exact against the oracle, also with a mask that moves
    every slot off the 64-pixel grid."""
    rng = np.random.default_rng(9090)
    S = 1024
    P = R * C
    c = rng.integers(10, 41, size=(S, P), dtype=np.uint16)
    blob = q().encode(c, 2, 512, R, C, layout=1)
    shifted = np.ones(P, np.uint8)
    shifted[0] = 0
    w = synth.Workload("largest", 2, 512, R, C, 2, 0, 0, 0, 0, 0, 0, 0, 0, 1)
    with q().Resident(blob) as res:
        for m in (None, shifted):
            check_com(res, c, w, m, None)
        res.finish()


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
def test_paired_moments_packed_over_rows_at_the_bound(dtype):
    """Masked CoM on a 16 x 192 paired resident whose one-stream-per-lane waves
    span four detector rows and 64 columns: the mask keeps columns 0-7 and
    56-63 of every row (16 pixels a row), so each wave's 64 pixels have row
    offsets 0-3 and column offsets 0-63 and share one packed word per scan
    with three fields. Counts are uniform in 10..40, so most escape the chosen
    model's window and are clamped to 15 in the packed word (the excess goes
    to the partials): the fields reach their bounds. Two more masks fall just
    outside the packed range and take the unpacked form: one adds column 64
    (a column offset of 64), one keeps 12 pixels a row (waves over five rows).
    Bit-exact against the oracle."""
    rng = np.random.default_rng(5151)
    R, C, S = 16, 192, 1024
    P = R * C
    c = rng.integers(10, 41, size=(S, P)).astype(dtype)
    c[:, 2 * C: 2 * C + 8] = 0  # EMPTY streams inside a packed wave
    blob = q().encode(c, 2, 512, R, C, layout=1)
    w = synth.Workload("over_rows", 2, 512, R, C, 2, 0, 0, 0, 0, 0, 0, 0, 0, 1)
    masks = []
    for keep in ([*range(0, 8), *range(56, 64)], [*range(0, 8), *range(56, 65)], [*range(0, 6), *range(58, 64)]):
        row = np.zeros(C, np.uint8)
        row[keep] = 1
        masks.append(np.tile(row, R))
    with q().Resident(blob) as res:
        for m in masks:
            check_com(res, c, w, m, None)
            assert np.array_equal(u(res.masked_sum(m)), oracle.masked_sum(c, m))
        res.finish()


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
@pytest.mark.parametrize("top", [127, 128])
def test_rans_moments_packed_rows_at_the_bound(dtype, top):
    """Full-detector CoM on a 4 x 256 byte-rANS resident: every two-stream wave
    lies in one detector row and spans 128 columns. Counts are mostly small with
    a sprinkle at `top` and two whole frames at `top`. With top = 127 the block
    codes no symbol above 127, so those waves keep one packed word per scan, and
    the full frames take both of its fields to their bounds (16 lanes x 2 x 127
    values, column offsets up to 127). With top = 128 they take the unpacked
    form. Bit-exact against the oracle, also with a mask that moves the slots
    off the 64-pixel grid."""
    rng = np.random.default_rng(777 + top)
    R, C, S = 4, 256, 1024
    P = R * C
    c = np.minimum(rng.geometric(0.25, size=(S, P)) - 1, top)
    c[rng.random((S, P)) < 0.02] = top
    c[7] = top
    c[600] = top
    c = c.astype(dtype)
    blob = q().encode(c, 2, 512, R, C, layout=0)
    shifted = np.ones(P, np.uint8)
    shifted[0] = 0
    w = synth.Workload("rows_rans", 2, 512, R, C, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    with q().Resident(blob) as res:
        for m in (None, shifted):
            check_com(res, c, w, m, None)
            mm = np.ones(P, np.uint8) if m is None else m
            assert np.array_equal(u(res.masked_sum(mm)), oracle.masked_sum(c, mm))
        res.finish()


@pytest.mark.parametrize("layout", [0, 1])
def test_uint64_sums_257_detector(layout):
    # 257 x 257 uint16: a full-detector sum can pass 2^32, so outputs are uint64
    P = 257 * 257
    rng = np.random.default_rng(21)
    S = 1024
    c = rng.poisson(0.2, size=(S, P)).astype(np.uint16)
    c[:, :257] = 65535                       # saturated detector row
    c[:, 257:514] = rng.integers(255, 65536, size=(S, 257))  # wide literals
    c[5] = 65535                             # one saturated frame: full sum 4,328,521,215
    valid = np.ones(P, np.uint8)
    valid[1000] = 0                          # one invalid pixel
    blob = q().encode(c, 2, 512, 257, 257, layout=layout)
    with q().Resident(blob, valid=valid) as res:
        assert res.info.sum_bits == 64
        full = np.ones(P, np.uint8)
        got = u(res.masked_sum(full))
        want = oracle.masked_sum(c, full, valid)
        assert np.array_equal(got, want)
        assert int(want[5]) == 4328521215 - 65535 and want.max() > 2**32
        assert np.array_equal(u(res.dense_df(full)), want)
        check_com(res, c, synth.Workload("x", 2, 512, 257, 257, 2, 0, 0, 0, 0, 0, 0, 0, 0, layout), None, valid)
        got = q().as_unsigned(res.decode_region(0, 1, 3, 8))
        assert np.array_equal(got, oracle.region(c, 512, 0, 1, 3, 8, valid))
        check_dp(res, c, valid)  # per-pixel sums of 1024 scans of 65535 pass 2^26: u64 storage


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("det", [(17, 17), (19, 19)])
def test_adversarial_streams(dtype, layout, det):
    from test_oracle import adversarial
    rng = np.random.default_rng(13)
    sr, sc = (2, 512) if layout == 1 else (3, 301)
    P = det[0] * det[1]
    c = adversarial(sr * sc, P, dtype, rng)
    valid = np.ones(P, np.uint8)
    valid[P // 2] = 0
    blob = q().encode(c, sr, sc, det[0], det[1], layout=layout)
    w = synth.Workload("adv", sr, sc, det[0], det[1], 1 if dtype == np.uint8 else 2, 0, 0, 0, 0, 0, 0, 0, 0, layout)
    masks = {"all": np.ones(P, np.uint8), "half": (np.arange(P) % 2).astype(np.uint8)}
    check_all_products(w, c, valid, blob, masks, masks["half"], [(0, sr, 0, sc), (1, 2, 5, 40)],
                       strides=(1, 2))


def test_raw_streams_among_dim_ones_two_per_lane():
    """Dim streams with a few RAW ones, over enough blocks that the plan gives
    every lane two streams: 72 blocks x 16 items of half a workgroup exceed the
    resident workgroups, while the selection stays below 0.4 encoded bytes per
    value. Waves holding a RAW stream take the mixed decode step, in its
    two-per-lane form, for sums, moments and a mask delta."""
    rng = np.random.default_rng(21)
    dr = dc = 64
    P, S = dr * dc, 72 * 512
    # eight distinct blocks, repeated: ones at rate 1/32, and 40 uniform streams
    base = (rng.integers(0, 32, size=(8 * 512, P), dtype=np.uint8) == 0).astype(np.uint16)
    raw = rng.choice(P, 40, replace=False)
    base[:, raw] = rng.integers(0, 65536, size=(base.shape[0], raw.size))
    c = np.tile(base, (S // base.shape[0], 1))
    blob = q().encode(c, 72, 512, dr, dc)
    w = synth.Workload("mixed", 72, 512, dr, dc, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    full = np.ones(P, np.uint8)
    disk = synth.disk_mask(dr, dc, 30, 33, 20)
    with q().Resident(blob) as res:
        assert res.info.mode_counts[2] >= 72 * raw.size  # the uniform streams are stored RAW
        for m in (full, disk):
            for k in (1, 3):
                assert np.array_equal(u(res.masked_sum(m, block_stride=k)), oracle.masked_sum(c, m, stride=k)), k
            check_com(res, c, w, m, None)
        prev = res.masked_sum(full)
        got = res.masked_sum_delta(full, prev, disk)
        assert np.array_equal(u(got), oracle.masked_sum(c, disk))
        res.finish()


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
def test_raw_streams_fill_waves(dtype):
    """200 of 256 streams RAW. Ordered first in each item, they fill three
    waves that decode sums and moments in the RAW-only form; the fourth wave
    mixes RAW and rANS streams. 903 scans give a complete block (decoded in
    two halves when a query is latency-bound) and a final block of 391 scans,
    a ragged chunk and, for uint8, a padded odd-length stream."""
    rng = np.random.default_rng(31)
    dr = dc = 16
    P, sr, sc = dr * dc, 3, 301
    S = sr * sc
    maxv = 255 if dtype == np.uint8 else 65535
    c = rng.poisson(0.4, size=(S, P)).astype(dtype)
    raw = np.sort(rng.choice(P, 200, replace=False))
    c[:, raw] = rng.integers(0, maxv + 1, size=(S, raw.size)).astype(dtype)
    blob = q().encode(c, sr, sc, dr, dc)
    w = synth.Workload("raw", sr, sc, dr, dc, 1 if dtype == np.uint8 else 2, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    valid = np.ones(P, np.uint8)
    valid[raw[7]] = 0
    masks = {"all": np.ones(P, np.uint8), "disk": synth.disk_mask(dr, dc, 8, 8, 5),
             "random": (rng.random(P) < 0.5).astype(np.uint8)}
    with q().Resident(blob, valid=valid) as res:
        assert res.info.mode_counts[2] >= 2 * raw.size
        for name, m in masks.items():
            for k in (1, 2):
                got = u(res.masked_sum(m, block_stride=k))
                assert np.array_equal(got, oracle.masked_sum(c, m, valid, stride=k)), (name, k)
            check_com(res, c, w, m, valid)
        check_com(res, c, w, None, valid)
        assert np.array_equal(u(res.dense_df(masks["disk"])), oracle.dense_df(c, masks["disk"], valid))
        prev = res.masked_sum(masks["all"])
        got = res.masked_sum_delta(masks["all"], prev, masks["disk"])
        assert np.array_equal(u(got), oracle.masked_sum(c, masks["disk"], valid))
        res.finish()


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
@pytest.mark.parametrize("S", [589, 712])
def test_raw_streams_short_final_block(dtype, S):
    """A final block of 77 scans (odd: a padded uint8 stream) or 200 scans:
    RAW-only waves read several streams per load (four for 77 scans, two for
    200), each stream cut by the per-lane byte mask at the block's end."""
    rng = np.random.default_rng(S)
    dr = dc = 16
    P = dr * dc
    maxv = 255 if dtype == np.uint8 else 65535
    c = rng.poisson(0.4, size=(S, P)).astype(dtype)
    raw = np.sort(rng.choice(P, 150, replace=False))
    c[:, raw] = rng.integers(0, maxv + 1, size=(S, raw.size)).astype(dtype)
    blob = q().encode(c, 1, S, dr, dc)
    w = synth.Workload("raw_short", 1, S, dr, dc, 1 if dtype == np.uint8 else 2, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    masks = {"all": np.ones(P, np.uint8), "disk": synth.disk_mask(dr, dc, 8, 8, 5)}
    with q().Resident(blob) as res:
        assert res.info.mode_counts[2] >= 2 * raw.size
        for name, m in masks.items():
            for k in (1, 2):
                got = u(res.masked_sum(m, block_stride=k))
                assert np.array_equal(got, oracle.masked_sum(c, m, stride=k)), (name, k)
            check_com(res, c, w, m, None)
        res.finish()


def test_raw_streams_without_a_plan():
    """A 257 x 257 detector (more pixels than a query plan covers): items are
    pixel tiles, and RAW streams (30 %, uniform uint16) are still ordered first
    within each tile and decoded by RAW-only waves; a final partial block too."""
    rng = np.random.default_rng(33)
    dr = dc = 257
    P, S = dr * dc, 768
    c = (rng.integers(0, 16, size=(S, P), dtype=np.uint8) == 0).astype(np.uint16)
    raw = np.sort(rng.choice(P, P * 3 // 10, replace=False))
    c[:, raw] = rng.integers(0, 65536, size=(S, raw.size), dtype=np.uint16)
    blob = q().encode(c, 3, 256, dr, dc)
    w = synth.Workload("raw257", 3, 256, dr, dc, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0)
    disk = synth.disk_mask(dr, dc, 128, 128, 60)
    with q().Resident(blob) as res:
        assert res.info.mode_counts[2] >= 2 * raw.size
        for m in (np.ones(P, np.uint8), disk):
            for k in (1, 2):
                assert np.array_equal(u(res.masked_sum(m, block_stride=k)), oracle.masked_sum(c, m, stride=k)), k
            check_com(res, c, w, m, None)
        res.finish()


def test_raw_stream_of_the_wrong_length_fails():
    """Moving the boundary between two RAW streams by one value keeps every
    extent even and ordered, so the container passes the host checks; the
    decode finds that neither stream holds exactly its block's values."""
    rng = np.random.default_rng(32)
    P, p = 256, 40  # pixels 40 and 41 share an offset group
    c = rng.integers(0, 65536, size=(1024, P)).astype(np.uint16)  # every stream RAW
    c[511, p] = 2  # the word that becomes pixel 41's header (mode RAW) in block 0
    blob = bytearray(q().encode(c, 2, 512, 16, 16).tobytes())
    h = oracle.header(bytes(blob))
    at = h["rel_off"] + 2 * (p + 1)
    struct.pack_into("<H", blob, at, struct.unpack_from("<H", blob, at)[0] - 2)
    qq = q()
    with qq.Resident(bytes(blob)) as res:
        for mask in (np.ones(P, np.uint8), np.eye(1, P, p, dtype=np.uint8)[0]):
            with pytest.raises(qq.QscValueError) as e:
                res.masked_sum(mask)
            assert e.value.code == qq.ERR_MALFORMED
        with pytest.raises(qq.QscValueError):
            res.com()


def test_sum_dp_edge_cases():
    w, counts, valid, blob = case("tiny_u8")
    with q().Resident(blob) as res:
        s, m = res.sum_dp(np.zeros(w.S, np.uint8))  # no scan selected
        assert not u(s).any() and not m.cpu().numpy().any()
        one = np.zeros(w.S, np.uint8)
        one[37] = 1  # a single scan: the sum is that frame
        s, m = res.sum_dp(one)
        assert np.array_equal(u(s), counts[37].astype(np.uint64))
        assert np.array_equal(m.cpu().numpy(), counts[37].astype(np.float32))
        a, _ = res.sum_dp()
        b, _ = res.sum_dp()
        assert np.array_equal(u(a), u(b))
        res.finish()


def test_empty_mask_and_determinism():
    w, counts, valid, blob = case("tiny_u8")
    with q().Resident(blob) as res:
        z = u(res.masked_sum(np.zeros(w.P, np.uint8)))
        assert (z == 0).all()
        bf = synth.query_masks(w)["bf"]
        a = u(res.masked_sum(bf))
        for _ in range(3):
            assert np.array_equal(u(res.masked_sum(bf)), a)


def corrupt_rans_word(blob):
    """Flip a bit in the state word of the first RANS stream."""
    b = bytearray(blob.tobytes())
    h = oracle.header(bytes(b))
    P = h["det_rows"] * h["det_cols"]
    G = (P + 31) // 32
    for p in range(P):
        g, i = divmod(p, 32)
        gb, = struct.unpack_from("<I", b, h["gbase_off"] + 4 * g)
        rel, = struct.unpack_from("<H", b, h["rel_off"] + 2 * (32 * g + i))
        off = h["payload_off"] + gb + rel
        if struct.unpack_from("<H", b, off)[0] == 1:
            b[off + 2] ^= 0x10
            return bytes(b), p
    raise AssertionError("no RANS stream")


def test_malformed_stream_fails_the_query():
    w, counts, valid, blob = case("tiny_u8")
    bad, p = corrupt_rans_word(blob)
    with pytest.raises(oracle.OracleError):
        oracle.decode(bad)
    qq = q()
    with qq.Resident(bad) as res:
        all_px = np.ones(w.P, np.uint8)
        with pytest.raises(qq.QscValueError) as e:
            res.masked_sum(all_px)
        assert e.value.code == qq.ERR_MALFORMED and f"pixel {p}" in str(e.value)
        # queued form: the error surfaces at finish(), then the resident is usable again
        res.masked_sum(all_px, wait=False)
        with pytest.raises(qq.QscValueError):
            res.finish()
        other = np.zeros(w.P, np.uint8)
        other[(p + 1) % w.P] = 1
        got = u(res.masked_sum(other))
        assert np.array_equal(got, oracle.masked_sum(counts, other))
        with pytest.raises(qq.QscValueError):
            res.decode_region(0, 16, 0, 16)
        with pytest.raises(qq.QscValueError):
            res.com()
        with pytest.raises(qq.QscValueError):
            res.sum_dp()
        with pytest.raises(qq.QscValueError):
            res.decode_blocks(0, 1)


def test_argument_errors():
    w, counts, valid, blob = case("tiny_u8")
    qq = q()
    with qq.Resident(blob) as res:
        with pytest.raises(ValueError):
            res.decode_region(0, 0, 0, 4)
        with pytest.raises(ValueError):
            res.decode_region(0, 17, 0, 4)
        with pytest.raises(ValueError):
            res.decode_region(0, 2, 0, 2, calibrated=True)  # not a scaled resident
        with pytest.raises(ValueError):
            res.masked_sum(np.ones(5, np.uint8))
        assert qq.lib.qsc_masked_sum(res._h, None, 1, None, None, 1) == qq.ERR_INVALID_ARG
        with pytest.raises(ValueError):
            res.decode_blocks(0, 1, "calibrated")  # not a scaled resident
        with pytest.raises(ValueError):
            res.decode_blocks(0, 2)  # one block only
        with pytest.raises(ValueError):
            res.sum_dp(np.ones(3, np.uint8))
        assert qq.lib.qsc_sum_dp(res._h, None, 0, None, None, None, 1) == qq.ERR_INVALID_ARG
