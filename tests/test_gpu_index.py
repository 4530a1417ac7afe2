"""GPU parity of masked sums answered through the polar interaction index.

With an index built, qsc_masked_sum sums the index fields a mask covers and
decodes only the residual pixels. Every result must equal the oracle's masked
sum bit for bit, and the GPU's own decode-only result on a resident without an
index. Masks that are exact unions of leaves (or of a root) exercise the
index fields alone; masks with no full leaf exercise the residual decode alone.
"""
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


def u(t):
    return q().as_unsigned(t).astype(np.uint64)


def leaf_union(order, leaves, P):
    m = np.zeros(P, np.uint8)
    for i in leaves:
        m[order[64 * i: 64 * (i + 1)]] = 1
    return m


def masks_for(w, order, rng):
    P = w.P
    cr, cc = w.det_rows // 2, w.det_cols // 2
    r = min(cr, cc)
    m = {
        "full": np.ones(P, np.uint8),
        "empty": np.zeros(P, np.uint8),
        "disk": synth.disk_mask(w.det_rows, w.det_cols, cr, cc, r // 3),
        "shifted disk": synth.disk_mask(w.det_rows, w.det_cols, cr + 3, cc - 5, r // 2),
        "annulus": synth.annulus_mask(w.det_rows, w.det_cols, cr, cc, r // 5, (4 * r) // 5),
        "random": (rng.random(P) < 0.4).astype(np.uint8),
        "leaves only": leaf_union(order, [0, 1, 2, 5, 9, len(order) // 64 - 1], P),
        "one root": leaf_union(order, range(16, 32), P),
        "checker": (np.arange(P) % 2).astype(np.uint8),  # no leaf is full: residual decode only
    }
    m.update({k: v for k, v in synth.query_masks(w).items()})
    return m


def check_index(w, counts, valid, blob, strides=(1, 3)):
    rng = np.random.default_rng(w.S)
    order = oracle.polar_order(w.det_rows, w.det_cols, w.det_rows // 2, w.det_cols // 2)
    masks = masks_for(w, order, rng)
    with q().Resident(blob, valid=valid) as plain, q().Resident(blob, valid=valid) as res:
        assert res.info.index_bytes == 0
        res.index_build()
        assert res.info.index_bytes > 0
        for name, m in masks.items():
            for k in strides:
                got = u(res.masked_sum(m, block_stride=k))
                assert np.array_equal(got, oracle.masked_sum(counts, m, valid, stride=k)), (name, k)
                assert np.array_equal(got, u(plain.masked_sum(m, block_stride=k))), (name, k)
        # other queries are unchanged by the index
        d = u(res.dense_df(masks["disk"]))
        assert np.array_equal(d, oracle.dense_df(counts, masks["disk"], valid))
        res.finish()


def case(name, sr=None, sc=None):
    w = synth.WORKLOADS[name]
    if sr is not None:
        w = w.with_scans(sr, sc)
    counts = synth.counts(w)
    blob = q().encode(counts, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
    return w, counts, synth.valid_pixels(w), blob


def test_index_tiny():
    check_index(*case("tiny_u8"))


def test_index_u16_128x128():
    check_index(*case("scan128_u16"), strides=(1, 4))


def test_index_with_invalid_pixels():
    w, counts, valid, blob = case("scan256_u16_sentinel", 12, 256)
    assert valid is not None
    check_index(w, counts, valid, blob)


def test_index_u8_low_dose_and_sweep():
    w, counts, valid, blob = case("scan512_u8_lowdose", 8, 512)
    sweep = synth.sweep_masks(w)
    with q().Resident(blob) as res:
        res.index_build((96, 96))
        for i, m in enumerate(sweep[::7]):
            assert np.array_equal(u(res.masked_sum(m)), oracle.masked_sum(counts, m)), i
        res.finish()


def test_index_paired_layout():
    check_index(*case("scan1024_u16_paired", 8, 1024), strides=(1, 2))


def test_index_errors():
    qq = q()
    w, counts, valid, blob = case("tiny_u8")
    with qq.Resident(blob) as res:
        with pytest.raises(ValueError):
            res.index_build((64, 0))  # outside the detector
        assert res.info.index_bytes == 0
        res.index_build((0, 63))  # a corner centre is fine
        res.index_build((32, 32))  # building again replaces the index
        m = synth.query_masks(w)["bf"]
        assert np.array_equal(u(res.masked_sum(m)), oracle.masked_sum(counts, m))
    # more than 65,535 pixels per detector
    c = np.zeros((512, 257 * 257), np.uint16)
    big = qq.encode(c, 1, 512, 257, 257)
    with qq.Resident(big) as res:
        with pytest.raises(qq.QscError) as e:
            res.index_build()
        assert e.value.code == qq.ERR_UNSUPPORTED
    # a malformed stream fails the build and leaves no index
    from test_gpu_parity import corrupt_rans_word
    bad, p = corrupt_rans_word(blob)
    with qq.Resident(bad) as res:
        with pytest.raises(qq.QscValueError):
            res.index_build()
        assert res.info.index_bytes == 0


def test_masked_sum_delta_follows_a_moving_mask():
    w, counts, valid, blob = case("scan256_u16_sentinel", 12, 256)
    shifts = [(0, 0), (2, 0), (2, 2), (-3, 1), (-3, 1), (5, -4)]
    masks = [synth.disk_mask(w.det_rows, w.det_cols, 96 + dr, 96 + dc, 30) for dr, dc in shifts]
    for stride in (1, 3):
        with q().Resident(blob, valid=valid) as res:
            prev = masks[0]
            out = res.masked_sum(prev, block_stride=stride)
            for m in masks[1:]:
                nxt = res.masked_sum_delta(prev, out, m, block_stride=stride)
                assert np.array_equal(u(nxt), oracle.masked_sum(counts, m, valid, stride=stride)), stride
                prev, out = m, nxt
            # in place, and back to an empty mask
            res.masked_sum_delta(prev, out, np.zeros(w.P, np.uint8), block_stride=stride, out=out)
            assert not u(out).any()
            res.finish()


def test_masked_sum_delta_without_a_plan():
    """A detector above 65,536 pixels is decoded without a query plan; deltas still hold."""
    rng = np.random.default_rng(11)
    dr = dc = 257
    counts = rng.poisson(0.3, size=(600, dr * dc)).astype(np.uint8)
    blob = q().encode(counts, 600, 1, dr, dc)
    a = synth.disk_mask(dr, dc, 128, 128, 40)
    b = synth.disk_mask(dr, dc, 131, 126, 40)
    with q().Resident(blob) as res:
        for stride in (1, 2):
            prev = res.masked_sum(a, block_stride=stride)
            got = res.masked_sum_delta(a, prev, b, block_stride=stride)
            assert np.array_equal(u(got), oracle.masked_sum(counts, b, stride=stride)), stride
        res.finish()
