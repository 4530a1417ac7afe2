"""GPU parity of the device encoder and of residents built from device containers.

qsc_encode_device must write the container the format's reference encoder
(the oracle's, `oracle.encode`) writes for the same values, byte for byte:
tables, offsets, every stream's mode and words, calibration. Cases cover
partial blocks, detectors that are not a multiple of 32 pixels, constant and
all-zero blocks, u16 escapes, a block whose table degenerates to one symbol
(its streams go raw), scaled float32 input with signed zeros and constant
regions, and the paired layout's five modes and model choice. A resident created from the device container answers queries like
the oracle; malformed device containers are refused.
"""
import ctypes

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


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def check_identical(data, sr, sc, dr, dc, scaled=False, layout=0):
    got = q().encode_device(dev(data), sr, sc, dr, dc, layout=layout, scaled=scaled).cpu().numpy()
    want = np.frombuffer(oracle.encode(data, sr, sc, dr, dc, layout=layout, scaled=scaled), dtype=np.uint8)
    assert got.size == want.size
    if not np.array_equal(got, want):
        first = int(np.nonzero(got != want)[0][0])
        raise AssertionError(f"containers differ first at byte {first} of {want.size}")
    return got


def test_workload_slices_byte_identical():
    for name, rows in (("tiny_u8", None), ("scan128_u16", 5), ("scan256_u16_sentinel", 4), ("scan512_u8_lowdose", 2)):
        w = synth.WORKLOADS[name]
        if rows is not None:
            w = w.with_scans(rows, w.scan_cols)  # 5 x 128 scans: one full block and a partial one
        check_identical(synth.counts(w), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols)


def test_adversarial_blocks_byte_identical():
    rng = np.random.default_rng(5)
    dr, dc = 7, 9  # 63 pixels: a partial group of 31
    S = 3 * 512 + 1
    x = rng.poisson(1.5, size=(S, dr * dc)).astype(np.uint16)
    x[:, 5] = 7                                   # a constant stream in every block
    x[:512] = 0                                   # block 0: all zero (empty table)
    x[512:1024] = np.where(rng.random((512, dr * dc)) < 0.5, 300, 400)  # only escapes: degenerate table
    x[1024:1536, 10:20] = rng.integers(0, 65536, size=(512, 10))       # wide escapes next to small counts
    check_identical(x, S, 1, dr, dc)
    check_identical(x[:1], 1, 1, dr, dc)          # one scan
    u8 = rng.poisson(0.3, size=(700, 33)).astype(np.uint8)
    u8[:, 0] = 255
    u8[::3, 1] = 255
    check_identical(u8, 700, 1, 3, 11)


def test_paired_byte_identical():
    w = synth.WORKLOADS["scan1024_u16_paired"].with_scans(1, 1024)  # two blocks
    check_identical(synth.counts(w), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=1)
    rng = np.random.default_rng(8)
    x = rng.poisson(0.7, size=(1024, 70)).astype(np.uint16)
    x[:, 0] = 0                                         # EMPTY
    x[:, 1] = 9                                         # CONST
    x[:, 2] = 0
    x[::97, 2] = 3                                      # SPARSE
    x[:, 3] = rng.integers(0, 65536, size=1024)         # RAW
    x[:, 4] = rng.poisson(18.0, size=1024)              # a high-rate model
    x[::5, 5] = 60000                                   # escapes with literals
    x[:512, 6:10] = rng.poisson(0.02, size=(512, 4))    # the lowest-rate models
    check_identical(x, 1024, 1, 7, 10, layout=1)
    u8 = rng.poisson(2.0, size=(512, 33)).astype(np.uint8)
    u8[::7, 0] = 250
    u8[:, 1] = rng.integers(0, 256, size=512)
    check_identical(u8, 512, 1, 3, 11, layout=1)


def test_scaled_byte_identical():
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(3, 256)
    check_identical(synth.scaled(w), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, scaled=True)
    rng = np.random.default_rng(6)
    x = rng.normal(size=(1024 + 100, 40)).astype(np.float32)
    x[:512] = 2.5                                 # a constant region
    x[512:1024:2, 3] = 0.0
    x[513:1024:2, 3] = -0.0                       # signed zeros at the minimum of their block
    x[512:1024] = np.abs(x[512:1024])
    x[1024:] = -0.0
    x[1030, 7] = 0.0
    check_identical(x, 1124, 1, 5, 8, scaled=True)


def test_resident_from_device_container():
    qq = q()
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(6, 256)
    counts, valid = synth.counts(w), synth.valid_pixels(w)
    blob = qq.encode_device(dev(counts), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols)
    masks = synth.query_masks(w)
    with qq.Resident(blob, valid=valid) as res, qq.Resident(blob.cpu().numpy(), valid=valid) as host:
        assert list(res.info.mode_counts) == list(host.info.mode_counts)
        assert res.info.payload_bytes == host.info.payload_bytes
        for name, m in masks.items():
            got = qq.as_unsigned(res.masked_sum(m, block_stride=2)).astype(np.uint64)
            assert np.array_equal(got, oracle.masked_sum(counts, m, valid, stride=2)), name
        row, col = res.com()
        orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, valid=valid)
        assert np.array_equal(row.cpu().numpy(), orow) and np.array_equal(col.cpu().numpy(), ocol)
        got = qq.as_unsigned(res.decode_region(1, 3, 250, 256))
        sub = np.concatenate([counts[r * w.scan_cols + 250: r * w.scan_cols + 256] for r in (1, 2)])
        assert np.array_equal(got, oracle.region(sub, 6, 0, 2, 0, 6, valid))
        res.finish()
    del blob  # the resident keeps its own copy
    wp = synth.WORKLOADS["scan1024_u16_paired"].with_scans(2, 1024)
    cp = synth.counts(wp)
    pblob = qq.encode_device(dev(cp), wp.scan_rows, wp.scan_cols, wp.det_rows, wp.det_cols, layout=1)
    with qq.Resident(pblob) as res:
        assert res.info.geom.layout == 1
        bf = synth.query_masks(wp)["bf"]
        assert np.array_equal(qq.as_unsigned(res.masked_sum(bf)).astype(np.uint64), oracle.masked_sum(cp, bf))
        res.finish()
    scaled = synth.scaled(w)
    sblob = qq.encode_device(dev(scaled), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, scaled=True)
    with qq.Resident(sblob) as res:
        got = res.decode_region(0, 1, 0, 4, calibrated=True).cpu().numpy()
        sc, off, codes = oracle.calibrate(scaled[:512])
        assert np.array_equal(got, oracle.reconstruct(codes.reshape(512, -1)[:4], sc, off).reshape(4, -1))


def test_device_encoder_errors():
    import torch
    qq = q()
    x = np.zeros((512, 64), np.uint16)
    with pytest.raises(qq.QscValueError):
        qq.encode_device(dev(x[:500]), 500, 1, 8, 8, layout=1)  # the paired layout needs whole blocks
    f = np.ones((512, 64), np.float32)
    f[100, 3] = np.nan
    with pytest.raises(qq.QscValueError):
        qq.encode_device(dev(f), 512, 1, 8, 8, scaled=True)
    with pytest.raises(ValueError):
        qq.encode_device(dev(x), 511, 1, 8, 8)  # wrong size
    # a capacity below the container size reports the size and writes no payload
    g = qq.Geometry(512, 1, 8, 8, 2, 0, 0)
    d = dev(np.random.default_rng(7).integers(0, 65536, size=(512, 64)).astype(np.uint16))  # every stream raw
    out = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    n = ctypes.c_uint64()
    rc = qq.lib.qsc_encode_device(ctypes.byref(g), d.data_ptr(), out.data_ptr(), 8192, ctypes.byref(n), None)
    assert rc == qq.ERR_INVALID_ARG and n.value > 8192
    # a device container with a reserved stream-header bit set is refused
    w = synth.WORKLOADS["tiny_u8"]
    blob = qq.encode_device(dev(synth.counts(w)), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols).clone()
    h = oracle.header(blob.cpu().numpy().tobytes())
    blob[h["payload_off"] + 1] = 0x80  # the first stream's header, high byte
    with pytest.raises(qq.QscValueError):
        qq.Resident(blob)
    blob[h["payload_off"] + 1] = 0
    blob[0] = ord("X")  # bad magic
    with pytest.raises(qq.QscValueError):
        qq.Resident(blob)


@pytest.mark.slow
def test_full_size_128x128_byte_identical():
    """The whole 128x128-scan u16 workload (604 M values) against the oracle encoder."""
    w = synth.WORKLOADS["scan128_u16"]
    check_identical(synth.counts(w), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols)


def test_borrowed_device_container():
    import torch
    qq = q()
    w = synth.WORKLOADS["scan128_u16"].with_scans(4, 128)
    counts = synth.counts(w)
    blob = qq.encode_device(dev(counts), w.scan_rows, w.scan_cols, w.det_rows, w.det_cols)
    keep = blob.clone()
    bf = synth.query_masks(w)["bf"]
    with qq.Resident(blob, borrow=True) as res, qq.Resident(keep) as copied:
        assert res.info.resident_bytes < copied.info.resident_bytes  # the container is not copied
        got = qq.as_unsigned(res.masked_sum(bf)).astype(np.uint64)
        assert np.array_equal(got, oracle.masked_sum(counts, bf))
        res.finish()
    assert torch.equal(blob, keep)  # the caller's container is unchanged and still usable
    # no room after the container for the decoders' read-ahead
    tight = blob.clone()
    n = ctypes.c_void_p()
    rc = qq.lib.qsc_resident_create_device_borrow(tight.data_ptr(), tight.numel(), tight.numel(), None, None,
                                                  ctypes.byref(n))
    assert rc == qq.ERR_INVALID_ARG
