"""The block feed (qsc_feed_*): whole-block frames decoded ahead on the
library's own stream, the paired-resident page's reconstruction feed
("Operation pipeline" item 6: PairedFeed, depth buffers ahead, events both
ways). Every item of a multi-block resident must equal oracle.frames for its
blocks, for several depths and item sizes (including a ragged last item), for
native, amplitude and calibrated frames and both layouts; work queued on the
consumer stream while an item is held must see that item, and a malformed
stream must fail the feed.
"""
import ctypes
import functools

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


@functools.lru_cache(maxsize=4)
def case(name, sr, sc, scaled=False):
    w = synth.WORKLOADS[name].with_scans(sr, sc)
    if scaled:
        x = synth.scaled(w)
        blob = q().encode(x, sr, sc, w.det_rows, w.det_cols, scaled=True)
        data, calib = oracle.decode(blob.tobytes()), oracle.calibration(blob.tobytes())
    else:
        data = synth.counts(w)
        blob = q().encode(data, sr, sc, w.det_rows, w.det_cols, layout=w.layout)
        calib = None
    return w, data, synth.valid_pixels(w), blob, calib


def run_feed(res, data, valid, first, n, per, kind, depth, calib=None):
    got_blocks = []
    for frames, s0 in res.feed(first, n, per, kind, depth):
        b0 = s0 // 512
        nb = min(per, first + n - b0)
        want = oracle.frames(data, b0, nb, valid, kind, calib)
        got = q().as_unsigned(frames) if kind == "native" else frames.cpu().numpy()
        assert np.array_equal(got, want), (b0, nb, kind, depth)
        got_blocks += list(range(b0, b0 + nb))
    assert got_blocks == list(range(first, first + n))


@pytest.mark.parametrize("per,depth", [(1, 1), (1, 2), (3, 2), (2, 3)])
def test_feed_byte_rans_every_block(per, depth):
    w, counts, valid, blob, _ = case("scan256_u16_sentinel", 40, 256)  # 20 blocks, sentinels excluded
    with q().Resident(blob, valid=valid) as res:
        n = res.info.n_blocks
        for kind in ("native", "amplitude"):
            run_feed(res, counts, valid, 0, n, per, kind, depth)
        run_feed(res, counts, valid, 5, 7, per, "native", depth)  # a range inside the resident
        res.finish()


def test_feed_byte_rans_partial_last_block():
    w = synth.WORKLOADS["scan128_u16"].with_scans(5, 300)  # 1500 scans: blocks of 512, 512, 476
    counts = synth.counts(w)
    blob = q().encode(counts, 5, 300, w.det_rows, w.det_cols)
    with q().Resident(blob) as res:
        run_feed(res, counts, None, 0, 3, 2, "native", 2)
        run_feed(res, counts, None, 0, 3, 1, "amplitude", 3)


@pytest.mark.parametrize("depth", [1, 2, 4])
def test_feed_paired_every_block(depth):
    w, counts, valid, blob, _ = case("scan1024_u16_paired", 4, 1024)  # 8 blocks
    with q().Resident(blob) as res:
        for kind in ("native", "amplitude"):
            run_feed(res, counts, valid, 0, 8, 1, kind, depth)
        run_feed(res, counts, valid, 1, 7, 3, "native", depth)


def test_feed_scaled_calibrated():
    w, codes, valid, blob, calib = case("scan256_u16_sentinel", 8, 256, scaled=True)  # 4 regions
    with q().Resident(blob, valid=valid) as res:
        run_feed(res, codes, valid, 0, 4, 1, "calibrated", 2, calib)
        run_feed(res, codes, valid, 0, 4, 2, "native", 2)


def test_feed_consumer_work_sees_the_item():
    """Queries and copies queued on the consumer stream while an item is held
    run after its decode and before its buffer is reused."""
    import torch
    w, counts, valid, blob, _ = case("scan256_u16_sentinel", 40, 256)
    bf = synth.query_masks(w)["bf"]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with q().Resident(blob, valid=valid) as res:
            kept = []
            for frames, s0 in res.feed(0, res.info.n_blocks, 2, "native", 2, stream=side):
                kept.append((s0, frames.clone()))  # queued on the consumer stream
                vi = res.masked_sum(bf, stream=side, wait=False)  # a query between items
            side.synchronize()
            res.finish(stream=side)
            assert np.array_equal(q().as_unsigned(vi).astype(np.uint64), oracle.masked_sum(counts, bf, valid))
    for s0, f in kept:
        b0 = s0 // 512
        assert np.array_equal(q().as_unsigned(f), oracle.frames(counts, b0, min(2, 20 - b0), valid))


def test_feed_malformed_stream_fails():
    import struct
    w, counts, valid, blob, _ = case("scan1024_u16_paired", 4, 1024)
    b = bytearray(blob.tobytes())
    h = oracle.header(bytes(b))
    # flip a code bit of one PAIRED stream of block 3 (its first stream's initial state)
    G = (w.P + 31) // 32
    base, = struct.unpack_from("<Q", b, h["dir_off"] + 16 * 3)
    p = 40 * 192 + 96
    gb, = struct.unpack_from("<I", b, h["gbase_off"] + 4 * (3 * G + p // 32))
    rel, = struct.unpack_from("<H", b, h["rel_off"] + 2 * ((3 * G + p // 32) * 32 + p % 32))
    off = h["payload_off"] + base + gb + rel
    assert struct.unpack_from("<H", b, off)[0] & 7 == 3
    b[off + 2] ^= 0x01
    bad = bytes(b)
    with pytest.raises(oracle.OracleError):
        oracle.decode(bad)
    qq = q()
    with qq.Resident(bad) as res:
        it = res.feed(0, 8, 1, "native", 2)
        with pytest.raises(qq.QscValueError) as e:
            for _ in it:
                pass
        assert e.value.code == qq.ERR_MALFORMED and f"block 3, pixel {p}" in str(e.value)
        # the resident still answers other blocks
        run_feed(res, counts, valid, 4, 4, 2, "native", 2)


def test_feed_argument_errors():
    import torch
    w, counts, valid, blob, _ = case("scan1024_u16_paired", 4, 1024)
    qq = q()
    with qq.Resident(blob) as res:
        buf = torch.empty(512 * w.P, dtype=torch.int16, device="cuda:0")
        ptrs = (ctypes.c_void_p * 2)(buf.data_ptr(), buf.data_ptr())
        h = ctypes.c_void_p()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        nbytes = buf.numel() * 2
        assert qq.lib.qsc_feed_create(res._h, 0, 9, 1, 0, 2, ptrs, nbytes, stream, ctypes.byref(h)) == qq.ERR_INVALID_ARG
        assert qq.lib.qsc_feed_create(res._h, 0, 8, 1, 0, 0, ptrs, nbytes, stream, ctypes.byref(h)) == qq.ERR_INVALID_ARG
        assert qq.lib.qsc_feed_create(res._h, 0, 8, 2, 0, 2, ptrs, nbytes, stream, ctypes.byref(h)) == qq.ERR_INVALID_ARG
        assert qq.lib.qsc_feed_create(res._h, 0, 8, 1, 1, 2, ptrs, nbytes, stream, ctypes.byref(h)) == qq.ERR_INVALID_ARG
        assert qq.lib.qsc_feed_create(res._h, 0, 8, 1, 0, 2, ptrs, nbytes, stream, ctypes.byref(h)) == qq.OK
        i, s0, n = ctypes.c_uint32(), ctypes.c_uint64(), ctypes.c_uint32()
        assert qq.lib.qsc_feed_next(h, ctypes.byref(i), ctypes.byref(s0), ctypes.byref(n)) == qq.OK and n.value == 512
        # a second next before the release is refused
        assert qq.lib.qsc_feed_next(h, ctypes.byref(i), ctypes.byref(s0), ctypes.byref(n)) == qq.ERR_INVALID_ARG
        assert qq.lib.qsc_feed_release(h) == qq.OK
        assert qq.lib.qsc_feed_release(h) == qq.ERR_INVALID_ARG
        assert qq.lib.qsc_feed_destroy(h) == qq.OK
