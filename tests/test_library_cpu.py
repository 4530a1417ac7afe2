"""Library checks that need no GPU: the C-ABI loads and exports every declared
symbol, the host encoder is byte-identical to the oracle encoder, and
resident_create rejects malformed containers before touching the device."""
import ctypes
import os
import re
import struct

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def qsc():
    import stem_compressed_count_amd as q
    return q


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qsc.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qsc_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    q = qsc()
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(q.lib, n), n
    assert set(names) == set(q.EXPORTS)
    assert q.abi() == "qsc-byte-rans-v1;qsc-paired-v1"


def test_library_is_gfx950_code():
    # the shared object carries an offload bundle for gfx950
    blob = open(qsc().LIB_PATH, "rb").read()
    assert b"gfx950" in blob


CASES = [
    ("tiny_u8", 16, 16, 0), ("scan128_u16", 4, 128, 0), ("scan256_u16_sentinel", 4, 128, 0), ("scan512_u8_lowdose", 2, 256, 0), ("scan512_u8_lowdose", 3, 301, 0),
]


@pytest.mark.parametrize("name,sr,sc,layout", CASES)
def test_encoder_matches_oracle_bytes(name, sr, sc, layout):
    w = synth.WORKLOADS[name].with_scans(sr, sc)
    c = synth.counts(w)
    a = qsc().encode(c, sr, sc, w.det_rows, w.det_cols, layout=layout).tobytes()
    assert a == oracle.encode(c, sr, sc, w.det_rows, w.det_cols, layout=layout)


def test_encoder_matches_oracle_paired_and_scaled():
    w = synth.Workload("p", 16, 64, 64, 64, 2, 5.0, 0.1, 32, 32, 20, 2, 0, 77, 1)
    c = synth.counts(w)
    assert qsc().encode(c, 16, 64, 64, 64, layout=1).tobytes() == oracle.encode(c, 16, 64, 64, 64, layout=1)
    x = synth.scaled(synth.WORKLOADS["scan256_u16_sentinel"].with_scans(2, 300))
    assert qsc().encode(x, 2, 300, 192, 192, scaled=True).tobytes() == oracle.encode(x, 2, 300, 192, 192, scaled=True)


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
@pytest.mark.parametrize("layout", [0, 1])
def test_encoder_matches_oracle_adversarial(dtype, layout):
    from test_oracle import adversarial
    rng = np.random.default_rng(11)
    sr, sc = (2, 512) if layout == 1 else (3, 301)
    for det in [(17, 17), (19, 19)]:
        c = adversarial(sr * sc, det[0] * det[1], dtype, rng)
        a = qsc().encode(c, sr, sc, det[0], det[1], layout=layout).tobytes()
        assert a == oracle.encode(c, sr, sc, det[0], det[1], layout=layout)
        assert np.array_equal(oracle.decode(a), c)


def test_encoder_streams_in_several_calls():
    w = synth.WORKLOADS["scan128_u16"].with_scans(6, 200)  # 1200 scans: blocks of 512, 512, 176
    c = synth.counts(w)
    q = qsc()
    enc = q.Encoder(6, 200, 192, 192, dtype=2)
    enc.add(c[:512])
    enc.add(c[512:])
    blob = enc.blob().tobytes()
    enc.close()
    assert blob == oracle.encode(c, 6, 200, 192, 192)
    enc = q.Encoder(6, 200, 192, 192, dtype=2)
    with pytest.raises(ValueError):
        enc.add(c[:100].astype(np.uint8))  # wrong dtype
    enc.add(c[:300])
    with pytest.raises(q.QscError):
        enc.add(c[300:])  # a partial block was already added
    enc.close()


def test_encoder_rejects_nan_and_bad_geometry():
    q = qsc()
    x = np.ones((512, 4), dtype=np.float32)
    x[3, 1] = np.nan
    with pytest.raises(q.QscValueError):
        q.encode(x, 1, 512, 2, 2, scaled=True)
    with pytest.raises(q.QscValueError):
        q.Encoder(3, 100, 2, 2, dtype=2, layout=1)  # paired needs complete 512-scan blocks
    with pytest.raises(q.QscValueError):
        q.Encoder(1, 10, 2000, 2, dtype=2)  # detector dimension above 1024


def test_float16_is_refused():
    """No float16 storage: neither native nor scaled encoding accepts float16 values
    (scaled-uint16 page, "What dtype means")."""
    q = qsc()
    x = np.ones((512, 4), dtype=np.float16)
    with pytest.raises(ValueError, match="float16"):
        q.encode(x, 1, 512, 2, 2)
    with pytest.raises(ValueError, match="float16"):
        q.encode(x, 1, 512, 2, 2, scaled=True)
    with pytest.raises(ValueError):
        q.encode(x.astype(np.int32), 1, 512, 2, 2)


def create_status(blob):
    q = qsc()
    b = np.frombuffer(blob, dtype=np.uint8)
    h = ctypes.c_void_p()
    return q.lib.qsc_resident_create(b.ctypes.data, b.size, None, None, ctypes.byref(h))


def test_resident_create_rejects_malformed_before_the_device():
    w = synth.WORKLOADS["tiny_u8"]
    c = synth.counts(w)
    blob = bytearray(oracle.encode(c, 16, 16, 64, 64))
    h = oracle.header(bytes(blob))
    q = qsc()
    # reserved stream header bit (paired-resident page, "Verification")
    bad = bytearray(blob)
    bad[h["payload_off"] + 1] |= 0x80
    assert create_status(bytes(bad)) == q.ERR_MALFORMED
    # invalid mode
    bad = bytearray(blob)
    bad[h["payload_off"]] = (bad[h["payload_off"]] & ~7) | 5
    assert create_status(bytes(bad)) == q.ERR_MALFORMED
    # shortened extent: the last stream's end moves before its start
    bad = bytearray(blob)
    struct.pack_into("<I", bad, h["dir_off"] + 12, 1)
    assert create_status(bytes(bad)) == q.ERR_MALFORMED
    # a relative offset that breaks monotonic order
    bad = bytearray(blob)
    struct.pack_into("<H", bad, h["rel_off"] + 2, 0xFFFF)
    assert create_status(bytes(bad)) == q.ERR_MALFORMED
    # frequency table not summing to 4096
    bad = bytearray(blob)
    bad[h["table_off"]] ^= 1
    assert create_status(bytes(bad)) == q.ERR_MALFORMED
    # another ABI is refused
    bad = bytearray(blob)
    bad[8:24] = b"qsc-byte-rans-v7"
    assert create_status(bytes(bad)) == q.ERR_UNSUPPORTED
    # truncated blob
    assert create_status(bytes(blob[:-2])) == q.ERR_MALFORMED


def test_paired_model_tables_are_validated():
    w = synth.Workload("p", 1, 512, 8, 8, 2, 5.0, 0.1, 4, 4, 2, 0, 0, 3, 1)
    c = synth.counts(w)
    blob = bytearray(oracle.encode(c, 1, 512, 8, 8, layout=1))
    h = oracle.header(bytes(blob))
    blob[h["table_off"] + 2] ^= 1  # one count of model 0 changed
    assert create_status(bytes(blob)) == qsc().ERR_MALFORMED


def test_device_encoder_bound_and_argument_errors():
    """Host logic of the device encoder: its capacity bound follows the format's
    section layout with every stream raw, and bad arguments fail before any GPU work."""
    q = qsc()
    for (sr, sc, dr, dc, dtype, layout, scaled) in [(3, 301, 7, 9, 2, 0, 0), (1, 700, 3, 11, 1, 0, 0),
                                                  (2, 512, 5, 8, 2, 1, 0), (1, 1124, 5, 8, 2, 0, 1)]:
        g = q.Geometry(sr, sc, dr, dc, dtype, layout, scaled)
        n = ctypes.c_uint64()
        assert q.lib.qsc_encode_device_bound(ctypes.byref(g), ctypes.byref(n)) == q.OK
        S, P, G = sr * sc, dr * dc, (dr * dc + 31) // 32
        nb = (S + 511) // 512
        up = lambda o: (o + 255) // 256 * 256
        payload_off = up(up(up(up(256 + 16 * nb) + (512 * nb if layout == 0 else 2 * 32 * 256)) + 4 * nb * G)
                         + 64 * nb * G)
        raw = sum(P * (2 + (2 * m if dtype == 2 else m + m % 2)) for m in
                  [min(512, S - 512 * b) for b in range(nb)])
        want = payload_off + raw
        if scaled:
            want = up(want) + 16 * nb
        assert n.value == want, (sr, sc, dr, dc, dtype, layout, scaled)
    bad = q.Geometry(3, 301, 7, 9, 3, 0, 0)  # dtype 3
    n = ctypes.c_uint64()
    assert q.lib.qsc_encode_device_bound(ctypes.byref(bad), ctypes.byref(n)) == q.ERR_INVALID_ARG
    g = q.Geometry(3, 301, 7, 9, 2, 0, 0)
    assert q.lib.qsc_encode_device(ctypes.byref(g), None, None, 0, ctypes.byref(n), None) == q.ERR_INVALID_ARG
    assert q.lib.qsc_encode_device(ctypes.byref(bad), ctypes.c_void_p(16), ctypes.c_void_p(16), 1 << 20,
                                   ctypes.byref(n), None) == q.ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert q.lib.qsc_resident_create_device(None, 4096, None, None, ctypes.byref(h)) == q.ERR_INVALID_ARG
    assert q.lib.qsc_resident_create_device_borrow(None, 4096, 8192, None, None, ctypes.byref(h)) == q.ERR_INVALID_ARG


def test_stream_split_and_pack_are_inverse():
    """The tests' container editor (tests/streams.py) rebuilds a container
    byte for byte from its streams, for both layouts and a partial group."""
    import streams
    rng = np.random.default_rng(12)
    for layout, sr, sc, det in [(0, 3, 301, (7, 9)), (1, 2, 512, (5, 13))]:
        c = rng.poisson(1.5, size=(sr * sc, det[0] * det[1])).astype(np.uint16)
        blob = oracle.encode(c, sr, sc, det[0], det[1], layout=layout)
        _, st = streams.split(blob)
        assert streams.pack(blob, st) == blob
        # a stream two bytes longer: the container stays structurally sound, and
        # the oracle finds exactly that stream malformed
        st[0][3] = st[0][3] + b"\0\0"
        with pytest.raises(oracle.OracleError) as e:
            oracle.decode(streams.pack(blob, st))
        assert e.value.code == oracle.ERR_MALFORMED and "block 0 pixel 3" in str(e.value)


def staged_lane(demand, start_word, n_steps=512, chunk_words=16, cadence=4):
    """One lane of the staged escape-heavy decode, as the kernel runs it: a ring
    of two chunks of `chunk_words` 16-bit words, both filled before the first
    step; at every `cadence` steps the chunk requested at the previous cadence
    is written, then the next chunk is requested if the ring half it goes to
    has been consumed. A step reads the word pair (wi, wi + 1) and consumes
    0-2 words. Returns the smallest number of written words ahead of wi seen
    at any step that consumed words (each such step needs that many)."""
    wi = start_word          # next word, counted from chunk 0
    fl = 2                   # chunks requested (and written: chunks 0 and 1)
    written = 2 * chunk_words
    pend = False
    worst = None
    for t in range(n_steps):
        if t and t % cadence == 0:
            if pend:
                written += chunk_words
                assert written - wi <= 2 * chunk_words, (t, wi, written)  # no unconsumed word is overwritten
            req = wi >= chunk_words * (fl - 1)   # the older half is free
            pend = req
            fl += req
        d = demand(t)
        if d:
            ahead = written - wi
            assert ahead >= d, (t, wi, written, d)
            worst = ahead if worst is None else min(worst, ahead)
        wi += d
    return worst


def test_staged_ring_never_reads_an_unwritten_word():
    """The staged decode's ring protocol (32-byte chunks, two per ring, a
    cadence of four steps, a chunk written one cadence after its request)
    keeps a lane's next two words written whatever the stream's rate: at most
    two words a step (a renormalisation word and an escape literal), checked
    for the worst case, idle stretches followed by bursts, and random rates,
    from every starting word of chunk 0; and a chunk is written only over
    words already consumed."""
    rng = np.random.default_rng(5)
    for start in range(16):
        assert staged_lane(lambda t: 2, start) >= 2
        for period in (3, 5, 13, 37, 61):
            staged_lane(lambda t: 0 if (t // period) % 2 else 2, start)
        for _ in range(20):
            p = rng.random()
            draws = (rng.random((512, 2)) < p).sum(axis=1)
            staged_lane(lambda t: int(draws[t]), start)
    # a cadence of eight steps with the same ring runs dry
    with pytest.raises(AssertionError):
        for start in range(16):
            staged_lane(lambda t: 2, start, cadence=8)
