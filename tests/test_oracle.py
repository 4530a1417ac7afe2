"""Pins of the CPU oracle against facts fixed outside it.

Each test ties one part of the oracle to something it cannot produce by
itself: hand-derived streams and model tables (tests/golden), NumPy brute
force, closed forms, numpy.rint, and round-trip identity of encode/decode over
every generator and a set of adversarial streams. A plausible mistake in the
oracle (a dropped term, a transposed index, a wrong rounding or mode rule)
fails at least one of them.
"""
import os
import struct

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals, freq, stream, counts, extra = None, {}, None, {}, {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "values":
            vals = [int(v) for v in rest]
        elif key == "freq":
            freq[int(rest[0])] = int(rest[1])
        elif key == "stream":
            stream = bytes(int(b, 16) for b in rest)
        elif key == "count":
            counts[int(rest[0])] = int(rest[1])
        else:
            extra[key] = [int(v) for v in rest]
    return vals, freq, stream, counts, extra


def pack_container(scan_rows, scan_cols, det_rows, det_cols, dtype, table, stream_list, layout=0):
    """A one-block container laid out by hand from FORMAT 1.1-1.3.

    Layout 0 takes the block's frequency table as {symbol: f}; layout 1 takes
    the 32 x 256 pair-model counts (a uint16 array) for its table section."""
    P = det_rows * det_cols
    G = (P + 31) // 32
    S = scan_rows * scan_cols
    assert S <= 512 and (layout == 0 or S == 512)

    def up(o):
        return (o + 255) // 256 * 256

    dir_off = 256
    table_off = up(dir_off + 16)
    gbase_off = up(table_off + (512 if layout == 0 else 2 * 32 * 256))
    rel_off = up(gbase_off + 4 * G)
    payload_off = up(rel_off + 64 * G)
    payload = b"".join(stream_list)
    total = payload_off + len(payload)
    blob = bytearray(total)
    blob[0:8] = b"QSCRES01"
    tag = b"qsc-byte-rans-v1" if layout == 0 else b"qsc-paired-v1"
    blob[8:8 + len(tag)] = tag
    struct.pack_into("<10I", blob, 40, 1, layout, scan_rows, scan_cols, det_rows, det_cols, dtype, 512, 1, 0)
    struct.pack_into("<8Q", blob, 80, dir_off, table_off, gbase_off, rel_off, payload_off, len(payload), 0, total)
    struct.pack_into("<QII", blob, dir_off, 0, S, len(payload))
    if layout == 0:
        for s, f in table.items():
            struct.pack_into("<H", blob, table_off + 2 * s, f)
    else:
        blob[table_off:table_off + 2 * 32 * 256] = np.asarray(table, dtype="<u2").tobytes()
    starts = np.cumsum([0] + [len(x) for x in stream_list])
    for g in range(G):
        gb = int(starts[32 * g])
        struct.pack_into("<I", blob, gbase_off + 4 * g, gb)
        for i in range(32):
            p = 32 * g + i
            st = int(starts[p]) if p < P else int(starts[P])
            struct.pack_into("<H", blob, rel_off + 2 * (32 * g + i), st - gb)
    blob[payload_off:] = payload
    return bytes(blob)


# ---------------------------------------------------------------------------
# codec pins
# ---------------------------------------------------------------------------

def test_golden_rans_u8_stream_encode_and_decode():
    vals, freq, stream, _, _ = read_golden("rans_u8_tiny.txt")
    counts = np.array(vals, dtype=np.uint8).reshape(8, 1)
    expect = pack_container(2, 4, 1, 1, 1, freq, [stream])
    blob = oracle.encode(counts, 2, 4, 1, 1)
    assert blob == expect
    assert np.array_equal(oracle.decode(expect), counts)


def test_golden_rans_u16_escape_decodes():
    vals, freq, stream, _, _ = read_golden("rans_u16_escape.txt")
    blob = pack_container(1, 2, 1, 1, 2, freq, [stream])
    assert oracle.decode(blob).ravel().tolist() == vals
    # the same values encode as RAW (smaller): header 2, then the two u16 values
    enc = oracle.encode(np.array(vals, dtype=np.uint16).reshape(2, 1), 1, 2, 1, 1)
    h = oracle.header(enc)
    assert enc[h["payload_off"]:] == struct.pack("<3H", 2, 0, 300)


def test_golden_pair_model0():
    _, _, _, counts, extra = read_golden("pair_model0.txt")
    n, a0, use = oracle.pair_models()
    assert a0[0] == extra["a0"][0]
    assert use[0] == sum(1 << k for k in extra["in_use"])
    want = np.zeros(256, dtype=np.uint16)
    for i, c in counts.items():
        want[i] = c
    assert np.array_equal(n[0], want)


def read_runs_golden(name):
    """A golden of value runs and stream bytes: 'run v n', 'hex b..', 'repeat k b..', '<key> ints'."""
    vals, stream, extra = [], bytearray(), {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "run":
            vals += [int(rest[0])] * int(rest[1])
        elif key == "hex":
            stream += bytes(int(b, 16) for b in rest)
        elif key == "repeat":
            stream += bytes(int(b, 16) for b in rest[1:]) * int(rest[0])
        else:
            extra[key] = [int(v) for v in rest]
    return vals, bytes(stream), extra


def paired_golden_blob(stream):
    n, _, _ = oracle.pair_models()
    return pack_container(1, 512, 1, 1, 2, n, [stream], layout=1)


def test_golden_paired_stream_decodes():
    vals, stream, _ = read_runs_golden("paired_u16_model0.txt")
    assert len(vals) == 512 and len(stream) == 2 + 326
    assert oracle.decode(paired_golden_blob(stream)).ravel().tolist() == vals


def test_golden_paired_stream_end_checks():
    """FORMAT 3.3 end check on the hand-worked stream: each change below breaks it."""
    _, stream, _ = read_runs_golden("paired_u16_model0.txt")
    cases = {}
    b = bytearray(stream)
    b[-1] |= 0x80  # a one in the zero padding
    cases["pad bit"] = bytes(b)
    cases["16 spare bits"] = stream + bytes(2)  # a whole spare word after the pad
    cases["shortened"] = stream[:-2]  # the last literal loses its top bits and the pad
    b = bytearray(stream)
    # the last literal (bits 2583-2598 of the section) 2 -> 1: a value in use inside the window
    bit = 16 + 2583  # 2 header bytes
    b[bit // 8] ^= 1 << (bit % 8)
    b[(bit + 1) // 8] ^= 1 << ((bit + 1) % 8)
    cases["in-window literal"] = bytes(b)
    b = bytearray(stream)
    # the final 10 bits read at t = 255 (bits 2573-2582) 0 -> 1: the state does not return to 0
    bit = 16 + 2573
    b[bit // 8] ^= 1 << (bit % 8)
    cases["final state"] = bytes(b)
    b = bytearray(stream)
    b[1] |= 0x01  # reserved header bit 8
    cases["reserved bit"] = bytes(b)
    for name, bad in cases.items():
        with pytest.raises(oracle.OracleError) as e:
            oracle.decode(paired_golden_blob(bad))
        assert e.value.code == oracle.ERR_MALFORMED, name


def test_pair_tables_every_state_decodes_to_a_valid_next_state():
    """FORMAT 3.2 for all 32 models: each state's entry (symbol, nbits, next-state
    base) leads into [0, 1024); per symbol the ranges [newX, newX + 2^nbits)
    tile [0, 1024) exactly (so every encoder state has exactly one decoder
    predecessor); each symbol holds n[i] states; and the encoder step of every
    symbol from every state x in [1024, 2048) lands on a state whose entry has
    that symbol, emits that entry's nbits, and decodes back to x - 1024."""
    counts, _, _ = oracle.pair_models()
    for m in range(32):
        sym, nb, nx = oracle.pair_decode_table(m)
        n = counts[m]
        assert np.array_equal(np.bincount(sym, minlength=256), n), m
        assert nb.max() <= 10
        assert np.all(nx.astype(np.int64) + (1 << nb.astype(np.int64)) <= 1024), m
        for i in np.nonzero(n)[0]:
            st = np.nonzero(sym == i)[0]
            lo = nx[st].astype(np.int64)
            hi = lo + (1 << nb[st].astype(np.int64))
            order = np.argsort(lo)
            assert lo[order][0] == 0 and hi[order][-1] == 1024, (m, i)
            assert np.array_equal(lo[order][1:], hi[order][:-1]), (m, i)
            k, bits, to = oracle.pair_encode_steps(m, int(i))
            assert np.all(sym[to] == i), (m, i)
            assert np.array_equal(nb[to].astype(np.uint32), k), (m, i)
            assert np.all(bits < (1 << k))
            assert np.array_equal(nx[to].astype(np.int64) + bits, np.arange(1024)), (m, i)


def table_golden_cases(name):
    """Cases of a table golden: (histogram, expected frequencies) per 'case' (one if none)."""
    cases, h, f = [], {}, {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "case":
            if h:
                cases.append((h, f))
            h, f = {}, {}
            continue
        r = [int(v) for v in rest]
        if key == "hist":
            h[r[0]] = r[1]
        elif key == "histrange":
            h.update({s: r[2] for s in range(r[0], r[1] + 1)})
        elif key == "freq":
            f[r[0]] = r[1]
        elif key == "freqrange":
            f.update({s: r[2] for s in range(r[0], r[1] + 1)})
    cases.append((h, f))
    return cases


def block_with_histogram(h, seed):
    """One uint8 block of 9 non-constant streams x 512 scans whose symbols have histogram h."""
    vals = np.concatenate([np.full(c, s, np.uint8) for s, c in sorted(h.items())])
    assert vals.size == 9 * 512
    rng = np.random.default_rng(seed)
    c = rng.permutation(vals).reshape(512, 9)
    assert not any((c[:, p] == c[0, p]).all() for p in range(9))
    return c


@pytest.mark.parametrize("name", ["rans_table_excess.txt", "rans_table_deficit.txt"])
def test_golden_rans_table_rules(name):
    """FORMAT 2.2 steps 3 and 4 on hand-worked histograms (excess with a tie; deficit
    to the largest h, not the largest remainder; deficit with a tie)."""
    for j, (h, f) in enumerate(table_golden_cases(name)):
        c = block_with_histogram(h, seed=40 + j)
        blob = oracle.encode(c, 1, 512, 3, 3)
        hd = oracle.header(blob)
        got = np.frombuffer(blob[hd["table_off"]:hd["table_off"] + 512], dtype=np.uint16)
        want = np.zeros(256, np.uint16)
        for s, v in f.items():
            want[s] = v
        assert np.array_equal(got, want), (name, j)
        assert np.array_equal(oracle.decode(blob), c)


@pytest.mark.parametrize("dtype", [np.uint16, np.uint8])
def test_mode_choice_at_the_sparse_paired_boundary(dtype):
    """FORMAT 3.4: PAIRED replaces SPARSE only when it is at least 2 bytes smaller.
    Stream sizes are even, so gaps of 0 and 2 bytes fix the rule. With model 0 a
    count of 1 is in the window and a count of 2 escapes to a literal; a lone 2
    codes in 10 + 10 + literal + a few one-bit (0,0) steps, under 48 bits for
    u16, so PAIRED is 8 bytes, SPARSE's size (a tie); a lone 1 saves the
    literal and codes in 6 bytes."""
    lit = 2 if dtype == np.uint16 else 1
    cases = [([(100, 2)], 2), ([(100, 1)], 3), ([(100, 1), (300, 2)], 3), ([(100, 2), (300, 2)], 2)]
    for nz, mode in cases:
        v = np.zeros(512, np.uint32)
        for pos, val in nz:
            v[pos] = val
        nnz = len(nz)
        sparse = 4 + 2 * nnz + (2 * nnz if lit == 2 else nnz + nnz % 2)
        model, paired = oracle.paired_size(v, 2 if lit == 2 else 1)
        assert model == 0
        assert sparse - paired == (2 if mode == 3 else 0), (nz, sparse, paired)
        blob = oracle.encode(v.astype(dtype).reshape(512, 1), 1, 512, 1, 1, layout=1)
        hd = oracle.header(blob)
        assert stream_modes(blob)[0][0] & 7 == mode, nz
        assert hd["payload_bytes"] == (paired if mode == 3 else sparse), nz
        assert np.array_equal(oracle.decode(blob).ravel(), v)


def test_pair_model_invariants():
    n, a0, use = oracle.pair_models()
    assert (n.sum(axis=1) == 1024).all()
    lam = 0.01 * 2000.0 ** (np.arange(32) / 31.0)
    assert np.isclose(lam[31], 20.0)
    assert np.array_equal(a0, np.maximum(0, np.floor(lam) - 7).astype(np.uint32))
    for m in range(32):
        support = [(a == 15 or (use[m] >> a) & 1) and (b == 15 or (use[m] >> b) & 1)
                   for a in range(16) for b in range(16)]
        assert np.array_equal(n[m] > 0, np.array(support, dtype=bool)), m
    # lambda = 20: all 15 window values (13..27) have Poisson mass >= 1/1024
    assert use[31] == (1 << 15) - 1


def test_rans_table_quantization_invariants():
    w = synth.WORKLOADS["tiny_u8"]
    c = synth.counts(w)
    blob = oracle.encode(c, 16, 16, 64, 64)
    h = oracle.header(blob)
    f = np.frombuffer(blob[h["table_off"]:h["table_off"] + 512], dtype=np.uint16)
    assert f.sum() == 4096
    # nonzero exactly on the symbols that occur in non-constant streams
    nonconst = [p for p in range(c.shape[1]) if not (c[:, p] == c[0, p]).all()]
    present = np.zeros(256, dtype=bool)
    present[np.unique(c[:, nonconst])] = True
    assert np.array_equal(f > 0, present)


ROUNDTRIP = [
    ("tiny_u8", 16, 16, 0),
    ("scan128_u16", 8, 64, 0),
    ("scan256_u16_sentinel", 8, 64, 0),
    ("scan512_u8_lowdose", 4, 128, 0),
]


@pytest.mark.parametrize("name,sr,sc,layout", ROUNDTRIP)
def test_roundtrip_generators(name, sr, sc, layout):
    w = synth.WORKLOADS[name].with_scans(sr, sc)
    c = synth.counts(w)
    blob = oracle.encode(c, sr, sc, w.det_rows, w.det_cols, layout=layout)
    assert np.array_equal(oracle.decode(blob), c)


def test_roundtrip_paired_generator():
    # the 1024x1024-scan paired generator on a 64 x 64 detector crop keeps the test fast
    w = synth.WORKLOADS["scan1024_u16_paired"]
    w = synth.Workload("p", 16, 64, 64, 64, 2, 5.0, 0.1, 32, 32, 20, 2, 0, 77, 1)
    c = synth.counts(w)
    blob = oracle.encode(c, 16, 64, 64, 64, layout=1)
    assert np.array_equal(oracle.decode(blob), c)
    # the paired layout codes this Poisson data below the byte-rANS layout
    assert len(blob) < len(oracle.encode(c, 16, 64, 64, 64, layout=0))


def adversarial(S, P, dtype, rng):
    """Streams that exercise every mode and escape path."""
    maxv = 255 if dtype == np.uint8 else 65535
    c = rng.poisson(0.3, size=(S, P)).astype(dtype)
    c[:, 0] = 0                          # all zero
    c[:, 1] = 7                          # constant
    c[:, 2] = maxv                       # saturated
    c[::2, 3] = maxv                     # alternating 0 / max
    c[:, 3][1::2] = 0
    c[:, 4] = 0
    c[S // 2, 4] = 200                   # one spike
    c[:, 5] = rng.integers(0, maxv + 1, size=S)  # incompressible, wide literals
    if P > 6:
        c[:, 6] = rng.poisson(20.0, size=S)      # high mean: escapes in the paired models
    if P > 7:
        c[:, 7] = rng.integers(250, 260, size=S).clip(0, maxv)  # around the u16 escape threshold
    return c


@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("det", [(17, 17), (19, 19)])
def test_roundtrip_adversarial(dtype, layout, det):
    rng = np.random.default_rng(5)
    sr, sc = (2, 512) if layout == 1 else (3, 301)  # byte-rANS: partial final block, odd length
    S, P = sr * sc, det[0] * det[1]
    c = adversarial(S, P, dtype, rng)
    blob = oracle.encode(c, sr, sc, det[0], det[1], layout=layout)
    assert np.array_equal(oracle.decode(blob), c)


def stream_modes(blob):
    """Mode of every stream of every block, read from the offsets and headers."""
    h = oracle.header(blob)
    P = h["det_rows"] * h["det_cols"]
    G = (P + 31) // 32
    modes = []
    for b in range(h["n_blocks"]):
        base, = struct.unpack_from("<Q", blob, h["dir_off"] + 16 * b)
        row = []
        for p in range(P):
            g, i = divmod(p, 32)
            gb, = struct.unpack_from("<I", blob, h["gbase_off"] + 4 * (b * G + g))
            rel, = struct.unpack_from("<H", blob, h["rel_off"] + 2 * ((b * G + g) * 32 + i))
            hdr, = struct.unpack_from("<H", blob, h["payload_off"] + base + gb + rel)
            row.append(hdr)
        modes.append(row)
    return np.array(modes)


def test_mode_choice_paired():
    # brute-force sizes decide the mode (FORMAT 3.4)
    S, P = 512, 8
    c = np.zeros((S, P), dtype=np.uint16)
    c[:, 1] = 9
    c[100, 2] = 3                       # one nonzero: sparse (8 bytes) beats any code section
    c[:, 3] = np.arange(S) % 2 + 1      # dense small values: paired
    c[:, 4] = (np.arange(S) * 7919) % 65536  # incompressible: raw
    blob = oracle.encode(c, 1, 512, 1, 8, layout=1)
    m = stream_modes(blob)[0] & 7
    assert m[0] == 0 and m[1] == 1 and m[2] == 2 and m[3] == 3 and m[4] == 4
    assert np.array_equal(oracle.decode(blob), c)


def test_mode_choice_rans():
    S, P = 512, 4
    c = np.zeros((S, P), dtype=np.uint8)
    c[:, 0] = 5                                   # constant
    c[:, 1] = np.random.default_rng(1).poisson(0.2, S)  # skewed: rANS
    c[:, 2] = np.arange(S) % 256                   # uniform bytes: raw (8 bits/value)
    blob = oracle.encode(c, 1, 512, 1, 4)
    m = stream_modes(blob)[0]
    assert m.tolist()[:3] == [0, 1, 2]


def test_malformed_streams_are_rejected():
    w = synth.WORKLOADS["tiny_u8"]
    c = synth.counts(w)
    blob = bytearray(oracle.encode(c, 16, 16, 64, 64))
    h = oracle.header(bytes(blob))
    # reserved header bit on the first stream
    bad = bytearray(blob)
    bad[h["payload_off"] + 1] |= 0x01
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(bytes(bad))
    assert e.value.code == oracle.ERR_MALFORMED
    # shortened extent: move the start of stream 1 one word earlier
    bad = bytearray(blob)
    rel1 = struct.unpack_from("<H", bad, h["rel_off"] + 2)[0]
    struct.pack_into("<H", bad, h["rel_off"] + 2, rel1 - 2)
    with pytest.raises(oracle.OracleError):
        oracle.decode(bytes(bad))
    # another ABI tag is refused
    bad = bytearray(blob)
    bad[8:24] = b"qsc-byte-rans-v9"
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(bytes(bad))
    assert e.value.code == oracle.ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# product pins
# ---------------------------------------------------------------------------

def test_masked_sum_matches_brute_force():
    w = synth.WORKLOADS["tiny_u8"]
    c = synth.counts(w)
    for name, m in synth.query_masks(w).items():
        assert np.array_equal(oracle.masked_sum(c, m), oracle.brute_masked_sum(c, m)), name
    valid = (np.arange(w.P) % 7 != 0).astype(np.uint8)
    m = synth.query_masks(w)["adf"]
    assert np.array_equal(oracle.masked_sum(c, m, valid), oracle.brute_masked_sum(c, m, valid))


def test_block_stride_definition():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 9, size=(3000, 6)).astype(np.uint8)
    m = np.ones(6, dtype=np.uint8)
    full = oracle.masked_sum(c, m)
    s4 = oracle.masked_sum(c, m, stride=4)
    blk = np.arange(3000) // 512
    assert np.array_equal(s4[blk % 4 == 0], full[blk % 4 == 0])
    assert (s4[blk % 4 != 0] == 0).all()
    assert np.array_equal(oracle.masked_sum(c, m, stride=1), c.sum(axis=1, dtype=np.uint64))


def test_uint64_closed_form():
    # a saturated uint16 frame: 257*257*65535 = 4,328,521,215 > 2^32; 256*256*65535 fits in uint32
    assert oracle.sum_bits(256 * 256, 2) == 32
    assert oracle.sum_bits(257 * 257, 2) == 64
    assert oracle.sum_bits(192 * 192, 2) == 32
    c = np.full((1, 257 * 257), 65535, dtype=np.uint16)
    s = oracle.masked_sum(c, np.ones(257 * 257, dtype=np.uint8))
    assert int(s[0]) == 4328521215


def test_dense_df_invariants():
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(2, 256)
    c = synth.counts(w)
    valid = synth.valid_pixels(w)
    bf = synth.query_masks(w)["bf"]
    df = synth.query_masks(w)["df"]
    total = oracle.masked_sum(c, np.ones(w.P, dtype=np.uint8), valid)
    assert np.array_equal(oracle.dense_df(c, df, valid) + oracle.masked_sum(c, bf, valid), total)
    assert np.array_equal(oracle.dense_df(c, df, valid), oracle.masked_sum(c, df, valid))
    # sentinels (65535 everywhere) are excluded by the validity mask
    assert total.max() < 65535 * 10


def test_com_closed_forms():
    R, C = 192, 192
    # one nonzero pixel at (r, c) -> exactly (r, c)
    x = np.zeros((3, R * C), dtype=np.uint16)
    x[0, 37 * C + 121] = 5
    x[1, 0] = 1
    row, col, m0 = oracle.com(x, R, C)
    assert (row[0], col[0]) == (37.0, 121.0)
    assert (row[1], col[1]) == (0.0, 0.0)
    assert (row[2], col[2], m0[2]) == (0.0, 0.0, 0)  # empty frame -> 0
    # a uniform frame -> the detector centre (95.5, 95.5)
    u = np.ones((1, R * C), dtype=np.uint8)
    row, col, _ = oracle.com(u, R, C)
    assert (row[0], col[0]) == (95.5, 95.5)
    # a disk symmetric about (96, 96) -> (96, 96)
    d = synth.disk_mask(R, C, 96, 96, 30).reshape(1, -1).astype(np.uint8)
    row, col, _ = oracle.com(d, R, C)
    assert (row[0], col[0]) == (96.0, 96.0)
    # masked CoM: mask the disk's right half away -> column shifts left, row stays
    half = synth.disk_mask(R, C, 96, 96, 30).copy()
    half[(np.arange(R * C) % C) > 96] = 0
    row, col, _ = oracle.com(d, R, C, mask=half)
    assert row[0] == 96.0 and col[0] < 96.0


def test_com_matches_brute_force():
    w = synth.WORKLOADS["tiny_u8"]
    c = synth.counts(w)
    bf = synth.query_masks(w)["bf"]
    for m in (None, bf):
        r1, c1, m1 = oracle.com(c, 64, 64, mask=m)
        r2, c2, m2 = oracle.brute_com(c, 64, 64, mask=m)
        assert np.array_equal(r1, r2) and np.array_equal(c1, c2) and np.array_equal(m1, m2)


def test_region_definition():
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(4, 16)
    c = synth.counts(w)
    valid = synth.valid_pixels(w)
    out = oracle.region(c, 16, 1, 3, 5, 9, valid)
    assert out.shape == (8, w.P)
    assert np.array_equal(out[0], np.where(valid == 1, c[1 * 16 + 5], 0))
    assert np.array_equal(out[7], np.where(valid == 1, c[2 * 16 + 8], 0))


# ---------------------------------------------------------------------------
# scaled uint16 pins
# ---------------------------------------------------------------------------

def test_scaled_ties_to_even_match_numpy_rint():
    # lo = 0 and hi = 65535/4 give scale = 0.25 exactly; x = (m + 1/2) * 0.25 is an exact tie
    x = np.array([0.0, 65535 * 0.25, 0.125, 0.375, 0.625, 0.875, 1000.125, 1000.375], dtype=np.float32)
    sc, off, codes = oracle.calibrate(x)
    assert sc == 0.25 and off == 0.0
    want = np.rint((x.astype(np.float64) - 0.0) / 0.25).astype(np.uint16)
    assert np.array_equal(codes, want)
    assert codes[2:6].tolist() == [0, 2, 2, 4]


def test_scaled_constant_negative_wide():
    sc, off, codes = oracle.calibrate(np.full(10, -3.5, dtype=np.float32))
    assert (sc, off) == (1.0, -3.5) and (codes == 0).all()
    x = np.array([-2.0, -1.0, 0.5, 1e-3, 1e6], dtype=np.float32)
    sc, off, codes = oracle.calibrate(x)
    assert off == -2.0 and sc == (1e6 + 2.0) / 65535
    assert codes[0] == 0 and codes[-1] == 65535
    want = np.clip(np.rint((x.astype(np.float64) + 2.0) / sc), 0, 65535).astype(np.uint16)
    assert np.array_equal(codes, want)
    with pytest.raises(oracle.OracleError):
        oracle.calibrate(np.array([1.0, np.nan], dtype=np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.calibrate(np.array([1.0, np.inf], dtype=np.float32))


def test_reconstruction_matches_numpy_float64():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 65536, size=10000).astype(np.uint16)
    for sc, off in [(0.731 / 3, -0.25), (1e-7, 12345.678), (3.3, -1e5)]:
        want = (codes.astype(np.float64) * sc + off).astype(np.float32)
        assert np.array_equal(oracle.reconstruct(codes, sc, off), want)


def test_scaled_roundtrip_and_error_bound():
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(4, 200)  # 800 scans: one full and one partial region
    x = synth.scaled(w)
    blob = oracle.encode(x, 4, 200, w.det_rows, w.det_cols, scaled=True)
    codes = oracle.decode(blob)
    cal = oracle.calibration(blob)
    assert cal.shape == (2, 2)
    for b in range(2):
        sl = slice(512 * b, min(800, 512 * (b + 1)))
        sc, off, want_codes = oracle.calibrate(x[sl])
        assert (sc, off) == tuple(cal[b])
        assert np.array_equal(codes[sl].ravel(), want_codes)
        rec = oracle.reconstruct(codes[sl], sc, off).reshape(x[sl].shape)
        # storage error of nearest rounding: at most half a step (plus float32 output rounding)
        err = np.abs(rec.astype(np.float64) - x[sl].astype(np.float64))
        assert err.max() <= 0.5 * sc + 1e-6 * np.abs(x[sl]).max()


def test_workload_masks_match_the_pages():
    # ~2827 BF radius-30 (pi*30^2) is 2821 pixels with an integer centre; full BF ~8809 is r = 53
    assert synth.disk_mask(192, 192, 96, 96, 30).sum() == 2821
    assert synth.disk_mask(192, 192, 96, 96, 53).sum() == 8809
    assert synth.disk_mask(64, 64, 32, 32, 8).sum() == 197
    assert synth.annulus_mask(64, 64, 32, 32, 14, 30).sum() == 2212
    assert synth.annulus_mask(192, 192, 96, 96, 60, 90).sum() == 14168
    assert len(synth.sweep_masks(synth.WORKLOADS["scan512_u8_lowdose"])) == 64


# ---------------------------------------------------------------------------
# sum / mean diffraction pattern (the dual of a virtual image)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [np.uint8, np.uint16])
def test_sum_dp_matches_numpy_brute_force(dtype):
    rng = np.random.default_rng(61)
    S, P = 1100, 37  # two full blocks and a partial one
    c = rng.poisson(3.0, size=(S, P)).astype(dtype)
    c[5] = np.iinfo(dtype).max
    valid = np.ones(P, np.uint8)
    valid[[0, 11]] = 0
    for scan_mask in (None, (rng.random(S) < 0.3).astype(np.uint8)):
        for stride in (1, 2):
            for v in (None, valid):
                got = oracle.sum_dp(c, scan_mask, v, stride)
                want = oracle.brute_sum_dp(c, scan_mask, v, stride)
                assert np.array_equal(got[0], want[0])
                assert np.array_equal(got[1], want[1])


def test_sum_dp_closed_forms():
    S, P = 1024, 9
    c = np.full((S, P), 3, np.uint16)
    s, m = oracle.sum_dp(c)
    assert np.all(s == 3 * S) and np.all(m == 3.0)
    # one bright frame among zeros: the mean is its value over the scan count
    z = np.zeros((S, P), np.uint16)
    z[700] = 65535
    s, m = oracle.sum_dp(z)
    assert np.all(s == 65535) and np.all(m == np.float32(65535 / 1024))
    # stride 2 visits block 0 only: the bright frame (block 1) drops out
    s, m = oracle.sum_dp(z, stride=2)
    assert not s.any() and not m.any()
    # an empty scan selection gives zeros
    s, m = oracle.sum_dp(z, scan_mask=np.zeros(S, np.uint8))
    assert not s.any() and not m.any()


def test_sum_dp_scaled_mean_is_the_mean_of_the_intensities():
    rng = np.random.default_rng(62)
    S, P = 1200, 24
    # integer-valued intensities holding 0 and 65535 in every region: the
    # calibration is exactly scale 1, offset 0, so the mean must be the plain mean
    x = rng.integers(0, 65536, size=(S, P)).astype(np.float32)
    x[0::512, 0] = 0.0
    x[1::512, 0] = 65535.0
    blob = oracle.encode(x, 1, S, 4, 6, scaled=True)
    codes, cal = oracle.decode(blob), oracle.calibration(blob)
    assert np.all(cal[:, 0] == 1.0) and np.all(cal[:, 1] == 0.0)
    sel = (rng.random(S) < 0.5).astype(np.uint8)
    _, mean = oracle.sum_dp(codes, sel, calib=cal)
    assert np.array_equal(mean, x[sel != 0].astype(np.float64).mean(axis=0).astype(np.float32))
    # general data: within half a code step of the mean of the raw intensities
    y = synth.scaled(synth.WORKLOADS["scan256_u16_sentinel"].with_scans(5, 240))[:, :200]
    blob = oracle.encode(y, 5, 240, 10, 20, scaled=True)
    codes, cal = oracle.decode(blob), oracle.calibration(blob)
    _, mean = oracle.sum_dp(codes, calib=cal)
    want = y.astype(np.float64).mean(axis=0)
    assert np.abs(mean - want).max() <= 0.5 * cal[:, 0].max() + 1e-6 * np.abs(want).max()


# ---------------------------------------------------------------------------
# frames of whole blocks (the reconstruction feed)
# ---------------------------------------------------------------------------

def test_frames_amplitude_is_the_correctly_rounded_square_root():
    c = np.arange(65536, dtype=np.uint16)[None, :]
    amp = oracle.frames(c, 0, 1, kind="amplitude")[0]
    # float32 sqrt equals the float64 sqrt rounded once to float32 (no double-rounding case
    # exists for square roots at these widths) and is exact on perfect squares
    assert np.array_equal(amp, np.sqrt(c[0].astype(np.float64)).astype(np.float32))
    k = np.arange(256)
    assert np.array_equal(amp[k * k], k.astype(np.float32))


def test_frames_are_the_decoded_scans():
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(5, 240)  # 1200 scans: blocks of 512, 512, 176
    c = synth.counts(w)
    valid = synth.valid_pixels(w)
    blob = oracle.encode(c, 5, 240, w.det_rows, w.det_cols)
    dec = oracle.decode(blob)
    f = oracle.frames(dec, 1, 2, valid)
    assert f.shape == (1200 - 512, w.P)
    want = c[512:].copy()
    want[:, valid == 0] = 0
    assert np.array_equal(f, want)


# ---------------------------------------------------------------------------
# polar interaction index
# ---------------------------------------------------------------------------

def test_polar_order_puts_centred_disks_first():
    order = oracle.polar_order(192, 192, 96, 96)
    assert np.array_equal(np.sort(order), np.arange(192 * 192))
    pos = np.empty_like(order)
    pos[order] = np.arange(order.size)
    for r in (0, 1, 8, 30, 53, 90):
        disk = np.nonzero(synth.disk_mask(192, 192, 96, 96, r))[0]
        assert pos[disk].max() == disk.size - 1  # a centred disk is exactly a prefix of the order
    # within one distance the angle increases
    kr, kc = np.divmod(order, 192)
    d2 = (kr - 96) ** 2 + (kc - 96) ** 2
    ang = np.arctan2(kr - 96, kc - 96)
    same = d2[1:] == d2[:-1]
    assert np.all(ang[1:][same] > ang[:-1][same])


def test_index_decomposition_partitions_the_mask_and_sums_exactly():
    rng = np.random.default_rng(71)
    det = 40
    P = det * det
    S = 1100
    c = rng.poisson(2.0, size=(S, P)).astype(np.uint16)
    c[:, 7] = 65535
    valid = np.ones(P, np.uint8)
    valid[[3, 400, 1000]] = 0
    order = oracle.polar_order(det, det, 20, 20)
    leaves, roots = oracle.index_fields(c, order, valid)
    assert leaves.shape == (S, 25) and roots.shape == (S, 2)
    assert np.array_equal(roots.sum(axis=1), leaves.sum(axis=1))
    assert np.array_equal(leaves.sum(axis=1), oracle.masked_sum(c, np.ones(P, np.uint8), valid))
    masks = {
        "full": np.ones(P, np.uint8),
        "empty": np.zeros(P, np.uint8),
        "disk": synth.disk_mask(det, det, 20, 20, 12),
        "shifted": synth.disk_mask(det, det, 23, 18, 12),
        "annulus": synth.annulus_mask(det, det, 20, 20, 6, 15),
        "random": (rng.random(P) < 0.5).astype(np.uint8),
    }
    for name, m in masks.items():
        r, l, residual = oracle.decompose(m, order, valid)
        # fields and residual partition mask & valid
        cover = np.zeros(P, int)
        for j in r:
            cover[order[1024 * j: 1024 * (j + 1)]] += 1
        for i in l:
            cover[order[64 * i: 64 * (i + 1)]] += 1
        cover += residual
        sel = (m != 0) & (valid != 0)
        assert np.array_equal(cover[valid != 0], sel[valid != 0].astype(int)), name
        for stride in (1, 2):
            assert np.array_equal(oracle.indexed_masked_sum(c, m, order, valid, stride),
                                  oracle.masked_sum(c, m, valid, stride)), (name, stride)
    r, l, residual = oracle.decompose(masks["full"], order, valid)
    assert r == [0, 1] and not l and not residual.any()
    r, l, residual = oracle.decompose(masks["disk"], order, valid)
    assert not r and len(l) >= 1 and residual.sum() < 64  # a centred disk: leaves plus one partial leaf
