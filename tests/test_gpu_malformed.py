"""GPU rejection of malformed streams that pass the host's structural checks.

The paired-resident page ("Contract", "Verification") makes a malformed stream
fail the query with no result, and names a reserved header bit and a shortened
stream extent among the cases. The host validates structure and headers at
resident creation; these corruptions change only stream contents, so the
kernels' end checks must find them:
- paired layout: a hand-worked model-0 stream (tests/golden) spliced into a
  real container, then its zero pad set, 16 spare bits appended, its extent
  shortened, a literal moved inside the window, its final state changed; a
  SPARSE stream with two positions out of order;
- byte-rANS uint16 with complete blocks (so latency-bound queries decode each
  stream as two halves from stored split points): a flipped state bit, an
  escape literal below 255, an extra word, a shortened extent.
Every case is first confirmed malformed by the oracle at the same (block,
pixel). On the GPU each must fail with the pixel named, under wait=1 and
under wait=0 followed by finish(), for small (split) and full-detector
selections, CoM, region reads and frames; afterwards a query that avoids the
bad stream on the same resident must still equal the oracle.
"""
import os
import struct

import numpy as np
import pytest

import oracle
import streams
import synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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


def golden_paired():
    vals, stream = [], bytearray()
    for line in open(os.path.join(GOLDEN, "paired_u16_model0.txt")):
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
    return np.array(vals, np.uint16), bytes(stream)


def flip_bits(s, *bits):
    """Flip bits of a stream, numbered from the first code bit after the 2-byte header."""
    b = bytearray(s)
    for bit in bits:
        bit += 16
        b[bit // 8] ^= 1 << (bit % 8)
    return bytes(b)


def expect_malformed(blob, b, p):
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(blob)
    assert e.value.code == oracle.ERR_MALFORMED and f"block {b} pixel {p}" in str(e.value)


def check_rejected(blob, counts, w, b, p, what):
    """The GPU path refuses every query that decodes stream (b, p) and still answers the others."""
    qq = q()
    P = w.det_rows * w.det_cols
    named = f"block {b}, pixel {p}"
    one = np.zeros(P, np.uint8)
    one[p] = 1
    near = np.zeros(P, np.uint8)
    near[max(0, p - 40): p + 40] = 1  # a small selection around it
    full = np.ones(P, np.uint8)
    with qq.Resident(blob) as res:
        for m in (one, near, full):
            with pytest.raises(qq.QscValueError) as e:
                res.masked_sum(m)
            assert e.value.code == qq.ERR_MALFORMED and named in str(e.value), (what, str(e.value))
        for k in (1, 2):
            if b % k == 0:
                with pytest.raises(qq.QscValueError):
                    res.masked_sum(near, block_stride=k)
        # queued: the error surfaces at finish(), with the pixel named
        res.masked_sum(near, wait=False)
        with pytest.raises(qq.QscValueError) as e:
            res.finish()
        assert named in str(e.value), what
        with pytest.raises(qq.QscValueError):
            res.com()
        with pytest.raises(qq.QscValueError):
            res.com(near)
        r, c = divmod(b * 512, w.scan_cols)  # the block's first scan
        with pytest.raises(qq.QscValueError):
            res.decode_region(r, r + 1, c, min(c + 8, w.scan_cols))
        with pytest.raises(qq.QscValueError):
            res.decode_blocks(b, 1)
        with pytest.raises(qq.QscValueError):
            res.sum_dp()
        # a selection without the bad pixel decodes normally on the same resident
        other = near.copy()
        other[p] = 0
        assert np.array_equal(u(res.masked_sum(other)), oracle.masked_sum(counts, other)), what
        row, col = res.com(other)
        orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, mask=other)
        assert np.array_equal(row.cpu().numpy(), orow) and np.array_equal(col.cpu().numpy(), ocol), what
        res.finish()


def paired_case():
    """A 4-block paired container on a 64 x 64 detector with the hand-worked
    stream at (block 1, pixel 1000) and a SPARSE stream at (block 2, pixel 77)."""
    w = synth.Workload("paired_malformed", 2, 1024, 64, 64, 2, 5.0, 0.1, 32, 32, 20, 2, 0, 91, 1)
    counts = synth.counts(w)
    counts[:, 77] = 0
    counts[1100, 77] = 2  # two lone counts of 2: SPARSE (PAIRED is no smaller)
    counts[1300, 77] = 2
    blob = oracle.encode(counts, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=1)
    gvals, gstream = golden_paired()
    _, st = streams.split(blob)
    st[1][1000] = gstream
    counts[512:1024, 1000] = gvals
    blob = streams.pack(blob, st)
    assert np.array_equal(oracle.decode(blob), counts)
    assert streams.modes(st)[2][77] == 2
    return w, counts, blob, st


def test_paired_clean_splice_matches_the_oracle():
    w, counts, blob, _ = paired_case()
    with q().Resident(blob) as res:
        full = np.ones(w.P, np.uint8)
        assert np.array_equal(u(res.masked_sum(full)), oracle.masked_sum(counts, full))
        row, col = res.com()
        orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols)
        assert np.array_equal(row.cpu().numpy(), orow) and np.array_equal(col.cpu().numpy(), ocol)
        got = q().as_unsigned(res.decode_blocks(1, 1))
        assert np.array_equal(got, counts[512:1024])


PAIRED_CORRUPTIONS = {
    # code section of the hand-worked stream: 2599 bits, then 9 zero pad bits
    "pad bit set": lambda s: flip_bits(s, 2607),
    "16 spare bits": lambda s: s + b"\0\0",
    "shortened extent": lambda s: s[:-2],
    "literal inside the window": lambda s: flip_bits(s, 2583, 2584),  # last literal 2 -> 1
    "final state not 0": lambda s: flip_bits(s, 2573),  # the 10 bits read at the last pair
    "initial state": lambda s: flip_bits(s, 0),
}


@pytest.mark.parametrize("what", sorted(PAIRED_CORRUPTIONS))
def test_paired_malformed_stream_fails_the_query(what):
    w, counts, blob, st = paired_case()
    st[1][1000] = PAIRED_CORRUPTIONS[what](st[1][1000])
    bad = streams.pack(blob, st)
    expect_malformed(bad, 1, 1000)
    check_rejected(bad, counts, w, 1, 1000, what)


def test_paired_sparse_positions_out_of_order():
    w, counts, blob, st = paired_case()
    s = bytearray(st[2][77])
    nnz = struct.unpack_from("<H", s, 2)[0]
    assert nnz == 2
    a, b = struct.unpack_from("<2H", s, 4)
    struct.pack_into("<2H", s, 4, b, a)
    st[2][77] = bytes(s)
    bad = streams.pack(blob, st)
    expect_malformed(bad, 2, 77)
    check_rejected(bad, counts, w, 2, 77, "sparse order")


def test_paired_reserved_header_bit_is_refused_at_creation():
    w, counts, blob, st = paired_case()
    s = bytearray(st[1][1000])
    s[1] |= 0x01
    st[1][1000] = bytes(s)
    bad = streams.pack(blob, st)
    expect_malformed(bad, 1, 1000)
    with pytest.raises(q().QscValueError) as e:
        q().Resident(bad)
    assert e.value.code == q().ERR_MALFORMED


def rans_case():
    """Two complete blocks of the 192 x 192 uint16 generator (so the resident keeps
    split points), byte-rANS, with escapes planted in one bright pixel."""
    w = synth.WORKLOADS["scan256_u16_sentinel"].with_scans(4, 256)
    counts = synth.counts(w)
    p_esc = 96 * 192 + 96
    counts[512 + np.arange(5, 512, 37), p_esc] = 300 + np.arange(14)  # escapes in block 1
    blob = oracle.encode(counts, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols)
    _, st = streams.split(blob)
    m = streams.modes(st)
    assert m[1][p_esc] == 1
    return w, counts, blob, st, p_esc


def rans_freq(blob, b):
    h = oracle.header(blob)
    return np.frombuffer(blob, "<u2", 256, h["table_off"] + 512 * b)


def test_rans_u16_split_resident_clean_matches_the_oracle():
    w, counts, blob, _, p_esc = rans_case()
    with q().Resident(blob) as res:
        near = np.zeros(w.P, np.uint8)
        near[p_esc - 40: p_esc + 40] = 1
        for m in (near, np.ones(w.P, np.uint8)):
            assert np.array_equal(u(res.masked_sum(m)), oracle.masked_sum(counts, m))
        row, col = res.com(near)
        orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, mask=near)
        assert np.array_equal(row.cpu().numpy(), orow) and np.array_equal(col.cpu().numpy(), ocol)


def test_rans_u16_escape_literal_below_255():
    w, counts, blob, st, p_esc = rans_case()
    lits = streams.rans_literal_offsets(st[1][p_esc], rans_freq(blob, 1), 512)
    assert len(lits) >= 14
    for which in (lits[0], lits[-1]):  # a literal in the first half and one in the second
        s = bytearray(st[1][p_esc])
        struct.pack_into("<H", s, which, 200)
        st2 = [list(r) for r in st]
        st2[1][p_esc] = bytes(s)
        bad = streams.pack(blob, st2)
        expect_malformed(bad, 1, p_esc)
        check_rejected(bad, counts, w, 1, p_esc, f"literal at byte {which}")


RANS_CORRUPTIONS = {
    "state bit": lambda s: s[:3] + bytes([s[3] ^ 0x04]) + s[4:],
    "extra word": lambda s: s + b"\x34\x12",
    "shortened extent": lambda s: s[:-2],
}


@pytest.mark.parametrize("what", sorted(RANS_CORRUPTIONS))
@pytest.mark.parametrize("b", [0, 1])
def test_rans_u16_malformed_stream_fails_the_query(what, b):
    w, counts, blob, st, p_esc = rans_case()
    m = streams.modes(st)
    p = int(np.nonzero(m[b] == 1)[0][len(np.nonzero(m[b] == 1)[0]) // 2])  # a RANS stream mid-detector
    st[b][p] = RANS_CORRUPTIONS[what](st[b][p])
    bad = streams.pack(blob, st)
    expect_malformed(bad, b, p)
    check_rejected(bad, counts, w, b, p, what)
