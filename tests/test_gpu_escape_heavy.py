"""Escape-heavy uint16 byte-rANS residents against the oracle.

When most blocks of a uint16 byte-rANS resident give the escape symbol (255)
at least a quarter of the 4096 table slots, sums and moments take the staged
decode: each stream is read in 32-byte chunks into a ring in LDS on a
four-step cadence, and every step takes its renormalisation word and literal
from the ring. The container here has that shape (scaled Poisson counts around
250 outside the bright disk and 360 inside), plus RAW streams (uniform 16-bit
values), constant streams, sentinel pixels excluded by the valid mask, two
complete blocks with split points and a ragged final block. Sums (several
strides, planned and latency-bound selections, the delta form), CoM (whole
detector, masks, a mask inside one detector row) and the no-allocation CoM
must equal the oracle exactly; malformed escape-heavy streams must fail the
query with the pixel named (the paired-resident page, "Contract").
"""
import struct

import numpy as np
import pytest

import oracle
import streams
import synth

pytestmark = pytest.mark.gpu

ESCAPE_HEAVY = 1024  # escape-symbol slots (of 4096) from which a block counts as escape-heavy


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


_CASE = {}


def escape_case():
    """(workload, counts, valid, container): 64 x 64 detector, 1400 scans (blocks of 512, 512, 376)."""
    if "c" not in _CASE:
        w = synth.Workload("escape_heavy", 14, 100, 64, 64, 2, 60.0, 42.0, 32, 32, 12, 1, 1, 2101, 0)
        rng = np.random.default_rng(2101)
        counts = synth.counts(w)
        valid = synth.valid_pixels(w)
        # a high dose: six times the generator's counts plus 0-5, so values
        # around 250 outside the disk and 360 inside (sentinels stay 65535)
        counts = np.where(counts == 65535, counts, counts * 6 + rng.integers(0, 6, counts.shape)).astype(np.uint16)
        ok = np.nonzero(valid)[0]
        raw_px = rng.choice(ok, 24, replace=False)
        counts[:, raw_px] = rng.integers(0, 65536, size=(w.S, raw_px.size), dtype=np.uint16)
        const_px = [int(p) for p in ok[[5, 900, 2000]] if p not in raw_px]
        counts[:, const_px] = 777
        low_px = [int(p) for p in ok[100:140] if p not in raw_px and p not in const_px]
        counts[:, low_px] = rng.poisson(3.0, size=(w.S, len(low_px)))  # plain streams in escape-heavy blocks
        blob = oracle.encode(counts, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols)
        _CASE["c"] = (w, counts, valid, blob)
    return _CASE["c"]


def block_freqs(blob):
    h = oracle.header(blob)
    return [np.frombuffer(blob, "<u2", 256, h["table_off"] + 512 * b) for b in range(h["n_blocks"])]


def masks(w):
    P = w.P
    m = {"full": np.ones(P, np.uint8),
         "disk": synth.disk_mask(w.det_rows, w.det_cols, 32, 32, 12),
         "annulus": synth.annulus_mask(w.det_rows, w.det_cols, 32, 32, 14, 28)}
    small = np.zeros(P, np.uint8)
    small[32 * 64 + 20: 32 * 64 + 40] = 1  # 20 pixels: a latency-bound query, stream halves side by side
    m["small"] = small
    row = np.zeros(P, np.uint8)
    row[40 * 64 + 3: 40 * 64 + 61] = 1  # inside one detector row
    m["row"] = row
    m["random"] = (np.random.default_rng(7).random(P) < 0.3).astype(np.uint8)
    return m


def test_container_is_escape_heavy():
    w, counts, valid, blob = escape_case()
    f = block_freqs(blob)
    assert sum(int(x[255]) >= ESCAPE_HEAVY for x in f) * 2 >= len(f)
    _, st = streams.split(blob)
    md = streams.modes(st)
    for b in range(len(st)):
        for mode in (0, 1, 2):  # CONST, RANS and RAW streams in every block
            assert (md[b] == mode).any(), (b, mode)


def check_com(res, counts, w, mask, valid, noalloc=False):
    row, col = (res.com_noalloc if noalloc else res.com)(mask)
    orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, mask=mask, valid=valid)
    assert np.array_equal(row.cpu().numpy(), orow) and np.array_equal(col.cpu().numpy(), ocol)


def test_escape_heavy_sums_and_moments():
    w, counts, valid, blob = escape_case()
    with q().Resident(blob, valid=valid) as res:
        for name, m in masks(w).items():
            for k in (1, 2, 3):
                got = u(res.masked_sum(m, block_stride=k))
                assert np.array_equal(got, oracle.masked_sum(counts, m, valid, stride=k)), (name, k)
            check_com(res, counts, w, m, valid)
        check_com(res, counts, w, None, valid)
        check_com(res, counts, w, None, valid, noalloc=True)
        check_com(res, counts, w, masks(w)["disk"], valid, noalloc=True)
        # the delta form: the disk moved by one pixel, from the previous sums
        disk = masks(w)["disk"]
        moved = np.roll(disk.reshape(64, 64), 1, axis=1).reshape(-1)
        prev = res.masked_sum(disk)
        got = u(res.masked_sum_delta(disk, prev, moved))
        assert np.array_equal(got, oracle.masked_sum(counts, moved, valid))
        res.finish()


def test_escape_heavy_queued_queries_agree():
    """Queries queued back to back (wait=0) on one resident give the waited results."""
    import torch
    w, counts, valid, blob = escape_case()
    ms = masks(w)
    with q().Resident(blob, valid=valid) as res:
        outs = [res.masked_sum(ms[n], wait=False) for n in ("full", "small", "row", "disk")]
        rc = res.com(ms["annulus"], wait=False)
        res.finish()
        torch.cuda.synchronize()
        for n, o in zip(("full", "small", "row", "disk"), outs):
            assert np.array_equal(u(o), oracle.masked_sum(counts, ms[n], valid)), n
        orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, mask=ms["annulus"], valid=valid)
        assert np.array_equal(rc[0].cpu().numpy(), orow) and np.array_equal(rc[1].cpu().numpy(), ocol)


def expect_malformed(blob, b, p):
    with pytest.raises(oracle.OracleError) as e:
        oracle.decode(blob)
    assert e.value.code == oracle.ERR_MALFORMED and f"block {b} pixel {p}" in str(e.value)


def literal_stream(blob, st, b):
    """(pixel, literal offsets) of a RANS stream of block b that holds at least 40 escape literals."""
    freq = block_freqs(blob)[b]
    md = streams.modes(st)
    for p in np.nonzero(md[b] == 1)[0][::7]:
        lits = streams.rans_literal_offsets(st[b][p], freq, 512 if b < 2 else 376)
        if len(lits) >= 40:
            return int(p), lits
    raise AssertionError("no escape-heavy stream")


CORRUPTIONS = {
    "literal below 255 (first)": lambda s, lits: s[:lits[0]] + struct.pack("<H", 200) + s[lits[0] + 2:],
    "literal below 255 (last)": lambda s, lits: s[:lits[-1]] + struct.pack("<H", 7) + s[lits[-1] + 2:],
    "state bit": lambda s, lits: s[:3] + bytes([s[3] ^ 0x04]) + s[4:],
    "extra word": lambda s, lits: s + b"\x34\x12",
    "shortened extent": lambda s, lits: s[:-2],
}


@pytest.mark.parametrize("what", sorted(CORRUPTIONS))
@pytest.mark.parametrize("b", [1, 2])  # a complete block (split points) and the ragged final block
def test_escape_heavy_malformed_stream_fails(what, b):
    w, counts, valid, blob = escape_case()
    _, st = streams.split(blob)
    p, lits = literal_stream(blob, st, b)
    st[b][p] = CORRUPTIONS[what](st[b][p], lits)
    bad = streams.pack(blob, st)
    expect_malformed(bad, b, p)
    qq = q()
    named = f"block {b}, pixel {p}"
    near = np.zeros(w.P, np.uint8)
    near[max(0, p - 30): p + 30] = 1
    one = np.zeros(w.P, np.uint8)
    one[p] = 1
    with qq.Resident(bad) as res:
        for m in (one, near, np.ones(w.P, np.uint8)):
            with pytest.raises(qq.QscValueError) as e:
                res.masked_sum(m)
            assert e.value.code == qq.ERR_MALFORMED and named in str(e.value), (what, str(e.value))
        with pytest.raises(qq.QscValueError) as e:
            res.com()
        assert named in str(e.value)
        with pytest.raises(qq.QscValueError):
            res.com(near)
        res.masked_sum(near, wait=False)
        with pytest.raises(qq.QscValueError) as e:
            res.finish()
        assert named in str(e.value)
        # selections without the bad stream still decode exactly on the same resident
        other = near.copy()
        other[p] = 0
        assert np.array_equal(u(res.masked_sum(other)), oracle.masked_sum(counts, other))
        row, col = res.com(other)
        orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, mask=other)
        assert np.array_equal(row.cpu().numpy(), orow) and np.array_equal(col.cpu().numpy(), ocol)
        res.finish()
