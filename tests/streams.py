"""Stream-level editing of containers for tests (FORMAT 1.2-1.3).

split() cuts a container into its header-and-table prefix and the byte string
of every (block, pixel) stream; pack() lays streams out again, recomputing the
block directory, group bases, relative offsets and sizes. Editing one stream
and packing therefore gives a container that is structurally valid (it passes
the host's checks) but holds exactly the stream contents the test chose.
Test helpers only: nothing here decodes or encodes values.
"""
import struct

import numpy as np

import oracle


def split(blob):
    """(header dict, streams[b][p] as bytes) of a container without calibration."""
    blob = bytes(blob)
    h = oracle.header(blob)
    assert h["calib_off"] == 0
    P = h["det_rows"] * h["det_cols"]
    G = (P + 31) // 32
    gbase = np.frombuffer(blob, "<u4", h["n_blocks"] * G, h["gbase_off"])
    rel = np.frombuffer(blob, "<u2", h["n_blocks"] * G * 32, h["rel_off"])
    streams = []
    for b in range(h["n_blocks"]):
        base, _, nbytes = struct.unpack_from("<QII", blob, h["dir_off"] + 16 * b)
        starts = [int(gbase[b * G + p // 32]) + int(rel[(b * G + p // 32) * 32 + p % 32]) for p in range(P)]
        ends = starts[1:] + [nbytes]
        off = h["payload_off"] + base
        streams.append([blob[off + s: off + e] for s, e in zip(starts, ends)])
    return h, streams


def pack(blob, streams):
    """The container with its payload replaced by streams[b][p] (same header and tables)."""
    blob = bytes(blob)
    h = oracle.header(blob)
    P = h["det_rows"] * h["det_cols"]
    G = (P + 31) // 32
    out = bytearray(blob[:h["payload_off"]])
    payload = bytearray()
    for b, row in enumerate(streams):
        base = len(payload)
        block = bytearray()
        for g in range(G):
            gb = len(block)
            struct.pack_into("<I", out, h["gbase_off"] + 4 * (b * G + g), gb)
            for i in range(32):
                p = 32 * g + i
                rel = len(block) - gb
                assert rel <= 0xFFFF
                struct.pack_into("<H", out, h["rel_off"] + 2 * ((b * G + g) * 32 + i), rel)
                if p < P:
                    assert len(row[p]) % 2 == 0
                    block += row[p]
        payload += block
        n_scans = struct.unpack_from("<I", blob, h["dir_off"] + 16 * b + 8)[0]
        struct.pack_into("<QII", out, h["dir_off"] + 16 * b, base, n_scans, len(block))
    out += payload
    struct.pack_into("<Q", out, 120, len(payload))
    struct.pack_into("<Q", out, 136, len(out))
    return bytes(out)


def modes(streams):
    """Mode (header bits 0-2) of every stream: (n_blocks, P) array."""
    return np.array([[struct.unpack_from("<H", s)[0] & 7 for s in row] for row in streams])


def rans_literal_offsets(stream, freq, n):
    """Byte offsets, inside a byte-rANS uint16 RANS stream, of its escape literals.

    Follows the decoder's reading order (FORMAT 2.3): per value the state
    update, a renormalisation word when the state drops below 2^16, then the
    literal of an escape symbol. Used only to find a word to corrupt."""
    f = np.asarray(freq, dtype=np.int64)
    c = np.concatenate([[0], np.cumsum(f)[:-1]])
    sym = np.repeat(np.arange(256), f)
    w = lambda o: struct.unpack_from("<H", stream, o)[0]
    x = w(2) | (w(4) << 16)
    pos, lits = 6, []
    for _ in range(n):
        t = x & 4095
        s = int(sym[t])
        x = int(f[s]) * (x >> 12) + t - int(c[s])
        if x < 65536:
            x = (x << 16) | w(pos)
            pos += 2
        if s == 255:
            lits.append(pos)
            pos += 2
    return lits
