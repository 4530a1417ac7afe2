"""qsc_com_noalloc against qsc_com, through the C ABI.

The no-allocation CoM keeps its moment partials in the library's static
device buffer. Two calls in a row, the second on a smaller resident (so the
buffer holds the first call's larger contents), must each equal qsc_com bit
for bit, with and without a mask, on both stream layouts; a resident above
the buffer's 1,048,576 scans is refused.
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


def noalloc(res, mask):
    """qsc_com_noalloc called through the C ABI with torch-owned buffers."""
    import torch
    qq = q()
    row = torch.full((res.S,), -1.0, dtype=torch.float32, device="cuda:0")
    col = torch.full((res.S,), -1.0, dtype=torch.float32, device="cuda:0")
    m = None if mask is None else torch.as_tensor(mask, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    rc = qq.lib.qsc_com_noalloc(res._h, None if m is None else ctypes.c_void_p(m.data_ptr()),
                                ctypes.c_void_p(row.data_ptr()), ctypes.c_void_p(col.data_ptr()),
                                ctypes.c_void_p(stream.cuda_stream), 1)
    assert rc == qq.OK, qq.lib.qsc_last_error(res._h)
    return row.cpu().numpy(), col.cpu().numpy()


def cases():
    big = synth.Workload("noalloc_paired", 4, 1024, 64, 64, 2, 5.0, 0.1, 32, 32, 20, 2, 0, 93, 1)  # 8 blocks
    small = synth.WORKLOADS["scan128_u16"].with_scans(16, 128)  # 2048 scans, byte-rANS, 192 x 192
    out = []
    for w in (big, small):
        counts = synth.counts(w)
        blob = q().encode(counts, w.scan_rows, w.scan_cols, w.det_rows, w.det_cols, layout=w.layout)
        out.append((w, counts, blob))
    return out


def test_com_noalloc_matches_com_on_two_calls_the_second_smaller():
    (wb, cb, bb), (ws, cs, bs) = cases()
    masks_b = [None, synth.disk_mask(64, 64, 32, 32, 12)]
    masks_s = [None, synth.disk_mask(192, 192, 96, 96, 30)]
    with q().Resident(bb) as big, q().Resident(bs) as small:
        for (res, w, counts, masks) in ((big, wb, cb, masks_b), (small, ws, cs, masks_s)):
            for mask in masks:
                got = noalloc(res, mask)
                ref = res.com(mask)
                ref = ref[0].cpu().numpy(), ref[1].cpu().numpy()
                assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
                orow, ocol, _ = oracle.com(counts, w.det_rows, w.det_cols, mask=mask)
                assert np.array_equal(got[0], orow) and np.array_equal(got[1], ocol)
        # once more on the big resident after the small one: nothing of the small call remains
        got = noalloc(big, None)
        orow, ocol, _ = oracle.com(cb, wb.det_rows, wb.det_cols)
        assert np.array_equal(got[0], orow) and np.array_equal(got[1], ocol)


def test_com_noalloc_refuses_more_scans_than_its_buffer():
    import torch
    qq = q()
    S = 1025 * 1024  # 1,049,600 scans > 1,048,576
    counts = (np.arange(S, dtype=np.uint32) % 3).astype(np.uint8).reshape(S, 1)
    blob = qq.encode(counts, 1025, 1024, 1, 1)
    with qq.Resident(blob) as res:
        row = torch.empty(S, dtype=torch.float32, device="cuda:0")
        col = torch.empty_like(row)
        rc = qq.lib.qsc_com_noalloc(res._h, None, ctypes.c_void_p(row.data_ptr()), ctypes.c_void_p(col.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), 1)
        assert rc == qq.ERR_INVALID_ARG
        assert b"1048576" in qq.lib.qsc_last_error(res._h)
        # the allocating form still answers it
        r, c = res.com()
        assert np.array_equal(r.cpu().numpy(), np.zeros(S, np.float32))
