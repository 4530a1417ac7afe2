"""Python binding of libqsc: ANS-resident 4D-STEM counts with fused GPU queries.

Argument marshalling only: every step of a query runs in the library's HIP
kernels. PyTorch supplies device memory and streams (tensor data pointers and
``torch.cuda.current_stream().cuda_stream``). Importing works without a GPU
(the encoder is host code); queries need a gfx950 device. There is no CPU
fallback: if libqsc.so is missing the import fails.

Entry points mirror include/qsc.h:
    encode(data, geometry) -> bytes          qsc_encoder_*
    encode_device(tensor, geometry)          qsc_encode_device_bound / qsc_encode_device
    Resident(blob, valid=None)               qsc_resident_create (host blob) or
                                             qsc_resident_create_device (device tensor); destroy / info
    Resident.masked_sum(mask, block_stride)  qsc_masked_sum
    Resident.dense_df(mask)                  qsc_dense_df
    Resident.com(mask=None)                  qsc_com
    Resident.com_noalloc(mask=None)          qsc_com_noalloc
    Resident.decode_region(r0, r1, c0, c1)   qsc_decode_region
    Resident.sum_dp(scan_mask, stride)       qsc_sum_dp
    Resident.decode_blocks(first, n, kind)   qsc_decode_blocks
    Resident.feed(first, n, per, kind, depth) qsc_feed_create / _next / _release / _destroy
    Resident.index_build(center)             qsc_index_build
    Resident.masked_sum_delta(prev, ...)     qsc_masked_sum_delta
    Resident.finish()                        qsc_finish
    Resident.query_bytes(mask, stride)       qsc_query_bytes
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsc.so")

OK, ERR_INVALID_ARG, ERR_MALFORMED, ERR_UNSUPPORTED, ERR_OOM, ERR_HIP = 0, -1, -2, -3, -4, -5
DEVICE_PAD = 16384  # zero bytes a borrowed device container needs after it


class QscError(RuntimeError):
    """A failed library call; ``code`` is the qsc_status."""

    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


class QscValueError(QscError, ValueError):
    """Malformed container/stream or invalid argument (the pages' ValueError)."""


class Geometry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("scan_rows", "scan_cols", "det_rows", "det_cols", "dtype", "layout", "scaled")]


class Info(ctypes.Structure):
    _fields_ = [("geom", Geometry), ("n_blocks", ctypes.c_uint32), ("sum_bits", ctypes.c_uint32),
                ("resident_bytes", ctypes.c_uint64), ("payload_bytes", ctypes.c_uint64),
                ("mode_counts", ctypes.c_uint64 * 8), ("index_bytes", ctypes.c_uint64)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(python -m stem_compressed_count_amd.build); there is no fallback path")
# torch's HIP runtime is loaded first, so that the library binds to the same
# runtime and device pointers pass between them (a second runtime loaded by
# the library alone would not know torch's allocations)
try:
    import torch  # noqa: F401
except ImportError:  # the host encoder and the pure host entry points still work
    pass
lib = ctypes.CDLL(LIB_PATH)

_vp, _u32, _u64, _i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
_SIGS = {
    "qsc_abi": ([], ctypes.c_char_p),
    "qsc_status_string": ([_i32], ctypes.c_char_p),
    "qsc_encoder_create": ([ctypes.POINTER(Geometry), ctypes.POINTER(_vp)], _i32),
    "qsc_encoder_add": ([_vp, _vp, _u64, ctypes.c_int], _i32),
    "qsc_encoder_size": ([_vp, ctypes.POINTER(_u64)], _i32),
    "qsc_encoder_write": ([_vp, _vp, _u64], _i32),
    "qsc_encoder_destroy": ([_vp], _i32),
    "qsc_resident_create": ([_vp, _u64, _vp, _vp, ctypes.POINTER(_vp)], _i32),
    "qsc_resident_create_device": ([_vp, _u64, _vp, _vp, ctypes.POINTER(_vp)], _i32),
    "qsc_resident_create_device_borrow": ([_vp, _u64, _u64, _vp, _vp, ctypes.POINTER(_vp)], _i32),
    "qsc_encode_device_bound": ([ctypes.POINTER(Geometry), ctypes.POINTER(_u64)], _i32),
    "qsc_encode_device": ([ctypes.POINTER(Geometry), _vp, _vp, _u64, ctypes.POINTER(_u64), _vp], _i32),
    "qsc_resident_destroy": ([_vp], _i32),
    "qsc_resident_info": ([_vp, ctypes.POINTER(Info)], _i32),
    "qsc_masked_sum": ([_vp, _vp, _u32, _vp, _vp, ctypes.c_int], _i32),
    "qsc_dense_df": ([_vp, _vp, _vp, _vp, ctypes.c_int], _i32),
    "qsc_com": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_int], _i32),
    "qsc_com_noalloc": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_int], _i32),
    "qsc_decode_region": ([_vp, _u32, _u32, _u32, _u32, ctypes.c_int, _vp, _vp, ctypes.c_int], _i32),
    "qsc_sum_dp": ([_vp, _vp, _u32, _vp, _vp, _vp, ctypes.c_int], _i32),
    "qsc_decode_blocks": ([_vp, _u32, _u32, ctypes.c_int, _vp, _vp, ctypes.c_int], _i32),
    "qsc_finish": ([_vp, _vp], _i32),
    "qsc_feed_create": ([_vp, _u32, _u32, _u32, ctypes.c_int, _u32, ctypes.POINTER(_vp), _u64, _vp,
                         ctypes.POINTER(_vp)], _i32),
    "qsc_feed_next": ([_vp, ctypes.POINTER(_u32), ctypes.POINTER(_u64), ctypes.POINTER(_u32)], _i32),
    "qsc_feed_release": ([_vp], _i32),
    "qsc_feed_destroy": ([_vp], _i32),
    "qsc_index_build": ([_vp, ctypes.c_int32, ctypes.c_int32, _vp], _i32),
    "qsc_masked_sum_delta": ([_vp, _vp, _vp, _vp, _u32, _vp, _vp, ctypes.c_int], _i32),
    "qsc_last_error": ([_vp], ctypes.c_char_p),
    "qsc_query_bytes": ([_vp, _vp, _u32, ctypes.POINTER(_u64), ctypes.POINTER(_u64)], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTS = tuple(_SIGS)


def abi():
    return lib.qsc_abi().decode()


def _raise(code, msg):
    text = f"{lib.qsc_status_string(code).decode()}: {msg}"
    if code in (ERR_MALFORMED, ERR_INVALID_ARG, ERR_UNSUPPORTED):
        raise QscValueError(code, text)
    raise QscError(code, text)


def encode(data, scan_rows, scan_cols, det_rows, det_cols, layout=0, scaled=False, threads=0):
    """Encode (S x P) uint8/uint16 counts, or float32 when scaled, into a container blob (numpy uint8).

    Other dtypes are refused, float16 included: there is no float16 storage (the
    scaled-uint16 page, "What dtype means": load and save refuse it), and scaled
    storage keeps 16-bit codes of float32 intensities."""
    dt = np.asarray(data).dtype
    if scaled and dt != np.float32:
        raise ValueError(f"scaled input must be float32, not {dt}")
    if not scaled and dt not in (np.uint8, np.uint16):
        raise ValueError(f"counts must be uint8 or uint16, not {dt}")
    enc = Encoder(scan_rows, scan_cols, det_rows, det_cols, dtype=2 if scaled else (1 if dt == np.uint8 else 2),
                  layout=layout, scaled=scaled)
    try:
        enc.add(data, threads)
        return enc.blob()
    finally:
        enc.close()


def encode_device(data, scan_rows, scan_cols, det_rows, det_cols, layout=0, scaled=False, stream=None):
    """Encode (S x P) values already on the GPU (a torch tensor: uint8, 16-bit integers, or float32 when
    scaled) into a container in device memory; returns a uint8 tensor holding exactly the container."""
    import torch
    if not isinstance(data, torch.Tensor) or not data.is_cuda or not data.is_contiguous():
        raise ValueError("data must be a contiguous CUDA tensor")
    if scaled:
        if data.dtype != torch.float32:
            raise ValueError("scaled input must be float32")
        dtype = 2
    elif data.dtype == torch.uint8:
        dtype = 1
    elif data.element_size() == 2 and not data.is_floating_point():
        dtype = 2
    else:
        raise ValueError("counts must be uint8 or 16-bit integers")
    g = Geometry(scan_rows, scan_cols, det_rows, det_cols, dtype, layout, 1 if scaled else 0)
    if data.numel() != scan_rows * scan_cols * det_rows * det_cols:
        raise ValueError("data must hold scans x detector pixels values")
    cap = _u64()
    rc = lib.qsc_encode_device_bound(ctypes.byref(g), ctypes.byref(cap))
    if rc:
        _raise(rc, "encode_device geometry")
    out = torch.empty(cap.value + DEVICE_PAD, dtype=torch.uint8, device=data.device)  # room to borrow it
    n = _u64()
    rc = lib.qsc_encode_device(ctypes.byref(g), data.data_ptr(), out.data_ptr(), cap.value, ctypes.byref(n),
                               _stream_handle(stream))
    if rc:
        _raise(rc, "encode_device")
    return out[:n.value]


class Encoder:
    """Streaming host encoder: add scans in order (multiples of 512 but the last), then blob()."""

    def __init__(self, scan_rows, scan_cols, det_rows, det_cols, dtype, layout=0, scaled=False):
        self.geom = Geometry(scan_rows, scan_cols, det_rows, det_cols, dtype, layout, 1 if scaled else 0)
        self.P = det_rows * det_cols
        self.scaled = scaled
        self._h = _vp()
        rc = lib.qsc_encoder_create(ctypes.byref(self.geom), ctypes.byref(self._h))
        if rc:
            _raise(rc, "encoder geometry")

    def add(self, data, threads=0):
        want = np.float32 if self.scaled else (np.uint8 if self.geom.dtype == 1 else np.uint16)
        a = np.ascontiguousarray(data)
        if a.dtype != want or a.size % self.P:
            raise ValueError(f"expected {np.dtype(want).name} data with {self.P} values per scan")
        rc = lib.qsc_encoder_add(self._h, a.ctypes.data, a.size // self.P, threads)
        if rc:
            _raise(rc, "encoder add")

    def blob(self):
        n = _u64()
        rc = lib.qsc_encoder_size(self._h, ctypes.byref(n))
        if rc:
            _raise(rc, "encoder size (were all scans added?)")
        out = np.empty(n.value, dtype=np.uint8)
        rc = lib.qsc_encoder_write(self._h, out.ctypes.data, n.value)
        if rc:
            _raise(rc, "encoder write")
        return out

    def close(self):
        if self._h:
            lib.qsc_encoder_destroy(self._h)
            self._h = _vp()

    def __del__(self):
        self.close()


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Resident:
    """An encoded acquisition resident in device memory (qsc_resident)."""

    def __init__(self, blob, valid=None, stream=None, borrow=False):
        """blob: a host container (bytes or numpy uint8), or a CUDA uint8 tensor holding one.
        borrow=True uses a device container in place (its storage needs 16384 spare bytes after it,
        as encode_device leaves) and keeps a reference to it for the resident's lifetime."""
        import torch
        v = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
        self._h = _vp()
        self._borrowed = None
        if isinstance(blob, torch.Tensor) and blob.is_cuda:
            if blob.dtype != torch.uint8 or not blob.is_contiguous():
                raise ValueError("a device container must be a contiguous uint8 tensor")
            if borrow:
                cap = blob.untyped_storage().nbytes() - blob.storage_offset()
                rc = lib.qsc_resident_create_device_borrow(blob.data_ptr(), blob.numel(), cap,
                                                           None if v is None else v.ctypes.data,
                                                           _stream_handle(stream), ctypes.byref(self._h))
                self._borrowed = blob
            else:
                rc = lib.qsc_resident_create_device(blob.data_ptr(), blob.numel(),
                                                    None if v is None else v.ctypes.data,
                                                    _stream_handle(stream), ctypes.byref(self._h))
        else:
            b = np.ascontiguousarray(np.frombuffer(blob, dtype=np.uint8) if isinstance(blob, (bytes, bytearray))
                                     else blob, dtype=np.uint8)
            rc = lib.qsc_resident_create(b.ctypes.data, b.size, None if v is None else v.ctypes.data,
                                         _stream_handle(stream), ctypes.byref(self._h))
        if rc:
            _raise(rc, "resident_create")
        info = self._info()
        self.info = info
        g = info.geom
        self.scan_rows, self.scan_cols, self.det_rows, self.det_cols = g.scan_rows, g.scan_cols, g.det_rows, g.det_cols
        self.S, self.P = g.scan_rows * g.scan_cols, g.det_rows * g.det_cols
        self.dtype = g.dtype
        self.scaled = bool(g.scaled)
        self.sum_dtype = torch.int64 if info.sum_bits == 64 else torch.int32
        self.device = torch.device("cuda", torch.cuda.current_device())

    # -- helpers
    def _info(self):
        info = Info()
        lib.qsc_resident_info(self._h, ctypes.byref(info))
        return info

    def _check(self, rc, what):
        if rc:
            _raise(rc, f"{what}: {lib.qsc_last_error(self._h).decode()}")

    def _mask(self, mask):
        import torch
        m = torch.as_tensor(mask, dtype=torch.uint8, device=self.device).contiguous()
        if m.numel() != self.P:
            raise ValueError(f"mask must have {self.P} entries")
        return m

    def _on(self, stream, *tensors):
        """A query queued on a stream other than the current one: that stream first
        waits for the current one (where the mask copies and new outputs were
        made), and the tensors are marked as used there, so the caching allocator
        does not hand their memory to other work before the query is done."""
        import torch
        if stream is None:
            return
        cur = torch.cuda.current_stream()
        if stream.cuda_stream == cur.cuda_stream:
            return
        stream.wait_stream(cur)
        for t in tensors:
            if t is not None:
                t.record_stream(stream)

    def _out(self, out, dtype, n):
        import torch
        if out is None:
            return torch.empty(n, dtype=dtype, device=self.device)
        if out.dtype != dtype or out.numel() != n or not out.is_contiguous() or out.device != self.device:
            raise ValueError(f"out must be a contiguous {dtype} tensor of {n} elements on {self.device}")
        return out

    # -- queries
    def masked_sum(self, mask, block_stride=1, out=None, stream=None, wait=True):
        """Exact per-scan sums over mask & valid (int32 storage of uint32, or int64 of uint64)."""
        m = self._mask(mask)
        o = self._out(out, self.sum_dtype, self.S)
        self._on(stream, m, o)
        self._check(lib.qsc_masked_sum(self._h, m.data_ptr(), block_stride, o.data_ptr(), _stream_handle(stream),
                                       int(wait)), "masked_sum")
        return o

    def masked_sum_delta(self, prev_mask, prev_out, mask, block_stride=1, out=None, stream=None, wait=True):
        """masked_sum(mask) from prev_out = masked_sum(prev_mask): only the changed pixels are decoded."""
        pm, m = self._mask(prev_mask), self._mask(mask)
        if prev_out.dtype != self.sum_dtype or prev_out.numel() != self.S or not prev_out.is_contiguous():
            raise ValueError(f"prev_out must be a contiguous {self.sum_dtype} tensor of {self.S} elements")
        o = self._out(out, self.sum_dtype, self.S)
        self._on(stream, pm, m, prev_out, o)
        self._check(lib.qsc_masked_sum_delta(self._h, pm.data_ptr(), prev_out.data_ptr(), m.data_ptr(), block_stride,
                                             o.data_ptr(), _stream_handle(stream), int(wait)), "masked_sum_delta")
        return o

    def dense_df(self, mask, out=None, stream=None, wait=True):
        m = self._mask(mask)
        o = self._out(out, self.sum_dtype, self.S)
        self._on(stream, m, o)
        self._check(lib.qsc_dense_df(self._h, m.data_ptr(), o.data_ptr(), _stream_handle(stream), int(wait)),
                    "dense_df")
        return o

    def com(self, mask=None, out_row=None, out_col=None, stream=None, wait=True):
        import torch
        m = None if mask is None else self._mask(mask)
        row = self._out(out_row, torch.float32, self.S)
        col = self._out(out_col, torch.float32, self.S)
        self._on(stream, m, row, col)
        self._check(lib.qsc_com(self._h, None if m is None else m.data_ptr(), row.data_ptr(), col.data_ptr(),
                                _stream_handle(stream), int(wait)), "com")
        return row, col

    def com_noalloc(self, mask=None, out_row=None, out_col=None, stream=None, wait=True):
        """com with the library's static moment buffer (qsc_com_noalloc): no device allocation
        inside the call; at most 1,048,576 scans; calls overlapping on one GPU race."""
        import torch
        m = None if mask is None else self._mask(mask)
        row = self._out(out_row, torch.float32, self.S)
        col = self._out(out_col, torch.float32, self.S)
        self._on(stream, m, row, col)
        self._check(lib.qsc_com_noalloc(self._h, None if m is None else m.data_ptr(), row.data_ptr(),
                                        col.data_ptr(), _stream_handle(stream), int(wait)), "com_noalloc")
        return row, col

    def decode_region(self, r0, r1, c0, c1, calibrated=False, out=None, stream=None, wait=True):
        """(h*w, P) counts of the scan rectangle; float32 intensities when calibrated (scaled residents)."""
        import torch
        if not (0 <= r0 < r1 <= self.scan_rows and 0 <= c0 < c1 <= self.scan_cols):
            raise ValueError("scan_region out of range or empty")
        n = (r1 - r0) * (c1 - c0) * self.P
        dt = torch.float32 if calibrated else (torch.uint8 if self.dtype == 1 else torch.int16)
        o = self._out(out, dt, n)
        self._on(stream, o)
        self._check(lib.qsc_decode_region(self._h, r0, r1, c0, c1, 1 if calibrated else 0, o.data_ptr(),
                                          _stream_handle(stream), int(wait)), "decode_region")
        return o.view((r1 - r0) * (c1 - c0), self.P)

    def decode_blocks(self, first_block, n_blocks, kind="native", out=None, stream=None, wait=True):
        """(scans, P) frames of whole blocks: "native" counts, "calibrated" (scaled) or "amplitude" float32 sqrt."""
        import torch
        kinds = {"native": 0, "calibrated": 1, "amplitude": 2}
        if kind not in kinds:
            raise ValueError(f"kind must be one of {sorted(kinds)}")
        s0 = first_block * 512
        n = max(0, min(self.S, (first_block + n_blocks) * 512) - s0) * self.P
        dt = torch.float32 if kinds[kind] else (torch.uint8 if self.dtype == 1 else torch.int16)
        o = self._out(out, dt, n)
        self._on(stream, o)
        self._check(lib.qsc_decode_blocks(self._h, first_block, n_blocks, kinds[kind], o.data_ptr(),
                                          _stream_handle(stream), int(wait)), "decode_blocks")
        return o.view(-1, self.P)

    def feed(self, first_block=0, n_blocks=None, blocks_per_item=1, kind="native", depth=2, stream=None):
        """Iterator over whole-block frames decoded depth items ahead on a stream of the
        library's (qsc_feed_*): yields (frames (scans, P) tensor, first scan). A yielded
        tensor is a view of one of the feed's buffers and is reused once the iteration
        moves on: copy it to keep it. Work queued on the consumer stream (the current one,
        or stream) while an item is held is ordered before its buffer is reused."""
        return Feed(self, first_block, self.info.n_blocks - first_block if n_blocks is None else n_blocks,
                    blocks_per_item, kind, depth, stream)

    def sum_dp(self, scan_mask=None, block_stride=1, out_sum=None, out_mean=None, stream=None, wait=True):
        """Sum (int64 storage of uint64) and mean (float32) diffraction pattern over the selected scans."""
        import torch
        m = None
        if scan_mask is not None:
            m = torch.as_tensor(scan_mask, dtype=torch.uint8, device=self.device).contiguous()
            if m.numel() != self.S:
                raise ValueError(f"scan_mask must have {self.S} entries")
        s = self._out(out_sum, torch.int64, self.P)
        mean = self._out(out_mean, torch.float32, self.P)
        self._on(stream, m, s, mean)
        self._check(lib.qsc_sum_dp(self._h, None if m is None else m.data_ptr(), block_stride, s.data_ptr(),
                                   mean.data_ptr(), _stream_handle(stream), int(wait)), "sum_dp")
        return s, mean

    def index_build(self, center=None, stream=None):
        """Build the polar interaction index around center (default: the detector's middle pixel)."""
        g = self.info.geom
        cr, cc = center if center is not None else (g.det_rows // 2, g.det_cols // 2)
        self._check(lib.qsc_index_build(self._h, int(cr), int(cc), _stream_handle(stream)), "index_build")
        self.info = self._info()

    def finish(self, stream=None):
        self._check(lib.qsc_finish(self._h, _stream_handle(stream)), "finish")

    def query_bytes(self, mask, block_stride=1):
        """(encoded bytes, logical counts) a masked_sum with this mask reads."""
        m = np.ascontiguousarray(mask, dtype=np.uint8)
        by, cn = _u64(), _u64()
        self._check(lib.qsc_query_bytes(self._h, m.ctypes.data, block_stride, ctypes.byref(by), ctypes.byref(cn)),
                    "query_bytes")
        return by.value, cn.value

    def close(self):
        if getattr(self, "_h", None) and lib is not None:  # lib is gone at interpreter exit
            lib.qsc_resident_destroy(self._h)
            self._h = _vp()
        self._borrowed = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        self.close()


class Feed:
    """Whole-block frames of a resident, decoded ahead on the library's own stream (qsc_feed_*)."""

    def __init__(self, res, first_block, n_blocks, blocks_per_item, kind, depth, stream):
        import torch
        kinds = {"native": 0, "calibrated": 1, "amplitude": 2}
        if kind not in kinds:
            raise ValueError(f"kind must be one of {sorted(kinds)}")
        self.res, self.P = res, res.P
        self._h = _vp()
        self._held = False
        dt = torch.float32 if kinds[kind] else (torch.uint8 if res.dtype == 1 else torch.int16)
        n = blocks_per_item * 512 * res.P
        self.bufs = [torch.empty(n, dtype=dt, device=res.device) for _ in range(max(0, depth))]
        self.stream = stream
        ptrs = (_vp * max(1, depth))(*[b.data_ptr() for b in self.bufs])
        res._check(lib.qsc_feed_create(res._h, first_block, n_blocks, blocks_per_item, kinds[kind], depth, ptrs,
                                       n * self.bufs[0].element_size() if self.bufs else 0,
                                       _stream_handle(stream), ctypes.byref(self._h)), "feed_create")

    def __iter__(self):
        return self

    def __next__(self):
        if not self._h:
            raise StopIteration
        if self._held:
            self.res._check(lib.qsc_feed_release(self._h), "feed_release")
            self._held = False
        i, s0, n = _u32(), _u64(), _u32()
        self.res._check(lib.qsc_feed_next(self._h, ctypes.byref(i), ctypes.byref(s0), ctypes.byref(n)), "feed_next")
        if n.value == 0:
            self.close()
            raise StopIteration
        self._held = True
        return self.bufs[i.value][:n.value * self.P].view(n.value, self.P), s0.value

    def close(self):
        """Waits for the feed's decodes; raises if a decoded stream was malformed."""
        if self._h:
            if self._held:
                lib.qsc_feed_release(self._h)
                self._held = False
            h, self._h = self._h, _vp()
            self.res._check(lib.qsc_feed_destroy(h), "feed")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def as_unsigned(t):
    """numpy view of a sum tensor as uint32/uint64 (the library's result type)."""
    a = t.cpu().numpy()
    return a.view(np.uint32 if a.dtype == np.int32 else np.uint64 if a.dtype == np.int64 else
                  np.uint16 if a.dtype == np.int16 else a.dtype)
