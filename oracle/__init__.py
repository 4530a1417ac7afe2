"""CPU oracle for the ANS-resident 4D-STEM query path.

TEST INFRASTRUCTURE ONLY: the library never imports this package. Tests, the
smoke check and the benchmark's CPU-baseline leg use it to produce expected
values. It wraps ``oracle.c`` (a plain scalar encoder/decoder written from
FORMAT.md, plus the dense product definitions) and adds NumPy brute-force
versions of the products for tiny inputs.

Pins (see tests/test_oracle.py): round-trip identity on every generator and on
adversarial streams; NumPy brute force and closed forms for the sums and CoM;
numpy.rint for ties-to-even codes; NumPy float64 reconstruction; table and
model invariants; hand-built streams decoded against hand-computed values.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_ARG, ERR_MALFORMED, ERR_UNSUPPORTED, ERR_OOM = 0, -1, -2, -3, -4
BLOCK = 512


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("scan_rows", "scan_cols", "det_rows", "det_cols", "dtype", "layout", "scaled")]


class OracleError(ValueError):
    def __init__(self, code, msg=""):
        super().__init__(f"oracle error {code} {msg}")
        self.code = code


def build(force=False):
    """Compile liboracle.so with gcc (plain C)."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        cmd = f"gcc -O2 -ffp-contract=off -fPIC -shared -o {_LIB_PATH}.tmp {src} -lm && mv {_LIB_PATH}.tmp {_LIB_PATH}"
        if os.system(cmd) != 0:
            raise RuntimeError("failed to build liboracle.so")


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp, u64, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
        lib.orc_encode.argtypes = [ctypes.POINTER(_Geom), vp, ctypes.POINTER(ctypes.POINTER(ctypes.c_uint8))]
        lib.orc_encode.restype = ctypes.c_int64
        lib.orc_free.argtypes = [vp]
        lib.orc_decode.argtypes = [vp, u64, vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        lib.orc_calibration.argtypes = [vp, u64, vp]
        lib.orc_masked_sum.argtypes = [vp, u32, u64, u64, vp, vp, u32, vp]
        lib.orc_com.argtypes = [vp, u32, u64, u32, u32, vp, vp, vp, vp, vp]
        lib.orc_sum_dp.argtypes = [vp, u32, u64, u64, vp, vp, u32, vp, vp, vp]
        lib.orc_calibrate.argtypes = [vp, u64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), vp]
        lib.orc_reconstruct.argtypes = [vp, u64, ctypes.c_double, ctypes.c_double, vp]
        lib.orc_reconstruct.restype = None
        lib.orc_pair_models.argtypes = [vp, vp, vp]
        lib.orc_pair_decode_table.argtypes = [ctypes.c_int, vp, vp, vp]
        lib.orc_pair_encode_steps.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
        lib.orc_paired_size.argtypes = [vp, u32, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_uint64)]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def encode(counts, scan_rows, scan_cols, det_rows, det_cols, layout=0, scaled=False):
    """Encode dense counts (S x P, uint8/uint16) or float32 (scaled) into a container blob (bytes)."""
    arr = np.ascontiguousarray(counts)
    if scaled:
        assert arr.dtype == np.float32
        dtype = 2
    else:
        dtype = {np.dtype(np.uint8): 1, np.dtype(np.uint16): 2}[arr.dtype]
    g = _Geom(scan_rows, scan_cols, det_rows, det_cols, dtype, layout, 1 if scaled else 0)
    out = ctypes.POINTER(ctypes.c_uint8)()
    n = _load().orc_encode(ctypes.byref(g), arr.ctypes.data, ctypes.byref(out))
    if n < 0:
        raise OracleError(n, "encode")
    blob = ctypes.string_at(out, n)
    _lib.orc_free(out)
    return blob


def header(blob):
    """Geometry fields of a container header."""
    h = np.frombuffer(blob[:256], dtype=np.uint8)
    u32 = h[40:80].view(np.uint32)
    u64 = h[80:144].view(np.uint64)
    return dict(version=int(u32[0]), layout=int(u32[1]), scan_rows=int(u32[2]), scan_cols=int(u32[3]),
                det_rows=int(u32[4]), det_cols=int(u32[5]), dtype=int(u32[6]), block_scans=int(u32[7]),
                n_blocks=int(u32[8]), flags=int(u32[9]), dir_off=int(u64[0]), table_off=int(u64[1]),
                gbase_off=int(u64[2]), rel_off=int(u64[3]), payload_off=int(u64[4]),
                payload_bytes=int(u64[5]), calib_off=int(u64[6]), total_bytes=int(u64[7]))


def decode(blob):
    """Dense native counts (S x P) of a blob; raises OracleError(MALFORMED) with the first bad stream."""
    h = header(blob)
    S, P = h["scan_rows"] * h["scan_cols"], h["det_rows"] * h["det_cols"]
    out = np.empty((S, P), dtype=np.uint8 if h["dtype"] == 1 else np.uint16)
    bb, bp = ctypes.c_int64(), ctypes.c_int64()
    buf = np.frombuffer(blob, dtype=np.uint8)
    rc = _load().orc_decode(buf.ctypes.data, len(blob), out.ctypes.data, ctypes.byref(bb), ctypes.byref(bp))
    if rc:
        raise OracleError(rc, f"decode block {bb.value} pixel {bp.value}")
    return out


def calibration(blob):
    """(n_blocks, 2) array of per-block (scale, offset) of a scaled blob."""
    h = header(blob)
    out = np.empty((h["n_blocks"], 2), dtype=np.float64)
    buf = np.frombuffer(blob, dtype=np.uint8)
    rc = _load().orc_calibration(buf.ctypes.data, len(blob), out.ctypes.data)
    if rc:
        raise OracleError(rc, "calibration")
    return out


def sum_bits(P, dtype):
    """64 when a full-detector sum could exceed 2^32 - 1, else 32."""
    maxv = 255 if dtype == 1 else 65535
    return 64 if P * maxv > 2**32 - 1 else 32


def masked_sum(counts, mask, valid=None, stride=1):
    """Exact per-scan sums over mask & valid (uint64); scans of skipped blocks are 0."""
    c = np.ascontiguousarray(counts)
    S, P = c.shape
    dtype = 1 if c.dtype == np.uint8 else 2
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    v = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    out = np.empty(S, dtype=np.uint64)
    rc = _load().orc_masked_sum(c.ctypes.data, dtype, S, P, m.ctypes.data, _ptr(v), stride, out.ctypes.data)
    if rc:
        raise OracleError(rc, "masked_sum")
    return out


def dense_df(counts, mask, valid=None):
    """Cached-total form of dense DF: total over valid minus the sum over valid & ~mask."""
    P = counts.shape[1]
    allm = np.ones(P, dtype=np.uint8)
    total = masked_sum(counts, allm, valid)
    comp = masked_sum(counts, (1 - np.asarray(mask, dtype=np.uint8)).astype(np.uint8), valid)
    return total - comp


def com(counts, det_rows, det_cols, mask=None, valid=None):
    """Exact-moment CoM: (row, col) float32 per scan, plus M0."""
    c = np.ascontiguousarray(counts)
    S = c.shape[0]
    dtype = 1 if c.dtype == np.uint8 else 2
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    v = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    row = np.empty(S, dtype=np.float32)
    col = np.empty(S, dtype=np.float32)
    m0 = np.empty(S, dtype=np.uint64)
    rc = _load().orc_com(c.ctypes.data, dtype, S, det_rows, det_cols, _ptr(m), _ptr(v), row.ctypes.data,
                         col.ctypes.data, m0.ctypes.data)
    if rc:
        raise OracleError(rc, "com")
    return row, col, m0


def sum_dp(counts, scan_mask=None, valid=None, stride=1, calib=None):
    """Sum (uint64) and mean (float32) diffraction pattern over the selected scans.

    calib: (n_blocks, 2) float64 (scale, offset) per 512-scan region of a scaled
    resident; the mean is then that of the reconstructed intensities.
    """
    c = np.ascontiguousarray(counts)
    S, P = c.shape
    dtype = 1 if c.dtype == np.uint8 else 2
    m = None if scan_mask is None else np.ascontiguousarray(scan_mask, dtype=np.uint8)
    v = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    cal = None if calib is None else np.ascontiguousarray(calib, dtype=np.float64)
    out = np.empty(P, dtype=np.uint64)
    mean = np.empty(P, dtype=np.float32)
    rc = _load().orc_sum_dp(c.ctypes.data, dtype, S, P, _ptr(m), _ptr(v), stride, _ptr(cal), out.ctypes.data,
                            mean.ctypes.data)
    if rc:
        raise OracleError(rc, "sum_dp")
    return out, mean


def region(counts, scan_cols, r0, r1, c0, c1, valid=None):
    """counts of the half-open scan rectangle, (h*w, P), invalid pixels zeroed."""
    rows = []
    for r in range(r0, r1):
        rows.append(counts[r * scan_cols + c0: r * scan_cols + c1])
    out = np.concatenate(rows, axis=0).copy()
    if valid is not None:
        out[:, np.asarray(valid) == 0] = 0
    return out


def frames(counts, first_block, n_blocks, valid=None, kind="native", calib=None):
    """Every scan of the block range as frames (scans, P), invalid pixels zeroed.

    kind "native": the counts; "amplitude": float32 square root of each count
    (NumPy's float32 sqrt, correctly rounded); "calibrated": code*scale+offset
    of each scan's region (calib: (n_blocks, 2) float64 of a scaled resident).
    """
    s0 = first_block * BLOCK
    s1 = min(counts.shape[0], (first_block + n_blocks) * BLOCK)
    out = counts[s0:s1].copy()
    if kind == "amplitude":
        out = np.sqrt(out.astype(np.float32))
    elif kind == "calibrated":
        rows = [reconstruct(out[i], *calib[(s0 + i) // BLOCK]) for i in range(out.shape[0])]
        out = np.stack(rows)
    if valid is not None:
        out[:, np.asarray(valid) == 0] = 0
    return out


# ---------------------------------------------------------------------------
# polar interaction index ("Paired-count resident layout", "Operation pipeline"
# items 3-4): exact per-scan sums over radial-angular pixel groups, 64-pixel
# leaves and 16-leaf roots; a mask is answered as index fields plus residual
# pixels that are decoded
# ---------------------------------------------------------------------------

LEAF = 64
ROOT = 16


def polar_order(det_rows, det_cols, cr, cc):
    """Pixels ordered by squared distance from (cr, cc), then by angle.

    The angle is atan2(kr - cr, kc - cc); distinct directions at one distance
    differ far more than its rounding error, so the order is exact.
    """
    kr, kc = np.meshgrid(np.arange(det_rows), np.arange(det_cols), indexing="ij")
    dr, dc = (kr - cr).ravel(), (kc - cc).ravel()
    d2 = dr.astype(np.int64) ** 2 + dc.astype(np.int64) ** 2
    ang = np.arctan2(dr.astype(np.float64), dc.astype(np.float64))
    return np.lexsort((ang, d2))


def index_fields(counts, order, valid=None):
    """Per-scan exact sums of the valid pixels of every leaf and every root: (S, leaves), (S, roots)."""
    c = counts.astype(np.uint64)
    if valid is not None:
        c = c * (np.asarray(valid) != 0)
    P = c.shape[1]
    n_leaves = (P + LEAF - 1) // LEAF
    leaves = np.stack([c[:, order[LEAF * i: LEAF * (i + 1)]].sum(axis=1) for i in range(n_leaves)], axis=1)
    n_roots = (n_leaves + ROOT - 1) // ROOT
    roots = np.stack([leaves[:, ROOT * i: ROOT * (i + 1)].sum(axis=1) for i in range(n_roots)], axis=1)
    return leaves, roots


def decompose(mask, order, valid=None):
    """(full roots, full leaves outside them, residual mask) of mask & valid.

    A leaf (root) is a field of the query when every valid pixel in it is
    selected and it has one; the residual is every selected valid pixel that
    no field covers.
    """
    P = len(order)
    v = np.ones(P, bool) if valid is None else np.asarray(valid) != 0
    sel = (np.asarray(mask) != 0) & v
    n_leaves = (P + LEAF - 1) // LEAF
    full_leaf = np.zeros(n_leaves, bool)
    for i in range(n_leaves):
        px = order[LEAF * i: LEAF * (i + 1)]
        full_leaf[i] = v[px].any() and np.array_equal(sel[px], v[px])
    n_roots = (n_leaves + ROOT - 1) // ROOT
    full_root = np.zeros(n_roots, bool)
    for j in range(n_roots):
        lv = np.arange(ROOT * j, min(n_leaves, ROOT * (j + 1)))
        px = order[LEAF * lv[0]: min(P, LEAF * (lv[-1] + 1))]
        full_root[j] = v[px].any() and np.array_equal(sel[px], v[px])
    leaves = [i for i in range(n_leaves) if full_leaf[i] and not full_root[i // ROOT]]
    roots = [j for j in range(n_roots) if full_root[j]]
    covered = np.zeros(P, bool)
    for i in range(n_leaves):
        if full_leaf[i] or full_root[i // ROOT]:
            covered[order[LEAF * i: LEAF * (i + 1)]] = True
    residual = (sel & ~covered).astype(np.uint8)
    return roots, leaves, residual


def indexed_masked_sum(counts, mask, order, valid=None, stride=1):
    """masked_sum answered the index way: field sums plus the residual pixels' sums."""
    leaves, roots = index_fields(counts, order, valid)
    r, l, residual = decompose(mask, order, valid)
    out = masked_sum(counts, residual, valid, stride)
    fields = roots[:, r].sum(axis=1) + leaves[:, l].sum(axis=1)
    S = counts.shape[0]
    visited = (np.arange(S) // BLOCK) % stride == 0
    return out + np.where(visited, fields, 0).astype(np.uint64)


def calibrate(x):
    """(scale, offset, codes) of one region of float32 values."""
    a = np.ascontiguousarray(x, dtype=np.float32).ravel()
    sc, off = ctypes.c_double(), ctypes.c_double()
    codes = np.empty(a.size, dtype=np.uint16)
    rc = _load().orc_calibrate(a.ctypes.data, a.size, ctypes.byref(sc), ctypes.byref(off), codes.ctypes.data)
    if rc:
        raise OracleError(rc, "calibrate")
    return sc.value, off.value, codes


def reconstruct(codes, scale, offset):
    """float32 of code*scale + offset, product and sum each rounded in float64."""
    c = np.ascontiguousarray(codes, dtype=np.uint16).ravel()
    out = np.empty(c.size, dtype=np.float32)
    _load().orc_reconstruct(c.ctypes.data, c.size, scale, offset, out.ctypes.data)
    return out


def pair_models():
    """(32, 256) uint16 pair counts, (32,) window bases and (32,) in-use bit masks of the paired layout."""
    n = np.empty((32, 256), dtype=np.uint16)
    a0 = np.empty(32, dtype=np.uint32)
    use = np.empty(32, dtype=np.uint32)
    _load().orc_pair_models(n.ctypes.data, a0.ctypes.data, use.ctypes.data)
    return n, a0, use


def pair_decode_table(m):
    """Decode entries of pair model m (FORMAT 3.2): (symbol, nbits, next-state base) per state, 1024 each."""
    sym = np.empty(1024, dtype=np.uint16)
    nb = np.empty(1024, dtype=np.uint8)
    nx = np.empty(1024, dtype=np.uint16)
    rc = _load().orc_pair_decode_table(m, sym.ctypes.data, nb.ctypes.data, nx.ctypes.data)
    if rc:
        raise OracleError(rc, "pair_decode_table")
    return sym, nb, nx


def pair_encode_steps(m, i):
    """The encoder step of pair symbol i of model m from every state x = 1024..2047:
    (emitted bit count, emitted bits, new state - 1024), each indexed by x - 1024."""
    k = np.empty(1024, dtype=np.uint32)
    bits = np.empty(1024, dtype=np.uint32)
    st = np.empty(1024, dtype=np.uint32)
    rc = _load().orc_pair_encode_steps(m, i, k.ctypes.data, bits.ctypes.data, st.ctypes.data)
    if rc:
        raise OracleError(rc, "pair_encode_steps")
    return k, bits, st


def paired_size(values, dtype):
    """(model, bytes) of the PAIRED form of one 512-value stream: the model the static
    cost picks and the stream size with its header (FORMAT 3.4)."""
    v = np.ascontiguousarray(values, dtype=np.uint32)
    assert v.size == BLOCK
    m, n = ctypes.c_int(), ctypes.c_uint64()
    rc = _load().orc_paired_size(v.ctypes.data, dtype, ctypes.byref(m), ctypes.byref(n))
    if rc:
        raise OracleError(rc, "paired_size")
    return m.value, n.value


# ---------------------------------------------------------------------------
# NumPy brute force for tiny inputs (independent of oracle.c)
# ---------------------------------------------------------------------------

def brute_masked_sum(counts, mask, valid=None, stride=1):
    sel = np.asarray(mask).astype(bool)
    if valid is not None:
        sel &= np.asarray(valid).astype(bool)
    out = counts.astype(np.uint64)[:, sel].sum(axis=1, dtype=np.uint64)
    blocks = np.arange(counts.shape[0]) // BLOCK
    out[blocks % stride != 0] = 0
    return out


def brute_sum_dp(counts, scan_mask=None, valid=None, stride=1):
    """NumPy sum and mean diffraction pattern over the selected scans."""
    S, P = counts.shape
    sel = (np.arange(S) // BLOCK) % stride == 0
    if scan_mask is not None:
        sel &= np.asarray(scan_mask) != 0
    total = counts[sel].astype(np.uint64).sum(axis=0)
    if valid is not None:
        total[np.asarray(valid) == 0] = 0
    n = int(sel.sum())
    mean = (total.astype(np.float64) / n).astype(np.float32) if n else np.zeros(P, np.float32)
    return total, mean


def brute_com(counts, det_rows, det_cols, mask=None, valid=None):
    sel = np.ones(det_rows * det_cols, dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    if valid is not None:
        sel &= np.asarray(valid).astype(bool)
    kr = (np.arange(det_rows * det_cols) // det_cols).astype(np.uint64)
    kc = (np.arange(det_rows * det_cols) % det_cols).astype(np.uint64)
    c = counts.astype(np.uint64)[:, sel]
    m0 = c.sum(axis=1)
    mr = (c * kr[sel]).sum(axis=1)
    mc = (c * kc[sel]).sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        row = np.where(m0 > 0, mr.astype(np.float64) / np.maximum(m0, 1).astype(np.float64), 0.0).astype(np.float32)
        col = np.where(m0 > 0, mc.astype(np.float64) / np.maximum(m0, 1).astype(np.float64), 0.0).astype(np.float32)
    return row, col, m0
