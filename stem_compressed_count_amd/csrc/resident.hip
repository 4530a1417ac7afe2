// C-ABI of the library: resident creation and the query entry points.
//
// The shape follows the pages' interface: a loaded acquisition stays ANS
// encoded on the GPU (quantem.widget ANS page; scaled-uint16 page), queries
// are enqueued and may be waited for later (paired-resident page, "Contract",
// row "queued queries"), a malformed stream fails the query with no result,
// and masked sums are exact uint32, or uint64 when a full-detector sum could
// pass 2^32 ("Contract", row "virtual image").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <string>
#include <tuple>
#include <cmath>
#include <memory>
#include <mutex>
#include <new>

#include "kernels.hpp"
#include "qsc_internal.hpp"

using namespace qsc;

struct qsc_resident {
    int device = 0;
    Geometry g;
    Sections sec;
    uint64_t mode_counts[8] = {0};
    // host copies of the directory and offsets (query byte accounting)
    std::vector<uint8_t> dir;
    std::vector<uint32_t> gbase;
    std::vector<uint16_t> rel;
    // device memory owned by the resident
    uint8_t *d_blob = nullptr;
    bool borrowed = false;  // d_blob belongs to the caller
    uint32_t *d_tables = nullptr;
    uint32_t *d_model_info = nullptr;
    uint8_t *d_valid = nullptr;
    unsigned long long *d_err = nullptr;
    uint32_t *d_plan = nullptr;  // per-tile selected-pixel counts of the current query
    uint32_t *d_split = nullptr; // byte-rANS split points (n_blocks x P x {state, byte offset})
    uint8_t *d_raw_blk = nullptr;  // byte-rANS: per block, nonzero when it holds a RAW stream
    uint32_t *d_dp_part = nullptr;  // diffraction pattern: n_blocks x P partial sums, then n_blocks scan counts
    float *d_amp = nullptr;         // sqrt of 0..65535, correctly rounded (amplitude frames)
    // polar interaction index (built on request)
    std::vector<uint8_t> h_valid;
    uint16_t *d_ix_perm = nullptr, *d_ix_leaf_valid = nullptr;
    uint32_t *d_ix_packed = nullptr, *d_ix_offset = nullptr, *d_ix_fields = nullptr;
    uint8_t *d_ix_width = nullptr, *d_ix_residual = nullptr;
    uint8_t *d_delta = nullptr;  // added and removed pixels of a mask change (2 x P bytes)
    DevIndex ix{};
    bool has_index = false;
    uint64_t index_bytes = 0;
    void *d_total = nullptr;
    bool total_ready = false;
    uint64_t *d_moments = nullptr;
    uint64_t device_bytes = 0;
    uint32_t n_valid = 0;
    DevResident dev{};
    std::string last_error;
};

namespace {

qsc_status fail(qsc_resident *res, qsc_status st, const std::string &msg) {
    if (res) res->last_error = msg;
    return st;
}

qsc_status hip_fail(qsc_resident *res, hipError_t e, const char *what) {
    return fail(res, e == hipErrorOutOfMemory ? QSC_ERR_OOM : QSC_ERR_HIP,
                std::string(what) + ": " + hipGetErrorString(e));
}

template <typename T>
hipError_t dalloc(qsc_resident *res, T **p, uint64_t bytes) {
    void *q = nullptr;
    hipError_t e = hipMalloc(&q, bytes ? bytes : 1);
    if (e == hipSuccess) {
        *p = static_cast<T *>(q);
        res->device_bytes += bytes;
    }
    return e;
}

void free_all(qsc_resident *res) {
    for (void *p : {res->borrowed ? nullptr : (void *)res->d_blob, (void *)res->d_split, (void *)res->d_raw_blk,
                    (void *)res->d_tables, (void *)res->d_model_info, (void *)res->d_valid, (void *)res->d_err, (void *)res->d_plan, (void *)res->d_dp_part, (void *)res->d_amp,
                    (void *)res->d_ix_perm, (void *)res->d_ix_leaf_valid, (void *)res->d_ix_packed,
                    (void *)res->d_ix_offset, (void *)res->d_ix_fields, (void *)res->d_ix_width,
                    (void *)res->d_ix_residual, (void *)res->d_delta, res->d_total,
                    (void *)res->d_moments})
        if (p) (void)hipFree(p);
}

// Current device must be the resident's; returns false if it cannot be set.
bool on_device(const qsc_resident *res) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return false;
    return cur == res->device || hipSetDevice(res->device) == hipSuccess;
}

qsc_status check_done(qsc_resident *res, hipStream_t st) {
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(res, e, "stream synchronize");
    unsigned long long err = 0;
    e = hipMemcpy(&err, res->d_err, sizeof(err), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(res, e, "error word readback");
    if (!err) return QSC_OK;
    (void)hipMemset(res->d_err, 0, sizeof(err));
    res->total_ready = false;  // a cache built by a failed decode is not kept
    const uint64_t b = (err >> 32) - 1, p = err & 0xFFFFFFFFull;
    return fail(res, QSC_ERR_MALFORMED,
                "malformed stream at block " + std::to_string(b) + ", pixel " + std::to_string(p));
}

qsc_status finish_query(qsc_resident *res, hipError_t launch, hipStream_t st, int wait) {
    if (launch != hipSuccess) return hip_fail(res, launch, "kernel launch");
    return wait ? check_done(res, st) : QSC_OK;
}

// A resident around a validated blob. blob holds at least the sections
// before the payload (host memory); the whole blob is copied to the device
// from host_blob or, when that is null, from dev_blob.
qsc_status build_resident(const Parsed &ps, const uint8_t *blob, const uint8_t *host_blob, const uint8_t *dev_blob,
                          uint64_t nbytes, const uint8_t *host_valid, void *hip_stream,
                          std::unique_ptr<qsc_resident> &res, bool borrow = false) {
    res.reset(new (std::nothrow) qsc_resident);
    if (!res) return QSC_ERR_OOM;
    const Geometry &g = ps.g;
    const Sections &s = ps.sec;
    res->g = g;
    res->sec = s;
    std::copy(ps.mode_counts, ps.mode_counts + 8, res->mode_counts);
    const uint64_t nb = g.n_blocks(), G = g.G();
    res->dir.assign(blob + s.dir, blob + s.dir + 16 * nb);
    res->gbase.resize(nb * G);
    std::memcpy(res->gbase.data(), blob + s.gbase, 4 * nb * G);
    res->rel.resize(nb * G * 32);
    std::memcpy(res->rel.data(), blob + s.rel, 64 * nb * G);
    if (hipGetDevice(&res->device) != hipSuccess) return QSC_ERR_HIP;
    hipStream_t strm = static_cast<hipStream_t>(hip_stream);
    hipError_t e;
    auto bail = [&](hipError_t err, const char *) {
        free_all(res.get());
        return err == hipErrorOutOfMemory ? QSC_ERR_OOM : QSC_ERR_HIP;
    };
    // the whole blob, plus zero padding that the decoders may read ahead into;
    // a borrowed device blob is used in place (its padding is zeroed here)
    if (borrow) {
        res->d_blob = const_cast<uint8_t *>(dev_blob);
        res->borrowed = true;
    } else {
        if ((e = dalloc(res.get(), &res->d_blob, nbytes + kDevicePad)) != hipSuccess) return bail(e, "blob");
        if ((e = hipMemcpy(res->d_blob, host_blob ? host_blob : dev_blob, nbytes,
                           host_blob ? hipMemcpyHostToDevice : hipMemcpyDeviceToDevice)) != hipSuccess)
            return bail(e, "upload");
    }
    if ((e = hipMemset(res->d_blob + nbytes, 0, kDevicePad)) != hipSuccess) return bail(e, "pad");
    // decode tables: the paired layout's 32 model tables; byte-rANS decoders
    // build each block's table in LDS from its 512-byte frequency table
    std::vector<uint32_t> info(kModels, 0);
    if (g.layout == 1) {
        std::vector<uint32_t> tables(kPairTable, 0);
        build_pair_tables(tables.data());
        tables[kPairIdle] = kPairIdle << 16;  // the idle entry: no bits, zero values, itself next
        const PairModels &pm = pair_models();
        for (uint32_t m = 0; m < kModels; m++) info[m] = pm.a0[m] | (pm.in_use[m] << 16);
        if ((e = dalloc(res.get(), &res->d_tables, 4 * tables.size())) != hipSuccess) return bail(e, "tables");
        if ((e = hipMemcpy(res->d_tables, tables.data(), 4 * tables.size(), hipMemcpyHostToDevice)) != hipSuccess)
            return bail(e, "tables upload");
    }
    if ((e = dalloc(res.get(), &res->d_model_info, 4 * kModels)) != hipSuccess) return bail(e, "model info");
    if ((e = hipMemcpy(res->d_model_info, info.data(), 4 * kModels, hipMemcpyHostToDevice)) != hipSuccess)
        return bail(e, "model info upload");
    std::vector<uint8_t> valid(g.P(), 1);
    if (host_valid)
        for (uint32_t p = 0; p < g.P(); p++) valid[p] = host_valid[p] ? 1 : 0;
    for (uint8_t v : valid) res->n_valid += v;
    res->h_valid = valid;
    if ((e = dalloc(res.get(), &res->d_valid, g.P())) != hipSuccess) return bail(e, "valid");
    if ((e = hipMemcpy(res->d_valid, valid.data(), g.P(), hipMemcpyHostToDevice)) != hipSuccess)
        return bail(e, "valid upload");
    if ((e = dalloc(res.get(), &res->d_plan, 4 * kPlanWords)) != hipSuccess) return bail(e, "query plan");
    if ((e = hipMemset(res->d_plan, 0, 4 * kPlanWords)) != hipSuccess) return bail(e, "query plan");
    if ((e = dalloc(res.get(), &res->d_err, 256)) != hipSuccess) return bail(e, "error word");
    if ((e = hipMemset(res->d_err, 0, 256)) != hipSuccess) return bail(e, "error word");
    if ((e = hipStreamSynchronize(strm)) != hipSuccess) return bail(e, "synchronize");

    DevResident &d = res->dev;
    d.payload = res->d_blob + s.payload;
    d.dir = res->d_blob + s.dir;
    d.gbase = reinterpret_cast<const uint32_t *>(res->d_blob + s.gbase);
    d.rel = reinterpret_cast<const uint16_t *>(res->d_blob + s.rel);
    d.tables = res->d_tables;
    d.freq = g.layout == 0 ? reinterpret_cast<const uint16_t *>(res->d_blob + s.table) : nullptr;
    d.model_info = res->d_model_info;
    d.valid = res->d_valid;
    d.calib = g.scaled ? reinterpret_cast<const double *>(res->d_blob + s.calib) : nullptr;
    d.err = res->d_err;
    d.plan = res->d_plan;
    d.S = g.S();
    d.P = g.P();
    d.G = g.G();
    d.det_cols = g.det_cols;
    d.scan_cols = g.scan_cols;
    d.n_blocks = g.n_blocks();
    d.dtype = g.dtype;
    d.layout = g.layout;
    d.split = nullptr;
    d.raw_blk = nullptr;
    // blocks holding RAW streams: queries give those streams waves of their
    // own. A resident without any keeps a null pointer, so its queries read
    // no flag at all.
    if (g.layout == 0) {
        if ((e = dalloc(res.get(), &res->d_raw_blk, g.n_blocks())) != hipSuccess) return bail(e, "RAW block flags");
        if ((e = hipMemsetAsync(res->d_raw_blk, 0, g.n_blocks(), strm)) != hipSuccess) return bail(e, "RAW block flags");
        if ((e = launch_raw_blocks(d, res->d_raw_blk, strm)) != hipSuccess) return bail(e, "RAW block flags");
        std::vector<uint8_t> flags(g.n_blocks());
        if ((e = hipMemcpyAsync(flags.data(), res->d_raw_blk, flags.size(), hipMemcpyDeviceToHost, strm)) != hipSuccess ||
            (e = hipStreamSynchronize(strm)) != hipSuccess)
            return bail(e, "RAW block flags");
        for (uint8_t f : flags)
            if (f) d.raw_blk = res->d_raw_blk;
    }
    // uint16 blocks whose tables give the escape symbol (255) at least a
    // quarter of the 4096 slots: when most blocks are such, sums and moments
    // take the staged decode, which reads each stream in 32-byte chunks
    d.esc_heavy = 0;
    if (g.layout == 0 && g.dtype == 2) {
        std::vector<uint16_t> fq(256ull * g.n_blocks());
        if ((e = hipMemcpy(fq.data(), d.freq, 2 * fq.size(), hipMemcpyDeviceToHost)) != hipSuccess)
            return bail(e, "frequency tables");
        uint64_t heavy = 0;
        for (uint32_t b = 0; b < g.n_blocks(); b++) heavy += fq[256ull * b + 255] >= 1024;
        d.esc_heavy = 2 * heavy >= g.n_blocks() ? 1u : 0u;
    }
    // split points of the byte-rANS streams of complete blocks: one decode of
    // their first halves, so that latency-bound queries decode both halves of
    // a stream side by side
    if (g.layout == 0 && g.S() >= kBlock) {
        if ((e = dalloc(res.get(), &res->d_split, 8ull * g.n_blocks() * g.P())) != hipSuccess) return bail(e, "split points");
        if ((e = launch_split_build(d, res->d_split, strm)) != hipSuccess) return bail(e, "split points");
        if ((e = hipStreamSynchronize(strm)) != hipSuccess) return bail(e, "split points");
        // streams are judged by the queries that decode them: whatever the
        // build's decode flagged is not carried into the first query
        if ((e = hipMemset(res->d_err, 0, sizeof(unsigned long long))) != hipSuccess) return bail(e, "error word");
        d.split = res->d_split;
    }
    return QSC_OK;
}

// Moment partials of qsc_com_noalloc: M0, Mr, Mc per scan, u64, for up to
// kNoAllocScans scans (24 MiB). Every GPU the library runs on holds one copy
// until the process ends. Host code never passes the array's name to a kernel:
// that is a host-side stand-in; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr uint64_t kNoAllocScans = 1ull << 20;
static __device__ __align__(256) uint64_t scratch[3 * kNoAllocScans];

constexpr int kMaxDevices = 64;

// Device address of this device's scratch (the current device must be it).
hipError_t scratch_address(int device, uint64_t **out) {
    static std::mutex mu;
    static uint64_t *ptrs[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[device] = static_cast<uint64_t *>(p);
    }
    *out = ptrs[device];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *qsc_abi(void) { return "qsc-byte-rans-v1;qsc-paired-v1"; }

const char *qsc_status_string(qsc_status s) {
    switch (s) {
    case QSC_OK: return "ok";
    case QSC_ERR_INVALID_ARG: return "invalid argument";
    case QSC_ERR_MALFORMED: return "malformed container or stream";
    case QSC_ERR_UNSUPPORTED: return "unsupported ABI or format version";
    case QSC_ERR_OOM: return "out of memory";
    case QSC_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

qsc_status qsc_resident_create(const void *host_blob, uint64_t nbytes, const uint8_t *host_valid, void *hip_stream,
                               qsc_resident **out) {
    if (!host_blob || !out) return QSC_ERR_INVALID_ARG;
    *out = nullptr;
    Parsed ps;
    std::string msg;
    const uint8_t *blob = static_cast<const uint8_t *>(host_blob);
    qsc_status st = parse_and_validate(blob, nbytes, &ps, &msg);
    if (st != QSC_OK) return st;  // no resident exists to carry the message
    std::unique_ptr<qsc_resident> res;
    if ((st = build_resident(ps, blob, blob, nullptr, nbytes, host_valid, hip_stream, res)) != QSC_OK) return st;
    *out = res.release();
    return QSC_OK;
}

static qsc_status create_from_device(const void *d_blob, uint64_t nbytes, const uint8_t *host_valid, void *hip_stream,
                              qsc_resident **out, bool borrow) {
    const uint8_t *dev = static_cast<const uint8_t *>(d_blob);
    if (nbytes < kHeaderBytes) return QSC_ERR_MALFORMED;
    // the header fixes the size of the sections before the payload
    uint8_t hdr[kHeaderBytes];
    if (hipMemcpy(hdr, dev, kHeaderBytes, hipMemcpyDeviceToHost) != hipSuccess) return QSC_ERR_HIP;
    Geometry g;
    g.layout = ld32(hdr + 44);
    g.scan_rows = ld32(hdr + 48);
    g.scan_cols = ld32(hdr + 52);
    g.det_rows = ld32(hdr + 56);
    g.det_cols = ld32(hdr + 60);
    g.dtype = ld32(hdr + 64);
    g.scaled = ld32(hdr + 76) & 1;
    if (!check_geometry(g).empty()) return QSC_ERR_MALFORMED;
    const Sections want = layout_sections(g, ld64(hdr + 120));
    if (want.payload != ld64(hdr + 112) || want.total != nbytes) return QSC_ERR_MALFORMED;
    std::vector<uint8_t> pre(want.payload), cal(g.scaled ? 16ull * g.n_blocks() : 0);
    if (hipMemcpy(pre.data(), dev, pre.size(), hipMemcpyDeviceToHost) != hipSuccess) return QSC_ERR_HIP;
    if (g.scaled && hipMemcpy(cal.data(), dev + want.calib, cal.size(), hipMemcpyDeviceToHost) != hipSuccess)
        return QSC_ERR_HIP;
    Parsed ps;
    std::string msg;
    qsc_status st = parse_and_validate(pre.data(), nbytes, &ps, &msg, false, g.scaled ? cal.data() : nullptr);
    if (st != QSC_OK) return st;
    std::unique_ptr<qsc_resident> res;
    if ((st = build_resident(ps, pre.data(), nullptr, dev, nbytes, host_valid, hip_stream, res, borrow)) != QSC_OK)
        return st;
    // stream headers on the device: reserved bits, modes, RANS only with a usable table
    const uint32_t nb = g.n_blocks();
    std::vector<uint8_t> usable(nb, 1);
    if (g.layout == 0)
        for (uint32_t b = 0; b < nb; b++) {
            uint32_t nz = 0, full = 0;
            for (int i = 0; i < 256; i++) {
                const uint32_t f = ld16(pre.data() + ps.sec.table + 512ull * b + 2 * i);
                nz += f != 0;
                full |= f == kRansM;
            }
            usable[b] = nz > 0 && !full;
        }
    uint8_t *d_usable = nullptr;
    unsigned long long *d_chk = nullptr;  // 8 mode counts, then the first bad stream
    hipError_t e = hipMalloc(&d_usable, nb);
    if (e == hipSuccess) e = hipMalloc(&d_chk, 9 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemcpy(d_usable, usable.data(), nb, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(d_chk, 0, 8 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemset(d_chk + 8, 0xFF, sizeof(unsigned long long));
    hipStream_t strm = static_cast<hipStream_t>(hip_stream);
    if (e == hipSuccess) e = launch_check_headers(res->dev, d_usable, d_chk, d_chk + 8, strm);
    unsigned long long chk[9] = {0};
    if (e == hipSuccess) e = hipStreamSynchronize(strm);
    if (e == hipSuccess) e = hipMemcpy(chk, d_chk, sizeof(chk), hipMemcpyDeviceToHost);
    if (d_usable) (void)hipFree(d_usable);
    if (d_chk) (void)hipFree(d_chk);
    if (e != hipSuccess) {
        free_all(res.get());
        return e == hipErrorOutOfMemory ? QSC_ERR_OOM : QSC_ERR_HIP;
    }
    if (chk[8] != ~0ull) {
        free_all(res.get());
        return QSC_ERR_MALFORMED;
    }
    std::copy(chk, chk + 8, res->mode_counts);
    *out = res.release();
    return QSC_OK;
}

qsc_status qsc_resident_create_device(const void *d_blob, uint64_t nbytes, const uint8_t *host_valid,
                                      void *hip_stream, qsc_resident **out) {
    if (!d_blob || !out) return QSC_ERR_INVALID_ARG;
    *out = nullptr;
    return create_from_device(d_blob, nbytes, host_valid, hip_stream, out, false);
}

qsc_status qsc_resident_create_device_borrow(void *d_blob, uint64_t nbytes, uint64_t capacity,
                                             const uint8_t *host_valid, void *hip_stream, qsc_resident **out) {
    if (!d_blob || !out) return QSC_ERR_INVALID_ARG;
    *out = nullptr;
    if (capacity < nbytes || capacity - nbytes < kDevicePad) return QSC_ERR_INVALID_ARG;
    return create_from_device(d_blob, nbytes, host_valid, hip_stream, out, true);
}

qsc_status qsc_resident_destroy(qsc_resident *res) {
    if (!res) return QSC_ERR_INVALID_ARG;
    on_device(res);
    (void)hipDeviceSynchronize();
    free_all(res);
    delete res;
    return QSC_OK;
}

qsc_status qsc_resident_info(const qsc_resident *res, qsc_info *info) {
    if (!res || !info) return QSC_ERR_INVALID_ARG;
    const Geometry &g = res->g;
    info->geom = qsc_geometry{g.scan_rows, g.scan_cols, g.det_rows, g.det_cols, g.dtype, g.layout, g.scaled};
    info->n_blocks = g.n_blocks();
    info->sum_bits = g.sum_bits();
    info->resident_bytes = res->device_bytes;
    info->payload_bytes = res->sec.payload_bytes;
    std::copy(res->mode_counts, res->mode_counts + 8, info->mode_counts);
    info->index_bytes = res->index_bytes;
    return QSC_OK;
}

qsc_status qsc_masked_sum(qsc_resident *res, const uint8_t *d_mask, uint32_t block_stride, void *d_out,
                          void *hip_stream, int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!d_mask || !d_out || block_stride < 1) return fail(res, QSC_ERR_INVALID_ARG, "masked_sum: bad argument");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int out64 = res->g.sum_bits() == 64;
    const hipError_t e =
        res->has_index ? launch_indexed_sum(res->dev, res->ix, d_mask, block_stride, d_out, out64, res->d_ix_fields,
                                            res->d_ix_residual, st)
                       : launch_query(res->dev, d_mask, 0, block_stride, Op::Sum, d_out, out64, 0, nullptr,
                                      res->g.S(), st);
    return finish_query(res, e, st, wait);
}

qsc_status qsc_masked_sum_delta(qsc_resident *res, const uint8_t *d_prev_mask, const void *d_prev_out,
                                const uint8_t *d_mask, uint32_t block_stride, void *d_out, void *hip_stream,
                                int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!d_prev_mask || !d_prev_out || !d_mask || !d_out || block_stride < 1)
        return fail(res, QSC_ERR_INVALID_ARG, "masked_sum_delta: bad argument");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int out64 = res->g.sum_bits() == 64;
    const uint32_t P = res->g.P();
    hipError_t e = hipSuccess;
    if (!res->d_delta && (e = dalloc(res, &res->d_delta, 2ull * P)) != hipSuccess)
        return hip_fail(res, e, "mask delta scratch");
    uint8_t *added = res->d_delta, *removed = res->d_delta + P;
    e = launch_mask_delta(d_prev_mask, d_mask, P, added, removed, st);
    // out = prev_out + the added pixels' sums - the removed pixels' sums, one launch
    if (e == hipSuccess)
        e = launch_query(res->dev, added, 0, block_stride, Op::Sum, d_out, out64, 0, d_prev_out, res->g.S(), st,
                         removed);
    return finish_query(res, e, st, wait);
}

qsc_status qsc_dense_df(qsc_resident *res, const uint8_t *d_mask, void *d_out, void *hip_stream, int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!d_mask || !d_out) return fail(res, QSC_ERR_INVALID_ARG, "dense_df: bad argument");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int out64 = res->g.sum_bits() == 64;
    const uint64_t width = out64 ? 8 : 4;
    hipError_t e = hipSuccess;
    if (!res->d_total && (e = dalloc(res, &res->d_total, width * res->g.S())) != hipSuccess)
        return hip_fail(res, e, "total cache");
    if (!res->total_ready) {
        // cold: full-detector total over the valid pixels, decoded once and kept
        e = launch_query(res->dev, nullptr, 0, 1, Op::Sum, res->d_total, out64, 0, nullptr, res->g.S(), st);
        if (e != hipSuccess) return hip_fail(res, e, "total cache build");
        res->total_ready = true;
    }
    // warm: out = total - sum over valid & ~mask
    e = launch_query(res->dev, d_mask, 1, 1, Op::Sum, d_out, out64, 1, res->d_total, res->g.S(), st);
    return finish_query(res, e, st, wait);
}

qsc_status qsc_com(qsc_resident *res, const uint8_t *d_mask, float *d_row, float *d_col, void *hip_stream, int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!d_row || !d_col) return fail(res, QSC_ERR_INVALID_ARG, "com: bad argument");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipSuccess;
    if (!res->d_moments && (e = dalloc(res, &res->d_moments, 3 * 8 * res->g.S())) != hipSuccess)
        return hip_fail(res, e, "moment buffer");
    e = launch_query(res->dev, d_mask, 0, 1, Op::Moments, res->d_moments, 1, 0, nullptr, 3 * res->g.S(), st);
    if (e == hipSuccess) e = launch_com_finalize(res->d_moments, res->g.S(), d_row, d_col, st);
    return finish_query(res, e, st, wait);
}

qsc_status qsc_com_noalloc(qsc_resident *res, const uint8_t *d_mask, float *d_row, float *d_col, void *hip_stream,
                           int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!d_row || !d_col) return fail(res, QSC_ERR_INVALID_ARG, "com_noalloc: bad argument");
    if (res->g.S() > kNoAllocScans)
        return fail(res, QSC_ERR_INVALID_ARG, "com_noalloc: more than 1048576 scans (its static moment buffer)");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    uint64_t *m = nullptr;
    hipError_t e = scratch_address(res->device, &m);
    if (e != hipSuccess) return hip_fail(res, e, "static moment buffer address");
    // the init kernel zeroes the 3 x S moments this call uses before the decode adds into them
    e = launch_query(res->dev, d_mask, 0, 1, Op::Moments, m, 1, 0, nullptr, 3 * res->g.S(), st);
    if (e == hipSuccess) e = launch_com_finalize(m, res->g.S(), d_row, d_col, st);
    return finish_query(res, e, st, wait);
}

qsc_status qsc_sum_dp(qsc_resident *res, const uint8_t *d_scan_mask, uint32_t block_stride, uint64_t *d_sum,
                      float *d_mean, void *hip_stream, int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!d_sum || block_stride < 1) return fail(res, QSC_ERR_INVALID_ARG, "sum_dp: bad argument");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const uint64_t nb = res->g.n_blocks(), P = res->g.P();
    hipError_t e = hipSuccess;
    if (!res->d_dp_part && (e = dalloc(res, &res->d_dp_part, 4 * (nb * P + nb))) != hipSuccess)
        return hip_fail(res, e, "diffraction-pattern scratch");
    e = launch_dp(res->dev, d_scan_mask, block_stride, res->d_dp_part, res->d_dp_part + nb * P, d_sum, d_mean, st);
    return finish_query(res, e, st, wait);
}

qsc_status qsc_decode_region(qsc_resident *res, uint32_t r0, uint32_t r1, uint32_t c0, uint32_t c1, int out_kind,
                             void *d_out, void *hip_stream, int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    const Geometry &g = res->g;
    if (!d_out || r0 >= r1 || c0 >= c1 || r1 > g.scan_rows || c1 > g.scan_cols || out_kind < 0 || out_kind > 1 ||
        (out_kind == 1 && !g.scaled))
        return fail(res, QSC_ERR_INVALID_ARG, "decode_region: bad rectangle or output kind");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    // blocks holding a scan of the rectangle
    std::vector<uint32_t> blocks;
    for (uint32_t r = r0; r < r1; r++) {
        const uint64_t sa = uint64_t(r) * g.scan_cols + c0, sb = uint64_t(r) * g.scan_cols + c1 - 1;
        for (uint64_t b = sa / kBlock; b <= sb / kBlock; b++)
            if (blocks.empty() || blocks.back() < b) blocks.push_back(uint32_t(b));
    }
    // invalid pixels read 0: the decode skips them, so clear the output first
    hipError_t e = hipSuccess;
    if (res->n_valid < g.P()) {
        const uint64_t elem = out_kind == 1 ? 4 : g.dtype;
        e = launch_zero_bytes(d_out, uint64_t(r1 - r0) * (c1 - c0) * g.P() * elem, st);
    }
    // the touched-block list travels as kernel launches of up to 64 blocks each (no device staging buffer)
    const RegionArgs ra{r0, r1, c0, c1, out_kind, d_out, 0, 0, nullptr};
    for (size_t i = 0; i < blocks.size() && e == hipSuccess; i += 64) {
        RegionBlocks rb{};
        rb.n = uint32_t(std::min<size_t>(64, blocks.size() - i));
        for (uint32_t k = 0; k < rb.n; k++) rb.b[k] = blocks[i + k];
        e = launch_region(res->dev, rb, ra, st);
    }
    return finish_query(res, e, st, wait);
}

qsc_status qsc_decode_blocks(qsc_resident *res, uint32_t first_block, uint32_t n_blocks, int out_kind, void *d_out,
                             void *hip_stream, int wait) {
    if (!res) return QSC_ERR_INVALID_ARG;
    const Geometry &g = res->g;
    if (!d_out || n_blocks < 1 || first_block >= g.n_blocks() || n_blocks > g.n_blocks() - first_block ||
        out_kind < 0 || out_kind > 2 || (out_kind == 1 && !g.scaled))
        return fail(res, QSC_ERR_INVALID_ARG, "decode_blocks: bad block range or output kind");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const uint64_t s0 = uint64_t(first_block) * kBlock;
    const uint64_t s1 = std::min<uint64_t>(g.S(), uint64_t(first_block + n_blocks) * kBlock);
    hipError_t e = hipSuccess;
    if (res->n_valid < g.P()) {  // invalid pixels read 0
        const uint64_t elem = out_kind ? 4 : g.dtype;
        e = launch_zero_bytes(d_out, (s1 - s0) * g.P() * elem, st);
    }
    if (out_kind == 2 && !res->d_amp) {
        // the host's IEEE square root, rounded once to float32, for every count
        std::vector<float> amp(65536);
        for (uint32_t c = 0; c < 65536; c++) amp[c] = std::sqrt(float(c));
        if ((e = dalloc(res, &res->d_amp, 4 * amp.size())) != hipSuccess) return hip_fail(res, e, "amplitude table");
        if ((e = hipMemcpy(res->d_amp, amp.data(), 4 * amp.size(), hipMemcpyHostToDevice)) != hipSuccess)
            return hip_fail(res, e, "amplitude table upload");
    }
    const RegionArgs ra{0, 0, 0, 0, out_kind, d_out, 1, s0, res->d_amp};
    for (uint32_t i = 0; i < n_blocks && e == hipSuccess; i += 64) {
        RegionBlocks rb{};
        rb.n = std::min<uint32_t>(64, n_blocks - i);
        for (uint32_t k = 0; k < rb.n; k++) rb.b[k] = first_block + i + k;
        e = launch_region(res->dev, rb, ra, st);
    }
    return finish_query(res, e, st, wait);
}

// ---------------------------------------------------------------- block feed
struct qsc_feed {
    qsc_resident *res = nullptr;
    hipStream_t prod = nullptr;  // the feed's own stream (default priority)
    hipStream_t cons = nullptr;  // the caller's stream
    std::vector<void *> bufs;
    std::vector<hipEvent_t> ready, freed;  // per buffer: decode done (producer), consumer done with it
    uint32_t first = 0, n_blocks = 0, per = 1, depth = 1, n_items = 0, issued = 0, consumed = 0;
    int kind = 0;
    bool holding = false;
};

static void feed_free(qsc_feed *f) {
    if (f->prod) (void)hipStreamSynchronize(f->prod);
    for (hipEvent_t e : f->ready)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : f->freed)
        if (e) (void)hipEventDestroy(e);
    if (f->prod) (void)hipStreamDestroy(f->prod);
    delete f;
}

// Decodes item f->issued into buffer issued % depth on the feed's stream, once
// the consumer has released that buffer's previous item.
static qsc_status feed_issue(qsc_feed *f) {
    const uint32_t j = f->issued, i = j % f->depth;
    if (j >= f->depth && hipStreamWaitEvent(f->prod, f->freed[i], 0) != hipSuccess)
        return fail(f->res, QSC_ERR_HIP, "feed: wait for a released buffer");
    const uint32_t b0 = f->first + j * f->per;
    const uint32_t nb = std::min(f->per, f->first + f->n_blocks - b0);
    const qsc_status st = qsc_decode_blocks(f->res, b0, nb, f->kind, f->bufs[i], f->prod, 0);
    if (st != QSC_OK) return st;
    if (hipEventRecord(f->ready[i], f->prod) != hipSuccess) return fail(f->res, QSC_ERR_HIP, "feed: record a decode");
    f->issued++;
    return QSC_OK;
}

qsc_status qsc_feed_create(qsc_resident *res, uint32_t first_block, uint32_t n_blocks, uint32_t blocks_per_item,
                           int out_kind, uint32_t depth, void *const *d_bufs, uint64_t buf_bytes,
                           void *consumer_stream, qsc_feed **out) {
    if (!res || !out) return QSC_ERR_INVALID_ARG;
    *out = nullptr;
    const Geometry &g = res->g;
    const uint64_t elem = out_kind ? 4 : g.dtype;
    if (n_blocks < 1 || first_block >= g.n_blocks() || n_blocks > g.n_blocks() - first_block ||
        blocks_per_item < 1 || depth < 1 || depth > 64 || out_kind < 0 || out_kind > 2 || (out_kind == 1 && !g.scaled) ||
        !d_bufs || buf_bytes < uint64_t(blocks_per_item) * kBlock * g.P() * elem)
        return fail(res, QSC_ERR_INVALID_ARG, "feed_create: bad block range, item size, depth, kind or buffers");
    for (uint32_t i = 0; i < depth; i++)
        if (!d_bufs[i]) return fail(res, QSC_ERR_INVALID_ARG, "feed_create: null buffer");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    qsc_feed *f = new (std::nothrow) qsc_feed;
    if (!f) return QSC_ERR_OOM;
    f->res = res;
    f->cons = static_cast<hipStream_t>(consumer_stream);
    f->bufs.assign(d_bufs, d_bufs + depth);
    f->first = first_block;
    f->n_blocks = n_blocks;
    f->per = blocks_per_item;
    f->depth = depth;
    f->n_items = (n_blocks + blocks_per_item - 1) / blocks_per_item;
    f->kind = out_kind;
    f->ready.assign(depth, nullptr);
    f->freed.assign(depth, nullptr);
    hipError_t e = hipStreamCreateWithFlags(&f->prod, hipStreamNonBlocking);
    for (uint32_t i = 0; i < depth && e == hipSuccess; i++) {
        e = hipEventCreateWithFlags(&f->ready[i], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&f->freed[i], hipEventDisableTiming);
    }
    // the buffers may still be in use by work the caller queued before
    hipEvent_t start = nullptr;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&start, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(start, f->cons);
    if (e == hipSuccess) e = hipStreamWaitEvent(f->prod, start, 0);
    if (start) (void)hipEventDestroy(start);
    if (e != hipSuccess) {
        feed_free(f);
        return hip_fail(res, e, "feed: stream and events");
    }
    qsc_status st = QSC_OK;
    while (st == QSC_OK && f->issued < std::min(f->depth, f->n_items)) st = feed_issue(f);
    if (st != QSC_OK) {
        feed_free(f);
        return st;
    }
    *out = f;
    return QSC_OK;
}

qsc_status qsc_feed_next(qsc_feed *f, uint32_t *buf_index, uint64_t *first_scan, uint32_t *n_scans) {
    if (!f || !buf_index || !first_scan || !n_scans) return QSC_ERR_INVALID_ARG;
    if (f->holding) return fail(f->res, QSC_ERR_INVALID_ARG, "feed_next: release the current item first");
    *buf_index = 0;
    *first_scan = 0;
    *n_scans = 0;
    if (f->consumed == f->n_items) return QSC_OK;
    const uint32_t i = f->consumed % f->depth;
    if (hipStreamWaitEvent(f->cons, f->ready[i], 0) != hipSuccess)
        return fail(f->res, QSC_ERR_HIP, "feed_next: wait for a decode");
    const uint64_t b0 = f->first + uint64_t(f->consumed) * f->per;
    const uint64_t s0 = b0 * kBlock;
    const uint64_t s1 = std::min<uint64_t>(f->res->g.S(), std::min<uint64_t>(b0 + f->per, f->first + f->n_blocks) * kBlock);
    *buf_index = i;
    *first_scan = s0;
    *n_scans = uint32_t(s1 - s0);
    f->holding = true;
    return QSC_OK;
}

qsc_status qsc_feed_release(qsc_feed *f) {
    if (!f) return QSC_ERR_INVALID_ARG;
    if (!f->holding) return fail(f->res, QSC_ERR_INVALID_ARG, "feed_release: no item is held");
    const uint32_t i = f->consumed % f->depth;
    if (hipEventRecord(f->freed[i], f->cons) != hipSuccess) return fail(f->res, QSC_ERR_HIP, "feed_release");
    f->consumed++;
    f->holding = false;
    return f->issued < f->n_items ? feed_issue(f) : QSC_OK;
}

qsc_status qsc_feed_destroy(qsc_feed *f) {
    if (!f) return QSC_ERR_INVALID_ARG;
    qsc_resident *res = f->res;
    const qsc_status st = on_device(res) ? check_done(res, f->prod) : QSC_ERR_HIP;
    feed_free(f);
    return st;
}

static void drop_index(qsc_resident *res) {
    for (void **p : {(void **)&res->d_ix_perm, (void **)&res->d_ix_leaf_valid, (void **)&res->d_ix_packed,
                     (void **)&res->d_ix_offset, (void **)&res->d_ix_fields, (void **)&res->d_ix_width,
                     (void **)&res->d_ix_residual})
        if (*p) {
            (void)hipFree(*p);
            *p = nullptr;
        }
    res->device_bytes -= res->index_bytes;
    res->index_bytes = 0;
    res->has_index = false;
    res->ix = DevIndex{};
}

qsc_status qsc_index_build(qsc_resident *res, int32_t center_row, int32_t center_col, void *hip_stream) {
    if (!res) return QSC_ERR_INVALID_ARG;
    const Geometry &g = res->g;
    const uint32_t P = g.P();
    if (P > 65535) return fail(res, QSC_ERR_UNSUPPORTED, "index_build: detectors above 65,535 pixels");
    if (center_row < 0 || center_col < 0 || uint32_t(center_row) >= g.det_rows || uint32_t(center_col) >= g.det_cols)
        return fail(res, QSC_ERR_INVALID_ARG, "index_build: center outside the detector");
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    drop_index(res);
    // polar order: squared distance, then angle; the sort is stable on pixel index for ties
    std::vector<std::tuple<int64_t, double, uint32_t>> key(P);
    for (uint32_t p = 0; p < P; p++) {
        const int64_t dr = int64_t(p / g.det_cols) - center_row, dc = int64_t(p % g.det_cols) - center_col;
        key[p] = {dr * dr + dc * dc, std::atan2(double(dr), double(dc)), p};
    }
    std::sort(key.begin(), key.end());
    const uint32_t n_leaves = (P + kLeaf - 1) / kLeaf, n_roots = (n_leaves + kRoot - 1) / kRoot;
    const uint32_t n_fields = n_leaves + n_roots, nb = g.n_blocks();
    std::vector<uint16_t> perm(P), leaf_valid(n_leaves, 0);
    for (uint32_t i = 0; i < P; i++) {
        perm[i] = uint16_t(std::get<2>(key[i]));
        leaf_valid[i / kLeaf] += res->h_valid[perm[i]];
    }
    const uint64_t bytes0 = res->device_bytes;
    auto bail = [&](qsc_status s, hipError_t e, const char *what) {
        drop_index(res);
        res->device_bytes = bytes0;
        return e != hipSuccess ? hip_fail(res, e, what) : fail(res, s, what);
    };
    hipError_t e;
    if ((e = dalloc(res, &res->d_ix_perm, 2ull * P)) != hipSuccess ||
        (e = dalloc(res, &res->d_ix_leaf_valid, 2ull * n_leaves)) != hipSuccess ||
        (e = dalloc(res, &res->d_ix_width, uint64_t(nb) * n_fields)) != hipSuccess ||
        (e = dalloc(res, &res->d_ix_offset, 4ull * nb * n_fields)) != hipSuccess ||
        (e = dalloc(res, &res->d_ix_fields, 4ull * (n_fields + 1) + n_leaves)) != hipSuccess ||
        (e = dalloc(res, &res->d_ix_residual, P)) != hipSuccess)
        return bail(QSC_OK, e, "index buffers");
    if ((e = hipMemcpy(res->d_ix_perm, perm.data(), 2ull * P, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(res->d_ix_leaf_valid, leaf_valid.data(), 2ull * n_leaves, hipMemcpyHostToDevice)) != hipSuccess)
        return bail(QSC_OK, e, "index upload");
    // exact field rows of every block (a temporary buffer), then their widths
    uint32_t *rows = nullptr;
    const uint64_t row_bytes = 4ull * nb * n_fields * kBlock;
    if ((e = hipMalloc(&rows, row_bytes)) != hipSuccess) return bail(QSC_OK, e, "index rows");
    e = hipMemsetAsync(rows, 0, row_bytes, st);
    if (e == hipSuccess) e = launch_index_leaves(res->dev, res->d_ix_perm, n_leaves, n_roots, rows, st);
    if (e == hipSuccess) e = launch_index_widths(nb, n_leaves, n_roots, rows, res->d_ix_width, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    unsigned long long err = 0;
    if (e == hipSuccess) e = hipMemcpy(&err, res->dev.err, sizeof(err), hipMemcpyDeviceToHost);
    if (e != hipSuccess || err) {
        (void)hipFree(rows);
        if (e != hipSuccess) return bail(QSC_OK, e, "index build");
        (void)check_done(res, st);  // reports the malformed stream and clears the error word
        const std::string why = res->last_error;
        drop_index(res);
        res->device_bytes = bytes0;
        return fail(res, QSC_ERR_MALFORMED, ("index_build: " + why).c_str());
    }
    std::vector<uint8_t> width(uint64_t(nb) * n_fields);
    std::vector<uint32_t> offset(width.size());
    if ((e = hipMemcpy(width.data(), res->d_ix_width, width.size(), hipMemcpyDeviceToHost)) != hipSuccess) {
        (void)hipFree(rows);
        return bail(QSC_OK, e, "index widths");
    }
    uint64_t dw = 0;
    for (size_t i = 0; i < width.size(); i++) {
        offset[i] = uint32_t(dw);
        dw += (uint64_t(kBlock) * width[i] + 31) / 32;
        if (dw >= (1ull << 32) - 4) {
            (void)hipFree(rows);
            return bail(QSC_ERR_UNSUPPORTED, hipSuccess, "index_build: index above 16 GB");
        }
    }
    // two spare dwords: a reader fetches the dword after a value's first
    if ((e = dalloc(res, &res->d_ix_packed, 4 * (dw + 2))) != hipSuccess ||
        (e = hipMemcpy(res->d_ix_offset, offset.data(), 4 * offset.size(), hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemsetAsync(res->d_ix_packed, 0, 4 * (dw + 2), st)) != hipSuccess) {
        (void)hipFree(rows);
        return bail(QSC_OK, e, "index pack buffers");
    }
    e = launch_index_pack(nb, n_fields, rows, res->d_ix_offset, res->d_ix_width, res->d_ix_packed, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipFree(rows);
    if (e != hipSuccess) return bail(QSC_OK, e, "index pack");
    res->ix = DevIndex{res->d_ix_perm, res->d_ix_leaf_valid, res->d_ix_packed, res->d_ix_offset, res->d_ix_width,
                       n_leaves, n_roots};
    res->index_bytes = res->device_bytes - bytes0;
    res->has_index = true;
    return QSC_OK;
}

qsc_status qsc_finish(qsc_resident *res, void *hip_stream) {
    if (!res) return QSC_ERR_INVALID_ARG;
    if (!on_device(res)) return fail(res, QSC_ERR_HIP, "cannot select the resident's device");
    return check_done(res, static_cast<hipStream_t>(hip_stream));
}

const char *qsc_last_error(const qsc_resident *res) { return res ? res->last_error.c_str() : "no resident"; }

qsc_status qsc_query_bytes(const qsc_resident *res, const uint8_t *host_mask, uint32_t block_stride, uint64_t *bytes,
                           uint64_t *counts) {
    if (!res || !host_mask || !bytes || !counts || block_stride < 1) return QSC_ERR_INVALID_ARG;
    const Geometry &g = res->g;
    const uint32_t P = g.P(), G = g.G(), nb = g.n_blocks();
    std::vector<uint32_t> sel;
    std::vector<uint8_t> valid(P, 1);
    // the resident keeps validity on the device only; fetch it once
    if (hipMemcpy(valid.data(), res->d_valid, P, hipMemcpyDeviceToHost) != hipSuccess) return QSC_ERR_HIP;
    for (uint32_t p = 0; p < P; p++)
        if (host_mask[p] && valid[p]) sel.push_back(p);
    uint64_t by = 0, cn = 0;
    for (uint32_t b = 0; b < nb; b += block_stride) {
        const uint8_t *d = res->dir.data() + 16ull * b;
        const uint32_t n = ld32(d + 8), nbytes = ld32(d + 12);
        by += 16 + (g.layout == 0 ? 512 : 0);  // directory entry and frequency table
        uint32_t last_group = 0xFFFFFFFFu;
        for (uint32_t p : sel) {
            const uint64_t gi = uint64_t(b) * G + (p >> 5);
            const uint64_t st = res->gbase[gi] + res->rel[gi * 32 + (p & 31)];
            uint64_t en;
            if (p + 1 < P) {
                const uint64_t gj = uint64_t(b) * G + ((p + 1) >> 5);
                en = res->gbase[gj] + res->rel[gj * 32 + ((p + 1) & 31)];
            } else {
                en = nbytes;
            }
            by += en - st + 2;  // stream bytes and its relative offset
            if ((p >> 5) != last_group) {
                by += 4;  // group base
                last_group = p >> 5;
            }
        }
        cn += uint64_t(n) * sel.size();
    }
    if (g.layout == 1) by += 2ull * kModels * 256;
    *bytes = by;
    *counts = cn;
    return QSC_OK;
}

}  // extern "C"
