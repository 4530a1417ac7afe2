// Host encoder for the resident container (FORMAT.md v1), multithreaded over
// 512-scan blocks.
//
// The paired-resident page ("Operation pipeline" items 1-2) feeds native
// counts as complete 512-scan blocks and codes every detector pixel's stream:
// paired counts under one of 32 Poisson pair models with 1024 tANS states, or
// an exact empty/constant/sparse/raw form; sparse stays preferred unless the
// paired stream saves at least two bytes ("Contract"). The byte-rANS layout is
// the default resident the same page names next to it. The scaled-uint16 page
// calibrates each float32 region in double precision, rounds codes to nearest
// with ties to even, and then ANS-codes the codes.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <thread>

#include "qsc_internal.hpp"

using namespace qsc;

namespace {

struct EncodedBlock {
    std::vector<uint8_t> payload;
    std::vector<uint32_t> gbase;
    std::vector<uint16_t> rel;
    uint16_t freq[256] = {0};
    uint32_t n_scans = 0;
    double scale = 0.0, offset = 0.0;
    qsc_status status = QSC_OK;
};

inline void emit16(std::vector<uint8_t> &o, uint32_t v) {
    o.push_back(uint8_t(v));
    o.push_back(uint8_t(v >> 8));
}

// ------------------------------------------------------------ byte-rANS

// FORMAT 2.2: frequencies from the histogram of the non-constant streams.
void quantize_freqs(const uint64_t *hist, uint16_t *f) {
    uint64_t total = 0;
    for (int s = 0; s < 256; s++) total += hist[s];
    std::fill(f, f + 256, uint16_t(0));
    if (!total) return;
    int64_t sum = 0;
    for (int s = 0; s < 256; s++)
        if (hist[s]) {
            f[s] = uint16_t(std::max<uint64_t>(1, hist[s] * kRansM / total));
            sum += f[s];
        }
    while (sum > int64_t(kRansM)) {
        int pick = -1;
        for (int s = 0; s < 256; s++)
            if (f[s] > 1 && (pick < 0 || f[s] > f[pick])) pick = s;
        f[pick]--;
        sum--;
    }
    if (sum < int64_t(kRansM)) {
        int pick = int(std::max_element(hist, hist + 256) - hist); // first maximum
        f[pick] = uint16_t(f[pick] + (kRansM - sum));
    }
}

struct RansCoder {
    uint32_t f[256], c[256];
    bool usable = false;
    explicit RansCoder(const uint16_t *freq) {
        uint32_t acc = 0, nz = 0;
        bool full = false;
        for (int s = 0; s < 256; s++) {
            f[s] = freq[s];
            c[s] = acc;
            acc += f[s];
            nz += f[s] != 0;
            full |= f[s] == kRansM;
        }
        usable = nz > 0 && !full;
    }
    // Words after the header of a RANS stream, in stream order (FORMAT 2.3-2.4).
    void encode(const uint32_t *v, uint32_t n, bool wide, std::vector<uint16_t> &stack,
                std::vector<uint16_t> &out) const {
        stack.clear();
        uint32_t x = kRansL;
        for (int32_t j = int32_t(n) - 1; j >= 0; j--) {
            uint32_t s = v[j];
            if (wide && s >= 255) {
                stack.push_back(uint16_t(s));
                s = 255;
            }
            const uint32_t fs = f[s];
            if (uint64_t(x) >= (uint64_t(fs) << 20)) {
                stack.push_back(uint16_t(x));
                x >>= 16;
            }
            const uint32_t q = x / fs;
            x = (q << 12) + (x - q * fs) + c[s];
        }
        out.clear();
        out.push_back(uint16_t(x));
        out.push_back(uint16_t(x >> 16));
        out.insert(out.end(), stack.rbegin(), stack.rend());
    }
};

uint64_t raw_size(uint32_t n, uint32_t dtype) { return dtype == 2 ? 2 + 2ull * n : 2 + n + (n & 1); }

void emit_values(std::vector<uint8_t> &o, const uint32_t *v, uint32_t n, uint32_t dtype) {
    if (dtype == 2) {
        for (uint32_t j = 0; j < n; j++) emit16(o, v[j]);
    } else {
        for (uint32_t j = 0; j < n; j++) o.push_back(uint8_t(v[j]));
        if (n & 1) o.push_back(0);
    }
}

// ------------------------------------------------------------ paired tANS

} // namespace

// The paired encode tables, built once from the format's pair models.
qsc::PairEncodeTables::PairEncodeTables() {
    const PairModels &pm = pair_models();
    for (uint32_t m = 0; m < kModels; m++) {
        uint16_t spread[kTansL];
        uint32_t pos = 0;
        for (uint32_t i = 0; i < 256; i++)
            for (uint32_t k = 0; k < pm.n[m][i]; k++) {
                spread[pos] = uint16_t(i);
                pos = (pos + 643) & (kTansL - 1);
            }
        uint32_t acc = 0;
        for (uint32_t i = 0; i < 256; i++) {
            first[m][i] = uint16_t(acc);
            acc += pm.n[m][i];
        }
        first[m][256] = uint16_t(acc);
        uint32_t fill[256];
        for (uint32_t i = 0; i < 256; i++) fill[i] = first[m][i];
        for (uint32_t X = 0; X < kTansL; X++) states[m][fill[spread[X]]++] = uint16_t(X);
        for (uint32_t i = 0; i < 256; i++)
            cost[m][i] = pm.n[m][i] ? uint32_t(std::ceil(256.0 * std::log2(1024.0 / double(pm.n[m][i])))) : 0;
    }
}

const PairEncodeTables &qsc::pair_encode_tables() {
    static PairEncodeTables t;
    return t;
}

namespace {

const PairEncodeTables &pair_tables() { return pair_encode_tables(); }

inline uint32_t wsym(uint32_t v, uint32_t a0, uint32_t use) {
    const uint32_t d = v - a0;
    return (v >= a0 && d < 15 && ((use >> d) & 1)) ? d : 15;
}

struct BitSink {
    std::vector<uint8_t> &out;
    uint64_t acc = 0;
    uint32_t nacc = 0;
    uint64_t bits = 0;
    explicit BitSink(std::vector<uint8_t> &o) : out(o) {}
    void put(uint32_t v, uint32_t nb) {
        if (!nb) return;
        acc |= uint64_t(v & ((1u << nb) - 1)) << nacc;
        nacc += nb;
        bits += nb;
        while (nacc >= 8) {
            out.push_back(uint8_t(acc));
            acc >>= 8;
            nacc -= 8;
        }
    }
    void pad16() {
        while (bits % 16) put(0, 1);
    }
};

// PAIRED stream (header included) for model m (FORMAT 3.2-3.3).
void paired_stream(uint32_t m, const uint32_t *v, uint32_t dtype, std::vector<uint8_t> &out) {
    const PairModels &pm = pair_models();
    const PairEncodeTables &pt = pair_tables();
    const uint32_t a0 = pm.a0[m], use = pm.in_use[m];
    uint16_t chunk_v[256];
    uint8_t chunk_n[256];
    uint32_t x = kTansL;
    for (int t = 255; t >= 0; t--) {
        const uint32_t i = wsym(v[2 * t], a0, use) * 16 + wsym(v[2 * t + 1], a0, use);
        const uint32_t ni = pm.n[m][i];
        uint32_t k = 0;
        while ((x >> k) >= 2 * ni) k++;
        chunk_v[t] = uint16_t(x & ((1u << k) - 1));
        chunk_n[t] = uint8_t(k);
        x = kTansL + pt.states[m][pt.first[m][i] + ((x >> k) - ni)];
    }
    out.clear();
    emit16(out, P_PAIRED | (m << 3));
    BitSink bs(out);
    const uint32_t lit = dtype == 2 ? 16 : 8;
    bs.put(x - kTansL, 10);
    for (int t = 0; t < 256; t++) {
        bs.put(chunk_v[t], chunk_n[t]);
        if (wsym(v[2 * t], a0, use) == 15) bs.put(v[2 * t], lit);
        if (wsym(v[2 * t + 1], a0, use) == 15) bs.put(v[2 * t + 1], lit);
    }
    bs.pad16();
}

// model with the smallest static cost, lowest index on ties (FORMAT 3.4)
uint32_t best_model(const uint32_t *v, uint32_t dtype) {
    const PairModels &pm = pair_models();
    const PairEncodeTables &pt = pair_tables();
    uint32_t keys[256];
    for (int t = 0; t < 256; t++) keys[t] = (v[2 * t] << 16) | v[2 * t + 1];
    std::sort(keys, keys + 256);
    uint32_t uk[256], uc[256], nu = 0;
    for (int t = 0; t < 256; t++) {
        if (nu && uk[nu - 1] == keys[t])
            uc[nu - 1]++;
        else {
            uk[nu] = keys[t];
            uc[nu] = 1;
            nu++;
        }
    }
    const uint64_t lit = 256ull * (dtype == 2 ? 16 : 8);
    uint32_t best = 0;
    uint64_t best_cost = ~0ull;
    for (uint32_t m = 0; m < kModels; m++) {
        uint64_t c = 0;
        for (uint32_t u = 0; u < nu; u++) {
            const uint32_t a = wsym(uk[u] >> 16, pm.a0[m], pm.in_use[m]);
            const uint32_t b = wsym(uk[u] & 0xFFFF, pm.a0[m], pm.in_use[m]);
            c += uint64_t(uc[u]) * (pt.cost[m][a * 16 + b] + (a == 15 ? lit : 0) + (b == 15 ? lit : 0));
        }
        if (c < best_cost) {
            best_cost = c;
            best = m;
        }
    }
    return best;
}

// ------------------------------------------------------------ one block

template <typename T>
void gather_group(const T *src, uint32_t n, uint32_t P, uint32_t p0, uint32_t cnt, uint32_t *dst /* cnt x 512 */) {
    for (uint32_t j = 0; j < n; j++) {
        const T *row = src + uint64_t(j) * P + p0;
        for (uint32_t i = 0; i < cnt; i++) dst[i * kBlock + j] = row[i];
    }
}

void encode_block(const Geometry &g, const void *data, uint32_t n, EncodedBlock &eb) {
    const uint32_t P = g.P(), G = g.G();
    eb.n_scans = n;
    eb.gbase.assign(G, 0);
    eb.rel.assign(size_t(G) * 32, 0);
    eb.payload.clear();
    std::vector<uint16_t> codes;
    const void *src = data;
    uint32_t dtype = g.dtype;
    if (g.scaled) {
        // calibrate the block region in double precision (FORMAT 1.5)
        const float *x = static_cast<const float *>(data);
        const uint64_t cnt = uint64_t(n) * P;
        double lo = 0, hi = 0;
        for (uint64_t i = 0; i < cnt; i++) {
            if (!std::isfinite(x[i])) {
                eb.status = QSC_ERR_INVALID_ARG;
                return;
            }
            const double d = x[i];
            if (i == 0 || d < lo) lo = d;
            if (i == 0 || d > hi) hi = d;
        }
        codes.resize(cnt);
        if (hi == lo) {
            eb.scale = 1.0;
            eb.offset = lo;
            std::fill(codes.begin(), codes.end(), uint16_t(0));
        } else {
            const double sc = (hi - lo) / 65535.0;
            eb.scale = sc;
            eb.offset = lo;
            for (uint64_t i = 0; i < cnt; i++) {
                double c = std::nearbyint((double(x[i]) - lo) / sc); // default rounding: nearest, ties to even
                codes[i] = uint16_t(std::min(65535.0, std::max(0.0, c)));
            }
        }
        src = codes.data();
        dtype = 2;
    }
    const bool wide = dtype == 2;
    std::vector<uint32_t> grp(32 * kBlock);
    auto load = [&](uint32_t gi, uint32_t cnt) {
        if (dtype == 1)
            gather_group(static_cast<const uint8_t *>(src), n, P, gi * 32, cnt, grp.data());
        else
            gather_group(static_cast<const uint16_t *>(src), n, P, gi * 32, cnt, grp.data());
    };
    auto constant = [&](const uint32_t *v) {
        for (uint32_t j = 1; j < n; j++)
            if (v[j] != v[0]) return false;
        return true;
    };

    if (g.layout == 0) {
        uint64_t hist[256] = {0};
        for (uint32_t gi = 0; gi < G; gi++) {
            const uint32_t cnt = std::min<uint32_t>(32, P - gi * 32);
            load(gi, cnt);
            for (uint32_t i = 0; i < cnt; i++) {
                const uint32_t *v = &grp[i * kBlock];
                if (constant(v)) continue;
                for (uint32_t j = 0; j < n; j++) hist[std::min<uint32_t>(v[j], 255)]++;
            }
        }
        quantize_freqs(hist, eb.freq);
    }
    const RansCoder coder(eb.freq);
    std::vector<uint16_t> stack, words;
    std::vector<uint8_t> pstream;
    stack.reserve(2 * kBlock);
    const uint64_t raw = raw_size(n, dtype);
    for (uint32_t gi = 0; gi < G; gi++) {
        const uint32_t cnt = std::min<uint32_t>(32, P - gi * 32);
        load(gi, cnt);
        const uint64_t gstart = eb.payload.size();
        eb.gbase[gi] = uint32_t(gstart);
        for (uint32_t i = 0; i < cnt; i++) {
            eb.rel[size_t(gi) * 32 + i] = uint16_t(eb.payload.size() - gstart);
            const uint32_t *v = &grp[i * kBlock];
            std::vector<uint8_t> &o = eb.payload;
            if (g.layout == 0) {
                if (constant(v)) {
                    emit16(o, R_CONST);
                    emit16(o, v[0]);
                    continue;
                }
                bool rans = false;
                if (coder.usable) {
                    coder.encode(v, n, wide, stack, words);
                    rans = 2 + 2ull * words.size() < raw;
                }
                if (rans) {
                    emit16(o, R_RANS);
                    for (uint16_t w : words) emit16(o, w);
                } else {
                    emit16(o, R_RAW);
                    emit_values(o, v, n, dtype);
                }
            } else {
                uint32_t nnz = 0;
                for (uint32_t j = 0; j < n; j++) nnz += v[j] != 0;
                if (!nnz) {
                    emit16(o, P_EMPTY);
                    continue;
                }
                if (constant(v)) {
                    emit16(o, P_CONST);
                    emit16(o, v[0]);
                    continue;
                }
                const uint64_t sparse = 4 + 2ull * nnz + (dtype == 2 ? 2ull * nnz : nnz + (nnz & 1));
                paired_stream(best_model(v, dtype), v, dtype, pstream);
                const uint64_t paired = pstream.size();
                uint32_t mode = P_SPARSE;
                uint64_t size = sparse;
                if (sparse >= paired + 2) {
                    mode = P_PAIRED;
                    size = paired;
                }
                if (raw < size) mode = P_RAW;
                if (mode == P_PAIRED) {
                    o.insert(o.end(), pstream.begin(), pstream.end());
                } else if (mode == P_SPARSE) {
                    emit16(o, P_SPARSE);
                    emit16(o, nnz);
                    for (uint32_t j = 0; j < n; j++)
                        if (v[j]) emit16(o, j);
                    if (dtype == 2) {
                        for (uint32_t j = 0; j < n; j++)
                            if (v[j]) emit16(o, v[j]);
                    } else {
                        for (uint32_t j = 0; j < n; j++)
                            if (v[j]) o.push_back(uint8_t(v[j]));
                        if (nnz & 1) o.push_back(0);
                    }
                } else {
                    emit16(o, P_RAW);
                    emit_values(o, v, n, dtype);
                }
            }
        }
        const uint64_t span = eb.payload.size() - gstart;
        for (uint32_t i = cnt; i < 32; i++) eb.rel[size_t(gi) * 32 + i] = uint16_t(span);
    }
}

} // namespace

struct qsc_encoder {
    Geometry g;
    uint64_t scans = 0;
    std::vector<EncodedBlock> blocks;
};

extern "C" {

qsc_status qsc_encoder_create(const qsc_geometry *geom, qsc_encoder **out) {
    if (!geom || !out) return QSC_ERR_INVALID_ARG;
    Geometry g;
    g.scan_rows = geom->scan_rows;
    g.scan_cols = geom->scan_cols;
    g.det_rows = geom->det_rows;
    g.det_cols = geom->det_cols;
    g.dtype = geom->dtype;
    g.layout = geom->layout;
    g.scaled = geom->scaled;
    if (!check_geometry(g).empty()) return QSC_ERR_INVALID_ARG;
    auto *e = new (std::nothrow) qsc_encoder;
    if (!e) return QSC_ERR_OOM;
    e->g = g;
    e->blocks.reserve(g.n_blocks());
    *out = e;
    return QSC_OK;
}

qsc_status qsc_encoder_add(qsc_encoder *enc, const void *host_data, uint64_t n_scans, int threads) {
    if (!enc || !host_data || n_scans == 0) return QSC_ERR_INVALID_ARG;
    const Geometry &g = enc->g;
    if (enc->scans % kBlock) return QSC_ERR_INVALID_ARG; // a partial block was already added
    if (enc->scans + n_scans > g.S()) return QSC_ERR_INVALID_ARG;
    const uint32_t nb = uint32_t((n_scans + kBlock - 1) / kBlock);
    if (threads <= 0) threads = int(std::max(1u, std::thread::hardware_concurrency()));
    threads = std::min<int>(threads, int(nb));
    const size_t first = enc->blocks.size();
    enc->blocks.resize(first + nb);
    const uint64_t vbytes = g.scaled ? 4 : g.dtype;
    std::atomic<uint32_t> next{0};
    auto work = [&]() {
        for (uint32_t b; (b = next.fetch_add(1)) < nb;) {
            const uint32_t n = uint32_t(std::min<uint64_t>(kBlock, n_scans - uint64_t(b) * kBlock));
            const uint8_t *src = static_cast<const uint8_t *>(host_data) + uint64_t(b) * kBlock * g.P() * vbytes;
            encode_block(g, src, n, enc->blocks[first + b]);
        }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < threads; t++) pool.emplace_back(work);
    work();
    for (auto &t : pool) t.join();
    qsc_status st = QSC_OK;
    for (uint32_t b = 0; b < nb; b++)
        if (enc->blocks[first + b].status != QSC_OK) st = enc->blocks[first + b].status;
    if (st != QSC_OK) {
        enc->blocks.resize(first);
        return st;
    }
    enc->scans += n_scans;
    return QSC_OK;
}

qsc_status qsc_encoder_size(const qsc_encoder *enc, uint64_t *nbytes) {
    if (!enc || !nbytes || enc->scans != enc->g.S()) return QSC_ERR_INVALID_ARG;
    uint64_t pay = 0;
    for (const auto &b : enc->blocks) pay += b.payload.size();
    *nbytes = layout_sections(enc->g, pay).total;
    return QSC_OK;
}

qsc_status qsc_encoder_write(const qsc_encoder *enc, void *host_out, uint64_t capacity) {
    uint64_t total;
    qsc_status st = qsc_encoder_size(enc, &total);
    if (st) return st;
    if (!host_out || capacity < total) return QSC_ERR_INVALID_ARG;
    const Geometry &g = enc->g;
    uint64_t pay = 0;
    for (const auto &b : enc->blocks) pay += b.payload.size();
    const Sections s = layout_sections(g, pay);
    uint8_t *o = static_cast<uint8_t *>(host_out);
    std::memset(o, 0, total);
    auto st32 = [&](uint64_t off, uint32_t v) { std::memcpy(o + off, &v, 4); };
    auto st64 = [&](uint64_t off, uint64_t v) { std::memcpy(o + off, &v, 8); };
    write_header(g, s, o);
    const uint32_t G = g.G();
    uint64_t base = 0;
    for (uint32_t b = 0; b < enc->blocks.size(); b++) {
        const EncodedBlock &eb = enc->blocks[b];
        st64(s.dir + 16ull * b, base);
        st32(s.dir + 16ull * b + 8, eb.n_scans);
        st32(s.dir + 16ull * b + 12, uint32_t(eb.payload.size()));
        if (g.layout == 0) std::memcpy(o + s.table + 512ull * b, eb.freq, 512);
        std::memcpy(o + s.gbase + 4ull * G * b, eb.gbase.data(), 4ull * G);
        std::memcpy(o + s.rel + 64ull * G * b, eb.rel.data(), 64ull * G);
        std::memcpy(o + s.payload + base, eb.payload.data(), eb.payload.size());
        if (g.scaled) {
            std::memcpy(o + s.calib + 16ull * b, &eb.scale, 8);
            std::memcpy(o + s.calib + 16ull * b + 8, &eb.offset, 8);
        }
        base += eb.payload.size();
    }
    if (g.layout == 1) {
        const PairModels &pm = pair_models();
        std::memcpy(o + s.table, pm.n, sizeof(pm.n));
    }
    return QSC_OK;
}

qsc_status qsc_encoder_destroy(qsc_encoder *enc) {
    delete enc;
    return QSC_OK;
}

} // extern "C"
