// Container parsing, validation and decode-table construction (host side).
//
// The container and both stream layouts are this library's own definition
// (FORMAT.md v1): the pages fix only their constraints (paired-resident page,
// "Operation pipeline" item 2 and "Contract": 512-scan blocks, per-pixel
// streams, a 2-byte stream header whose reserved bits must be rejected,
// grouped offsets of one 32-bit base plus 32 relative 16-bit offsets, 32
// Poisson pair models with 1024 states, exact alternative stream forms).
#include <algorithm>
#include <cmath>
#include <mutex>
#include <numeric>

#include "qsc_internal.hpp"

namespace qsc {

static const char *kAbiRans = "qsc-byte-rans-v1";
static const char *kAbiPaired = "qsc-paired-v1";

std::string check_geometry(const Geometry &g) {
    if (g.det_rows < 1 || g.det_rows > 1024 || g.det_cols < 1 || g.det_cols > 1024)
        return "detector dimensions must be in 1..1024";
    if (g.scan_rows < 1 || g.scan_cols < 1) return "scan dimensions must be positive";
    if (g.S() >= (1ull << 31)) return "too many scans";
    if (g.dtype != 1 && g.dtype != 2) return "dtype must be 1 (uint8) or 2 (uint16)";
    if (g.layout > 1) return "layout must be 0 (byte-rANS) or 1 (paired)";
    if (g.layout == 1 && g.S() % kBlock) return "the paired layout needs complete 512-scan blocks";
    if (g.scaled > 1) return "scaled must be 0 or 1";
    if (g.scaled && (g.layout != 0 || g.dtype != 2)) return "scaled storage needs layout 0 and uint16 codes";
    return "";
}

static uint64_t up256(uint64_t o) { return (o + 255) / 256 * 256; }

Sections layout_sections(const Geometry &g, uint64_t payload_bytes) {
    const uint64_t nb = g.n_blocks(), G = g.G();
    Sections s;
    s.dir = kHeaderBytes;
    s.table = up256(s.dir + 16 * nb);
    s.gbase = up256(s.table + (g.layout == 0 ? 512 * nb : 2ull * kModels * 256));
    s.rel = up256(s.gbase + 4 * nb * G);
    s.payload = up256(s.rel + 64 * nb * G);
    s.payload_bytes = payload_bytes;
    s.total = s.payload + payload_bytes;
    if (g.scaled) {
        s.calib = up256(s.total);
        s.total = s.calib + 16 * nb;
    }
    return s;
}

void write_header(const Geometry &g, const Sections &s, uint8_t *out) {
    std::memset(out, 0, kHeaderBytes);
    auto st32 = [&](uint64_t off, uint32_t v) { std::memcpy(out + off, &v, 4); };
    auto st64 = [&](uint64_t off, uint64_t v) { std::memcpy(out + off, &v, 8); };
    std::memcpy(out, "QSCRES01", 8);
    const char *tag = g.layout == 0 ? kAbiRans : kAbiPaired;
    std::memcpy(out + 8, tag, std::strlen(tag));
    const uint32_t hdr[10] = {1, g.layout, g.scan_rows, g.scan_cols, g.det_rows, g.det_cols, g.dtype, kBlock,
                              g.n_blocks(), g.scaled};
    for (int i = 0; i < 10; i++) st32(40 + 4 * i, hdr[i]);
    const uint64_t offs[8] = {s.dir, s.table, s.gbase, s.rel, s.payload, s.payload_bytes, s.calib, s.total};
    for (int i = 0; i < 8; i++) st64(80 + 8 * i, offs[i]);
}

// ---------------------------------------------------------------- pair models

static PairModels compute_pair_models() {
    PairModels pm{};
    for (uint32_t m = 0; m < kModels; m++) {
        const double lam = 0.01 * std::pow(2000.0, double(m) / 31.0);
        int base = int(std::floor(lam)) - 7;
        if (base < 0) base = 0;
        // Poisson pmf by the recurrence p(k) = p(k-1) * lam / k
        double pmf[48];
        pmf[0] = std::exp(-lam);
        for (int k = 1; k < base + 15; k++) pmf[k] = (pmf[k - 1] * lam) / double(k);
        double q[16];
        uint32_t use = 0;
        double kept = 0.0;
        for (int k = 0; k < 15; k++) {
            q[k] = pmf[base + k];
            if (q[k] >= 1.0 / 1024.0) {
                use |= 1u << k;
                kept += q[k];
            }
        }
        q[15] = std::max(0.0, 1.0 - kept);
        auto usable = [&](int s) { return s == 15 || ((use >> s) & 1); };
        bool sup[256];
        double rem[256];
        int32_t cnt[256];
        int64_t sum = 0;
        for (int i = 0; i < 256; i++) {
            sup[i] = usable(i >> 4) && usable(i & 15);
            cnt[i] = 0;
            rem[i] = 0.0;
            if (!sup[i]) continue;
            const double y = 1024.0 * (q[i >> 4] * q[i & 15]);
            const double fl = std::floor(y);
            rem[i] = y - fl;
            cnt[i] = std::max<int32_t>(1, int32_t(fl));
            sum += cnt[i];
        }
        while (sum > int64_t(kTansL)) { // take from the largest count, lowest index first
            int best = -1;
            for (int i = 0; i < 256; i++)
                if (sup[i] && (best < 0 || cnt[i] > cnt[best])) best = i;
            cnt[best]--;
            sum--;
        }
        if (sum < int64_t(kTansL)) { // largest remainders, lowest index on ties, cycling if needed
            std::vector<int> order;
            for (int i = 0; i < 256; i++)
                if (sup[i]) order.push_back(i);
            std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return rem[a] > rem[b]; });
            for (size_t k = 0; sum < int64_t(kTansL); k = (k + 1) % order.size()) {
                cnt[order[k]]++;
                sum++;
            }
        }
        for (int i = 0; i < 256; i++) pm.n[m][i] = uint16_t(cnt[i]);
        pm.a0[m] = uint32_t(base);
        pm.in_use[m] = use;
    }
    return pm;
}

const PairModels &pair_models() {
    static PairModels pm = compute_pair_models();
    return pm;
}

// ---------------------------------------------------------------- device tables

void build_pair_tables(uint32_t *out) {
    const PairModels &pm = pair_models();
    for (uint32_t m = 0; m < kModels; m++) {
        uint16_t spread[kTansL];
        uint32_t pos = 0;
        for (uint32_t i = 0; i < 256; i++)
            for (uint32_t k = 0; k < pm.n[m][i]; k++) {
                spread[pos] = uint16_t(i);
                pos = (pos + 643) & (kTansL - 1);
            }
        uint32_t next[256];
        for (uint32_t i = 0; i < 256; i++) next[i] = pm.n[m][i];
        for (uint32_t X = 0; X < kTansL; X++) {
            const uint32_t i = spread[X];
            const uint32_t y = next[i]++;
            const uint32_t nb = 10 - (31 - __builtin_clz(y));
            const uint32_t newX = (y << nb) - kTansL;
            const uint32_t a = i >> 4, b = i & 15;
            // code length, window values, escape flag, and the next state's table index
            out[m * kTansL + X] = nb | (a << 6) | (b << 10) | ((a == 15 || b == 15) ? 1u << 15 : 0u) |
                                  ((m * kTansL + newX) << 16);
        }
    }
}

// ---------------------------------------------------------------- validation

qsc_status parse_and_validate(const uint8_t *blob, uint64_t nbytes, Parsed *out, std::string *msg, bool streams,
                              const uint8_t *calib) {
    auto fail = [&](qsc_status st, const std::string &m) {
        *msg = m;
        return st;
    };
    if (!blob || nbytes < kHeaderBytes) return fail(QSC_ERR_MALFORMED, "blob shorter than its header");
    if (std::memcmp(blob, "QSCRES01", 8)) return fail(QSC_ERR_MALFORMED, "bad magic");
    char tag[33];
    std::memcpy(tag, blob + 8, 32);
    tag[32] = 0;
    Geometry g;
    g.layout = ld32(blob + 44);
    const char *want = g.layout == 0 ? kAbiRans : g.layout == 1 ? kAbiPaired : nullptr;
    if (!want || std::strcmp(tag, want) != 0 || ld32(blob + 40) != 1)
        return fail(QSC_ERR_UNSUPPORTED, std::string("unsupported ABI tag or version: ") + tag);
    for (int i = 8 + int(std::strlen(tag)); i < 40; i++)
        if (blob[i]) return fail(QSC_ERR_MALFORMED, "ABI tag not NUL padded");
    g.scan_rows = ld32(blob + 48);
    g.scan_cols = ld32(blob + 52);
    g.det_rows = ld32(blob + 56);
    g.det_cols = ld32(blob + 60);
    g.dtype = ld32(blob + 64);
    const uint32_t flags = ld32(blob + 76);
    if (flags & ~1u) return fail(QSC_ERR_MALFORMED, "unknown flag bits");
    g.scaled = flags & 1;
    std::string why = check_geometry(g);
    if (!why.empty()) return fail(QSC_ERR_MALFORMED, "header geometry: " + why);
    if (ld32(blob + 68) != kBlock) return fail(QSC_ERR_MALFORMED, "block_scans must be 512");
    if (ld32(blob + 72) != g.n_blocks()) return fail(QSC_ERR_MALFORMED, "n_blocks does not match the scans");
    for (int i = 144; i < 256; i++)
        if (blob[i]) return fail(QSC_ERR_MALFORMED, "reserved header bytes not zero");
    Sections s;
    s.dir = ld64(blob + 80);
    s.table = ld64(blob + 88);
    s.gbase = ld64(blob + 96);
    s.rel = ld64(blob + 104);
    s.payload = ld64(blob + 112);
    s.payload_bytes = ld64(blob + 120);
    s.calib = ld64(blob + 128);
    s.total = ld64(blob + 136);
    const Sections want_s = layout_sections(g, s.payload_bytes);
    if (s.dir != want_s.dir || s.table != want_s.table || s.gbase != want_s.gbase || s.rel != want_s.rel ||
        s.payload != want_s.payload || s.calib != want_s.calib || s.total != want_s.total || s.total != nbytes)
        return fail(QSC_ERR_MALFORMED, "section offsets do not match the format layout");

    const uint32_t nb = g.n_blocks(), G = g.G(), P = g.P();
    // block directory
    uint64_t expect_base = 0;
    for (uint32_t b = 0; b < nb; b++) {
        const uint8_t *d = blob + s.dir + 16ull * b;
        const uint64_t base = ld64(d);
        const uint32_t n = ld32(d + 8), bytes = ld32(d + 12);
        const uint64_t want_n = std::min<uint64_t>(kBlock, g.S() - uint64_t(b) * kBlock);
        if (base != expect_base || n != want_n)
            return fail(QSC_ERR_MALFORMED, "block directory entry " + std::to_string(b) + " inconsistent");
        expect_base += bytes;
    }
    if (expect_base != s.payload_bytes) return fail(QSC_ERR_MALFORMED, "block sizes do not add up to the payload");
    // tables
    if (g.layout == 0) {
        for (uint32_t b = 0; b < nb; b++) {
            uint32_t sum = 0;
            for (int i = 0; i < 256; i++) sum += ld16(blob + s.table + 512ull * b + 2 * i);
            if (sum != 0 && sum != kRansM)
                return fail(QSC_ERR_MALFORMED, "frequency table of block " + std::to_string(b) + " does not sum to 4096");
        }
    } else {
        const PairModels &pm = pair_models();
        for (uint32_t m = 0; m < kModels; m++)
            for (int i = 0; i < 256; i++)
                if (ld16(blob + s.table + 2 * (256ull * m + i)) != pm.n[m][i])
                    return fail(QSC_ERR_MALFORMED, "pair model tables differ from the format's models");
    }
    // grouped offsets and stream headers
    for (auto &c : out->mode_counts) c = 0;
    for (uint32_t b = 0; b < nb; b++) {
        const uint8_t *d = blob + s.dir + 16ull * b;
        const uint64_t base = ld64(d);
        const uint32_t bytes = ld32(d + 12);
        bool table_usable = true;
        if (g.layout == 0) {
            uint32_t nz = 0, big = 0;
            for (int i = 0; i < 256; i++) {
                const uint32_t f = ld16(blob + s.table + 512ull * b + 2 * i);
                nz += f != 0;
                big |= f == kRansM;
            }
            table_usable = nz > 0 && !big;
        }
        uint64_t prev_end = 0;
        for (uint32_t gi = 0; gi < G; gi++) {
            const uint64_t gb = ld32(blob + s.gbase + 4 * (uint64_t(b) * G + gi));
            if (gb != prev_end) return fail(QSC_ERR_MALFORMED, "group base out of order in block " + std::to_string(b));
            const uint8_t *rel = blob + s.rel + 2 * ((uint64_t(b) * G + gi) * 32);
            if (ld16(rel) != 0) return fail(QSC_ERR_MALFORMED, "first relative offset of a group is not 0");
            const uint32_t used = std::min<uint32_t>(32, P - gi * 32);
            uint64_t group_end;
            if (gi + 1 < G)
                group_end = ld32(blob + s.gbase + 4 * (uint64_t(b) * G + gi + 1));
            else
                group_end = bytes;
            if (group_end < gb || group_end - gb > 65535 || group_end > bytes)
                return fail(QSC_ERR_MALFORMED, "group span out of range in block " + std::to_string(b));
            for (uint32_t i = used; i < 32; i++)
                if (ld16(rel + 2 * i) != group_end - gb)
                    return fail(QSC_ERR_MALFORMED, "unused offsets of a partial group must point at its end");
            for (uint32_t i = 0; i < used; i++) {
                const uint64_t st = gb + ld16(rel + 2 * i);
                const uint64_t en = i + 1 < used ? gb + ld16(rel + 2 * (i + 1)) : group_end;
                const uint32_t p = gi * 32 + i;
                auto where = [&]() { return " (block " + std::to_string(b) + ", pixel " + std::to_string(p) + ")"; };
                if (en < st + 2 || (st & 1) || (en & 1)) return fail(QSC_ERR_MALFORMED, "stream extent invalid" + where());
                if (!streams) continue;  // the stream headers are checked elsewhere
                const uint32_t hdr = ld16(blob + s.payload + base + st);
                const uint32_t mode = hdr & 7, model = (hdr >> 3) & 31;
                if (hdr >> 8) return fail(QSC_ERR_MALFORMED, "reserved stream header bits set" + where());
                if (g.layout == 0) {
                    if (mode > R_RAW || model) return fail(QSC_ERR_MALFORMED, "invalid stream mode" + where());
                    if (mode == R_RANS && !table_usable)
                        return fail(QSC_ERR_MALFORMED, "RANS stream with an unusable table" + where());
                } else {
                    if (mode > P_RAW || (model && mode != P_PAIRED))
                        return fail(QSC_ERR_MALFORMED, "invalid stream mode" + where());
                }
                out->mode_counts[mode]++;
            }
            prev_end = group_end;
        }
        if (prev_end != bytes) return fail(QSC_ERR_MALFORMED, "streams do not cover block " + std::to_string(b));
    }
    // calibration must be finite
    if (g.scaled)
        for (uint32_t i = 0; i < 2 * nb; i++) {
            double v;
            std::memcpy(&v, (calib ? calib : blob + s.calib) + 8ull * i, 8);
            if (!std::isfinite(v)) return fail(QSC_ERR_MALFORMED, "non-finite calibration");
        }
    out->g = g;
    out->sec = s;
    out->blob = blob;
    out->nbytes = nbytes;
    return QSC_OK;
}

} // namespace qsc
