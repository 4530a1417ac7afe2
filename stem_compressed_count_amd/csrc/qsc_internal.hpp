// Internal host-side definitions shared by the library's translation units.
#pragma once
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/qsc.h"

namespace qsc {

constexpr uint32_t kBlock = 512;      // scans per block
constexpr uint32_t kRansM = 4096;     // byte-rANS table size (12-bit precision)
constexpr uint32_t kRansL = 1u << 16; // byte-rANS state lower bound
constexpr uint32_t kTansL = 1024;     // paired tANS states
constexpr uint32_t kModels = 32;      // paired pair models
constexpr uint64_t kHeaderBytes = 256;
constexpr uint64_t kDevicePad = 16384; // zero bytes after the payload on the device (decoder read-ahead)

// stream modes (FORMAT 2.4, 3.4)
enum : uint32_t { R_CONST = 0, R_RANS = 1, R_RAW = 2 };
enum : uint32_t { P_EMPTY = 0, P_CONST = 1, P_SPARSE = 2, P_PAIRED = 3, P_RAW = 4 };

struct Geometry {
    uint32_t scan_rows = 0, scan_cols = 0, det_rows = 0, det_cols = 0;
    uint32_t dtype = 0, layout = 0, scaled = 0;
    uint64_t S() const { return uint64_t(scan_rows) * scan_cols; }
    uint32_t P() const { return det_rows * det_cols; }
    uint32_t G() const { return (P() + 31) / 32; }
    uint32_t n_blocks() const { return uint32_t((S() + kBlock - 1) / kBlock); }
    uint32_t maxval() const { return dtype == 1 ? 255u : 65535u; }
    uint32_t sum_bits() const { return uint64_t(P()) * maxval() > 0xFFFFFFFFull ? 64 : 32; }
};

// Validates a geometry; returns an empty string or the reason it is refused.
std::string check_geometry(const Geometry &g);

// Section offsets of a blob (FORMAT 1.1).
struct Sections {
    uint64_t dir = 0, table = 0, gbase = 0, rel = 0, payload = 0, payload_bytes = 0, calib = 0, total = 0;
};

// Section layout the encoder writes for a geometry and payload size.
Sections layout_sections(const Geometry &g, uint64_t payload_bytes);

// The 256-byte container header (FORMAT 1.1) of a geometry and its sections.
void write_header(const Geometry &g, const Sections &s, uint8_t *out256);

// A parsed and structurally validated blob.
struct Parsed {
    Geometry g;
    Sections sec;
    const uint8_t *blob = nullptr;
    uint64_t nbytes = 0;
    uint64_t mode_counts[8] = {0};
};

// Full host validation (FORMAT 1.x headers, offsets, tables, stream headers).
// Returns QSC_OK or an error with a message. With streams = false the stream
// headers are not read (blob then needs to hold only the sections before the
// payload) and the calibration is read from calib when that is not null.
qsc_status parse_and_validate(const uint8_t *blob, uint64_t nbytes, Parsed *out, std::string *msg,
                              bool streams = true, const uint8_t *calib = nullptr);

// Paired pair models (FORMAT 3.1): counts[32][256], window bases, in-use masks.
struct PairModels {
    uint16_t n[kModels][256];
    uint32_t a0[kModels];
    uint32_t in_use[kModels];
};
const PairModels &pair_models();

// Paired encode tables (FORMAT 3.2, 3.4): per model, the states of each pair
// symbol's occurrences in spread order (states[first[i] .. first[i+1])), and
// the static cost ceil(256 * log2(1024 / n[i])) in 1/256 bits.
struct PairEncodeTables {
    uint16_t first[kModels][257];
    uint16_t states[kModels][kTansL];
    uint32_t cost[kModels][256];
    PairEncodeTables();
};
const PairEncodeTables &pair_encode_tables();

// Device decode-table entries.
//  byte-rANS (per block, two planes of 4096 entries): f | symbol << 24, then slot - c
//  paired (per model, 1024 entries): a | b << 8 | nbits << 16 | newX << 20 | escape << 31
void build_pair_tables(uint32_t *out /* 32 x 1024 */);

// little-endian access
inline uint16_t ld16(const uint8_t *p) { return uint16_t(p[0] | (p[1] << 8)); }
inline uint32_t ld32(const uint8_t *p) { return uint32_t(ld16(p)) | (uint32_t(ld16(p + 2)) << 16); }
inline uint64_t ld64(const uint8_t *p) { return uint64_t(ld32(p)) | (uint64_t(ld32(p + 4)) << 32); }

} // namespace qsc
