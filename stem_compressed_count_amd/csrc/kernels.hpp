// Device-side parameter blocks and kernel launchers (gfx950).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qsc {

// Paired decode tables on the device: 32 models x 1024 states, then one idle
// entry (values 0, no bits, next state 0) padded to 16 bytes.
constexpr uint32_t kPairTable = 32 * 1024 + 4;
// LDS index of the paired layout's idle entry (after the 32 model tables): no
// code bits, zero values, and itself as the next entry
constexpr uint32_t kPairIdle = 32 * 1024;

// Query plan: the selected pixels are counted per 64-pixel tile (at most
// kMaxPlanTiles tiles, so detectors up to 65,536 pixels; larger ones decode
// every pixel tile), then cut into work items of equal numbers of selected
// pixels in pixel order.
constexpr uint32_t kPlanFine = 64;
constexpr uint32_t kMaxPlanTiles = 1024;
// plan buffer: the counts (a second, subtracted mask's follow), then as many
// words of the selected pixels' encoded bytes in the first block
constexpr uint32_t kPlanBytes = 2 * kMaxPlanTiles;
constexpr uint32_t kPlanWords = 4 * kMaxPlanTiles;

// Device view of a resident (all pointers are device memory).
struct DevResident {
    const uint8_t *payload;  // stream bytes, followed by zero padding
    const uint8_t *dir;      // n_blocks x {u64 base, u32 n_scans, u32 nbytes}
    const uint32_t *gbase;   // n_blocks x G
    const uint16_t *rel;     // n_blocks x G x 32
    const uint16_t *freq;    // byte-rANS: n_blocks x 256 frequencies (the container's table section)
    const uint32_t *tables;  // paired: kPairTable entries (null for byte-rANS)
    const uint32_t *model_info; // paired: per model a0 | in_use << 16
    const uint8_t *valid;    // P bytes, nonzero = valid
    const double *calib;     // scaled: n_blocks x {scale, offset}
    unsigned long long *err; // first malformed stream: (block + 1) << 32 | pixel, 0 = none
    uint32_t *plan;          // query plan: selected pixels per 64-pixel tile (kPlanWords words)
    const uint32_t *split;   // byte-rANS: per (block, pixel), the state and byte offset of the stream after
                             // its first kSplit scans (two words), or null when not built
    const uint8_t *raw_blk;  // byte-rANS: per block, nonzero when it holds a RAW stream (null: none does)
    uint32_t esc_heavy;      // byte-rANS uint16: most blocks give the escape symbol at least 1/4 of the table
    uint64_t S;
    uint32_t P, G, det_cols, scan_cols, n_blocks, dtype, layout;
};

// Region reads (a scan rectangle), Frames (whole blocks) and Amp (whole
// blocks as square-root amplitudes) write decoded values; each is its own
// instantiation, so the rectangle tests and the table gather stay out of the
// loops that do not need them.
enum class Op : int { Sum = 0, Moments = 1, Region = 2, Dp = 3, Index = 4, Amp = 5, Frames = 6, Split = 7 };

// Scans after which byte-rANS streams of complete blocks keep a split point:
// a latency-bound query decodes each stream's two halves side by side.
constexpr uint32_t kSplit = 256;

// Buffers of the queries beyond sums and moments.
//  diffraction pattern: the selected scans (null: every scan), the
//  per-(visited block, pixel) partial sums and the per-visited-block count of
//  selected scans it fills;
//  index build: the polar pixel order and the field rows it fills.
struct AuxArgs {
    const uint8_t *scan_mask;
    uint32_t *part;  // n_visited x P
    uint32_t *nb;    // n_visited
    const uint16_t *perm;  // P
    uint32_t *rows;        // n_blocks x n_fields x 512
    uint32_t n_fields;
    const uint8_t *neg_mask;  // planned sums: pixels whose values are subtracted (P bytes), or null
    uint32_t halves;          // region reads: items of half a workgroup whose streams' halves decode side by side
};

// A region read: half-open scan rectangle, output buffer and kind (0 native
// dtype, 1 float32 code*scale+offset of the scan's region, 2 float32 square
// root of the count, looked up in amp: 65536 correctly rounded values). With
// frames set, every scan of the listed blocks is written instead, at row
// s - s_first.
struct RegionArgs {
    uint32_t r0, r1, c0, c1;
    int out_kind;
    void *out;
    int frames;
    uint64_t s_first;
    const float *amp;
};

// Blocks touched by a region read, passed by value to one launch.
struct RegionBlocks {
    uint32_t n;
    uint32_t b[64];
};

// Launch wrappers (enqueue only; return hipSuccess or the launch error).
//  One reduce query: out is zeroed (or copied from init, n_init elements of 4
//  or 8 bytes) and the pixel tiles the mask selects nothing from are planned
//  out; then every pixel with (mask[p] != 0) != complement (all pixels when
//  mask is null) and valid[p] of every visited block (b % stride == 0) is
//  decoded and added (negate: subtracted) into out: u32/u64 per scan for
//  Op::Sum, u64 [3][S] moments for Op::Moments.
//  With neg_mask (Op::Sum, n_init > 0), the valid pixels of neg_mask are
//  decoded in the same launch and subtracted instead.
hipError_t launch_query(const DevResident &r, const uint8_t *mask, int complement, uint32_t stride, Op op, void *out,
                        int out64, int negate, const void *init, uint64_t n_init, hipStream_t st,
                        const uint8_t *neg_mask = nullptr);
//  Masks of a change from prev to mask: added = mask & ~prev, removed = prev & ~mask (P bytes each).
hipError_t launch_mask_delta(const uint8_t *prev, const uint8_t *mask, uint32_t P, uint8_t *added, uint8_t *removed,
                             hipStream_t st);
//  CoM from exact moments.
hipError_t launch_com_finalize(const uint64_t *moments, uint64_t S, float *row, float *col, hipStream_t st);
//  decode of a scan rectangle over the listed touched blocks.
hipError_t launch_region(const DevResident &r, const RegionBlocks &blocks, const RegionArgs &ra, hipStream_t st);
//  Sum (u64[P]) and mean (f32[P], nullable) diffraction pattern over the
//  selected scans of the visited blocks; part holds n_visited x P u32 and nb
//  n_visited u32 of device scratch.
hipError_t launch_dp(const DevResident &r, const uint8_t *scan_mask, uint32_t stride, uint32_t *part, uint32_t *nb,
                     uint64_t *sum, float *mean, hipStream_t st);
// Polar interaction index of a resident: pixels in radial-angular order, 64-pixel
// leaves, 16-leaf roots; fields = leaves then roots, each block's field rows
// bit-packed at dword offsets.
constexpr uint32_t kLeaf = 64, kRoot = 16;
struct DevIndex {
    const uint16_t *perm;        // P: pixel at each polar position
    const uint16_t *leaf_valid;  // n_leaves: valid pixels per leaf
    const uint32_t *packed;      // bit-packed field rows
    const uint32_t *offset;      // n_blocks x n_fields dword offsets into packed
    const uint8_t *width;        // n_blocks x n_fields bits per value
    uint32_t n_leaves, n_roots;
};
//  index build, step 1: exact per-scan leaf sums of every block into rows
//  (n_blocks x (n_leaves + n_roots) x 512 u32, root rows filled in step 2).
hipError_t launch_index_leaves(const DevResident &r, const uint16_t *perm, uint32_t n_leaves, uint32_t n_roots,
                               uint32_t *rows, hipStream_t st);
//  step 2: root rows and the bit width of every field row.
hipError_t launch_index_widths(uint32_t n_blocks, uint32_t n_leaves, uint32_t n_roots, uint32_t *rows,
                               uint8_t *width, hipStream_t st);
//  step 3: pack every field row at its dword offset.
hipError_t launch_index_pack(uint32_t n_blocks, uint32_t n_fields, const uint32_t *rows, const uint32_t *offset,
                             const uint8_t *width, uint32_t *packed, hipStream_t st);
//  masked_sum through the index: fields covered by mask & valid are summed from
//  the index, the residual pixels decoded; scratch: fields holds n_leaves +
//  n_roots + 1 u32 (the field list) then n_leaves bytes (leaf flags),
//  residual P bytes.
hipError_t launch_indexed_sum(const DevResident &r, const DevIndex &ix, const uint8_t *mask, uint32_t stride,
                              void *out, int out64, uint32_t *fields, uint8_t *residual, hipStream_t st);
//  zero n bytes (region outputs of residents with invalid pixels)
// Split points of every byte-rANS stream of the complete blocks (out: n_blocks
// x P x {state, byte offset}); one decode of the first kSplit scans.
hipError_t launch_split_build(const DevResident &r, uint32_t *out, hipStream_t st);
// Stream-header checks of a resident built from a device container.
// Marks (nonzero) the blocks that hold a RAW stream; out is zeroed by the caller.
hipError_t launch_raw_blocks(const DevResident &r, uint8_t *out, hipStream_t st);
hipError_t launch_check_headers(const DevResident &r, const uint8_t *usable, unsigned long long *counts,
                                unsigned long long *bad, hipStream_t st);
hipError_t launch_zero_bytes(void *out, uint64_t n, hipStream_t st);

int device_cu_count();

} // namespace qsc
