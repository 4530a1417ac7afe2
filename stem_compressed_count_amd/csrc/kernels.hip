// Fused ANS decode + virtual-detector reduction kernels for gfx950 (CDNA4).
//
// Hot path of the paired-resident page ("Operation pipeline", steps 3-4): each
// workgroup takes one work item, (visited 512-scan block, a run of the
// selected pixels cut by the query plan) or for region reads (block, pixel
// tile), gathers the pixels that the mask and valid_pixels keep (wave ballots
// into an LDS list), stages the block's decode table in LDS and decodes every
// selected stream with one lane per stream. A lane keeps a 64-bit bit
// reservoir refilled 32 bits at a time from a prefetched dword on a
// wave-uniform cadence, and per-scan partial sums are reduced across the wave
// by a transpose-reduce (the page's warp-wide packed reduction per 32 scans,
// done here on 64-lane waves with the gfx950 lane-swap instructions and DPP).
// Streams stored in exact non-entropy forms (constant, sparse) are folded into
// LDS partials directly instead of stepping through the scans. Outputs are
// exact integers; the reduction order never matters.
//
// The products follow the optimization-matrix page, "Product Coverage": sparse
// BF/ADF masks as selected-pixel sums, dense DF as a cached full-detector total
// minus the complement, CoM from fused moment sums, and region reads that
// write the decoded values of the requested scans.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "kernels.hpp"

namespace qsc {

namespace {

constexpr uint32_t kBlk = 512;
constexpr uint16_t kHole = 0xFFFF;  // a selection-list lane without a pixel (index leaves with invalid pixels)
constexpr uint32_t kRansWG = 256;   // threads per byte-rANS workgroup
constexpr uint32_t kPairWG = 1024;  // threads per paired workgroup (one per CU: all 32 tables in LDS)

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

__device__ __forceinline__ void report(const DevResident &r, uint32_t b, uint32_t p) {
    atomicCAS(r.err, 0ull, ((unsigned long long)(b + 1) << 32) | p);
}

struct Extent {
    uint64_t start, end;
};

__device__ __forceinline__ Extent locate(const DevResident &r, uint32_t b, uint32_t p, uint64_t base,
                                         uint32_t nbytes) {
    const uint64_t gi = (uint64_t)b * r.G + (p >> 5);
    Extent e;
    e.start = base + r.gbase[gi] + r.rel[gi * 32 + (p & 31)];
    if (p + 1 < r.P) {
        const uint64_t gj = (uint64_t)b * r.G + ((p + 1) >> 5);
        e.end = base + r.gbase[gj] + r.rel[gj * 32 + ((p + 1) & 31)];
    } else {
        e.end = base + nbytes;
    }
    return e;
}

// a * b + c on 24-bit operands (v_mad_u32_u24, full rate), for operands the
// compiler cannot bound itself: past the selects of a mixed decode step it
// widens __umul24 to 32-bit multiplies, which run at a quarter of the rate
__device__ __forceinline__ uint32_t mad24(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// a * b + c on sign-extended 24-bit operands (v_mad_i32_i24, full rate), low 32
// bits: the modulo-2^32 product of operands in [-2^23, 2^23)
__device__ __forceinline__ uint32_t mad24s(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

__device__ __forceinline__ uint32_t ld16(const uint8_t *pay, uint64_t off) {
    return *reinterpret_cast<const uint16_t *>(pay + off);
}

// ------------------------------------------------------------------ bit reservoir
// Next bits of the stream sit at the bottom of r; n bits are valid. The stream
// is read through a buffer resource over one block's payload: 32-bit offsets,
// one add per refill, and reads past the block return zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;

// Block base and size are the same in every lane; readfirstlane keeps the
// descriptor in scalar registers (a per-lane descriptor would serialise loads).
__device__ __forceinline__ Rsrc block_rsrc(const uint8_t *block, uint32_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(block);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    // the range check is per dword and a block may end on a 2-byte boundary: cover
    // its last partial dword (the next block or the device padding follows it)
    const uint32_t nb = __builtin_amdgcn_readfirstlane(nbytes + 16u);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)nb, 0x00020000);
}

__device__ __forceinline__ uint32_t bload(Rsrc rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0);
}

struct BBits {
    uint64_t r;
    uint32_t n;
    uint32_t off;  // block offset of the prefetched dword pf
    uint32_t pf;
};

__device__ __forceinline__ void bbits_init(BBits &s, Rsrc rs, uint32_t start) {
    const uint32_t a = start & ~3u;
    const uint32_t d0 = bload(rs, a), d1 = bload(rs, a + 4);
    s.r = ((uint64_t)d1 << 32) | d0;
    s.n = 64;
    if (start & 2) {
        s.r >>= 16;
        s.n = 48;
    }
    s.off = a + 8;
    s.pf = bload(rs, s.off);
}

__device__ __forceinline__ void bbits_refill(BBits &s, Rsrc rs) {
    if (s.n <= 32) {
        s.r |= (uint64_t)s.pf << s.n;
        s.n += 32;
        s.off += 4;
        s.pf = bload(rs, s.off);
    }
}

// bits consumed since the stream start (block offset start)
__device__ __forceinline__ uint32_t bbits_used(const BBits &s, uint32_t start) {
    return 8u * (s.off - (start & ~3u)) - s.n - ((start & 2) ? 16u : 0u);
}

// Loads one dword of every 128-byte line of a stream so the whole stream is in
// flight towards the caches at once: the decode then waits for one memory
// latency per tile instead of one per line. The values only feed a dummy sum.
__device__ __forceinline__ uint32_t touch_stream(Rsrc rs, uint32_t start, uint32_t len) {
    uint32_t t[9];
#pragma unroll
    for (int i = 0; i < 9; i++) t[i] = (uint32_t)i * 128u < len ? bload(rs, (start & ~3u) + 128u * i) : 0u;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 9; i++) s += t[i];
    return s;
}

template <typename B>
__device__ __forceinline__ uint32_t pop16(B &s) {
    const uint32_t w = (uint32_t)s.r & 0xFFFFu;
    s.r >>= 16;
    s.n -= 16;
    return w;
}

template <typename B>
__device__ __forceinline__ uint32_t popn(B &s, uint32_t nb) {
    const uint32_t v = (uint32_t)s.r & ((1u << nb) - 1u);
    s.r >>= nb;
    s.n -= nb;
    return v;
}

// The 16-bit literal after an escape symbol, from a reservoir known to hold it.
__device__ __forceinline__ uint32_t rans_literal(BBits &s, uint32_t &bad) {
    const uint32_t lit = pop16(s);
    bad |= lit < 255u;
    return lit;
}

// The 16-bit literal after an escape symbol; refills first so it is always there.
__device__ __forceinline__ uint32_t rans_escape(BBits &s, Rsrc rs, uint32_t &bad) {
    bbits_refill(s, rs);
    const uint32_t lit = pop16(s);
    bad |= lit < 255u;
    return lit;
}

// ------------------------------------------------------------------ wave reductions
// Transpose-reduce of CH per-lane accumulators over the 64 lanes of a wave:
// every level pairs two registers and halves their count, so no value is ever
// moved twice. Cross-row levels use the gfx950 lane-swap instructions
// (v_permlane32_swap: lanes l and l+32; v_permlane16_swap: rows of 16), in-row
// levels a DPP-sourced add. Afterwards each lane holds the wave total of one
// scan of the chunk; which one is lane_scan() (found by reducing an index
// probe once, so the result does not depend on the swap direction).
__device__ __forceinline__ uint32_t bf32(uint32_t a, uint32_t b) {
    const auto s = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return s[0] + s[1];
}
__device__ __forceinline__ uint32_t bf16(uint32_t a, uint32_t b) {
    const auto s = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return s[0] + s[1];
}
// DPP level: lanes with (lane & BIT) == 0 keep a, the others keep b; CTRL
// pairs each lane with one of the opposite half.
template <int CTRL, int BIT>
__device__ __forceinline__ uint32_t bfdpp(uint32_t a, uint32_t b) {
    const bool up = lane_id() & BIT;
    const uint32_t keep = up ? b : a, send = up ? a : b;
    return keep + (uint32_t)__builtin_amdgcn_mov_dpp((int)send, CTRL, 0xF, 0xF, false);
}
constexpr int kRowRor8 = 0x128;     // lane i <- i^8 within a row of 16
constexpr int kHalfMirror = 0x141;  // lane i <- 7-i within each 8 lanes (pairs bit 2)
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]

// The first levels: the two lane-swap levels and the first DPP level. After
// them each of the CH / 8 remaining registers holds sums of at most 8 lanes'
// values (the moments reduce those in 32 bits for any detector).
template <int CH>
__device__ __forceinline__ void transpose_head(uint32_t (&a)[CH]) {
    static_assert(CH == 32 || CH == 16 || CH == 8, "chunk of 8, 16 or 32 scans");
#pragma unroll
    for (int i = 0; i < CH / 2; i++) a[i] = bf32(a[i], a[i + CH / 2]);
#pragma unroll
    for (int i = 0; i < CH / 4; i++) a[i] = bf16(a[i], a[i + CH / 4]);
#pragma unroll
    for (int i = 0; i < CH / 8; i++) a[i] = bfdpp<kRowRor8, 8>(a[i], a[i + CH / 8]);
}
// The remaining levels, over a[0 .. CH / 8).
template <int CH>
__device__ __forceinline__ uint32_t transpose_tail(const uint32_t *a) {
    uint32_t v;
    if constexpr (CH == 32) {
        v = bfdpp<kQuadXor2, 2>(bfdpp<kHalfMirror, 4>(a[0], a[2]), bfdpp<kHalfMirror, 4>(a[1], a[3]));
        v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, false);
    } else if constexpr (CH == 16) {
        v = bfdpp<kHalfMirror, 4>(a[0], a[1]);
        v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, false);
    } else {
        v = a[0];
        v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kHalfMirror, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor2, 0xF, 0xF, false);
        v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kQuadXor1, 0xF, 0xF, false);
    }
    return v;
}
template <int CH>
__device__ __forceinline__ uint32_t wave_transpose_sum(uint32_t (&a)[CH]) {
    transpose_head<CH>(a);
    return transpose_tail<CH>(a);
}

// Sum of one value over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Smallest value over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, (uint32_t)__shfl_xor(v, off));
    return v;
}

// Scan (within the chunk) whose total lane_id() holds after wave_transpose_sum,
// and whether this lane is the one that writes it.
template <int CH>
__device__ __forceinline__ uint32_t lane_scan() {
    uint32_t probe[CH];
#pragma unroll
    for (int i = 0; i < CH; i++) probe[i] = lane_id() == 0 ? (uint32_t)i : 0u;
    return wave_transpose_sum<CH>(probe) & (CH - 1);
}
template <int CH>
__device__ __forceinline__ bool lane_writes() {
    return (lane_id() & (64 / CH - 1)) == 0;
}

// Adds the wave totals of one chunk to the LDS partials. A lane's moment term
// is at most 4 slots x 65535 x (dim - 1); over 64 lanes that stays below 2^32
// while both detector dimensions are at most 256 (split = false), and over
// the 8 lanes of the head levels below 2^31 for any detector (dim <= 1024).
// Larger detectors split the head's sums into 16-bit halves for the tail
// levels (8 x 2^16 < 2^32) and recombine them in 64 bits.
// ROWU: every pixel of the wave lies in detector row kru, so the row moment of
// a scan is kru times its total and ar is not used.
template <int CH, Op OP, bool ROWU = false>
__device__ __forceinline__ void chunk_to_lds(uint32_t (&a0)[CH], uint32_t (&ar)[OP == Op::Moments ? CH : 1],
                                             uint32_t (&ac)[OP == Op::Moments ? CH : 1], uint32_t my, bool writer,
                                             bool split, uint32_t *m0, unsigned long long *mr,
                                             unsigned long long *mc, uint32_t kru = 0) {
    const uint32_t t0 = wave_transpose_sum<CH>(a0);
    if (writer && t0) atomicAdd(&m0[my], t0);
    if constexpr (OP == Op::Moments) {
        // the head levels add at most 8 lanes' terms: below 2^31 for any detector
        // (up to 1024 per side); only the tail needs 16-bit halves on large ones
        if constexpr (!ROWU) transpose_head<CH>(ar);
        transpose_head<CH>(ac);
        unsigned long long tr = 0, tc;
        if constexpr (ROWU) tr = (unsigned long long)t0 * kru;
        if (!split) {
            if constexpr (!ROWU) tr = transpose_tail<CH>(ar);
            tc = transpose_tail<CH>(ac);
        } else {
            constexpr int R = CH / 8;
            uint32_t lo[R], hi[R];
            if constexpr (!ROWU) {
#pragma unroll
                for (int i = 0; i < R; i++) {
                    lo[i] = ar[i] & 0xFFFFu;
                    hi[i] = ar[i] >> 16;
                }
                tr = ((unsigned long long)transpose_tail<CH>(hi) << 16) + transpose_tail<CH>(lo);
            }
#pragma unroll
            for (int i = 0; i < R; i++) {
                lo[i] = ac[i] & 0xFFFFu;
                hi[i] = ac[i] >> 16;
            }
            tc = ((unsigned long long)transpose_tail<CH>(hi) << 16) + transpose_tail<CH>(lo);
        }
        if (writer && tr) atomicAdd(&mr[my], tr);
        if (writer && tc) atomicAdd(&mc[my], tc);
    }
}
// ------------------------------------------------------------------ LDS partials of one work item
template <Op OP>
struct Partials {
    uint32_t *m0;            // [512]
    unsigned long long *mr;  // [512] (moments only)
    unsigned long long *mc;
    uint32_t *c0;            // constant per scan (constant streams)
    unsigned long long *cr, *cc;
};

template <Op OP>
__device__ __forceinline__ void add_event(const Partials<OP> &pt, int pos, uint32_t v, uint32_t kr, uint32_t kc) {
    if (pos < 0) {
        atomicAdd(pt.c0, v);
        if (OP == Op::Moments) {
            atomicAdd(pt.cr, (unsigned long long)v * kr);
            atomicAdd(pt.cc, (unsigned long long)v * kc);
        }
    } else {
        atomicAdd(&pt.m0[pos], v);
        if (OP == Op::Moments) {
            atomicAdd(&pt.mr[pos], (unsigned long long)v * kr);
            atomicAdd(&pt.mc[pos], (unsigned long long)v * kc);
        }
    }
}

// ------------------------------------------------------------------ diffraction-pattern tiles
// One (visited block, tile) item of a diffraction-pattern query: the block's
// row of per-pixel partial sums, its selected scans as 16 bitmask words in LDS
// and their number.
struct DpTile {
    uint32_t *row;
    const uint32_t *bits;
    uint32_t n_sel;
};

__device__ __forceinline__ uint32_t scan_bit(const DpTile &dt, uint32_t j) { return (dt.bits[j >> 5] >> (j & 31u)) & 1u; }

// Selected scans of a block as 16 bitmask words (scan j is bit j % 32 of word
// j / 32): one ballot per wave, then the caller synchronises and counts.
template <int WG>
__device__ __forceinline__ void dp_scan_bits(const uint8_t *scan_mask, uint64_t s0, uint32_t n, uint32_t *bits) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    for (uint32_t base = 0; base < 512; base += WG) {
        const uint32_t j = base + tid;
        const bool f = j < n && (!scan_mask || scan_mask[s0 + j] != 0);
        const unsigned long long bal = __ballot(f);
        const uint32_t word = (base + 64 * wave) >> 5;
        if (lane == 0 && word < 16) {
            bits[word] = (uint32_t)bal;
            bits[word + 1] = (uint32_t)(bal >> 32);
        }
    }
}

__device__ __forceinline__ uint32_t dp_count(const uint32_t *bits) {
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) c += __popc(bits[i]);
    return c;
}

// ------------------------------------------------------------------ region output
constexpr bool is_frames(Op op) { return op == Op::Frames || op == Op::Amp; }
constexpr bool is_region(Op op) { return op == Op::Region || is_frames(op); }

// Value v of pixel p in the output row starting at element `row` (one scan):
// the row's address is uniform and the pixel's byte offset a 32-bit lane
// value, so the store needs no 64-bit address arithmetic per lane.
// The amplitudes of counts 0-255 in LDS, staged once per workgroup by the
// amplitude kernels (only their instantiations allocate it): frames of counts
// read their square roots without a global load, whose wait would also hold
// back the reservoir's refill.
__device__ __forceinline__ float *amp_cache() {
    __shared__ float a[256];
    return a;
}
template <int WG>
__device__ __forceinline__ void amp_stage(const RegionArgs &ra) {
    float *a = amp_cache();
    for (uint32_t i = threadIdx.x; i < 256; i += WG) a[i] = ra.amp[i];
}

template <bool WIDE, bool AMP>
__device__ __forceinline__ void region_put(const RegionArgs &ra, uint64_t row, uint32_t p, uint32_t v, double scale,
                                           double offset) {
    // the row is the same in every lane: readfirstlane keeps it in scalar
    // registers, so each lane's address is that base plus its pixel offset
    const uint32_t row_lo = __builtin_amdgcn_readfirstlane((uint32_t)row);
    const uint32_t row_hi = __builtin_amdgcn_readfirstlane((uint32_t)(row >> 32));
    row = ((uint64_t)row_hi << 32) | row_lo;
    uint8_t *out = static_cast<uint8_t *>(ra.out);
    if constexpr (AMP) {
        // counts are at most 65535; the rare larger ones in the wave load their
        // amplitude from the full table and store it over the cached one
        float *dst = reinterpret_cast<float *>(out + 4 * row + 4u * p);
        const uint32_t c = v & 0xFFFFu;
        *dst = amp_cache()[c & 255u];
        if (__builtin_amdgcn_ballot_w64(c > 255u)) {
            if (c > 255u) *dst = ra.amp[c];
        }
    } else if (ra.out_kind == 1) {
        *reinterpret_cast<float *>(out + 4 * row + 4u * p) = (float)__dadd_rn(__dmul_rn((double)v, scale), offset);
    } else if (WIDE) {
        *reinterpret_cast<uint16_t *>(out + 2 * row + 2u * p) = (uint16_t)v;
    } else {
        out[row + p] = (uint8_t)v;
    }
}

// Scan walk of one block for a region read (FRAMES false: scans inside the
// rectangle, at their row of the rectangle) or a frames read (every scan, at
// row s - s_first): (row, col) and index s of scan s0 + j, and the
// calibration of the block.
template <bool FRAMES>
struct RegionWalk {
    uint32_t row, col;
    uint64_t s;
    uint32_t scan_cols;
    uint32_t r0, r1, c0, c1;
    uint64_t s_first;
    double scale, offset;
    __device__ __forceinline__ bool inside() const {
        return FRAMES || (row >= r0 && row < r1 && col >= c0 && col < c1);
    }
    __device__ __forceinline__ uint64_t index(uint32_t P) const {
        if constexpr (FRAMES) return (s - s_first) * P;
        return ((uint64_t)(row - r0) * (c1 - c0) + (col - c0)) * P;
    }
    __device__ __forceinline__ void next() {
        if constexpr (FRAMES) {
            s++;
        } else if (++col == scan_cols) {
            col = 0;
            row++;
        }
    }
    __device__ __forceinline__ void seek(const DevResident &r, uint64_t s_) {
        s = s_;
        if constexpr (!FRAMES) {
            row = (uint32_t)(s_ / r.scan_cols);
            col = (uint32_t)(s_ % r.scan_cols);
        }
    }
};

template <bool FRAMES>
__device__ __forceinline__ RegionWalk<FRAMES> region_walk(const DevResident &r, uint32_t b, const RegionArgs &ra) {
    RegionWalk<FRAMES> rw;
    rw.scan_cols = r.scan_cols;
    rw.seek(r, (uint64_t)b * kBlk);
    rw.r0 = ra.r0;
    rw.r1 = ra.r1;
    rw.c0 = ra.c0;
    rw.c1 = ra.c1;
    rw.s_first = ra.s_first;
    rw.scale = 1.0;
    rw.offset = 0.0;
    if (ra.out_kind == 1) {
        rw.scale = r.calib[2 * b];
        rw.offset = r.calib[2 * b + 1];
    }
    return rw;
}

// A stream whose scans hold one value (constant, or zero): written directly.
template <bool WIDE, Op OP>
__device__ __forceinline__ void region_fill(const DevResident &r, uint32_t b, uint32_t n, uint32_t p, uint32_t v,
                                            const RegionArgs &ra) {
    constexpr bool AMP = OP == Op::Amp;
    auto rw = region_walk<is_frames(OP)>(r, b, ra);
    for (uint32_t j = 0; j < n; j++, rw.next())
        if (rw.inside()) region_put<WIDE, AMP>(ra, rw.index(r.P), p, v, rw.scale, rw.offset);
}

// ------------------------------------------------------------------ staged stream window
// A uint16 byte-rANS stream whose symbol 255 (escape) is frequent spends up to
// 32 bits a step: a renormalisation word and a 16-bit literal. Refilled one
// dword at a time from a lane's own stream, it sends one cache-line request
// per 4 bytes, and with thousands of streams in flight per CU each line has
// left the L1 before its next dword is read: the L1 then misses on nearly
// every access and its queue of misses bounds the decode.
//
// The staged form moves each stream in 32-byte chunks instead. Every kStageC
// steps (a cadence the whole wave shares) a lane whose older ring half has
// been consumed requests the next chunk with two 16-byte loads, and at the
// next cadence writes it into its ring in LDS. Every lane issues the loads at
// every cadence, and a lane with no request addresses past the buffer range
// (the hardware returns zero and reads no memory), so the compiler's wait
// before the write counts them exactly. A step reads its two candidate words
// (renormalisation, literal) as one word pair from the ring. A step consumes
// at most two words, and a cadence of 4 steps with a two-chunk ring keeps a
// lane's next two words written before it reads them.
constexpr uint32_t kStageC = 4;    // steps between cadence points
constexpr uint32_t kStageDw = 17;  // ring dwords per stream: two chunks of 8 and a copy of dword 0
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

__device__ __forceinline__ u32x4 bload4(Rsrc rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
}

// Slot s of a block's decode table as fe = f | symbol << 24 (v_mad_u32_u24
// reads only f) and bias = s - c[symbol]: two words per slot, read together, or
// (T32) one word f | bias << 12 | symbol << 24.
template <bool T32>
__device__ __forceinline__ void tbl_read(const uint32_t *tbl, uint32_t s, uint32_t &fe, uint32_t &bias) {
    if constexpr (T32) {
        const uint32_t w = tbl[s];
        fe = w & 0xFF000FFFu;
        bias = __builtin_amdgcn_ubfe(w, 12, 12);
    } else {
        const uint2 w = reinterpret_cast<const uint2 *>(tbl)[s];
        fe = w.x;
        bias = w.y;
    }
}

struct Stage {
    uint32_t wi;    // next word of the stream, counted from the start of chunk 0
    uint32_t fl;    // chunks requested (the latest is written at the next cadence)
    uint32_t c0;    // chunk 0's offset in the staging range (a 32-byte boundary)
    uint32_t endc;  // the stream's end in that range: no chunk starts at or past it
    bool pend;      // a chunk is in flight
    u32x4 q0, q1;   // its two halves
};

// Dword i of a lane's ring, stored lane-major (dword i of the 64 lanes side by
// side) so the lanes of a wave fall in distinct banks whatever their i.
__device__ __forceinline__ void ring_put8(uint32_t *q, const u32x4 &a, const u32x4 &b) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        q[64 * i] = a[i];
        q[64 * (4 + i)] = b[i];
    }
}

// ------------------------------------------------------------------ byte-rANS tile
// Per-slot state kept in registers across the 512 steps (kept small: the tile
// holds up to two slots per lane).
struct RSlot {
    uint32_t x;     // rANS state
    uint32_t hold;  // second byte of a RAW uint8 word
    uint32_t p;     // detector pixel
    uint32_t org;   // stream start within the block payload
    uint32_t len;   // stream bytes
    BBits s;
    bool raw;       // RAW stream, or an idle slot (raw over an empty range: every read is 0)
    bool live;      // a RANS or RAW stream is decoded in this slot
};

// Every slot steps through the same instructions whatever its mode: a RAW
// stream is a renormalisation that always takes a word, and an idle slot is a
// RAW stream whose reads fall outside the buffer range and return zero. With
// no per-slot branches the K table reads of a step issue together.
//
// half: 0 decodes whole streams; 1 the first kSplit scans of each stream
// (checked against its split point); 2 the rest, resumed from the split point
// (a complete block's streams then take two lanes, one per half).
//
// STG: escape-heavy waves take the staged form, with `ring` the workgroup's
// stream rings (kStageDw x 64 dwords per wave), and the block table has one
// word per slot.
template <int K, bool WIDE, Op OP, bool STG = false>
__device__ __forceinline__ void rans_tile(const DevResident &r, const uint16_t *sel, uint32_t p0, uint32_t n_sel, uint32_t first, uint32_t b,
                          uint32_t n, uint64_t base, uint32_t nbytes, const uint32_t *tbl, const Partials<OP> &pt,
                          const RegionArgs &ra, const DpTile &dt, uint32_t half = 0, bool raw_block = false,
                          uint32_t *ring = nullptr, bool touch = true) {
    const Rsrc rs = block_rsrc(r.payload + base, nbytes);
    const uint32_t lane = lane_id();
    const uint32_t maxv = WIDE ? 65535u : 255u;
    RSlot sl[K];
    uint32_t bad = 0, touched = 0, cst = 0;
#pragma unroll
    for (int k = 0; k < K; k++) {
        RSlot &z = sl[k];
        z.x = 0;
        z.hold = 0;
        z.p = 0;
        z.raw = true;
        z.live = false;
        z.s.r = 0;
        z.s.n = 64;
        // outside the range (a block is far below 2 GB) and it cannot wrap back in: loads return 0
        z.s.off = 0x80000000u;
        z.s.pf = 0;
        const uint32_t i = first + k * 64 + lane;
        if (i >= n_sel || sel[i] == kHole) continue;
        z.p = p0 + sel[i];
        const Extent e = locate(r, b, z.p, base, nbytes);
        z.org = (uint32_t)(e.start - base);
        z.len = (uint32_t)(e.end - e.start);
        const uint32_t hdr = ld16(r.payload, e.start);
        const uint32_t mode = hdr & 7u;
        if (mode == 0) {  // CONST
            if (half == 2 || OP == Op::Split) continue;  // folded once, by the first half
            const uint32_t v = ld16(r.payload, e.start + 2);
            if (z.len != 4 || v > maxv) {
                report(r, b, z.p);
                continue;
            }
            if constexpr (is_region(OP)) {
                region_fill<WIDE, OP>(r, b, n, z.p, v, ra);
            } else if constexpr (OP == Op::Dp) {
                dt.row[z.p] = v * dt.n_sel;
            } else if constexpr (OP == Op::Index) {
                cst += v;  // a constant stream adds v to every scan of the leaf row
            } else {
                const uint32_t kr = z.p / r.det_cols;
                if (v) add_event<OP>(pt, -1, v, kr, z.p - kr * r.det_cols);
            }
            continue;
        }
        z.live = true;
        z.raw = mode == 2;
        // a RAW stream that a RAW-only wave of a sum (or of moments on a detector
        // of at most 256 per side) reads with whole-wave loads: no prefetch here,
        // since the in-order load counter would make the first wait of that form
        // wait for all of it
        const bool raw_whole = (OP == Op::Sum || OP == Op::Moments) && K == 1 && raw_block && z.raw &&
                               (OP == Op::Sum || (r.det_cols <= 256 && r.P / r.det_cols <= 256));
        if (half == 2) {
            // resume where the first half ends: a RAW stream at its value kSplit, a
            // RANS stream at its split point (state, byte offset from the stream start)
            const uint64_t si = 2 * ((uint64_t)b * r.P + z.p);
            const uint32_t off = z.raw ? 2u + kSplit * (WIDE ? 2u : 1u) : r.split[si + 1];
            if (!raw_whole && touch) touched += touch_stream(rs, z.org + off, z.len > off ? z.len - off : 0u);
            bbits_init(z.s, rs, z.org + off);
            if (!z.raw) z.x = r.split[si];
        } else {
            if (!raw_whole && touch) touched += touch_stream(rs, z.org, z.len);
            bbits_init(z.s, rs, z.org);
            pop16(z.s);  // header
            if (mode == 1) {
                z.x = pop16(z.s);
                z.x |= pop16(z.s) << 16;
            }
        }
        bbits_refill(z.s, rs);
    }
    uint32_t kr[OP == Op::Moments ? K : 1], kc[OP == Op::Moments ? K : 1];
    if (OP == Op::Moments) {
#pragma unroll
        for (int k = 0; k < K; k++) {
            kr[k] = sl[k].p / r.det_cols;
            kc[k] = sl[k].p - kr[k] * r.det_cols;
        }
    }
    // moments of a wave whose pixels share one detector row (a wave of
    // consecutive pixels that does not cross a row end): the row moment comes
    // from the per-scan totals, one multiply per scan instead of one per value
    bool rowu = false;
    uint32_t kru = 0;
    if constexpr (OP == Op::Moments) {
        const uint64_t lv = __builtin_amdgcn_ballot_w64(sl[0].live);
        if (lv) {
            kru = (uint32_t)__builtin_amdgcn_readlane((int)kr[0], (int)__builtin_ctzll(lv));
            bool diff = false;
#pragma unroll
            for (int k = 0; k < K; k++) diff |= sl[k].live && kr[k] != kru;
            rowu = !__builtin_amdgcn_ballot_w64(diff);
        }
    }
    // Packed row moments: in such a wave, when the block codes no symbol above
    // 127 and the live columns span at most 128, one accumulator per scan holds
    // the sum of the values (bits 0-11) and their column moment relative to the
    // wave's first live column (bits 12-31): one 24-bit multiply-add per value
    // with the weight 1 + (column offset << 12). Over 16 lanes of two slots both
    // fields stay below their widths (16 x 2 x 127 = 4064 < 2^12, 4064 x 127 <
    // 2^20), so the first four reduction levels run packed and the last two per
    // field. Only the plain form (no escapes, no RAW slots) takes it.
    bool rowp = false;
    uint32_t kcw = 0, wgt[OP == Op::Moments ? K : 1];
    if constexpr (OP == Op::Moments && !STG) {
        if (rowu && (tbl[2 * 4095] >> 24) <= 127u) {
            uint32_t m = 0xFFFFFFFFu;
#pragma unroll
            for (int k = 0; k < K; k++)
                if (sl[k].live) m = min(m, kc[k]);
            kcw = wave_min(m);
            bool far = false;
#pragma unroll
            for (int k = 0; k < K; k++) far |= sl[k].live && kc[k] - kcw > 127u;
            rowp = !__builtin_amdgcn_ballot_w64(far);
#pragma unroll
            for (int k = 0; k < K; k++) wgt[k] = sl[k].live ? 1u + ((kc[k] - kcw) << 12) : 0u;
        }
    }

    // byte-rANS decode step (FORMAT 2.3). The block table holds two words per
    // slot, side by side and read by one 64-bit LDS load: f | symbol << 24
    // (v_mad_u32_u24 reads only the low 24 bits, so the symbol rides along) and
    // slot - c[symbol] (one word per slot under STG: see tbl_read). A renormalisation appends the next 16-bit word with one
    // byte permute; an escape (symbol 255 of a uint16 stream) reads its literal.
    //
    // One step of every slot: values in v[], escapes resolved. Three forms of
    // the same step, chosen once per wave:
    //  kMixed   some slot is RAW or idle: every slot runs the unified step;
    //  kEscape  all slots are rANS and the block's table codes symbol 255;
    //  kPlain   all slots are rANS and no escape can occur.
    //  kStaged  (STG) as kEscape, with the stream words read from LDS rings.
    constexpr int kMixed = 0, kEscape = 1, kPlain = 2, kStaged = 3;
    static_assert(!STG || K == 1, "the staged form decodes one stream per lane");
    Stage sg[STG ? K : 1];
    uint32_t *rk[STG ? K : 1];
    if constexpr (STG) rk[0] = ring + (threadIdx.x >> 6) * kStageDw * 64 + lane;
    auto step = [&](auto form, bool even, uint32_t (&v)[K]) {
        constexpr int F = decltype(form)::value;
        if constexpr (F == kStaged) {
            // the step of the escape form, its two candidate words taken from
            // the ring as one pair (words wi and wi + 1)
            uint32_t e[K], bias[K], w2[K];
#pragma unroll
            for (int k = 0; k < K; k++) {
                tbl_read<STG>(tbl, sl[k].x & 4095u, e[k], bias[k]);
                const uint32_t *q = rk[k] + ((sg[k].wi >> 1) & 15u) * 64u;
                w2[k] = __builtin_amdgcn_alignbit(q[64], q[0], sg[k].wi << 4);
            }
#pragma unroll
            for (int k = 0; k < K; k++) {
                RSlot &z = sl[k];
                const uint32_t xn = __umul24(e[k], z.x >> 12) + bias[k];
                const bool need = xn < 65536u;
                z.x = need ? __builtin_amdgcn_perm(xn, w2[k], 0x05040100u) : xn;
                const uint32_t lit = need ? w2[k] >> 16 : w2[k] & 0xFFFFu;
                const uint32_t sym = e[k] >> 24;
                const bool esc = sym == 255u;
                v[k] = esc ? lit : sym;
                bad |= (uint32_t)(esc && lit < 255u);
                sg[k].wi += (uint32_t)need + (uint32_t)esc;
            }
            return;
        }
        uint32_t e[K], bias[K];
#pragma unroll
        for (int k = 0; k < K; k++) tbl_read<STG>(tbl, sl[k].x & 4095u, e[k], bias[k]);
        bool esc_any = false;
        bool esc[K];
#pragma unroll
        for (int k = 0; k < K; k++) {
            RSlot &z = sl[k];
            const uint32_t xn = __umul24(e[k], z.x >> 12) + bias[k];
            const uint32_t sym = e[k] >> 24;
            const uint32_t w = (uint32_t)z.s.r;
            bool need;
            if constexpr (F == kMixed) {
                // a RAW uint8 word covers an even scan and the odd scan after it
                const bool raw_take = WIDE || even;
                need = z.raw ? raw_take : xn < 65536u;
            } else {
                need = xn < 65536u;
            }
            z.x = need ? __builtin_amdgcn_perm(xn, w, 0x05040100u) : xn;
            const uint32_t sh = need ? 16u : 0u;
            z.s.r >>= sh;
            z.s.n -= sh;
            if constexpr (F == kMixed) {
                uint32_t rv;
                if (WIDE) {
                    rv = w & 0xFFFFu;
                } else if (even) {
                    rv = w & 0xFFu;
                    z.hold = z.raw ? (w >> 8) & 0xFFu : z.hold;
                } else {
                    rv = z.hold;
                }
                v[k] = z.raw ? rv : sym;
                esc[k] = WIDE && !z.raw && sym == 255u;
            } else {
                v[k] = sym;
                esc[k] = F == kEscape && sym == 255u;
            }
            esc_any |= esc[k];
        }
        if (WIDE && F != kPlain && __builtin_amdgcn_ballot_w64(esc_any)) {  // rare: escapes of uint16 streams
#pragma unroll
            for (int k = 0; k < K; k++)
                if (esc[k]) v[k] = F == kEscape ? rans_literal(sl[k].s, bad) : rans_escape(sl[k].s, rs, bad);
        }
    };
    // Refill on a wave-uniform cadence: two steps use at most 32 bits (an escape
    // refills on its own), so the dword prefetched at the previous cadence point
    // has a full period to arrive.
    auto refill = [&]() {
#pragma unroll
        for (int k = 0; k < K; k++) bbits_refill(sl[k].s, rs);
    };
    // The plain form's sums and moments refill on demand in waves of dim
    // streams: a step takes at most one 16-bit word, so the wave refills when
    // some lane holds fewer than 16 bits, and then every lane with room for a
    // dword takes one. The lanes' refills fall together, every several steps
    // instead of every second one. A wave holding a stream of more than 5
    // coded bits per value (renormalising in a third of its steps or more)
    // would refill about every step that way, so it keeps the cadence.
    bool dim = true;
#pragma unroll
    for (int k = 0; k < K; k++) dim &= !sl[k].live || sl[k].raw || 8u * sl[k].len <= 5u * n;
    const bool ondemand = !__builtin_amdgcn_ballot_w64(!dim);
    auto refill_low = [&]() {
        bool low = false;
#pragma unroll
        for (int k = 0; k < K; k++) low |= sl[k].s.n < 16u;
        if (__builtin_amdgcn_ballot_w64(low)) refill();
    };
    // The staged form's range: the block from the 32-byte boundary at or
    // below its start, so chunk loads are aligned.
    const uint32_t delta = STG ? (uint32_t)reinterpret_cast<uint64_t>(r.payload + base) & 31u : 0u;
    const Rsrc rs2 = STG ? block_rsrc(r.payload + base - delta, nbytes + delta) : rs;
    // its cadence: write the chunk that landed, then request the next where
    // the ring half it goes to has been consumed (see the staged window above)
    auto cadence = [&]() {
#pragma unroll
        for (int k = 0; k < K; k++) {
            const Stage &g = sg[k];
            if (g.pend) {
                const uint32_t half_i = (g.fl - 1u) & 1u;
                ring_put8(rk[k] + half_i * 8u * 64u, g.q0, g.q1);
                if (half_i == 0) rk[k][16 * 64] = g.q0[0];
            }
        }
#pragma unroll
        for (int k = 0; k < K; k++) {
            Stage &g = sg[k];
            const bool req = sl[k].live && g.wi >= 16u * (g.fl - 1u) && g.c0 + 32u * g.fl < g.endc;
            const uint32_t o = req ? g.c0 + 32u * g.fl : 0x80000000u;
            g.q0 = bload4(rs2, o);
            g.q1 = bload4(rs2, o + 16u);
            g.pend = req;
            g.fl += req ? 1u : 0u;
        }
    };
    // the staged form's start: the words after those the reservoir has taken
    // (header and state, or the split point), chunks 0 and 1 in the ring
    auto stage_init = [&]() {
#pragma unroll
        for (int k = 0; k < K; k++) {
            Stage &g = sg[k];
            const RSlot &z = sl[k];
            const uint32_t rel = z.org + bbits_used(z.s, z.org) / 8u + delta;
            g.c0 = rel & ~31u;
            g.wi = (rel - g.c0) >> 1;
            g.endc = z.live ? z.org + z.len + delta : 0u;
            g.fl = 2;
            g.pend = false;
            const uint32_t o = z.live ? g.c0 : 0x80000000u;
            const u32x4 a = bload4(rs2, o), bq = bload4(rs2, o + 16u), c = bload4(rs2, o + 32u), d = bload4(rs2, o + 48u);
            ring_put8(rk[k], a, bq);
            ring_put8(rk[k] + 8u * 64u, c, d);
            rk[k][16 * 64] = a[0];
        }
    };

    auto run = [&](auto form, auto rowu, auto od) {
        constexpr bool ROWU = decltype(rowu)::value != 0;  // moments of a wave inside one detector row
        constexpr bool ROWP = decltype(rowu)::value == 2;  // packed row moments
        constexpr bool OD = decltype(od)::value;           // sums and moments refill on demand (plain form, dim wave)
        // the escape form refills after every step: a step then starts with at
        // least 33 bits, enough for a renormalisation word and a literal, so an
        // escape reads its literal without a load of its own
        constexpr bool every = decltype(form)::value == kEscape;
        constexpr bool staged = decltype(form)::value == kStaged;  // sums and moments only
        if constexpr (is_region(OP)) {
            // values of scans inside the rectangle go straight to the output;
            // frames store every step, and a shorter unroll keeps their
            // calibrated (float64) path out of spills
            constexpr int CH = is_frames(OP) ? 4 : 16;
            auto rw = region_walk<is_frames(OP)>(r, b, ra);
            // a split item's lanes cover kSplit scans from 0 (first half) or kSplit (second)
            const uint32_t nsteps = half == 0 ? n : (half == 1 ? kSplit : n - kSplit);
            if (half == 2) rw.seek(r, (uint64_t)b * kBlk + kSplit);
            auto put = [&](const uint32_t (&v)[K]) {
                if (rw.inside()) {
                    const uint64_t idx = rw.index(r.P);
#pragma unroll
                    for (int k = 0; k < K; k++)
                        if (sl[k].live) region_put<WIDE, OP == Op::Amp>(ra, idx, sl[k].p, v[k], rw.scale, rw.offset);
                }
                rw.next();
            };
            const uint32_t nfull = nsteps / CH;
            for (uint32_t c = 0; c < nfull; c++) {
                if constexpr (is_frames(OP)) {
                    // Stores wait in the same in-order counter as loads, so a refill
                    // would also wait for the stores of the steps just before it:
                    // frames store each pair of steps after its refill, so those
                    // stores get a whole cadence to complete, like the prefetch.
                    // (A rectangle stores few steps; there the order is unchanged.)
#pragma unroll
                    for (int jj = 0; jj < CH; jj += 2) {
                        uint32_t v0[K], v1[K];
                        step(form, true, v0);
                        if (every) refill();
                        __builtin_amdgcn_sched_barrier(0);
                        step(form, false, v1);
                        refill();
                        put(v0);
                        put(v1);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
#pragma unroll
                    for (int jj = 0; jj < CH; jj++) {
                        uint32_t v[K];
                        step(form, (jj & 1) == 0, v);
                        put(v);
                        if (every || (jj & 1)) refill();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            for (uint32_t j = nfull * CH; j < nsteps; j++) {
                uint32_t v[K];
                step(form, (j & 1) == 0, v);
                put(v);
                if (every || (j & 1) || j + 1 == nsteps) refill();
            }
        } else if constexpr (OP == Op::Dp) {
            // per-lane sums over the selected scans, no reduction across lanes
            constexpr int CH = 32;
            uint32_t acc[K];
#pragma unroll
            for (int k = 0; k < K; k++) acc[k] = 0;
            const uint32_t nfull = n / CH;
            for (uint32_t c = 0; c < nfull; c++) {
                const uint32_t word = dt.bits[c];
#pragma unroll
                for (int jj = 0; jj < CH; jj++) {
                    uint32_t v[K];
                    step(form, (jj & 1) == 0, v);
                    const uint32_t m = (word >> jj) & 1u;
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        acc[k] = __umul24(v[k], m) + acc[k];
                        asm volatile("" : "+v"(acc[k]));  // keep the sum in the loop (see the reduce chunks)
                    }
                    if (every || (jj & 1)) refill();
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            for (uint32_t j = nfull * CH; j < n; j++) {
                uint32_t v[K];
                step(form, (j & 1) == 0, v);
                const uint32_t m = scan_bit(dt, j);
#pragma unroll
                for (int k = 0; k < K; k++) acc[k] = __umul24(v[k], m) + acc[k];
                if (every || (j & 1) || j + 1 == n) refill();
            }
#pragma unroll
            for (int k = 0; k < K; k++)
                if (sl[k].live) dt.row[sl[k].p] = acc[k];
        } else if constexpr (OP == Op::Split) {
            // decode the first kSplit scans only; the state and position are stored below
            for (uint32_t j = 0; j < kSplit; j++) {
                uint32_t v[K];
                step(form, (j & 1) == 0, v);
                if (every || (j & 1)) refill();
            }
        } else {
            constexpr int CH = 16;
            const uint32_t my = lane_scan<CH>();
            const bool writer = lane_writes<CH>();
            const bool split = r.det_cols > 256 || r.P / r.det_cols > 256;
            // the scans this lane's half covers: [j0, j0 + nsteps)
            const uint32_t j0 = half == 2 ? kSplit : 0u, nsteps = half == 0 ? n : (half == 1 ? kSplit : n - kSplit);
            const uint32_t nfull = nsteps / CH;
            const uint32_t cw = OP == Op::Index ? wave_sum(cst) : 0u;  // the leaf's constant streams
            for (uint32_t c = 0; c < nfull; c++) {
                uint32_t a0[CH];
                uint32_t ar[OP == Op::Moments ? CH : 1], ac[OP == Op::Moments ? CH : 1];
#pragma unroll
                for (int i = 0; i < CH; i++) {
                    a0[i] = 0;
                    if (OP == Op::Moments) {
                        ar[i] = 0;
                        ac[i] = 0;
                    }
                }
#pragma unroll
                for (int jj = 0; jj < CH; jj++) {
                    uint32_t v[K];
                    step(form, (jj & 1) == 0, v);  // chunks start at even scans
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        if constexpr (ROWP) {
                            a0[jj] = mad24(v[k], wgt[k], a0[jj]);
                            continue;
                        }
                        a0[jj] += v[k];
                        if (OP == Op::Moments) {
                            // 24-bit multiplies run at full rate
                            if constexpr (decltype(form)::value == kMixed) {
                                ar[jj] = mad24(v[k], kr[k], ar[jj]);
                                ac[jj] = mad24(v[k], kc[k], ac[jj]);
                            } else {
                                if constexpr (!ROWU) ar[jj] += __umul24(v[k], kr[k]);
                                ac[jj] += __umul24(v[k], kc[k]);
                            }
                        }
                    }
                    // materialise the sums here: deferring them to the chunk end keeps every step's table entry live
                    asm volatile("" : "+v"(a0[jj]));
                    if constexpr (OP == Op::Moments && !ROWU) asm volatile("" : "+v"(ar[jj]), "+v"(ac[jj]));
                    if constexpr (OP == Op::Moments && ROWU && !ROWP) asm volatile("" : "+v"(ac[jj]));
                    if constexpr (staged) {
                        if (jj % kStageC == kStageC - 1) cadence();
                    } else if constexpr (OD) {
                        refill_low();
                    } else if (every || (jj & 1)) {
                        refill();
                    }
                    // keep the scheduler's interleaving to the K independent slots of one step
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (OP == Op::Index) {
                    // one leaf per wave: its per-scan totals go to the leaf's index row
                    const uint32_t t0 = wave_transpose_sum<CH>(a0) + cw;
                    if (writer && t0) atomicAdd(&dt.row[(first >> 6) * kBlk + c * CH + my], t0);
                } else if constexpr (ROWP) {
                    transpose_head<CH>(a0);
                    const uint32_t pv = bfdpp<kHalfMirror, 4>(a0[0], a0[1]);  // 16 lanes
                    uint32_t t0 = pv & 0xFFFu, tc = pv >> 12;
                    t0 += (uint32_t)__builtin_amdgcn_mov_dpp((int)t0, kQuadXor2, 0xF, 0xF, false);
                    tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor2, 0xF, 0xF, false);
                    t0 += (uint32_t)__builtin_amdgcn_mov_dpp((int)t0, kQuadXor1, 0xF, 0xF, false);
                    tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor1, 0xF, 0xF, false);
                    if (writer && t0) {
                        // totals at most 64 x 2 x 127, column moments below 2^21 + 2^24
                        const uint32_t j = j0 + c * CH + my;
                        atomicAdd(&pt.m0[j], t0);
                        atomicAdd(&pt.mc[j], (unsigned long long)mad24(kcw, t0, tc));
                        atomicAdd(&pt.mr[j], (unsigned long long)mad24(kru, t0, 0u));
                    }
                } else {
                    chunk_to_lds<CH, OP, ROWU>(a0, ar, ac, my, writer, split, pt.m0 + j0 + c * CH,
                                               pt.mr + j0 + c * CH, pt.mc + j0 + c * CH, kru);
                }
            }
            // ragged end of a final partial block (never split): one scan at a time, reduced per scan
            for (uint32_t j = nfull * CH; j < nsteps; j++) {
                uint32_t v[K];
                step(form, (j & 1) == 0, v);
                uint32_t t0 = 0, tr = 0, tc = 0;
#pragma unroll
                for (int k = 0; k < K; k++) {
                    t0 += v[k];
                    if (OP == Op::Moments) {
                        tr += __umul24(v[k], kr[k]);
                        tc += __umul24(v[k], kc[k]);
                    }
                }
                if constexpr (OP == Op::Index) {
                    t0 = wave_sum(t0) + cw;
                    if (lane == 0 && t0) atomicAdd(&dt.row[(first >> 6) * kBlk + j], t0);
                    if constexpr (OD)
                        refill_low();
                    else if (every || (j & 1) || j + 1 == n)
                        refill();
                    continue;
                }
                if (t0) atomicAdd(&pt.m0[j], t0);
                if (OP == Op::Moments) {
                    if (tr) atomicAdd(&pt.mr[j], (unsigned long long)tr);
                    if (tc) atomicAdd(&pt.mc[j], (unsigned long long)tc);
                }
                if constexpr (staged) {
                    if (j % kStageC == kStageC - 1) cadence();
                } else if constexpr (OD) {
                    refill_low();
                } else if (every || (j & 1) || j + 1 == n) {
                    refill();
                }
            }
        }
    };

    // RAW-only waves of sums and moments (a block's RAW streams are ordered
    // first, so they fill waves of their own): no reservoir and no per-step
    // branch.
    if constexpr ((OP == Op::Sum || OP == Op::Moments) && K == 1) {
        bool rans_live = false;
#pragma unroll
        for (int k = 0; k < K; k++) rans_live |= sl[k].live && !sl[k].raw;
        if (raw_block && !__builtin_amdgcn_ballot_w64(rans_live)) {
            constexpr uint32_t W = WIDE ? 2u : 1u;  // bytes per value
            const bool split = r.det_cols > 256 || r.P / r.det_cols > 256;
            const uint32_t j0 = half == 2 ? kSplit : 0u, nsteps = half == 0 ? n : (half == 1 ? kSplit : n - kSplit);
            if (OP == Op::Sum || !split) {
                // The wave reads its streams together: a stream's range of nsteps
                // scans takes G = 64, 32 or 16 lanes (8 scans each; enough for
                // nsteps), so one load instruction covers 64 / G streams. Lane l
                // loads the 8 values of scans [8 (l mod G), 8 (l mod G) + 8) of its
                // group's stream (one 8 W-byte load and the next dword, 4-byte
                // aligned and shifted into place), and keeps the totals of those 8
                // scans over all the streams of its group: no reduction across
                // lanes is needed. Over at most 64 streams, a moment total stays
                // below 2^32 while both detector dimensions are at most 256.
                // Streams are taken in lane order (a scalar bit scan; offsets,
                // rows and columns read from their lanes), each one's loads issued
                // two iterations ahead; past the last stream the loads fall
                // outside the buffer and add zeros.
                constexpr uint32_t E = 8;       // values per lane per stream
                constexpr int NW = 2 * (int)W;  // their dwords
                const uint32_t G = nsteps > 256 ? 64u : (nsteps > 128 ? 32u : 16u);
                const uint32_t gl = lane & (G - 1), grp = lane / G, ng = 64u / G;
                const uint32_t span = nsteps * W;
                uint32_t km[NW];
#pragma unroll
                for (int i = 0; i < NW; i++) {
                    const int rem = (int)span - (int)(8u * W * gl + 4u * (uint32_t)i);
                    km[i] = rem >= 4 ? ~0u : (rem <= 0 ? 0u : (1u << (8 * rem)) - 1u);
                }
                uint32_t a0[E], ar[OP == Op::Moments ? E : 1], ac[OP == Op::Moments ? E : 1];
#pragma unroll
                for (uint32_t t = 0; t < E; t++) {
                    a0[t] = 0;
                    if constexpr (OP == Op::Moments) {
                        ar[t] = 0;
                        ac[t] = 0;
                    }
                }
                const uint32_t so = sl[0].live ? sl[0].org + 2u + j0 * W : 0u;  // this lane's stream, first value of the range
                uint64_t left = __builtin_amdgcn_ballot_w64(sl[0].live);
                const uint32_t nl = (uint32_t)__builtin_popcountll(left);
                struct Pick {
                    uint32_t vs, sh, kr, kc;
                };
                // the next stream of each group, in this lane's registers
                auto pick = [&]() {
                    Pick s{0x80000000u, 0u, 0u, 0u};
#pragma unroll
                    for (uint32_t g = 0; g < 4; g++) {
                        if (g >= ng || !left) break;
                        const int l = (int)__builtin_ctzll(left);
                        left &= left - 1;
                        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)so, l);
                        const bool mine = grp == g;
                        s.vs = mine ? o & ~3u : s.vs;
                        s.sh = mine ? (o & 3u) * 8u : s.sh;
                        if constexpr (OP == Op::Moments) {
                            const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)kr[0], l);
                            const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)kc[0], l);
                            s.kr = mine ? a : s.kr;
                            s.kc = mine ? c : s.kc;
                        }
                    }
                    return s;
                };
                auto load = [&](uint32_t (&d)[NW + 1], const Pick &s) {
                    const uint32_t o = s.vs + 8u * W * gl;
                    if constexpr (WIDE) {
                        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)o, 0, 0);
                        d[0] = v[0];
                        d[1] = v[1];
                        d[2] = v[2];
                        d[3] = v[3];
                    } else {
                        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)o, 0, 0);
                        d[0] = v[0];
                        d[1] = v[1];
                    }
                    d[NW] = bload(rs, o + 4u * NW);
                };
                auto add = [&](const uint32_t (&d)[NW + 1], const Pick &s) {
#pragma unroll
                    for (int i = 0; i < NW; i++) {
                        const uint32_t e = __builtin_amdgcn_alignbit(d[i + 1], d[i], s.sh) & km[i];
#pragma unroll
                        for (int q = 0; q < (int)(4 / W); q++) {
                            const int t = i * (int)(4 / W) + q;
                            const uint32_t v = WIDE ? __builtin_amdgcn_ubfe(e, 16 * q, 16) : __builtin_amdgcn_ubfe(e, 8 * q, 8);
                            a0[t] += v;
                            if constexpr (OP == Op::Moments) {
                                ar[t] = mad24(v, s.kr, ar[t]);
                                ac[t] = mad24(v, s.kc, ac[t]);
                            }
                        }
                    }
                };
                uint32_t dA[NW + 1], dB[NW + 1], dC[NW + 1];
                Pick sA = pick(), sB = pick(), sC;
                load(dA, sA);
                load(dB, sB);
                for (uint32_t i = 0; i < nl; i += 3 * ng) {
                    sC = pick();
                    load(dC, sC);
                    add(dA, sA);
                    sA = pick();
                    load(dA, sA);
                    add(dB, sB);
                    sB = pick();
                    load(dB, sB);
                    add(dC, sC);
                }
#pragma unroll
                for (uint32_t t = 0; t < E; t++) {
                    const uint32_t j = gl * E + t;
                    if (j >= nsteps) continue;
                    if (a0[t]) atomicAdd(&pt.m0[j0 + j], a0[t]);
                    if constexpr (OP == Op::Moments) {
                        if (ar[t]) atomicAdd(&pt.mr[j0 + j], (unsigned long long)ar[t]);
                        if (ac[t]) atomicAdd(&pt.mc[j0 + j], (unsigned long long)ac[t]);
                    }
                }
            } else {
                // Moments on larger detectors: each slot's values are read a 16-scan
                // chunk at a time (two 16-byte loads and one dword, 4-byte aligned,
                // shifted into place with a funnel shift) and reduced across lanes
                // per chunk; each chunk's loads are issued two chunks ahead,
                // unconditionally, so every wait is for a load two chunks old.
                constexpr int CH = 16;
                constexpr int ND = CH * (int)W / 4;     // dwords of one chunk's values
                const uint32_t my = lane_scan<CH>();
                const bool writer = lane_writes<CH>();
                const uint32_t nfull = nsteps / CH;
                uint32_t vs[K], sh[K];
#pragma unroll
                for (int k = 0; k < K; k++) {
                    // an idle slot reads outside the buffer range: zeros
                    const uint32_t s0 = sl[k].live ? sl[k].org + 2u + j0 * W : 0x80000000u;
                    vs[k] = s0 & ~3u;
                    sh[k] = (s0 & 3u) * 8u;
                }
                uint32_t bufA[K][ND + 1], bufB[K][ND + 1], bufC[K][ND + 1];
                auto load = [&](uint32_t (&d)[K][ND + 1], uint32_t c) {
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        const uint32_t o = vs[k] + c * (CH * W);
#pragma unroll
                        for (int q = 0; q < ND / 4; q++) {
                            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(o + 16u * q), 0, 0);
                            d[k][4 * q] = v[0];
                            d[k][4 * q + 1] = v[1];
                            d[k][4 * q + 2] = v[2];
                            d[k][4 * q + 3] = v[3];
                        }
                        d[k][ND] = bload(rs, o + 4u * ND);
                    }
                };
                auto chunk = [&](const uint32_t (&d)[K][ND + 1], uint32_t c) {
                    uint32_t a0[CH];
                    uint32_t ar[OP == Op::Moments ? CH : 1], ac[OP == Op::Moments ? CH : 1];
#pragma unroll
                    for (int i = 0; i < CH; i++) {
                        a0[i] = 0;
                        if (OP == Op::Moments) {
                            ar[i] = 0;
                            ac[i] = 0;
                        }
                    }
#pragma unroll
                    for (int k = 0; k < K; k++) {
#pragma unroll
                        for (int i = 0; i < ND; i++) {
                            const uint32_t e = __builtin_amdgcn_alignbit(d[k][i + 1], d[k][i], sh[k]);
#pragma unroll
                            for (int q = 0; q < (int)(4 / W); q++) {
                                const int j = i * (int)(4 / W) + q;
                                const uint32_t v = WIDE ? __builtin_amdgcn_ubfe(e, 16 * q, 16) : __builtin_amdgcn_ubfe(e, 8 * q, 8);
                                a0[j] += v;
                                if constexpr (OP == Op::Moments) {
                                    ar[j] = mad24(v, kr[k], ar[j]);
                                    ac[j] = mad24(v, kc[k], ac[j]);
                                }
                            }
                        }
                    }
                    chunk_to_lds<CH, OP>(a0, ar, ac, my, writer, split, pt.m0 + j0 + c * CH, pt.mr + j0 + c * CH,
                                         pt.mc + j0 + c * CH);
                };
                // three buffers, each chunk's loads issued two chunks ahead; three
                // chunks per iteration, so the buffers rotate without copies; loads
                // past a stream's end stay inside the block or return zeros
                load(bufA, 0);
                load(bufB, 1);
                uint32_t c = 0;
                for (; c + 2 < nfull; c += 3) {
                    load(bufC, c + 2);
                    chunk(bufA, c);
                    load(bufA, c + 3);
                    chunk(bufB, c + 1);
                    load(bufB, c + 4);
                    chunk(bufC, c + 2);
                }
                if (c < nfull) chunk(bufA, c);
                if (c + 1 < nfull) chunk(bufB, c + 1);
                // ragged end of a final partial block: one scan at a time
                for (uint32_t j = nfull * CH; j < nsteps; j++) {
                    uint32_t t0 = 0, tr = 0, tc = 0;
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        const uint32_t s0 = sl[k].live ? sl[k].org + 2u + (j0 + j) * W : 0x80000000u;
                        const uint32_t e = bload(rs, s0 & ~3u) >> ((s0 & 3u) * 8u);
                        const uint32_t v = WIDE ? (e & 0xFFFFu) : (e & 0xFFu);
                        t0 += v;
                        if constexpr (OP == Op::Moments) {
                            tr = mad24(v, kr[k], tr);
                            tc = mad24(v, kc[k], tc);
                        }
                    }
                    if (t0) atomicAdd(&pt.m0[j0 + j], t0);
                    if constexpr (OP == Op::Moments) {
                        if (tr) atomicAdd(&pt.mr[j0 + j], (unsigned long long)tr);
                        if (tc) atomicAdd(&pt.mc[j0 + j], (unsigned long long)tc);
                    }
                }
            }
            asm volatile("" ::"v"(touched));
            // end checks (FORMAT 2.4): the stream holds exactly the block's values,
            // and a uint8 stream with an odd count ends in a zero pad byte
#pragma unroll
            for (int k = 0; k < K; k++) {
                const RSlot &z = sl[k];
                if (!z.live) continue;
                bool ok = z.len == 2u + n * W + (WIDE ? 0u : (n & 1u));
                if (!WIDE && (n & 1u) && ok) {
                    const uint32_t s0 = z.org + 2u + n;
                    ok = ((bload(rs, s0 & ~3u) >> ((s0 & 3u) * 8u)) & 0xFFu) == 0u;
                }
                if (!ok) report(r, b, z.p);
            }
            return;
        }
    }

    // The form is uniform over the wave. An idle slot (x = 0, reads outside the
    // buffer) decodes the symbol of table slot 0 forever, so the rANS-only forms
    // can carry it when that symbol is 0 (the smallest coded value is 0).
    bool raw = false, idle = false;
#pragma unroll
    for (int k = 0; k < K; k++) {
        raw |= sl[k].live && sl[k].raw;
        idle |= !sl[k].live;
    }
    const bool idle_ok = (tbl[0] >> 24) == 0u;
    auto run_rows = [&](auto form, auto od) {
        using rows0 = std::integral_constant<int, 0>;
        if constexpr (OP == Op::Moments) {
            if constexpr (decltype(form)::value == kPlain) {
                if (rowp)
                    run(form, std::integral_constant<int, 2>{}, od);
                else if (rowu)
                    run(form, std::integral_constant<int, 1>{}, od);
                else
                    run(form, rows0{}, od);
            } else {
                if (rowu)
                    run(form, std::integral_constant<int, 1>{}, od);
                else
                    run(form, rows0{}, od);
            }
        } else {
            run(form, rows0{}, od);
        }
    };
    if (__builtin_amdgcn_ballot_w64(raw || (idle && !idle_ok))) {
        run(std::integral_constant<int, kMixed>{}, std::false_type{}, std::false_type{});
    } else if (WIDE && (tbl[(STG ? 1 : 2) * 4095] >> 24) == 255u) {
        // symbols are laid out in increasing order, so the last slot holds the
        // largest coded symbol: 255 there means escapes can occur
        if constexpr (STG) {
            stage_init();
            run_rows(std::integral_constant<int, kStaged>{}, std::false_type{});
            // hand the end position to the reservoir, where the end checks read it
#pragma unroll
            for (int k = 0; k < K; k++) {
                sl[k].s.off = sg[k].c0 + 2u * sg[k].wi - delta;
                sl[k].s.n = 0;
            }
        } else {
            run_rows(std::integral_constant<int, kEscape>{}, std::false_type{});
        }
    } else if constexpr (OP == Op::Sum || OP == Op::Moments || OP == Op::Index) {
        if (ondemand)
            run_rows(std::integral_constant<int, kPlain>{}, std::true_type{});
        else
            run_rows(std::integral_constant<int, kPlain>{}, std::false_type{});
    } else {
        run_rows(std::integral_constant<int, kPlain>{}, std::false_type{});
    }
    asm volatile("" ::"v"(touched));
    if constexpr (OP == Op::Split) {
        // the split point: state and byte offset after kSplit scans
#pragma unroll
        for (int k = 0; k < K; k++) {
            const RSlot &z = sl[k];
            if (!z.live) continue;
            const uint64_t si = 2 * ((uint64_t)b * r.P + z.p);
            dt.row[si] = z.x;
            dt.row[si + 1] = bbits_used(z.s, z.org) / 8u;
        }
        return;
    }
    // end checks (FORMAT 2.3-2.4); a first half ends at its split point
#pragma unroll
    for (int k = 0; k < K; k++) {
        const RSlot &z = sl[k];
        if (!z.live) continue;
        bool ok;
        if (half == 1) {
            const uint64_t si = 2 * ((uint64_t)b * r.P + z.p);
            const uint32_t off = z.raw ? 2u + kSplit * (WIDE ? 2u : 1u) : r.split[si + 1];
            ok = bbits_used(z.s, z.org) == 8u * off && (z.raw || z.x == r.split[si]);
        } else {
            ok = bbits_used(z.s, z.org) == 8u * z.len;
            if (!z.raw) ok = ok && z.x == 65536u;
            if (z.raw && !WIDE && (n & 1)) ok = ok && z.hold == 0;
        }
        if (!ok || bad) report(r, b, z.p);
    }
}

// ------------------------------------------------------------------ paired tile
// Any lane of the wave whose entry (or OR of entries) flags an escape: one
// 16-bit signed compare of the entry's low half (bit 15 is its sign).
__device__ __forceinline__ bool any_escape(uint32_t e) {
    uint64_t m;
    asm("v_cmp_gt_i16_e64 %0, 0, %1" : "=s"(m) : "v"(e));
    return m != 0;
}

// Bit reservoir of a paired stream: the valid bits sit below a single marker
// bit, so consuming bits is one 64-bit shift (the marker moves with them) and
// the count of valid bits is only needed at the refill and at the end.
struct MBits {
    uint64_t r;    // valid bits, the marker, zeros
    uint32_t off;  // block offset of the prefetched dword pf
    uint32_t pf;
};

// From a counted reservoir holding fewer than 64 bits.
__device__ __forceinline__ MBits mbits_from(const BBits &s) { return MBits{s.r | (1ull << s.n), s.off, s.pf}; }

__device__ __forceinline__ uint32_t mbits_count(const MBits &s) { return 63u - (uint32_t)__builtin_clzll(s.r); }

// At most 31 valid bits (the marker in the low word): the prefetched dword
// goes above them, and the marker 32 bits higher.
__device__ __forceinline__ void mbits_refill(MBits &s, Rsrc rs) {
    if ((uint32_t)(s.r >> 32) == 0u) {
        const uint32_t lo = (uint32_t)s.r;
        const uint32_t n = 31u - (uint32_t)__builtin_clz(lo);             // the marker's position
        const uint64_t ins = ((((uint64_t)1) << 32) | s.pf) << n;          // the new bits and marker
        s.r = ((uint64_t)(uint32_t)(ins >> 32) << 32) | ((lo ^ (1u << n)) | (uint32_t)ins);
        s.off += 4;
        s.pf = bload(rs, s.off);
    }
}

__device__ __forceinline__ uint32_t mbits_pop(MBits &s, uint32_t nb) {
    const uint32_t v = __builtin_amdgcn_ubfe((uint32_t)s.r, 0, nb);
    s.r >>= nb;
    return v;
}

// bits consumed since the stream start (block offset start)
__device__ __forceinline__ uint32_t mbits_used(const MBits &s, uint32_t start) {
    return 8u * (s.off - (start & ~3u)) - mbits_count(s) - ((start & 2) ? 16u : 0u);
}

// One tANS step's code bits: the entry's code length of bits from the
// reservoir; returns the next state's entry index.
__device__ __forceinline__ uint32_t take_code(MBits &s, uint32_t e) {
    const uint32_t v = __builtin_amdgcn_ubfe((uint32_t)s.r, 0, e);  // width = e[4:0] = code length
    s.r >>= (e & 63u);                                                // amount = e[5:0] = code length
    return (e >> 16) + v;
}

struct PSlot {
    uint32_t idx;   // LDS index of the tANS state's entry: model * 1024 + state (the idle entry unless PAIRED)
    uint32_t e;     // that entry, read one step ahead
    uint32_t meta;  // mode (3 PAIRED, 4 RAW, 7 idle) | model << 3
    uint32_t a0;    // window base of the slot's model (0 unless PAIRED)
    uint32_t p;
    uint32_t org;  // stream start within the block payload
    uint32_t len;
    MBits s;
};

// Paired decode-table entry: code length in bits 0-3 (bits 4-5 zero, so the
// entry itself is the width operand of a bit-field extract and the amount of
// a 64-bit shift), window values a, b (15 = escape) in bits 6-9 and 10-13,
// bit 15 set when either value escapes, and in bits 16-31 the LDS index of
// the next state's base entry (model * 1024 + next-state base). One shift
// and one add give the next lookup's index.
__device__ __forceinline__ uint32_t pe_a(uint32_t e) { return __builtin_amdgcn_ubfe(e, 6, 4); }
__device__ __forceinline__ uint32_t pe_b(uint32_t e) { return __builtin_amdgcn_ubfe(e, 10, 4); }
__device__ __forceinline__ bool pe_escape(uint32_t e) { return (int16_t)e < 0; }


__device__ __forceinline__ uint32_t window_sym(uint32_t v, uint32_t a0, uint32_t use) {
    const uint32_t d = v - a0;
    return (v >= a0 && d < 15u && ((use >> d) & 1u)) ? d : 15u;
}

// An escaped count: its literal, returned relative to the model's window base.
template <bool WIDE>
__device__ __forceinline__ uint32_t pair_literal(MBits &s, Rsrc rs, uint32_t info, uint32_t &bad) {
    mbits_refill(s, rs);
    const uint32_t lit = mbits_pop(s, WIDE ? 16u : 8u);
    const uint32_t a0 = info & 0xFFFFu;
    bad |= window_sym(lit, a0, info >> 16) != 15u;
    return lit - a0;
}

template <int K, bool WIDE, Op OP>
__device__ __forceinline__ void paired_tile(const DevResident &r, const uint16_t *sel, uint32_t p0, uint32_t n_sel, uint32_t first, uint32_t b,
                            uint64_t base, uint32_t nbytes, const uint32_t *tbl, const Partials<OP> &pt,
                            const RegionArgs &ra, const DpTile &dt) {
    const Rsrc rs = block_rsrc(r.payload + base, nbytes);
    const uint32_t lane = lane_id();
    const uint32_t maxv = WIDE ? 65535u : 255u;
    PSlot sl[K];
    uint32_t bad = 0, touched = 0, cst = 0;
    // window-base contributions, added once per chunk instead of once per value
    uint32_t base0 = 0, baseR = 0, baseC = 0;
#pragma unroll
    for (int k = 0; k < K; k++) {
        PSlot &z = sl[k];
        z.meta = 7;
        z.idx = kPairIdle;  // the idle entry after the 32 model tables: no bits, zero values, itself next
        z.p = 0;
        z.a0 = 0;
        // an idle slot reads outside the buffer range (zeros) and consumes no bits
        z.s.r = 1ull << 63;
        z.s.off = 0x80000000u;
        z.s.pf = 0;
        const uint32_t i = first + k * 64 + lane;
        if (i >= n_sel || sel[i] == kHole) continue;
        z.p = p0 + sel[i];
        const uint32_t kr = z.p / r.det_cols, kc = z.p - kr * r.det_cols;
        const Extent e = locate(r, b, z.p, base, nbytes);
        z.org = (uint32_t)(e.start - base);
        z.len = (uint32_t)(e.end - e.start);
        const uint32_t hdr = ld16(r.payload, e.start);
        const uint32_t mode = hdr & 7u;
        if (mode >= 3) touched += touch_stream(rs, z.org, z.len);
        if (mode == 0) {  // EMPTY
            if (z.len != 2) report(r, b, z.p);
            if constexpr (is_region(OP)) region_fill<WIDE, OP>(r, b, kBlk, z.p, 0, ra);
            if constexpr (OP == Op::Dp) dt.row[z.p] = 0;
            continue;
        }
        if (mode == 1) {  // CONST
            const uint32_t v = ld16(r.payload, e.start + 2);
            if (z.len != 4 || v == 0 || v > maxv)
                report(r, b, z.p);
            else if constexpr (is_region(OP))
                region_fill<WIDE, OP>(r, b, kBlk, z.p, v, ra);
            else if constexpr (OP == Op::Dp)
                dt.row[z.p] = v * dt.n_sel;
            else if constexpr (OP == Op::Index)
                cst += v;
            else
                add_event<OP>(pt, -1, v, kr, kc);
            continue;
        }
        if (mode == 2) {  // SPARSE: add the nonzeros straight into the LDS partials
            const uint32_t nnz = z.len >= 4 ? ld16(r.payload, e.start + 2) : 0;
            const uint32_t need = 4u + 2u * nnz + (WIDE ? 2u * nnz : nnz + (nnz & 1u));
            if (nnz == 0 || nnz > kBlk || need != z.len) {
                report(r, b, z.p);
                continue;
            }
            int prev = -1;
            bool ok = true;
            uint32_t dsum = 0;
            if constexpr (is_region(OP)) region_fill<WIDE, OP>(r, b, kBlk, z.p, 0, ra);
            for (uint32_t t = 0; t < nnz; t++) {
                const int pos = (int)ld16(r.payload, e.start + 4 + 2 * t);
                const uint32_t v = WIDE ? ld16(r.payload, e.start + 4 + 2 * nnz + 2 * t)
                                        : r.payload[e.start + 4 + 2 * nnz + t];
                if (pos <= prev || pos >= (int)kBlk || v == 0) {
                    ok = false;
                    break;
                }
                if constexpr (is_region(OP)) {
                    auto rw = region_walk<is_frames(OP)>(r, b, ra);
                    const uint64_t s = (uint64_t)b * kBlk + (uint32_t)pos;
                    rw.seek(r, s);
                    if (rw.inside()) region_put<WIDE, OP == Op::Amp>(ra, rw.index(r.P), z.p, v, rw.scale, rw.offset);
                } else if constexpr (OP == Op::Dp) {
                    dsum += v * scan_bit(dt, (uint32_t)pos);
                } else if constexpr (OP == Op::Index) {
                    atomicAdd(&dt.row[(first >> 6) * kBlk + (uint32_t)pos], v);
                } else {
                    add_event<OP>(pt, pos, v, kr, kc);
                }
                prev = pos;
            }
            if (ok && !WIDE && (nnz & 1)) ok = r.payload[e.start + 4 + 3 * nnz] == 0;
            if (!ok) report(r, b, z.p);
            if constexpr (OP == Op::Dp) dt.row[z.p] = dsum;
            continue;
        }
        z.meta = hdr & 0xFFu;  // mode and model
        BBits cs;
        bbits_init(cs, rs, z.org);
        pop16(cs);  // header
        if (mode == 3) {
            const uint32_t a0 = tbl[kPairTable + ((hdr >> 3) & 31u)] & 0xFFFFu;
            z.idx = (((hdr >> 3) & 31u) << 10) + popn(cs, 10);
            z.a0 = a0;
            base0 += a0;
            baseR += a0 * kr;
            baseC += a0 * kc;
        }
        z.s = mbits_from(cs);  // at most 48 bits are left after the header
        mbits_refill(z.s, rs);
    }
    // the first table entry of every slot (the idle entry for slots without a PAIRED stream)
#pragma unroll
    for (int k = 0; k < K; k++) sl[k].e = tbl[sl[k].idx];
    uint32_t kr[OP == Op::Moments ? K : 1], kc[OP == Op::Moments ? K : 1];
    if (OP == Op::Moments) {
#pragma unroll
        for (int k = 0; k < K; k++) {
            kr[k] = sl[k].p / r.det_cols;
            kc[k] = sl[k].p - kr[k] * r.det_cols;
        }
    }
    // moments of a wave whose pixels share one detector row: the row moment
    // comes from the per-scan totals (as in the byte-rANS tile)
    bool rowu = false;
    uint32_t kru = 0;
    if constexpr (OP == Op::Moments) {
        const uint64_t lv = __builtin_amdgcn_ballot_w64((sl[0].meta & 7u) != 7u);
        if (lv) {
            kru = (uint32_t)__builtin_amdgcn_readlane((int)kr[0], (int)__builtin_ctzll(lv));
            bool diff = false;
#pragma unroll
            for (int k = 0; k < K; k++) diff |= (sl[k].meta & 7u) != 7u && kr[k] != kru;  // mode 7: idle
            rowu = !__builtin_amdgcn_ballot_w64(diff);
        }
    }
    // Packed moments: in a wave inside one detector row whose live columns span
    // at most 128, one 32-bit accumulator per scan holds the sum of the values
    // (low half) and their column moment relative to the wave's first live
    // column (high half): one 24-bit multiply-add per value with the weight
    // 1 + (column offset << 16). Window values are at most 15 (escaped counts
    // beyond that are clamped to 15 and their excess goes to the partials
    // directly), so over 16 lanes of two slots each both halves stay below
    // 2^16 (16 x 2 x 15 = 480; 16 x 15 x (127 + 126) < 65536): the first four
    // reduction levels run on the packed words, the last two on each half.
    // The window bases enter once per scan as wave totals.
    bool packed = false;
    uint32_t kcw = 0, B0 = 0, Bc = 0, wgt[OP == Op::Moments ? K : 1];
    // Packed per slot: in a two-slot wave that crosses a row end, each slot's
    // 64 pixels may still lie in one row (64-pixel runs of a full detector
    // whose width is a multiple of 64). Both slots then share one accumulator
    // per scan with three fields: bits 0-8 the sum of the values, bits 9-16
    // the second slot's sum, bits 17-31 the column moment relative to each
    // slot's own first live column (a span of at most 63). The weight of a
    // value is 1 (+ 2^9 in the second slot) + (column offset << 17). Over 16
    // lanes of two slots the fields stay below their widths (480 < 2^9,
    // 240 < 2^8, 16 x 2 x 15 x 63 = 30240 < 2^15), so the first four
    // reduction levels run on the packed words and the last two per field.
    // The row moment is each slot's row times its total.
    bool pack2 = false;
    uint32_t krs[K], kcs[K], Br = 0;
    if constexpr (OP == Op::Moments && K == 2) {
        if (!rowu) {
            bool diff = false, far = false;
#pragma unroll
            for (int k = 0; k < K; k++) {
                const bool live = (sl[k].meta & 7u) != 7u;
                const uint64_t lv = __builtin_amdgcn_ballot_w64(live);
                krs[k] = lv ? (uint32_t)__builtin_amdgcn_readlane((int)kr[k], (int)__builtin_ctzll(lv)) : 0u;
                kcs[k] = wave_min(live ? kc[k] : 0xFFFFFFFFu);
                diff |= live && kr[k] != krs[k];
                far |= live && kc[k] - kcs[k] > 63u;
            }
            pack2 = !__builtin_amdgcn_ballot_w64(diff || far);
            if (pack2) {
#pragma unroll
                for (int k = 0; k < K; k++)
                    wgt[k] = (sl[k].meta & 7u) != 7u ? 1u + (k ? 1u << 9 : 0u) + ((kc[k] - kcs[k]) << 17) : 0u;
                B0 = wave_sum(base0);
                Bc = wave_sum(baseC);
                Br = wave_sum(baseR);
            }
        }
    }
    // Packed over rows: a one-stream-per-lane wave that spans up to four
    // detector rows and 64 columns (a row or two of a disk mask) keeps one
    // accumulator per scan with three fields relative to the wave's first live
    // row and column: bits 0-7 the sum of the values, bits 8-17 the row moment,
    // bits 18-31 the column moment (weight 1 + (row offset << 8) + (column
    // offset << 18), below 2^24). Over 16 lanes the fields stay below their
    // widths (240 < 2^8, 16 x 15 x 3 = 720 < 2^10, 16 x 15 x 63 = 15120 < 2^14),
    // so the first four reduction levels run packed and the last two per field.
    bool pack3 = false;
    uint32_t kr0 = 0, kc0 = 0;
    if constexpr (OP == Op::Moments && K == 1) {
        if (!rowu) {
            const bool live = (sl[0].meta & 7u) != 7u;
            kr0 = wave_min(live ? kr[0] : 0xFFFFFFFFu);
            kc0 = wave_min(live ? kc[0] : 0xFFFFFFFFu);
            const bool far = live && (kr[0] - kr0 > 3u || kc[0] - kc0 > 63u);
            pack3 = __builtin_amdgcn_ballot_w64(live) && !__builtin_amdgcn_ballot_w64(far);
            if (pack3) {
                wgt[0] = live ? 1u + ((kr[0] - kr0) << 8) + ((kc[0] - kc0) << 18) : 0u;
                B0 = wave_sum(base0);
                Bc = wave_sum(baseC);
                Br = wave_sum(baseR);
            }
        }
    }
    if constexpr (OP == Op::Moments) {
        if (rowu) {
            uint32_t m = 0xFFFFFFFFu;
#pragma unroll
            for (int k = 0; k < K; k++)
                if ((sl[k].meta & 7u) != 7u) m = min(m, kc[k]);
            kcw = wave_min(m);
            bool far = false;
#pragma unroll
            for (int k = 0; k < K; k++) far |= (sl[k].meta & 7u) != 7u && kc[k] - kcw > 127u;
            packed = !__builtin_amdgcn_ballot_w64(far);
#pragma unroll
            for (int k = 0; k < K; k++) wgt[k] = (sl[k].meta & 7u) != 7u ? 1u + ((kc[k] - kcw) << 16) : 0u;
            if (packed) {
                B0 = wave_sum(base0);
                Bc = wave_sum(baseC);
            }
        }
    }

    // One pair step of every slot: window-relative values for PAIRED slots,
    // absolute values for RAW slots, zeros for idle ones. Two forms, chosen
    // once per wave: kPMixed when some slot is RAW (per-slot branches), kPPlain
    // otherwise (every slot, idle ones included, runs the same table step).
    constexpr int kPMixed = 0, kPPlain = 1;
    // Returns whether some slot of the wave read an escape literal at this step.
    auto step = [&](auto form, uint32_t t, uint32_t (&v0)[K], uint32_t (&v1)[K]) -> bool {
        constexpr int F = decltype(form)::value;
        bool escaped = true;
        if constexpr (F == kPPlain) {
            // the entry read a step ahead gives the code bits and the next
            // state at once; the next entry's read is issued right away, and
            // this step's values, escapes and refill run while it is in flight
            uint32_t e[K];
            uint32_t esc_any = 0;
#pragma unroll
            for (int k = 0; k < K; k++) {
                PSlot &z = sl[k];
                e[k] = z.e;
                z.idx = take_code(z.s, e[k]);
                z.e = tbl[z.idx];
            }
#pragma unroll
            for (int k = 0; k < K; k++) {
                v0[k] = pe_a(e[k]);
                v1[k] = pe_b(e[k]);
                esc_any |= e[k];
            }
            escaped = any_escape(esc_any);
            if (escaped) {  // values outside the model window
#pragma unroll
                for (int k = 0; k < K; k++) {
                    // the per-lane test stays inside the wave's branch (the compiler
                    // would otherwise compute it at every step, escapes or not)
                    uint32_t ek = e[k];
                    asm volatile("" : "+v"(ek));
                    if (pe_escape(ek)) {
                        PSlot &z = sl[k];
                        const uint32_t info = tbl[kPairTable + (z.meta >> 3)];
                        if (v0[k] == 15u) v0[k] = pair_literal<WIDE>(z.s, rs, info, bad);
                        if (v1[k] == 15u) v1[k] = pair_literal<WIDE>(z.s, rs, info, bad);
                        mbits_refill(z.s, rs);  // keep 32+ bits until the next cadence point
                    }
                }
            }
            // Codes are at most 10 bits. The wave refills when some lane holds
            // fewer than 10 bits (the marker below bit 10), and then every lane
            // with room for a dword takes one: the refills of a wave's lanes fall
            // together, so a wave of dim streams refills every ten or more pairs
            // instead of at every cadence point, and each refill's load has had
            // that long to arrive.
            bool low = false;
#pragma unroll
            for (int k = 0; k < K; k++) low |= sl[k].s.r < 1024u;
            if (__builtin_amdgcn_ballot_w64(low)) {
#pragma unroll
                for (int k = 0; k < K; k++) {
                    // keep the reservoir test inside the wave's branch (else it
                    // runs at every step)
                    uint32_t hi = (uint32_t)(sl[k].s.r >> 32);
                    asm volatile("" : "+v"(hi));
                    sl[k].s.r = ((uint64_t)hi << 32) | (uint32_t)sl[k].s.r;
                    mbits_refill(sl[k].s, rs);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < K; k++) {
                PSlot &z = sl[k];
                const uint32_t mode = z.meta & 7u;
                v0[k] = 0;
                v1[k] = 0;
                if (mode == 3) {
                    const uint32_t e = z.e;
                    z.idx = take_code(z.s, e);
                    z.e = tbl[z.idx];
                    v0[k] = pe_a(e);
                    v1[k] = pe_b(e);
                    if (pe_escape(e)) {
                        const uint32_t info = tbl[kPairTable + (z.meta >> 3)];
                        if (v0[k] == 15u) v0[k] = pair_literal<WIDE>(z.s, rs, info, bad);
                        if (v1[k] == 15u) v1[k] = pair_literal<WIDE>(z.s, rs, info, bad);
                        mbits_refill(z.s, rs);
                    }
                    if (t % 3 == 2) mbits_refill(z.s, rs);
                } else if (mode == 4) {
                    if (WIDE) {
                        v0[k] = mbits_pop(z.s, 16);
                        mbits_refill(z.s, rs);
                        v1[k] = mbits_pop(z.s, 16);
                    } else {
                        const uint32_t w = mbits_pop(z.s, 16);
                        v0[k] = w & 0xFFu;
                        v1[k] = w >> 8;
                    }
                    mbits_refill(z.s, rs);
                }
            }
        }
        return escaped;
    };

    auto run = [&](auto form, auto rowu, auto packed_t) {
        constexpr bool ROWU = decltype(rowu)::value;  // moments of a wave inside one detector row
        constexpr bool PACKED = decltype(packed_t)::value == 1;  // one packed accumulator (a row-uniform wave)
        constexpr bool PACK2 = decltype(packed_t)::value == 2;   // one per slot (each slot's pixels in one row)
        constexpr bool PACK3 = decltype(packed_t)::value == 3;   // one over up to four rows (one slot per lane)
        if constexpr (is_region(OP)) {
            auto rw = region_walk<is_frames(OP)>(r, b, ra);
            for (uint32_t t = 0; t < kBlk / 2; t++) {
                uint32_t v0[K], v1[K];
                step(form, t, v0, v1);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    if (rw.inside()) {
                        const uint64_t idx = rw.index(r.P);
#pragma unroll
                        for (int k = 0; k < K; k++) {
                            const uint32_t mode = sl[k].meta & 7u;
                            if (mode == 3 || mode == 4)
                                region_put<WIDE, OP == Op::Amp>(ra, idx, sl[k].p, sl[k].a0 + (h ? v1[k] : v0[k]),
                                                 rw.scale, rw.offset);
                        }
                    }
                    rw.next();
                }
            }
        } else if constexpr (OP == Op::Dp) {
            // per-lane sums over the selected scans; a PAIRED slot's window base
            // counts once per selected scan
            uint32_t acc[K];
#pragma unroll
            for (int k = 0; k < K; k++) acc[k] = sl[k].a0 * dt.n_sel;
            for (uint32_t c = 0; c < kBlk / 32; c++) {
                const uint32_t word = dt.bits[c];
#pragma unroll
                for (int tt = 0; tt < 16; tt++) {
                    uint32_t v0[K], v1[K];
                    step(form, c * 16 + tt, v0, v1);
                    // window-relative values wrap below zero for literals under the
                    // window base, so select with full-width masks (sums stay exact mod 2^32)
                    const uint32_t m0 = 0u - ((word >> (2 * tt)) & 1u), m1 = 0u - ((word >> (2 * tt + 1)) & 1u);
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        acc[k] += (v0[k] & m0) + (v1[k] & m1);
                        asm volatile("" : "+v"(acc[k]));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int k = 0; k < K; k++) {
                const uint32_t mode = sl[k].meta & 7u;
                if (mode == 3 || mode == 4) dt.row[sl[k].p] = acc[k];
            }
        } else if constexpr (OP == Op::Moments && PACK2) {
            constexpr int CH = 16;
            const uint32_t my = lane_scan<CH>();
            const bool writer = lane_writes<CH>();
            for (uint32_t c = 0; c < kBlk / CH; c++) {
                uint32_t acc[CH];
#pragma unroll
                for (int i = 0; i < CH; i++) acc[i] = 0;
#pragma unroll
                for (int tt = 0; tt < CH / 2; tt++) {
                    uint32_t v0[K], v1[K];
                    if (step(form, c * (CH / 2) + tt, v0, v1)) {
                        // counts beyond the packed range: 15 stays packed, the excess
                        // (negative below the window) goes to the partials with its moments
#pragma unroll
                        for (int k = 0; k < K; k++) {
#pragma unroll
                            for (int h = 0; h < 2; h++) {
                                uint32_t &v = h ? v1[k] : v0[k];
                                if (v > 15u) {
                                    const uint32_t s = c * CH + 2 * tt + h;
                                    const long long x = (int32_t)(v - 15u);
                                    atomicAdd(&pt.m0[s], v - 15u);
                                    atomicAdd(&pt.mc[s], (unsigned long long)(x * (long long)kc[k]));
                                    atomicAdd(&pt.mr[s], (unsigned long long)(x * (long long)kr[k]));
                                    v = 15u;
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        acc[2 * tt] = mad24(v0[k], wgt[k], acc[2 * tt]);
                        acc[2 * tt + 1] = mad24(v1[k], wgt[k], acc[2 * tt + 1]);
                    }
                    asm volatile("" : "+v"(acc[2 * tt]), "+v"(acc[2 * tt + 1]));
                    __builtin_amdgcn_sched_barrier(0);
                }
                transpose_head<CH>(acc);
                const uint32_t v = bfdpp<kHalfMirror, 4>(acc[0], acc[1]);  // 16 lanes
                uint32_t ts = v & 0x1FFu, t1 = __builtin_amdgcn_ubfe(v, 9, 8), tc = v >> 17;
                ts += (uint32_t)__builtin_amdgcn_mov_dpp((int)ts, kQuadXor2, 0xF, 0xF, false);
                t1 += (uint32_t)__builtin_amdgcn_mov_dpp((int)t1, kQuadXor2, 0xF, 0xF, false);
                tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor2, 0xF, 0xF, false);
                ts += (uint32_t)__builtin_amdgcn_mov_dpp((int)ts, kQuadXor1, 0xF, 0xF, false);
                t1 += (uint32_t)__builtin_amdgcn_mov_dpp((int)t1, kQuadXor1, 0xF, 0xF, false);
                tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor1, 0xF, 0xF, false);
                const uint32_t m0 = ts + B0;
                if (writer && m0) {
                    // one wave's moments of one scan fit 32 bits: slot totals at most
                    // 64 x 15, column moments below 2^16, window-base sums at most
                    // 128 x 13 x 1023 (model bases are at most 13, detector sides at most 1024)
                    const uint32_t s = c * CH + my, t0 = ts - t1;
                    atomicAdd(&pt.m0[s], m0);
                    atomicAdd(&pt.mc[s], (unsigned long long)mad24(kcs[0], t0, mad24(kcs[1], t1, Bc + tc)));
                    atomicAdd(&pt.mr[s], (unsigned long long)mad24(krs[0], t0, mad24(krs[1], t1, Br)));
                }
            }
        } else if constexpr (OP == Op::Moments && PACK3) {
            constexpr int CH = 16;
            const uint32_t my = lane_scan<CH>();
            const bool writer = lane_writes<CH>();
            for (uint32_t c = 0; c < kBlk / CH; c++) {
                uint32_t acc[CH];
#pragma unroll
                for (int i = 0; i < CH; i++) acc[i] = 0;
#pragma unroll
                for (int tt = 0; tt < CH / 2; tt++) {
                    uint32_t v0[K], v1[K];
                    if (step(form, c * (CH / 2) + tt, v0, v1)) {
                        // counts beyond the packed range: 15 stays packed, the excess
                        // (negative below the window) goes to the partials with its moments
#pragma unroll
                        for (int h = 0; h < 2; h++) {
                            uint32_t &v = h ? v1[0] : v0[0];
                            if (v > 15u) {
                                const uint32_t s = c * CH + 2 * tt + h;
                                const long long x = (int32_t)(v - 15u);
                                atomicAdd(&pt.m0[s], v - 15u);
                                atomicAdd(&pt.mc[s], (unsigned long long)(x * (long long)kc[0]));
                                atomicAdd(&pt.mr[s], (unsigned long long)(x * (long long)kr[0]));
                                v = 15u;
                            }
                        }
                    }
                    acc[2 * tt] = mad24(v0[0], wgt[0], acc[2 * tt]);
                    acc[2 * tt + 1] = mad24(v1[0], wgt[0], acc[2 * tt + 1]);
                    asm volatile("" : "+v"(acc[2 * tt]), "+v"(acc[2 * tt + 1]));
                    __builtin_amdgcn_sched_barrier(0);
                }
                transpose_head<CH>(acc);
                const uint32_t v = bfdpp<kHalfMirror, 4>(acc[0], acc[1]);  // 16 lanes
                uint32_t ts = v & 0xFFu, tr = __builtin_amdgcn_ubfe(v, 8, 10), tc = v >> 18;
                ts += (uint32_t)__builtin_amdgcn_mov_dpp((int)ts, kQuadXor2, 0xF, 0xF, false);
                tr += (uint32_t)__builtin_amdgcn_mov_dpp((int)tr, kQuadXor2, 0xF, 0xF, false);
                tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor2, 0xF, 0xF, false);
                ts += (uint32_t)__builtin_amdgcn_mov_dpp((int)ts, kQuadXor1, 0xF, 0xF, false);
                tr += (uint32_t)__builtin_amdgcn_mov_dpp((int)tr, kQuadXor1, 0xF, 0xF, false);
                tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor1, 0xF, 0xF, false);
                const uint32_t m0 = ts + B0;
                if (writer && m0) {
                    // 32 bits suffice: totals at most 64 x 15, relative moments below
                    // 64 x 15 x 63, window-base sums at most 64 x 13 x 1023
                    const uint32_t s = c * CH + my;
                    atomicAdd(&pt.m0[s], m0);
                    atomicAdd(&pt.mc[s], (unsigned long long)mad24(kc0, ts, Bc + tc));
                    atomicAdd(&pt.mr[s], (unsigned long long)mad24(kr0, ts, Br + tr));
                }
            }
        } else if constexpr (OP == Op::Moments && PACKED) {
            constexpr int CH = 16;
            const uint32_t my = lane_scan<CH>();
            const bool writer = lane_writes<CH>();
            for (uint32_t c = 0; c < kBlk / CH; c++) {
                uint32_t acc[CH];
#pragma unroll
                for (int i = 0; i < CH; i++) acc[i] = 0;
#pragma unroll
                for (int tt = 0; tt < CH / 2; tt++) {
                    uint32_t v0[K], v1[K];
                    if (step(form, c * (CH / 2) + tt, v0, v1)) {
                        // escaped counts beyond the packed range (window-relative, so a
                        // count below the window base is negative): 15 stays packed, the
                        // excess goes to the partials with its moments
#pragma unroll
                        for (int k = 0; k < K; k++) {
#pragma unroll
                            for (int h = 0; h < 2; h++) {
                                uint32_t &v = h ? v1[k] : v0[k];
                                if (v > 15u) {
                                    const uint32_t s = c * CH + 2 * tt + h;
                                    const long long x = (int32_t)(v - 15u);
                                    atomicAdd(&pt.m0[s], v - 15u);
                                    atomicAdd(&pt.mc[s], (unsigned long long)(x * (long long)kc[k]));
                                    atomicAdd(&pt.mr[s], (unsigned long long)(x * (long long)kru));
                                    v = 15u;
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        acc[2 * tt] = mad24(v0[k], wgt[k], acc[2 * tt]);
                        acc[2 * tt + 1] = mad24(v1[k], wgt[k], acc[2 * tt + 1]);
                    }
                    asm volatile("" : "+v"(acc[2 * tt]), "+v"(acc[2 * tt + 1]));
                    __builtin_amdgcn_sched_barrier(0);
                }
                transpose_head<CH>(acc);
                const uint32_t v = bfdpp<kHalfMirror, 4>(acc[0], acc[1]);  // 16 lanes
                uint32_t t0 = v & 0xFFFFu, tc = v >> 16;
                t0 += (uint32_t)__builtin_amdgcn_mov_dpp((int)t0, kQuadXor2, 0xF, 0xF, false);
                tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor2, 0xF, 0xF, false);
                t0 += (uint32_t)__builtin_amdgcn_mov_dpp((int)t0, kQuadXor1, 0xF, 0xF, false);
                tc += (uint32_t)__builtin_amdgcn_mov_dpp((int)tc, kQuadXor1, 0xF, 0xF, false);
                const uint32_t m0 = t0 + B0;
                if (writer && m0) {
                    const uint32_t s = c * CH + my;
                    atomicAdd(&pt.m0[s], m0);
                    atomicAdd(&pt.mc[s], (unsigned long long)mad24(kcw, t0, Bc + tc));
                    atomicAdd(&pt.mr[s], (unsigned long long)mad24(kru, m0, 0u));
                }
            }
        } else {
            // paired workgroups have 128 VGPRs per lane: moments reduce every 8 scans
            constexpr int CH = OP == Op::Moments ? 8 : 16;
            const uint32_t my = lane_scan<CH>();
            const bool writer = lane_writes<CH>();
            const bool split = r.det_cols > 256 || r.P / r.det_cols > 256;
            const uint32_t cw = OP == Op::Index ? wave_sum(cst) : 0u;  // the leaf's constant streams
            for (uint32_t c = 0; c < kBlk / CH; c++) {
                uint32_t a0[CH];
                uint32_t ar[OP == Op::Moments ? CH : 1], ac[OP == Op::Moments ? CH : 1];
#pragma unroll
                for (int i = 0; i < CH; i++) {
                    a0[i] = base0;
                    if (OP == Op::Moments) {
                        ar[i] = baseR;
                        ac[i] = baseC;
                    }
                }
#pragma unroll
                for (int tt = 0; tt < CH / 2; tt++) {
                    uint32_t v0[K], v1[K];
                    step(form, c * (CH / 2) + tt, v0, v1);
#pragma unroll
                    for (int k = 0; k < K; k++) {
                        a0[2 * tt] += v0[k];
                        a0[2 * tt + 1] += v1[k];
                        if (OP == Op::Moments) {
                            // window-relative values lie in [-65535, 65535] (an escape below
                            // the window is negative) and pixel coordinates below 1024: signed
                            // 24-bit products give the same sums modulo 2^32 at full rate
                            if constexpr (!ROWU) {
                                ar[2 * tt] = mad24s(v0[k], kr[k], ar[2 * tt]);
                                ar[2 * tt + 1] = mad24s(v1[k], kr[k], ar[2 * tt + 1]);
                            }
                            ac[2 * tt] = mad24s(v0[k], kc[k], ac[2 * tt]);
                            ac[2 * tt + 1] = mad24s(v1[k], kc[k], ac[2 * tt + 1]);
                        }
                    }
                    // materialise the sums here (see the byte-rANS tile)
                    asm volatile("" : "+v"(a0[2 * tt]), "+v"(a0[2 * tt + 1]));
                    if constexpr (OP == Op::Moments && !ROWU)
                        asm volatile("" : "+v"(ar[2 * tt]), "+v"(ar[2 * tt + 1]), "+v"(ac[2 * tt]), "+v"(ac[2 * tt + 1]));
                    if constexpr (OP == Op::Moments && ROWU) asm volatile("" : "+v"(ac[2 * tt]), "+v"(ac[2 * tt + 1]));
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (OP == Op::Index) {
                    const uint32_t t0 = wave_transpose_sum<CH>(a0) + cw;
                    if (writer && t0) atomicAdd(&dt.row[(first >> 6) * kBlk + c * CH + my], t0);
                } else {
                    chunk_to_lds<CH, OP, ROWU>(a0, ar, ac, my, writer, split, pt.m0 + c * CH, pt.mr + c * CH,
                                               pt.mc + c * CH, kru);
                }
            }
        }
    };

    bool raw = false;
#pragma unroll
    for (int k = 0; k < K; k++) raw |= (sl[k].meta & 7u) == 4u;
    auto run_rows = [&](auto form) {
        constexpr bool PLAIN = decltype(form)::value == kPPlain;
        using none = std::integral_constant<int, 0>;
        if constexpr (OP == Op::Moments) {
            if (rowu) {
                if constexpr (PLAIN) {
                    if (packed)
                        run(form, std::true_type{}, std::integral_constant<int, 1>{});
                    else
                        run(form, std::true_type{}, none{});
                } else {
                    run(form, std::true_type{}, none{});
                }
            } else if constexpr (PLAIN && K == 2) {
                if (pack2)
                    run(form, std::false_type{}, std::integral_constant<int, 2>{});
                else
                    run(form, std::false_type{}, none{});
            } else if constexpr (PLAIN && K == 1) {
                if (pack3)
                    run(form, std::false_type{}, std::integral_constant<int, 3>{});
                else
                    run(form, std::false_type{}, none{});
            } else {
                run(form, std::false_type{}, none{});
            }
        } else {
            run(form, std::false_type{}, none{});
        }
    };
    if (__builtin_amdgcn_ballot_w64(raw))
        run_rows(std::integral_constant<int, kPMixed>{});
    else
        run_rows(std::integral_constant<int, kPPlain>{});
    asm volatile("" ::"v"(touched));
    // end checks (FORMAT 3.3-3.4)
#pragma unroll
    for (int k = 0; k < K; k++) {
        PSlot &z = sl[k];
        const uint32_t mode = z.meta & 7u;
        if (mode != 3 && mode != 4) continue;
        const uint32_t used = mbits_used(z.s, z.org), total = 8u * z.len;
        bool ok;
        if (mode == 4) {
            ok = used == total;
        } else {
            ok = (z.idx & 1023u) == 0 && used <= total && total - used < 16;  // state 0 of the model
            if (ok && total > used) {
                mbits_refill(z.s, rs);
                ok = mbits_pop(z.s, total - used) == 0;
            }
        }
        if (!ok || bad) report(r, b, z.p);
    }
}

// ------------------------------------------------------------------ query plan
// The init kernel counts the selected pixels of every 64-pixel tile. Each
// reduce workgroup then numbers the selected pixels in pixel order (a prefix
// sum over the counts) and cuts them into work items of exactly `cap` pixels
// (the last item keeps the rest), so every item of a visited block decodes
// `cap` streams, however the mask scatters them over the detector, and no
// item is spent on pixels the mask misses. An item is described by its first
// tile and the selected pixels of that tile before the item's first.
//
// Item size: half the workgroup, the workgroup (one stream per lane), or twice
// it (two per lane). An item's decode is a chain of dependent steps, so the
// time of a round of resident workgroups hardly depends on the streams per
// lane while they are few; two per lane take about 1.7 times as long as one
// (measured). The plan estimates rounds times that factor; on a tie the
// smaller items spread the work over more compute units.
struct PlanArgs {
    const uint8_t *mask;
    const uint8_t *mask2;  // a second (subtracted) mask counted after the first, or null
    const uint8_t *valid;
    int complement;
    uint32_t P, n_tiles;  // 64-pixel tiles of one mask
    uint32_t *counts;     // null: no plan
    const uint32_t *gbase0;  // block 0's group bases, relative offsets and directory entry: the
    const uint16_t *rel0;    // selected streams' sizes there tell bright (densely coded) data from dim
    const uint8_t *dir0;
};

constexpr float kTwoSlotTime = 1.7f;

struct PlanView {
    uint32_t n_items, n_first;  // items per visited block; of them, items of the first mask
    uint32_t cap;               // selected pixels per item
    uint32_t end[2];            // per mask, the end of its last non-empty tile (pixels)
    bool halves;                // decode each stream's two halves side by side (split points)
    bool sparse;                // at most a quarter of the pixels are selected (per mask)
};

// Most items a plan can hold: two masks of kMaxPlanTiles tiles cut in halves of a workgroup.
template <int WG>
constexpr uint32_t kMaxItems = 2 * kMaxPlanTiles * kPlanFine / (WG / 2);

// With `two`, the counts of a second mask follow those of the first, and its
// items (whose values the query subtracts) start after the first mask's:
// its pixel numbering starts at the first multiple of cap past the first's.
//
// one_slot: items of at most one stream per lane.
//
// can_split: the streams have split points. When every item of half-workgroup
// size fits one round of the resident workgroups, the query is latency-bound:
// each item then takes half a workgroup of streams and the other half of the
// lanes decodes their second halves, so the chain of dependent steps halves.
template <int WG>
__device__ __forceinline__ PlanView plan_cut(const uint32_t *counts, uint32_t P, uint32_t n_visited, bool two,
                                             bool can_split, uint16_t *desc, uint32_t *wtot, bool one_slot = false) {
    constexpr uint32_t kPer = 2 * kMaxPlanTiles / WG;
    constexpr uint32_t kWaves = WG / 64;
    __shared__ uint32_t wpart[5][kWaves];  // per wave: the second mask's sum, each mask's last tile, bytes
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t n_tiles = (P + kPlanFine - 1) / kPlanFine, n_all = two ? 2 * n_tiles : n_tiles;
    uint32_t c[kPer], s = 0, s2 = 0, last[2] = {0, 0}, bytes = 0;
#pragma unroll
    for (uint32_t j = 0; j < kPer; j++) {
        const uint32_t t = tid * kPer + j;
        c[j] = t < n_all ? counts[t] : 0u;
        bytes += t < n_all ? counts[kPlanBytes + t] : 0u;
        s += c[j];
        const uint32_t second = t >= n_tiles;
        s2 += second ? c[j] : 0u;
        if (c[j]) last[second] = t - (second ? n_tiles : 0u) + 1;
    }
    // exclusive prefix of the per-thread sums over both masks, the second
    // mask's total, and the end of each mask's last non-empty tile
    uint32_t x = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= (uint32_t)off) x += y;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        s2 += __shfl_xor(s2, off);
        bytes += __shfl_xor(bytes, off);
        last[0] = max(last[0], (uint32_t)__shfl_xor(last[0], off));
        last[1] = max(last[1], (uint32_t)__shfl_xor(last[1], off));
    }
    __syncthreads();  // wtot may still be read by the previous user
    if (lane == 63) wtot[wave] = x;
    if (lane == 0) {
        wpart[0][wave] = s2;
        wpart[1][wave] = last[0];
        wpart[2][wave] = last[1];
        wpart[3][wave] = bytes;
    }
    __syncthreads();
    uint32_t before = 0, total = 0, total2 = 0, end0 = 0, end1 = 0;
    uint64_t total_bytes = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; w++) {
        before += w < wave ? wtot[w] : 0u;
        total += wtot[w];
        total2 += wpart[0][w];
        end0 = max(end0, wpart[1][w]);
        end1 = max(end1, wpart[2][w]);
        total_bytes += wpart[3][w];
    }
    const uint32_t total1 = total - total2;
    const float slots = (float)gridDim.x;
    auto cost = [&](uint32_t cap) {
        const float items = (float)((total1 + cap - 1) / cap + (total2 + cap - 1) / cap) * (float)n_visited;
        return ceilf(items / slots) * (cap > (uint32_t)WG ? kTwoSlotTime : 1.0f);
    };
    uint32_t cap = WG / 2;
    if (cost(WG) < cost(cap)) cap = WG;
    // Two streams per lane pay for dim data only (measured): streams coded in
    // more than 0.4 bytes per decoded value (block 0's 512 scans per stream)
    // make them about twice as slow. 1024-lane workgroups fill a
    // compute unit alone and pay only when most pixels are selected.
    const bool dim = total_bytes * 10 <= (uint64_t)total * kBlk * 4;
    if (!one_slot && (WG < 1024 ? dim : 2 * total >= P) && cost(2 * WG) < cost(cap)) cap = 2 * WG;
    const bool halves = can_split && cap == WG / 2 && cost(WG / 2) <= 1.0f;
    const uint32_t n_first = (total1 + cap - 1) / cap, pad = n_first * cap - total1;
    // tile t starts item k when it holds the pixel numbered k * cap
    uint32_t e = before + x - s;  // selected pixels before this thread's first tile
#pragma unroll
    for (uint32_t j = 0; j < kPer; j++) {
        const uint32_t t = tid * kPer + j;
        const bool second = t >= n_tiles;
        const uint32_t ee = e + (second ? pad : 0u);
        if (c[j]) {
            const uint32_t k = (ee + cap - 1) / cap;
            if (k * cap < ee + c[j]) desc[k] = (uint16_t)(((t - (second ? n_tiles : 0u)) << 6) | (k * cap - ee));
        }
        e += c[j];
    }
    __syncthreads();
    return PlanView{n_first + (total2 + cap - 1) / cap, n_first, cap,
                    {min(end0 * kPlanFine, P), min(end1 * kPlanFine, P)}, halves, 4ull * total <= (two ? 2ull : 1ull) * P};
}

// The pixels of one planned item: from tile (desc >> 6) on, skipping that
// tile's first (desc & 63) selected pixels, the next `cap` selected ones
// (fewer for the last item), as offsets from the tile's first pixel.
template <int WG>
__device__ __forceinline__ uint32_t select_range(const DevResident &r, const uint8_t *mask, int complement,
                                                 uint32_t desc, uint32_t cap, uint32_t end, uint32_t &p0,
                                                 uint16_t *sel, uint32_t *wtot) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const unsigned long long below = (1ull << lane) - 1ull;
    const uint32_t skip = desc & 63u, want = skip + cap;
    p0 = (desc >> 6) * kPlanFine;
    uint32_t seen = 0;  // selected pixels from p0 on, skipped ones included
    for (uint32_t base = p0; base < end && seen < want; base += WG) {
        const uint32_t p = base + tid;
        bool f = false;
        if (p < end) f = r.valid[p] != 0 && (mask ? ((mask[p] != 0) != (complement != 0)) : true);
        const unsigned long long bal = __ballot(f);
        if (lane == 0) wtot[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t before = seen, all = seen;
#pragma unroll
        for (uint32_t w = 0; w < WG / 64; w++) {
            const uint32_t c = wtot[w];
            before += w < wave ? c : 0u;
            all += c;
        }
        const uint32_t ord = before + (uint32_t)__popcll(bal & below);
        if (f && ord >= skip && ord < want) sel[ord - skip] = (uint16_t)(p - p0);
        __syncthreads();
        seen = all;
    }
    return seen > skip ? min(seen, want) - skip : 0u;
}

// Units of `unit` selected pixels (one mask): tile t starts unit k when it
// holds the pixel numbered k * unit; udesc[k] is that tile and the selected
// pixels of it before the unit's first, as for the items above. Returns the
// number of units.
template <int WG>
__device__ __forceinline__ uint32_t plan_units(const uint32_t *counts, uint32_t P, uint32_t unit, uint16_t *udesc,
                                               uint32_t *wtot) {
    constexpr uint32_t kPer = 2 * kMaxPlanTiles / WG;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t n_tiles = (P + kPlanFine - 1) / kPlanFine;
    uint32_t c[kPer], s = 0;
#pragma unroll
    for (uint32_t j = 0; j < kPer; j++) {
        const uint32_t t = tid * kPer + j;
        c[j] = t < n_tiles ? counts[t] : 0u;
        s += c[j];
    }
    uint32_t x = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= (uint32_t)off) x += y;
    }
    __syncthreads();  // wtot may still be read by the previous user
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (uint32_t w = 0; w < WG / 64; w++) {
        before += w < wave ? wtot[w] : 0u;
        total += wtot[w];
    }
    uint32_t e = before + x - s;
#pragma unroll
    for (uint32_t j = 0; j < kPer; j++) {
        const uint32_t t = tid * kPer + j;
        if (c[j]) {
            const uint32_t k = (e + unit - 1) / unit;
            if (k * unit < e + c[j]) udesc[k] = (uint16_t)((t << 6) | (k * unit - e));
        }
        e += c[j];
    }
    __syncthreads();
    return (total + unit - 1) / unit;
}

// The pixels of one unit, gathered by one wave alone into its own slice of
// the list (offsets from the unit's first tile), 64 pixels per ballot.
__device__ __forceinline__ uint32_t select_unit(const DevResident &r, const uint8_t *mask, int complement,
                                                uint32_t desc, uint32_t unit, uint32_t end, uint32_t &p0,
                                                uint16_t *wsel) {
    const uint32_t lane = lane_id();
    const unsigned long long below = (1ull << lane) - 1ull;
    const uint32_t skip = desc & 63u, want = skip + unit;
    p0 = (desc >> 6) * kPlanFine;
    uint32_t seen = 0;  // selected pixels from p0 on, skipped ones included
    for (uint32_t base = p0; base < end && seen < want; base += 64) {
        const uint32_t p = base + lane;
        bool f = false;
        if (p < end) f = r.valid[p] != 0 && (mask ? ((mask[p] != 0) != (complement != 0)) : true);
        const unsigned long long bal = __ballot(f);
        const uint32_t ord = seen + (uint32_t)__popcll(bal & below);
        if (f && ord >= skip && ord < want) wsel[ord - skip] = (uint16_t)(p - p0);
        seen += (uint32_t)__popcll(bal);
    }
    // the wave's own list: its writes are read by other lanes of the same wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return seen > skip ? min(seen, want) - skip : 0u;
}

// ------------------------------------------------------------------ index groups
// One work item of the index build: WG consecutive polar positions, lane l of
// wave w at position (group * WG / 64 + w) * 64 + l, so every wave decodes one
// leaf. Invalid pixels and positions past the detector are holes.
template <int WG>
__device__ __forceinline__ uint32_t index_group(const DevResident &r, const uint16_t *perm, uint32_t group,
                                                uint16_t *sel) {
    const uint32_t pos = group * WG + threadIdx.x;
    uint16_t px = kHole;
    if (pos < r.P) {
        const uint16_t p = perm[pos];
        if (r.valid[p]) px = p;
    }
    sel[threadIdx.x] = px;
    __syncthreads();
    return WG;
}

// ------------------------------------------------------------------ byte-rANS table in LDS
// A block's decode table built from its 256 frequencies (FORMAT 2.2-2.3): slot
// t of symbol s (c[s] <= t < c[s] + f[s]) holds f | s << 24 and t - c[s]. The
// frequencies' exclusive prefix sums c go to cum (257 words of LDS); then each
// thread fills 4096 / WG consecutive slots, starting from the symbol that a
// binary search over c finds for its first one. A table that sums to 0 (no
// RANS stream may use it) is all zero. f is thread s's frequency, loaded by
// the caller early (before the item's pixel selection) so that its latency
// overlaps that work: 512 bytes per build instead of a 32 KB expanded table.
// T32: one word per slot, f | (t - c[s]) << 12 | s << 24 (a 16 KB table).
template <int WG, bool T32 = false>
__device__ __forceinline__ void rans_table_build(uint32_t f, uint32_t *tbl, uint32_t *cum, uint32_t *wtot) {
    static_assert(WG == 256, "one symbol per thread");
    constexpr uint32_t kSlots = 4096 / WG;
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint32_t x = f;  // inclusive prefix within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= (uint32_t)off) x += y;
    }
    __syncthreads();  // wtot and cum may still be read by the previous user
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (uint32_t w = 0; w < WG / 64; w++) {
        before += w < wave ? wtot[w] : 0u;
        total += wtot[w];
    }
    cum[tid] = before + x - f;
    if (tid == WG - 1) cum[WG] = before + x;
    __syncthreads();
    const uint32_t t0 = tid * kSlots;
    uint2 *out = reinterpret_cast<uint2 *>(tbl);
    if (total == 0) {
#pragma unroll
        for (uint32_t j = 0; j < kSlots; j++) {
            if constexpr (T32)
                tbl[t0 + j] = 0u;
            else
                out[t0 + j] = make_uint2(0u, 0u);
        }
        return;
    }
    // the last symbol whose range starts at or before t0 (its range holds t0)
    uint32_t lo = 0, hi = WG - 1;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if (cum[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    uint32_t sym = lo, c = cum[sym], e = cum[sym + 1];
#pragma unroll
    for (uint32_t j = 0; j < kSlots; j++) {
        const uint32_t t = t0 + j;
        while (t >= e) {
            sym++;
            c = e;
            e = cum[sym + 1];
        }
        if constexpr (T32)
            tbl[t] = ((e - c) & 0xFFFu) | ((t - c) << 12) | (sym << 24);
        else
            out[t] = make_uint2(((e - c) & 0xFFFu) | (sym << 24), t - c);
    }
}

// ------------------------------------------------------------------ reduce kernels
template <Op OP>
struct SharedPartials {
    uint32_t m0[kBlk];
    unsigned long long mr[OP == Op::Moments ? kBlk : 1];
    unsigned long long mc[OP == Op::Moments ? kBlk : 1];
    uint32_t c0;
    unsigned long long cr, cc;
};

template <Op OP>
__device__ __forceinline__ void zero_partials(SharedPartials<OP> &sp, uint32_t n) {
    for (uint32_t j = threadIdx.x; j < n; j += blockDim.x) {
        sp.m0[j] = 0;
        if (OP == Op::Moments) {
            sp.mr[j] = 0;
            sp.mc[j] = 0;
        }
    }
    if (threadIdx.x == 0) {
        sp.c0 = 0;
        sp.cr = 0;
        sp.cc = 0;
    }
}

template <Op OP>
__device__ __forceinline__ void flush_partials(SharedPartials<OP> &sp, uint32_t n, uint64_t s0, uint64_t S, void *out,
                                               int out64, int negate) {
    for (uint32_t j = threadIdx.x; j < n; j += blockDim.x) {
        const uint64_t s = s0 + j;
        if (OP == Op::Sum) {
            uint64_t v = (uint64_t)sp.m0[j] + sp.c0;
            if (!v) continue;
            if (out64)
                atomicAdd(reinterpret_cast<unsigned long long *>(out) + s,
                          (unsigned long long)(negate ? (0ull - v) : v));
            else
                atomicAdd(reinterpret_cast<uint32_t *>(out) + s, (uint32_t)(negate ? (0u - (uint32_t)v) : (uint32_t)v));
        } else {
            unsigned long long *m = reinterpret_cast<unsigned long long *>(out);
            const unsigned long long v0 = (unsigned long long)sp.m0[j] + sp.c0;
            const unsigned long long vr = sp.mr[j] + sp.cr, vc = sp.mc[j] + sp.cc;
            if (v0) atomicAdd(m + s, v0);
            if (vr) atomicAdd(m + S + s, vr);
            if (vc) atomicAdd(m + 2 * S + s, vc);
        }
    }
}

// Selection of one pixel tile: writes the tile-local offsets of the pixels with
// (mask[p] != 0) != complement (every pixel when mask is null) and valid[p],
// in increasing order, to sel (LDS) and returns their number. Wave ballots
// give each selected pixel its slot; nothing outside the workgroup is needed.
template <int WG>
__device__ __forceinline__ uint32_t select_tile(const DevResident &r, const uint8_t *mask, int complement, uint32_t p0,
                                                uint32_t cnt, uint16_t *sel, uint32_t *wtot) {
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const unsigned long long below = (1ull << lane) - 1ull;
    uint32_t total = 0;
    for (uint32_t base = 0; base < cnt; base += WG) {
        const uint32_t off = base + tid;
        bool f = false;
        if (off < cnt) {
            const uint32_t p = p0 + off;
            f = r.valid[p] != 0 && (mask ? ((mask[p] != 0) != (complement != 0)) : true);
        }
        const unsigned long long bal = __ballot(f);
        if (lane == 0) wtot[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t before = total, all = total;
#pragma unroll
        for (uint32_t w = 0; w < WG / 64; w++) {
            const uint32_t c = wtot[w];
            before += w < wave ? c : 0u;
            all += c;
        }
        if (f) sel[before + (uint32_t)__popcll(bal & below)] = (uint16_t)off;
        __syncthreads();
        total = all;
    }
    return total;
}

// Sums fit four workgroups per CU (36 KB of LDS, at most 128 VGPRs); the
// moment partials (44 KB of LDS) fit three. The extra waves hide latency when
// few streams are selected.
// Reorders an item's pixel list so that its RAW streams come first, keeping
// the order within each group. A wave whose streams are all rANS can then run
// a rANS-only decode form, while a RAW stream among them would send the whole
// wave to the unified step. Every thread reads its entries (i = tid and
// tid + WG) before the barrier and writes them to their new places after it.
template <int WG>
__device__ __forceinline__ void raw_first(const DevResident &r, uint32_t b, uint64_t base, uint32_t nbytes,
                                          uint32_t p0, uint32_t n_sel, uint16_t *sel) {
    constexpr uint32_t kWaves = WG / 64;
    __shared__ uint32_t rc[2 * kWaves];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint32_t v[2];
    bool raw[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const uint32_t i = tid + j * WG;
        v[j] = i < n_sel ? sel[i] : kHole;
        raw[j] = false;
        if (v[j] != kHole) {
            const Extent e = locate(r, b, p0 + v[j], base, nbytes);
            raw[j] = (ld16(r.payload, e.start) & 7u) == 2u;
        }
    }
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(raw[0]), m1 = __builtin_amdgcn_ballot_w64(raw[1]);
    if (lane == 0) {
        rc[wave] = (uint32_t)__popcll(m0);
        rc[kWaves + wave] = (uint32_t)__popcll(m1);
    }
    __syncthreads();  // every entry is read and counted
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t before0 = 0, all0 = 0, before1 = 0, total = 0;
#pragma unroll
    for (uint32_t w = 0; w < kWaves; w++) {
        before0 += w < wave ? rc[w] : 0u;
        all0 += rc[w];
        before1 += w < wave ? rc[kWaves + w] : 0u;
        total += rc[w] + rc[kWaves + w];
    }
    // raw entries before entry i, for i = tid and tid + WG
    const uint32_t rb0 = before0 + (uint32_t)__popcll(m0 & below);
    const uint32_t rb1 = all0 + before1 + (uint32_t)__popcll(m1 & below);
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const uint32_t i = tid + j * WG, rb = j ? rb1 : rb0;
        if (i < n_sel) sel[raw[j] ? rb : total + (i - rb)] = (uint16_t)v[j];
    }
    __syncthreads();
}

// The work items of a query: n_live items of each of n_visited blocks. With
// at least as many blocks as workgroups, workgroup g takes every item of
// blocks g, g + grid, ... in turn, so it decodes consecutive items of one block
// and keeps that block's LDS partials (and decode table) between them;
// otherwise item w of the grid-strided sequence is item w / n_visited of block
// w % n_visited (a grid that is a multiple of the blocks still keeps each
// workgroup on one block). Returns false when the workgroup has no k-th item.
__device__ __forceinline__ bool work_item(uint32_t k, uint32_t n_live, uint32_t n_visited, uint32_t &vb, uint32_t &t) {
    if (n_visited >= gridDim.x) {
        vb = (k / n_live) * gridDim.x + blockIdx.x;
        t = k % n_live;
        return vb < n_visited;
    }
    const uint32_t w = blockIdx.x + k * gridDim.x;
    vb = w % n_visited;
    t = w / n_visited;
    return w < n_live * n_visited;
}

// Whether sums and moments may keep a block's LDS partials over several items:
// a scan's u32 total over every pixel of the detector cannot pass 2^32 - 1
// (the rule that keeps a virtual image in 32 bits).
__device__ __forceinline__ bool hold_partials(const DevResident &r) {
    return (uint64_t)r.P * (r.dtype == 2 ? 65535u : 255u) <= 0xFFFFFFFFull;
}

// STG: sums and moments of residents whose blocks are mostly escape-heavy: one
// stream per lane, 17 KB of stream rings and a table of one word per slot, so
// the LDS allows as many workgroups per CU as without.
template <bool WIDE, Op OP, bool STG = false>
__global__ __launch_bounds__(kRansWG, OP == Op::Moments ? 3 : 4) void k_reduce_rans(DevResident r, const uint8_t *mask, int complement,
                                                         uint32_t stride, uint32_t n_visited, uint32_t tile_px,
                                                         const uint32_t *plan, void *out, int out64, int negate,
                                                         RegionBlocks rb, RegionArgs ra, AuxArgs da) {
    __shared__ __align__(16) uint32_t tbl[STG ? 4096 : 2 * 4096];  // per slot: f | symbol << 24, slot - c[symbol]
    __shared__ SharedPartials<OP> sp;
    __shared__ uint16_t sel[2 * kRansWG];
    __shared__ uint32_t wtot[kRansWG / 64];
    __shared__ uint32_t sbits[OP == Op::Dp ? 16 : 1];
    __shared__ uint16_t desc[kMaxItems<kRansWG>];
    __shared__ uint32_t ring[STG ? (kRansWG / 64) * kStageDw * 64 : 1];
    // planned: items of `cap` selected pixels; else every pixel tile of
    // tile_px. With a subtracted mask, its items follow those of mask.
    const bool two = da.neg_mask != nullptr;
    uint32_t n_first = (r.P + tile_px - 1) / tile_px, n_live = two ? 2 * n_first : n_first, cap = 0, end[2] = {0, 0};
    bool halves = false;
    // the staged form prefetches streams only for sparse selections: over most
    // of the detector the prefetched lines leave the L2 before their chunks
    // are read
    bool touch = true;
    if (plan) {
        const PlanView pv =
            plan_cut<kRansWG>(plan, r.P, n_visited, two, (OP == Op::Sum || OP == Op::Moments) && r.split, desc, wtot, STG);
        touch = !STG || pv.sparse;
        n_live = pv.n_items;
        n_first = pv.n_first;
        cap = pv.cap;
        end[0] = pv.end[0];
        end[1] = pv.end[1];
        halves = pv.halves;
    } else if constexpr (OP == Op::Region) {
        halves = da.halves && r.split;  // a latency-bound region read: items of half a workgroup
    }
    const Partials<OP> pt{sp.m0, sp.mr, sp.mc, &sp.c0, &sp.cr, &sp.cc};
    if constexpr (OP == Op::Amp) amp_stage<kRansWG>(ra);  // read after the item loop's first barrier
    uint32_t loaded = 0xFFFFFFFFu;
    // the block (and sign) whose sums the LDS partials hold; flushed when the block changes
    constexpr bool kAcc = OP == Op::Sum || OP == Op::Moments;
    const bool hold = hold_partials(r);
    uint32_t held_b = 0xFFFFFFFFu, held_n = 0;
    bool held_sub = false;
    uint32_t vb, t;
    for (uint32_t k = 0; n_live && work_item(k, n_live, n_visited, vb, t); k++) {
        const uint32_t b = is_region(OP) ? rb.b[vb] : vb * stride;
        const uint32_t fq = b != loaded ? r.freq[256ull * b + threadIdx.x] : 0u;  // the table build's input
        const bool sub = two && t >= n_first;  // an item of the subtracted mask
        const uint8_t *m = sub ? da.neg_mask : mask;
        uint32_t p0 = OP == Op::Index ? 0 : (sub && !plan ? t - n_first : t) * tile_px;
        __syncthreads();
        const uint32_t n_sel =
            OP == Op::Index ? index_group<kRansWG>(r, da.perm, t, sel)
            : plan ? select_range<kRansWG>(r, m, complement, desc[t], cap, end[sub], p0, sel, wtot)
                   : select_tile<kRansWG>(r, m, complement, p0, min(tile_px, r.P - p0), sel, wtot);
        const uint8_t *d = r.dir + 16ull * b;
        const uint64_t base = *reinterpret_cast<const uint64_t *>(d);
        const uint32_t n = *reinterpret_cast<const uint32_t *>(d + 8);
        const uint32_t nbytes = *reinterpret_cast<const uint32_t *>(d + 12);
        // blocks holding RAW streams (a resident without any has no flags)
        const bool raw_block = OP != Op::Index && OP != Op::Split && r.raw_blk && r.raw_blk[b];
        if (OP == Op::Split && n != kBlk) continue;  // a final partial block has no split points
        DpTile dt{nullptr, sbits, 0};
        if constexpr (OP == Op::Index) dt.row = da.rows + ((uint64_t)b * da.n_fields + (uint64_t)t * (kRansWG / 64)) * kBlk;
        if constexpr (OP == Op::Split) dt.row = da.rows;
        if constexpr (OP == Op::Dp) {
            dp_scan_bits<kRansWG>(da.scan_mask, (uint64_t)b * kBlk, n, sbits);
            __syncthreads();
            dt.row = da.part + (uint64_t)vb * r.P;
            dt.n_sel = dp_count(sbits);
            if (threadIdx.x == 0 && t == 0) da.nb[vb] = dt.n_sel;  // once per visited block
        }
        if (n_sel == 0) continue;
        if (kAcc && held_b != 0xFFFFFFFFu && (held_b != b || held_sub != sub)) {
            flush_partials<OP>(sp, held_n, (uint64_t)held_b * kBlk, r.S, out, out64, negate ^ (int)held_sub);
            held_b = 0xFFFFFFFFu;
            __syncthreads();
        }
        if (b != loaded) {
            // no partials are held here (they belong to the block), so they lend
            // the build room for the prefix sums; they are zeroed after it
            rans_table_build<kRansWG, STG>(fq, tbl, sp.m0, wtot);
            loaded = b;
            __syncthreads();  // the table is complete, and cum is read before the partials are zeroed
        }
        // a block with RAW streams: put them in waves of their own (an index
        // leaf must stay one wave, and the split-point build does not care)
        if (raw_block) raw_first<kRansWG>(r, b, base, nbytes, p0, n_sel, sel);
        if (kAcc && held_b == 0xFFFFFFFFu) {
            zero_partials<OP>(sp, n);
            held_b = b;
            held_n = n;
            held_sub = sub;
        }
        __syncthreads();
        // at most two slots per lane: with three decode forms, more do not fit 3 waves per SIMD
        const uint32_t K = (STG || OP == Op::Index || n_sel <= kRansWG) ? 1 : 2;  // an index leaf is one wave
        // split items (at most half a workgroup of streams): waves 0-1 decode the
        // first halves of the streams, waves 2-3 the second halves
        const uint32_t wave = threadIdx.x >> 6;
        const bool split_item = halves && n == kBlk;
        const uint32_t half = split_item ? 1u + (wave >> 1) : 0u;
        const uint32_t first = split_item ? (wave & 1u) * 64u : wave * 64 * K;
        if (first < n_sel) {  // whole waves without a stream skip the decode
            if (!STG && K == 2)
                rans_tile<STG ? 1 : 2, WIDE, OP, STG>(r, sel, p0, n_sel, first, b, n, base, nbytes, tbl, pt, ra, dt, 0,
                                                      raw_block, ring);
            else
                rans_tile<1, WIDE, OP, STG>(r, sel, p0, n_sel, first, b, n, base, nbytes, tbl, pt, ra, dt, half, raw_block,
                                            ring, touch);
        }
        __syncthreads();
        if (kAcc && !hold) {
            flush_partials<OP>(sp, n, (uint64_t)b * kBlk, r.S, out, out64, negate ^ (int)sub);
            held_b = 0xFFFFFFFFu;
        }
    }
    if (kAcc && held_b != 0xFFFFFFFFu)
        flush_partials<OP>(sp, held_n, (uint64_t)held_b * kBlk, r.S, out, out64, negate ^ (int)held_sub);
}

template <bool WIDE, Op OP>
__global__ __launch_bounds__(kPairWG) void k_reduce_paired(DevResident r, const uint8_t *mask, int complement,
                                                           uint32_t stride, uint32_t n_visited, uint32_t tile_px,
                                                           const uint32_t *plan, void *out, int out64, int negate,
                                                           RegionBlocks rb, RegionArgs ra, AuxArgs da) {
    // the 32 decode tables and the idle entry, then each model's window info:
    // an escape reads it from LDS, not from global memory, because a global load
    // inside the unrolled step made the compiler wait for every load in flight,
    // the reservoir prefetch included, at each step
    __shared__ uint32_t tbl[kPairTable + 32];
    __shared__ SharedPartials<OP> sp;
    __shared__ uint16_t sel[2 * kPairWG];
    __shared__ uint32_t wtot[kPairWG / 64];
    __shared__ uint32_t sbits[OP == Op::Dp ? 16 : 1];
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(r.tables);
        uint4 *dst = reinterpret_cast<uint4 *>(tbl);
        for (uint32_t i = threadIdx.x; i < kPairTable / 4; i += kPairWG) dst[i] = src[i];
        if (threadIdx.x < 32) tbl[kPairTable + threadIdx.x] = r.model_info[threadIdx.x];
    }
    __shared__ uint16_t desc[kMaxItems<kPairWG>];
    __shared__ uint16_t udesc[(OP == Op::Sum || OP == Op::Moments) ? kMaxPlanTiles : 1];
    __shared__ uint32_t next_unit;
    // planned: items of `cap` selected pixels; else every pixel tile of
    // tile_px. With a subtracted mask, its items follow those of mask.
    const bool two = da.neg_mask != nullptr;
    uint32_t n_first = (r.P + tile_px - 1) / tile_px, n_live = two ? 2 * n_first : n_first, cap = 0, end[2] = {0, 0};
    if (plan) {
        const PlanView pv = plan_cut<kPairWG>(plan, r.P, n_visited, two, false, desc, wtot);
        n_live = pv.n_items;
        n_first = pv.n_first;
        cap = pv.cap;
        end[0] = pv.end[0];
        end[1] = pv.end[1];
    }
    const Partials<OP> pt{sp.m0, sp.mr, sp.mc, &sp.c0, &sp.cr, &sp.cc};
    if constexpr (OP == Op::Amp) amp_stage<kPairWG>(ra);  // read after the item loop's first barrier
    // the block (and sign) whose sums the LDS partials hold; flushed when the block changes
    constexpr bool kAcc = OP == Op::Sum || OP == Op::Moments;
    const bool hold = hold_partials(r);
    uint32_t held_b = 0xFFFFFFFFu;
    bool held_sub = false;
    // Sums and moments of one mask: a workgroup takes whole blocks (or, with
    // fewer visited blocks than workgroups, an equal share of one block's
    // units), and each of its waves takes units of 64 or 128 selected pixels
    // (one or two streams per lane) one after another, selecting each unit's
    // pixels itself. The waves meet only at the end of the block or share,
    // where the partials are flushed: with a barrier after every work item,
    // waves spent a quarter of their time waiting for the slowest wave of the
    // item. Running apart, the waves fetch more stream lines again from past
    // the L2, but those reads stay far below the HBM rate.
    if constexpr (kAcc) {
        if (plan && !two && hold) {
            const uint32_t unit = cap > kPairWG ? 128u : 64u;
            const uint32_t n_units = plan_units<kPairWG>(plan, r.P, unit, udesc, wtot);
            const uint32_t shares = n_visited >= gridDim.x ? 1u : gridDim.x / n_visited;
            const uint32_t wave = threadIdx.x >> 6;
            uint16_t *wsel = sel + wave * 128u;
            const DpTile dt{nullptr, sbits, 0};
            for (uint32_t w = blockIdx.x; w < n_visited * shares; w += gridDim.x) {
                const uint32_t vb = w / shares, part = w % shares;
                const uint32_t b = vb * stride;
                const uint8_t *d = r.dir + 16ull * b;
                const uint64_t base = *reinterpret_cast<const uint64_t *>(d);
                const uint32_t nbytes = *reinterpret_cast<const uint32_t *>(d + 12);
                zero_partials<OP>(sp, kBlk);
                if (threadIdx.x == 0) next_unit = 0;
                __syncthreads();
                // the c-th unit of this share: two-stream units go to whichever wave
                // asks next (dim full-detector waves run far ahead of bright ones);
                // one-stream units (a disk's) in a fixed interleave, measured faster
                for (uint32_t k = 0;; k++) {
                    uint32_t c = k * (kPairWG / 64) + wave;
                    if (unit == 128u) {
                        if ((threadIdx.x & 63u) == 0) c = atomicAdd(&next_unit, 1u);
                        c = (uint32_t)__builtin_amdgcn_readfirstlane((int)c);
                    }
                    const uint32_t u = (c / (kPairWG / 64)) * shares * (kPairWG / 64) + part * (kPairWG / 64) +
                                       c % (kPairWG / 64);
                    if (u >= n_units) break;
                    uint32_t p0 = 0;
                    const uint32_t n_sel = select_unit(r, mask, complement, udesc[u], unit, end[0], p0, wsel);
                    if (n_sel == 0) continue;
                    if (unit == 128u)
                        paired_tile<2, WIDE, OP>(r, wsel, p0, n_sel, 0, b, base, nbytes, tbl, pt, ra, dt);
                    else
                        paired_tile<1, WIDE, OP>(r, wsel, p0, n_sel, 0, b, base, nbytes, tbl, pt, ra, dt);
                }
                __syncthreads();
                flush_partials<OP>(sp, kBlk, (uint64_t)b * kBlk, r.S, out, out64, negate);
                __syncthreads();
            }
            return;
        }
    }
    // a block's items go to neighbouring workgroups (w / n_live), so a wave of
    // workgroups reads few blocks at a time: measured faster here than keeping
    // a workgroup on one block; the partials are held only while the block stays
    const uint32_t n_work = n_live * n_visited;
    for (uint32_t w = blockIdx.x; w < n_work; w += gridDim.x) {
        const uint32_t vb = w / n_live, t = w % n_live;
        const uint32_t b = is_region(OP) ? rb.b[vb] : vb * stride;
        const bool sub = two && t >= n_first;  // an item of the subtracted mask
        const uint8_t *m = sub ? da.neg_mask : mask;
        uint32_t p0 = OP == Op::Index ? 0 : (sub && !plan ? t - n_first : t) * tile_px;
        __syncthreads();
        const uint32_t n_sel =
            OP == Op::Index ? index_group<kPairWG>(r, da.perm, t, sel)
            : plan ? select_range<kPairWG>(r, m, complement, desc[t], cap, end[sub], p0, sel, wtot)
                   : select_tile<kPairWG>(r, m, complement, p0, min(tile_px, r.P - p0), sel, wtot);
        const uint8_t *d = r.dir + 16ull * b;
        const uint64_t base = *reinterpret_cast<const uint64_t *>(d);
        const uint32_t nbytes = *reinterpret_cast<const uint32_t *>(d + 12);
        DpTile dt{nullptr, sbits, 0};
        if constexpr (OP == Op::Index) dt.row = da.rows + ((uint64_t)b * da.n_fields + (uint64_t)t * (kPairWG / 64)) * kBlk;
        if constexpr (OP == Op::Dp) {
            dp_scan_bits<kPairWG>(da.scan_mask, (uint64_t)b * kBlk, kBlk, sbits);
            __syncthreads();
            dt.row = da.part + (uint64_t)vb * r.P;
            dt.n_sel = dp_count(sbits);
            if (threadIdx.x == 0 && t == 0) da.nb[vb] = dt.n_sel;  // once per visited block
        }
        if (n_sel == 0) continue;
        if (kAcc && held_b != 0xFFFFFFFFu && (held_b != b || held_sub != sub)) {
            flush_partials<OP>(sp, kBlk, (uint64_t)held_b * kBlk, r.S, out, out64, negate ^ (int)held_sub);
            held_b = 0xFFFFFFFFu;
            __syncthreads();
        }
        if (kAcc && held_b == 0xFFFFFFFFu) {
            zero_partials<OP>(sp, kBlk);
            held_b = b;
            held_sub = sub;
        }
        __syncthreads();
        // at most two slots per lane: 1024-thread workgroups have 128 VGPRs per lane
        const uint32_t K = (OP == Op::Index || n_sel <= kPairWG) ? 1 : 2;  // an index leaf is one wave
        const uint32_t first = (threadIdx.x >> 6) * 64 * K;
        if (first < n_sel) {
            if (K == 2)
                paired_tile<2, WIDE, OP>(r, sel, p0, n_sel, first, b, base, nbytes, tbl, pt, ra, dt);
            else
                paired_tile<1, WIDE, OP>(r, sel, p0, n_sel, first, b, base, nbytes, tbl, pt, ra, dt);
        }
        __syncthreads();
        if (kAcc && !hold) {
            flush_partials<OP>(sp, kBlk, (uint64_t)b * kBlk, r.S, out, out64, negate ^ (int)sub);
            held_b = 0xFFFFFFFFu;
        }
    }
    if (kAcc && held_b != 0xFFFFFFFFu)
        flush_partials<OP>(sp, kBlk, (uint64_t)held_b * kBlk, r.S, out, out64, negate ^ (int)held_sub);
}

// out[i] = init[i], or 0 without init (u32 or u64 elements); with a plan,
// wave w of workgroup g counts the selected pixels of 64-pixel tile 4g + w
// (grid-strided; the tiles of a second mask follow those of the first).
__global__ void __launch_bounds__(256) k_init(void *out, int out64, const void *init, uint64_t n, PlanArgs pa) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        if (out64)
            reinterpret_cast<uint64_t *>(out)[i] = init ? reinterpret_cast<const uint64_t *>(init)[i] : 0;
        else
            reinterpret_cast<uint32_t *>(out)[i] = init ? reinterpret_cast<const uint32_t *>(init)[i] : 0;
    }
    if (!pa.counts) return;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t n_all = pa.mask2 ? 2 * pa.n_tiles : pa.n_tiles;
    for (uint32_t t = blockIdx.x * 4 + wave; t < n_all; t += gridDim.x * 4) {
        const bool second = t >= pa.n_tiles;
        const uint8_t *mask = second ? pa.mask2 : pa.mask;
        const uint32_t p = (t - (second ? pa.n_tiles : 0u)) * kPlanFine + lane;
        bool f = false;
        if (p < pa.P) f = pa.valid[p] != 0 && (mask ? ((mask[p] != 0) != (pa.complement != 0)) : true);
        const uint32_t c = (uint32_t)__popcll(__ballot(f));
        // encoded bytes of the tile's selected streams in block 0
        uint32_t len = 0;
        if (f) {
            const uint32_t s0 = pa.gbase0[p >> 5] + pa.rel0[p];
            const uint32_t s1 = p + 1 < pa.P ? pa.gbase0[(p + 1) >> 5] + pa.rel0[p + 1]
                                             : *reinterpret_cast<const uint32_t *>(pa.dir0 + 12);
            len = s1 - s0;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) len += __shfl_xor(len, off);
        if (lane == 0) {
            pa.counts[t] = c;
            pa.counts[kPlanBytes + t] = len;
        }
    }
}

__global__ void k_zero_bytes(uint8_t *out, uint64_t n) {
    const uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x, step = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t head = (16 - (reinterpret_cast<uint64_t>(out) & 15)) & 15;
    if (n <= head + 16) {
        for (uint64_t i = i0; i < n; i += step) out[i] = 0;
        return;
    }
    for (uint64_t i = i0; i < head; i += step) out[i] = 0;
    uint4 *body = reinterpret_cast<uint4 *>(out + head);
    const uint64_t nv = (n - head) / 16;
    for (uint64_t i = i0; i < nv; i += step) body[i] = make_uint4(0, 0, 0, 0);
    for (uint64_t i = head + 16 * nv + i0; i < n; i += step) out[i] = 0;
}

// Diffraction pattern from the per-(visited block, pixel) partial sums: the
// exact u64 sum, and the mean over the selected scans in float64 rounded to
// float32 (for scaled residents, of the reconstructed intensities, block by
// block in increasing order, each product and sum rounded in float64).
__global__ void k_dp_finalize(const uint32_t *part, const uint32_t *nb, uint32_t n_visited, uint32_t stride,
                              uint32_t P, const uint8_t *valid, const double *calib, uint64_t *sum, float *mean) {
    const uint32_t p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    uint64_t s = 0, n = 0;
    double acc = 0.0;
    const bool ok = valid[p] != 0;
    for (uint32_t vb = 0; vb < n_visited; vb++) {
        n += nb[vb];
        if (!ok) continue;
        const uint32_t c = part[(uint64_t)vb * P + p];
        s += c;
        if (calib) {
            const uint64_t b = (uint64_t)vb * stride;
            const double t1 = __dmul_rn(calib[2 * b], (double)c);
            const double t2 = __dmul_rn((double)nb[vb], calib[2 * b + 1]);
            acc = __dadd_rn(acc, __dadd_rn(t1, t2));
        }
    }
    sum[p] = ok ? s : 0;
    if (mean) mean[p] = (ok && n) ? (float)__ddiv_rn(calib ? acc : (double)s, (double)n) : 0.0f;
}

// ------------------------------------------------------------------ polar index: build
// Root rows (sums of 16 leaf rows) and the bit width of every field row.
__global__ void __launch_bounds__(512) k_index_widths(uint32_t n_leaves, uint32_t n_roots, uint32_t *rows,
                                                      uint8_t *width) {
    const uint32_t n_fields = n_leaves + n_roots;
    const uint32_t b = blockIdx.y, f = blockIdx.x, j = threadIdx.x;
    uint32_t *row = rows + ((uint64_t)b * n_fields + f) * kBlk;
    uint32_t v;
    if (f < n_leaves) {
        v = row[j];
    } else {
        const uint32_t l0 = (f - n_leaves) * kRoot, l1 = min(l0 + kRoot, n_leaves);
        v = 0;
        for (uint32_t l = l0; l < l1; l++) v += rows[((uint64_t)b * n_fields + l) * kBlk + j];
        row[j] = v;
    }
    // bits of the row's largest value
    uint32_t m = v;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor(m, off));
    __shared__ uint32_t wmax[kBlk / 64];
    if ((j & 63u) == 0) wmax[j >> 6] = m;
    __syncthreads();
    if (j == 0) {
        for (uint32_t w = 1; w < kBlk / 64; w++) m = max(m, wmax[w]);
        m = max(m, wmax[0]);
        width[(uint64_t)b * n_fields + f] = (uint8_t)(m ? 32 - __clz(m) : 0);
    }
}

// Field row (b, f) packed: value j at bits [j*w, j*w + w) of its dword run.
__global__ void __launch_bounds__(256) k_index_pack(uint32_t n_fields, const uint32_t *rows, const uint32_t *offset,
                                                    const uint8_t *width, uint32_t *packed) {
    const uint64_t bf = (uint64_t)blockIdx.y * n_fields + blockIdx.x;
    const uint32_t w = width[bf];
    if (!w) return;
    const uint32_t *row = rows + bf * kBlk;
    uint32_t *dst = packed + offset[bf];
    const uint32_t n_dw = (kBlk * w + 31) / 32;
    for (uint32_t d = threadIdx.x; d < n_dw; d += blockDim.x) {
        const uint32_t bit0 = 32 * d, bit1 = bit0 + 32;
        uint32_t word = 0;
        for (uint32_t j = bit0 / w; j < kBlk && j * w < bit1; j++) {
            const int sh = (int)(j * w) - (int)bit0;  // position of the value's bit 0 within the dword
            const uint32_t v = row[j];
            word |= sh >= 0 ? (v << sh) : (v >> -sh);
        }
        dst[d] = word;
    }
}

// ------------------------------------------------------------------ polar index: query
// Decomposition of mask & valid into index fields and residual pixels, in two
// kernels. k_index_leaf_flags: one wave per leaf counts the leaf's selected
// valid pixels (a ballot over its 64 polar positions), flags the leaf full when
// every valid pixel is selected, and writes the residual mask of its pixels:
// selected, valid and not in a full leaf (a full root's leaves are all full or
// without valid pixels, so the leaf flag decides).
constexpr uint32_t kMaxLeaves = 1024;  // detectors up to 65,535 pixels
__global__ void __launch_bounds__(256) k_index_leaf_flags(const DevResident r, DevIndex ix, const uint8_t *mask,
                                                          uint8_t *leaf_full, uint8_t *residual) {
    const uint32_t l = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63u;
    if (l >= ix.n_leaves) return;
    const uint32_t pos = l * kLeaf + lane;
    uint32_t p = 0;
    bool sel = false, val = false;
    if (pos < r.P) {
        p = ix.perm[pos];
        val = r.valid[p] != 0;
        sel = val && mask[p] != 0;
    }
    const uint32_t n_sel = (uint32_t)__popcll(__ballot(sel));
    const bool full = ix.leaf_valid[l] != 0 && n_sel == ix.leaf_valid[l];
    if (pos < r.P) residual[p] = sel && !full;
    if (lane == 0) leaf_full[l] = full;
}

// k_index_list: roots (every leaf full or without valid pixels, one valid
// pixel at least) and the field list: full roots, then full leaves outside
// them; fields[0] holds the count.
__global__ void __launch_bounds__(1024) k_index_list(DevIndex ix, const uint8_t *leaf_full, uint32_t *fields) {
    __shared__ uint8_t full[kMaxLeaves];
    __shared__ uint8_t root_full[kMaxLeaves / kRoot];
    __shared__ uint32_t wtot[1024 / 64];
    const uint32_t tid = threadIdx.x;
    for (uint32_t l = tid; l < ix.n_leaves; l += blockDim.x) full[l] = leaf_full[l];
    __syncthreads();
    for (uint32_t q = tid; q < ix.n_roots; q += blockDim.x) {
        bool all = true, any_valid = false;
        for (uint32_t l = q * kRoot; l < min((q + 1) * kRoot, ix.n_leaves); l++) {
            any_valid |= ix.leaf_valid[l] != 0;
            all &= full[l] || ix.leaf_valid[l] == 0;
        }
        root_full[q] = all && any_valid;
    }
    __syncthreads();
    const uint32_t lane = tid & 63u, wave = tid >> 6;
    const unsigned long long below = (1ull << lane) - 1ull;
    const uint32_t n_cand = ix.n_roots + ix.n_leaves;
    uint32_t total = 0;
    for (uint32_t base = 0; base < n_cand; base += blockDim.x) {
        const uint32_t c = base + tid;
        bool f = false;
        uint32_t id = 0;
        if (c < ix.n_roots) {
            f = root_full[c];
            id = ix.n_leaves + c;
        } else if (c < n_cand) {
            const uint32_t l = c - ix.n_roots;
            f = full[l] && !root_full[l / kRoot];
            id = l;
        }
        const unsigned long long bal = __ballot(f);
        if (lane == 0) wtot[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t before = total, all = total;
        for (uint32_t w = 0; w < blockDim.x / 64; w++) {
            before += w < wave ? wtot[w] : 0u;
            all += wtot[w];
        }
        if (f) fields[1 + before + (uint32_t)__popcll(bal & below)] = id;
        __syncthreads();
        total = all;
    }
    if (tid == 0) fields[0] = total;
}

// Sum of the listed fields of each visited block, added into out (u32/u64 per scan).
constexpr uint32_t kFieldChunk = 64;
__global__ void __launch_bounds__(256) k_index_sum(DevIndex ix, const uint32_t *fields, uint32_t stride,
                                                   uint32_t n_blocks, uint64_t S, void *out, int out64) {
    const uint32_t n_sel = fields[0];
    const uint32_t f0 = blockIdx.y * kFieldChunk;
    if (f0 >= n_sel) return;
    const uint32_t f1 = min(f0 + kFieldChunk, n_sel);
    const uint32_t b = blockIdx.x * stride;
    if (b >= n_blocks) return;
    const uint32_t n_fields = ix.n_leaves + ix.n_roots;
    for (uint32_t j = threadIdx.x; j < kBlk; j += blockDim.x) {
        const uint64_t s = (uint64_t)b * kBlk + j;
        if (s >= S) break;
        uint64_t acc = 0;
        for (uint32_t i = f0; i < f1; i++) {
            const uint64_t bf = (uint64_t)b * n_fields + fields[1 + i];
            const uint32_t w = ix.width[bf];
            if (!w) continue;
            const uint32_t bit = j * w;
            const uint32_t *src = ix.packed + ix.offset[bf] + (bit >> 5);
            // two dwords hold any value of at most 32 bits; the packed buffer is padded
            const uint64_t two = (uint64_t)src[0] | ((uint64_t)src[1] << 32);
            acc += (uint32_t)(two >> (bit & 31u)) & (w == 32 ? 0xFFFFFFFFu : ((1u << w) - 1u));
        }
        if (!acc) continue;
        if (out64)
            atomicAdd(reinterpret_cast<unsigned long long *>(out) + s, (unsigned long long)acc);
        else
            atomicAdd(reinterpret_cast<uint32_t *>(out) + s, (uint32_t)acc);
    }
}

// Masks of a change between two detector masks.
__global__ void k_mask_delta(const uint8_t *prev, const uint8_t *mask, uint32_t P, uint8_t *added, uint8_t *removed) {
    for (uint32_t p = blockIdx.x * blockDim.x + threadIdx.x; p < P; p += gridDim.x * blockDim.x) {
        const bool a = prev[p] != 0, b = mask[p] != 0;
        added[p] = b && !a;
        removed[p] = a && !b;
    }
}

// Stream headers of a resident built from a device container (FORMAT 1.4,
// 2.4, 3.4): reserved bits clear, a mode the layout defines, the model bits
// only on a paired stream, and byte-rANS streams only with a usable table.
// counts[mode] gets the valid streams; bad the first bad (block << 32 | pixel).
__global__ void __launch_bounds__(256) k_raw_blocks(DevResident r, uint8_t *out) {
    const uint32_t b = blockIdx.y, p = blockIdx.x * 256 + threadIdx.x;
    bool raw = false;
    if (p < r.P) {
        const uint64_t base = *reinterpret_cast<const uint64_t *>(r.dir + 16ull * b);
        const uint64_t gi = (uint64_t)b * r.G + (p >> 5);
        const uint64_t st = base + r.gbase[gi] + r.rel[gi * 32 + (p & 31u)];
        raw = (*reinterpret_cast<const uint16_t *>(r.payload + st) & 7u) == 2u;
    }
    if (__builtin_amdgcn_ballot_w64(raw) && (threadIdx.x & 63u) == 0) out[b] = 1;
}

__global__ void __launch_bounds__(256) k_check_headers(DevResident r, const uint8_t *usable, unsigned long long *counts,
                                                       unsigned long long *bad) {
    __shared__ uint32_t c[8];
    if (threadIdx.x < 8) c[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t b = blockIdx.y, p = blockIdx.x * 256 + threadIdx.x;
    if (p < r.P) {
        const uint64_t base = *reinterpret_cast<const uint64_t *>(r.dir + 16ull * b);
        const uint64_t gi = (uint64_t)b * r.G + (p >> 5);
        const uint64_t st = base + r.gbase[gi] + r.rel[gi * 32 + (p & 31u)];
        const uint32_t hdr = *reinterpret_cast<const uint16_t *>(r.payload + st);
        const uint32_t mode = hdr & 7u, model = (hdr >> 3) & 31u;
        bool ok = (hdr >> 8) == 0;
        if (r.layout == 0)
            ok = ok && mode <= 2 && model == 0 && !(mode == 1 && !usable[b]);  // 0 CONST, 1 RANS, 2 RAW
        else
            ok = ok && mode <= 4 && !(model && mode != 3);  // 3 PAIRED
        if (ok)
            atomicAdd(&c[mode], 1u);
        else
            atomicMin(bad, ((unsigned long long)b << 32) | p);
    }
    __syncthreads();
    if (threadIdx.x < 8 && c[threadIdx.x]) atomicAdd(counts + threadIdx.x, (unsigned long long)c[threadIdx.x]);
}

__global__ void k_com_finalize(const uint64_t *m, uint64_t S, float *row, float *col) {
    for (uint64_t s = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; s < S; s += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t m0 = m[s];
        if (m0 == 0) {
            row[s] = 0.0f;
            col[s] = 0.0f;
        } else {
            row[s] = (float)((double)m[S + s] / (double)m0);
            col[s] = (float)((double)m[2 * S + s] / (double)m0);
        }
    }
}

}  // namespace

// ------------------------------------------------------------------ launchers
int device_cu_count() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            cus = prop.multiProcessorCount;
        if (cus <= 0) cus = 256;
    }
    return cus;
}

// Pixel-tile size: the largest tile whose count of (block, tile) items fills
// the resident workgroup slots in whole rounds.
static uint32_t pick_tile(uint32_t P, uint32_t n_visited, uint32_t slots, const uint32_t *cands, int ncand) {
    uint32_t best = cands[ncand - 1];
    double best_eff = -1.0;
    for (int i = 0; i < ncand; i++) {
        const double items = (double)((P + cands[i] - 1) / cands[i]) * n_visited;
        const double rounds = items / slots;
        const double eff = rounds / std::ceil(rounds);
        if (eff >= 0.85) return cands[i];
        if (eff > best_eff) {
            best_eff = eff;
            best = cands[i];
        }
    }
    return best;
}

// Workgroups of a kernel that the device holds at once (occupancy x CUs),
// computed once per kernel.
template <typename F>
static uint32_t resident_wgs(F kern, int threads) {
    static std::mutex mu;
    static std::unordered_map<const void *, uint32_t> cache;
    const void *key = reinterpret_cast<const void *>(kern);
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, threads, 0) != hipSuccess || per < 1) per = 1;
    const uint32_t n = (uint32_t)per * (uint32_t)device_cu_count();
    cache.emplace(key, n);
    return n;
}

// One query: the init kernel (outputs + plan), then the reduce. The tile size
// is chosen for whole rounds of the resident workgroups and the grid never
// exceeds them.
template <typename F>
static void launch_items(F kern, int threads, const uint32_t *cands, int ncand, hipStream_t st, const DevResident &r,
                         const uint8_t *mask, int complement, uint32_t stride, uint32_t n_visited, void *out, int out64,
                         int negate, const void *init, uint64_t n_init, const RegionBlocks &rb, const RegionArgs &ra,
                         const AuxArgs &da) {
    const uint32_t slots = resident_wgs(kern, threads);
    // a planned query counts 64-pixel tiles and the reduce cuts the items;
    // without a plan (region reads, or too many tiles) every pixel tile
    // of the host's size is an item
    const uint32_t n_fine = (r.P + kPlanFine - 1) / kPlanFine;
    const bool planned = n_init && n_fine <= kMaxPlanTiles;
    const uint32_t tile = planned ? kPlanFine : pick_tile(r.P, n_visited, slots, cands, ncand);
    const uint32_t n_tiles = (r.P + tile - 1) / tile, n_masks = da.neg_mask ? 2 : 1;
    uint32_t *plan = planned ? r.plan : nullptr;
    if (n_init) {
        const PlanArgs pa{mask, da.neg_mask, r.valid, complement, r.P, n_tiles, plan, r.gbase, r.rel, r.dir};
        const uint32_t grid = (uint32_t)std::max<uint64_t>(
            planned ? (n_masks * n_tiles + 3) / 4 : 1,
            std::max<uint64_t>(1, std::min<uint64_t>(2048, (n_init + 255) / 256)));
        hipLaunchKernelGGL(k_init, dim3(grid), dim3(256), 0, st, out, out64, init, n_init, pa);
    }
    // planned items number at most one per 64-pixel tile and mask
    const uint64_t items = (uint64_t)n_masks * n_tiles * n_visited;
    const uint32_t grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(items, slots));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, st, r, mask, complement, stride, n_visited, tile, plan, out,
                       out64, negate, rb, ra, da);
}

template <bool W, Op O>
static void launch_layout(const DevResident &r, const uint8_t *mask, int complement, uint32_t stride,
                          uint32_t n_visited, void *out, int out64, int negate, const void *init, uint64_t n_init,
                          const RegionBlocks &rb, const RegionArgs &ra, hipStream_t st, const AuxArgs &da = AuxArgs{}) {
    if (r.layout == 0) {
        const uint32_t cands[2] = {2 * kRansWG, kRansWG};
        if constexpr (W && (O == Op::Sum || O == Op::Moments)) {
            if (r.esc_heavy) {  // one stream per lane
                launch_items(k_reduce_rans<W, O, true>, kRansWG, cands + 1, 1, st, r, mask, complement, stride,
                             n_visited, out, out64, negate, init, n_init, rb, ra, da);
                return;
            }
        }
        launch_items(k_reduce_rans<W, O>, kRansWG, cands, 2, st, r, mask, complement, stride, n_visited, out, out64,
                     negate, init, n_init, rb, ra, da);
    } else {
        const uint32_t cands[2] = {2 * kPairWG, kPairWG};
        launch_items(k_reduce_paired<W, O>, kPairWG, cands, 2, st, r, mask, complement, stride, n_visited, out, out64,
                     negate, init, n_init, rb, ra, da);
    }
}

hipError_t launch_query(const DevResident &r, const uint8_t *mask, int complement, uint32_t stride, Op op, void *out,
                        int out64, int negate, const void *init, uint64_t n_init, hipStream_t st,
                        const uint8_t *neg_mask) {
    const uint32_t n_visited = (r.n_blocks + stride - 1) / stride;
    const RegionBlocks rb{};
    const RegionArgs ra{};
    const bool wide = r.dtype == 2;
    AuxArgs da{};
    da.neg_mask = neg_mask;
#define QSC_LAUNCH(W, O) \
    launch_layout<W, O>(r, mask, complement, stride, n_visited, out, out64, negate, init, n_init, rb, ra, st, da)
    if (op == Op::Sum) {
        if (wide) QSC_LAUNCH(true, Op::Sum); else QSC_LAUNCH(false, Op::Sum);
    } else {
        if (wide) QSC_LAUNCH(true, Op::Moments); else QSC_LAUNCH(false, Op::Moments);
    }
#undef QSC_LAUNCH
    return hipGetLastError();
}

hipError_t launch_com_finalize(const uint64_t *moments, uint64_t S, float *row, float *col, hipStream_t st) {
    const uint32_t grid = (uint32_t)std::min<uint64_t>(4096, (S + 255) / 256);
    hipLaunchKernelGGL(k_com_finalize, dim3(std::max(1u, grid)), dim3(256), 0, st, moments, S, row, col);
    return hipGetLastError();
}

hipError_t launch_region(const DevResident &r, const RegionBlocks &blocks, const RegionArgs &ra, hipStream_t st) {
    // a rectangle whose items of half-workgroup tiles fit one round of the
    // resident workgroups is latency-bound: decode both halves of each stream
    // side by side
    if (r.layout == 0 && r.split && !ra.frames && ra.out_kind != 2) {
        AuxArgs da{};
        da.halves = 1;
        const uint32_t cands[1] = {kRansWG / 2};
        const uint64_t items = (uint64_t)((r.P + kRansWG / 2 - 1) / (kRansWG / 2)) * blocks.n;
        if (r.dtype == 2 && items <= resident_wgs(k_reduce_rans<true, Op::Region>, kRansWG)) {
            launch_items(k_reduce_rans<true, Op::Region>, kRansWG, cands, 1, st, r, nullptr, 0, 1, blocks.n, nullptr,
                         0, 0, nullptr, 0, blocks, ra, da);
            return hipGetLastError();
        }
        if (r.dtype != 2 && items <= resident_wgs(k_reduce_rans<false, Op::Region>, kRansWG)) {
            launch_items(k_reduce_rans<false, Op::Region>, kRansWG, cands, 1, st, r, nullptr, 0, 1, blocks.n, nullptr,
                         0, 0, nullptr, 0, blocks, ra, da);
            return hipGetLastError();
        }
    }
#define QSC_REGION(W, O) launch_layout<W, O>(r, nullptr, 0, 1, blocks.n, nullptr, 0, 0, nullptr, 0, blocks, ra, st)
    if (ra.out_kind == 2) {
        if (r.dtype == 2) QSC_REGION(true, Op::Amp); else QSC_REGION(false, Op::Amp);
    } else if (ra.frames) {
        if (r.dtype == 2) QSC_REGION(true, Op::Frames); else QSC_REGION(false, Op::Frames);
    } else {
        if (r.dtype == 2) QSC_REGION(true, Op::Region); else QSC_REGION(false, Op::Region);
    }
#undef QSC_REGION
    return hipGetLastError();
}

hipError_t launch_dp(const DevResident &r, const uint8_t *scan_mask, uint32_t stride, uint32_t *part, uint32_t *nb,
                     uint64_t *sum, float *mean, hipStream_t st) {
    const uint32_t n_visited = (r.n_blocks + stride - 1) / stride;
    const AuxArgs da{scan_mask, part, nb};
    // the init kernel zeroes the per-block scan counts and plans the valid pixels
    if (r.dtype == 2)
        launch_layout<true, Op::Dp>(r, nullptr, 0, stride, n_visited, nb, 0, 0, nullptr, n_visited, RegionBlocks{},
                                    RegionArgs{}, st, da);
    else
        launch_layout<false, Op::Dp>(r, nullptr, 0, stride, n_visited, nb, 0, 0, nullptr, n_visited, RegionBlocks{},
                                     RegionArgs{}, st, da);
    hipLaunchKernelGGL(k_dp_finalize, dim3((r.P + 255) / 256), dim3(256), 0, st, part, nb, n_visited, stride, r.P,
                       r.valid, r.calib, sum, mean);
    return hipGetLastError();
}

hipError_t launch_index_leaves(const DevResident &r, const uint16_t *perm, uint32_t n_leaves, uint32_t n_roots,
                               uint32_t *rows, hipStream_t st) {
    AuxArgs da{};
    da.perm = perm;
    da.rows = rows;
    da.n_fields = n_leaves + n_roots;
    const uint32_t n_visited = r.n_blocks;
    const RegionBlocks rb{};
    const RegionArgs ra{};
    // one item = one group of leaves (a workgroup's waves), no plan: tile_px is the group size
    if (r.layout == 0) {
        const uint32_t cands[1] = {kRansWG};
        if (r.dtype == 2)
            launch_items(k_reduce_rans<true, Op::Index>, kRansWG, cands, 1, st, r, nullptr, 0, 1, n_visited, nullptr,
                         0, 0, nullptr, 0, rb, ra, da);
        else
            launch_items(k_reduce_rans<false, Op::Index>, kRansWG, cands, 1, st, r, nullptr, 0, 1, n_visited, nullptr,
                         0, 0, nullptr, 0, rb, ra, da);
    } else {
        const uint32_t cands[1] = {kPairWG};
        if (r.dtype == 2)
            launch_items(k_reduce_paired<true, Op::Index>, kPairWG, cands, 1, st, r, nullptr, 0, 1, n_visited,
                         nullptr, 0, 0, nullptr, 0, rb, ra, da);
        else
            launch_items(k_reduce_paired<false, Op::Index>, kPairWG, cands, 1, st, r, nullptr, 0, 1, n_visited,
                         nullptr, 0, 0, nullptr, 0, rb, ra, da);
    }
    return hipGetLastError();
}

hipError_t launch_index_widths(uint32_t n_blocks, uint32_t n_leaves, uint32_t n_roots, uint32_t *rows,
                               uint8_t *width, hipStream_t st) {
    hipLaunchKernelGGL(k_index_widths, dim3(n_leaves + n_roots, n_blocks), dim3(kBlk), 0, st, n_leaves, n_roots, rows,
                       width);
    return hipGetLastError();
}

hipError_t launch_index_pack(uint32_t n_blocks, uint32_t n_fields, const uint32_t *rows, const uint32_t *offset,
                             const uint8_t *width, uint32_t *packed, hipStream_t st) {
    hipLaunchKernelGGL(k_index_pack, dim3(n_fields, n_blocks), dim3(256), 0, st, n_fields, rows, offset, width, packed);
    return hipGetLastError();
}

hipError_t launch_indexed_sum(const DevResident &r, const DevIndex &ix, const uint8_t *mask, uint32_t stride,
                              void *out, int out64, uint32_t *fields, uint8_t *residual, hipStream_t st) {
    // the leaf flags sit after the field list in the same scratch
    uint8_t *leaf_full = reinterpret_cast<uint8_t *>(fields + ix.n_leaves + ix.n_roots + 1);
    hipLaunchKernelGGL(k_index_leaf_flags, dim3((ix.n_leaves + 3) / 4), dim3(256), 0, st, r, ix, mask, leaf_full,
                       residual);
    hipLaunchKernelGGL(k_index_list, dim3(1), dim3(1024), 0, st, ix, leaf_full, fields);
    // zero the output and decode the residual pixels, then add the index fields
    hipError_t e = launch_query(r, residual, 0, stride, Op::Sum, out, out64, 0, nullptr, r.S, st);
    if (e != hipSuccess) return e;
    const uint32_t n_visited = (r.n_blocks + stride - 1) / stride;
    const uint32_t chunks = (ix.n_leaves + ix.n_roots + kFieldChunk - 1) / kFieldChunk;
    hipLaunchKernelGGL(k_index_sum, dim3(n_visited, chunks), dim3(256), 0, st, ix, fields, stride, r.n_blocks, r.S,
                       out, out64);
    return hipGetLastError();
}

hipError_t launch_mask_delta(const uint8_t *prev, const uint8_t *mask, uint32_t P, uint8_t *added, uint8_t *removed,
                             hipStream_t st) {
    hipLaunchKernelGGL(k_mask_delta, dim3(std::max(1u, std::min(1024u, (P + 255) / 256))), dim3(256), 0, st, prev,
                       mask, P, added, removed);
    return hipGetLastError();
}

hipError_t launch_split_build(const DevResident &r, uint32_t *out, hipStream_t st) {
    AuxArgs da{};
    da.rows = out;
    const RegionBlocks rb{};
    const RegionArgs ra{};
    // every pixel tile of every block, no plan (the partial final block is skipped)
    const uint32_t cands[1] = {kRansWG};
    if (r.dtype == 2)
        launch_items(k_reduce_rans<true, Op::Split>, kRansWG, cands, 1, st, r, nullptr, 0, 1, r.n_blocks, nullptr, 0, 0,
                     nullptr, 0, rb, ra, da);
    else
        launch_items(k_reduce_rans<false, Op::Split>, kRansWG, cands, 1, st, r, nullptr, 0, 1, r.n_blocks, nullptr, 0,
                     0, nullptr, 0, rb, ra, da);
    return hipGetLastError();
}

hipError_t launch_raw_blocks(const DevResident &r, uint8_t *out, hipStream_t st) {
    hipLaunchKernelGGL(k_raw_blocks, dim3((r.P + 255) / 256, r.n_blocks), dim3(256), 0, st, r, out);
    return hipGetLastError();
}

hipError_t launch_check_headers(const DevResident &r, const uint8_t *usable, unsigned long long *counts,
                                unsigned long long *bad, hipStream_t st) {
    hipLaunchKernelGGL(k_check_headers, dim3((r.P + 255) / 256, r.n_blocks), dim3(256), 0, st, r, usable, counts, bad);
    return hipGetLastError();
}

hipError_t launch_zero_bytes(void *out, uint64_t n, hipStream_t st) {
    const uint32_t grid = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(2048, (n / 16 + 255) / 256));
    hipLaunchKernelGGL(k_zero_bytes, dim3(grid), dim3(256), 0, st, reinterpret_cast<uint8_t *>(out), n);
    return hipGetLastError();
}

}  // namespace qsc
