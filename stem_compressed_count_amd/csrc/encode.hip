// Device encoder: containers of both stream layouts (FORMAT.md) built from
// values already in device memory, byte-identical to the host encoder.
//
// The paired-resident page ("Operation pipeline" items 1-2) has counts arrive
// as complete 512-scan blocks and be coded per detector-pixel stream with a
// per-block frequency table; the scaled-uint16 page calibrates each float32
// region to uint16 codes first. Here every step runs on the GPU:
//   calibration (scaled only): per-block min/max with first-index ties, the
//     f64 scale and offset, and the codes;
//   k_enc_scan: one lane per (block, pixel) stream reads its values once,
//     flags constant streams and histograms the symbols of the others;
//   k_enc_table: one wave per block quantises the histogram to 4096;
//   k_enc_size: one lane per stream runs the rANS coder in reverse to count
//     its words and picks CONST, RANS or RAW;
//   k_enc_offsets / k_enc_dir: prefix sums give the grouped offsets, block
//     sizes and bases;
//   k_enc_write: one lane per stream writes its header and payload, the rANS
//     words straight to their final place (the last pushed word first).
// The paired layout (FORMAT 3) replaces the table and size steps: one lane per
// stream finds EMPTY / CONST, the SPARSE size, the static cost of all 32 pair
// models at once (32 accumulators, one pass over the pairs), then runs the
// tANS coder of the cheapest model in reverse for its exact bit count; the
// writer runs it again and fills the code section from its end, 16 bits at a
// time, since the pairs are coded last to first but read first to last.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "qsc_internal.hpp"

using namespace qsc;

namespace {

constexpr uint32_t kWG = 256;

struct EncGeom {
    uint64_t S;
    uint32_t P, G, nb;
};

__device__ __forceinline__ uint32_t block_scans(const EncGeom &g, uint32_t b) {
    return (uint32_t)min<uint64_t>(kBlock, g.S - (uint64_t)b * kBlock);
}

template <typename T>
__device__ __forceinline__ uint32_t value_at(const T *data, const EncGeom &g, uint32_t b, uint32_t j, uint32_t p) {
    return data[((uint64_t)b * kBlock + j) * g.P + p];
}

__device__ __forceinline__ uint32_t raw_bytes(uint32_t n, bool wide) { return wide ? 2 + 2 * n : 2 + n + (n & 1u); }

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)v, off);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_min64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), off) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)v, off);
        v = o < v ? o : v;
    }
    return v;
}

// ------------------------------------------------------------------ calibration (FORMAT 1.5)
// Order-preserving key of a finite float; +0 and -0 share a key, so the
// tie-break below keeps the first of them like a sequential scan does.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Per block: the smallest value with the lowest index (lo: key << 32 | index)
// and the largest with the lowest index (hi: key << 32 | ~index), by atomics
// over workgroups; bad = 1 if any value is NaN or infinite.
__global__ __launch_bounds__(kWG) void k_cal_minmax(const float *x, EncGeom g, uint32_t chunk,
                                                    unsigned long long *lo, unsigned long long *hi, uint32_t *bad) {
    const uint32_t b = blockIdx.y;
    const uint64_t n = (uint64_t)block_scans(g, b) * g.P;
    const float *xb = x + (uint64_t)b * kBlock * g.P;
    const uint64_t i0 = (uint64_t)blockIdx.x * chunk, i1 = min<uint64_t>(n, i0 + chunk);
    uint64_t mn = ~0ull, mx = 0;
    bool nonfinite = false;
    for (uint64_t i = i0 + threadIdx.x; i < i1; i += kWG) {
        const float v = xb[i];
        if (!isfinite(v)) {
            nonfinite = true;
            continue;
        }
        const uint64_t k = (uint64_t)order_key(v) << 32;
        mn = min(mn, k | (uint32_t)i);
        mx = max(mx, k | (uint32_t)~(uint32_t)i);
    }
    mn = wave_min64(mn);
    mx = wave_max64(mx);
    const bool any_bad = __ballot(nonfinite) != 0;
    __shared__ unsigned long long smn[kWG / 64], smx[kWG / 64];
    __shared__ uint32_t sbad[kWG / 64];
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    if (lane == 0) {
        smn[wave] = mn;
        smx[wave] = mx;
        sbad[wave] = any_bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t bd = 0;
        for (uint32_t w = 0; w < kWG / 64; w++) {
            mn = min(mn, (uint64_t)smn[w]);
            mx = max(mx, (uint64_t)smx[w]);
            bd |= sbad[w];
        }
        if (mn != ~0ull) atomicMin(lo + b, (unsigned long long)mn);
        if (mx != 0) atomicMax(hi + b, (unsigned long long)mx);
        if (bd) atomicOr(bad, 1u);
    }
}

// scale and offset of every block, in float64 as the format fixes them
__global__ void k_cal_params(const float *x, EncGeom g, const unsigned long long *lo, const unsigned long long *hi,
                             double *calib) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= g.nb) return;
    if (lo[b] == ~0ull || hi[b] == 0) {  // no finite value: the encode fails on the bad flag
        calib[2 * b] = 1.0;
        calib[2 * b + 1] = 0.0;
        return;
    }
    const float *xb = x + (uint64_t)b * kBlock * g.P;
    const double vlo = (double)xb[(uint32_t)lo[b]];
    const double vhi = (double)xb[~(uint32_t)hi[b]];
    calib[2 * b] = vhi == vlo ? 1.0 : (vhi - vlo) / 65535.0;
    calib[2 * b + 1] = vlo;
}

// codes = clamp(round-half-even((x - offset) / scale)); a constant region
// (hi == lo) codes every value as 0, which this formula also gives
__global__ __launch_bounds__(kWG) void k_cal_codes(const float *x, EncGeom g, const double *calib, uint16_t *codes) {
    const uint64_t n = g.S * g.P;
    for (uint64_t i = (uint64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (uint64_t)gridDim.x * kWG) {
        const uint32_t b = (uint32_t)(i / ((uint64_t)kBlock * g.P));
        const double sc = calib[2 * b], off = calib[2 * b + 1];
        double c = rint(((double)x[i] - off) / sc);
        c = c < 0.0 ? 0.0 : (c > 65535.0 ? 65535.0 : c);
        codes[i] = (uint16_t)c;
    }
}

// ------------------------------------------------------------------ byte-rANS (FORMAT 2)
// meta: bit 31 set for a constant stream, its value in the low 16 bits.
// hist: per block, the symbol counts of the non-constant streams.
template <typename T>
__global__ __launch_bounds__(kWG) void k_enc_scan(const T *data, EncGeom g, uint32_t *hist, uint32_t *meta) {
    __shared__ uint32_t h[256];
    const uint32_t b = blockIdx.y, p = blockIdx.x * kWG + threadIdx.x, n = block_scans(g, b);
    h[threadIdx.x] = 0;
    __syncthreads();
    if (p < g.P) {
        const uint32_t v0 = value_at(data, g, b, 0, p);
        bool eq = true;
        for (uint32_t j = 0; j < n; j++) {
            const uint32_t v = value_at(data, g, b, j, p);
            eq &= v == v0;
            atomicAdd(&h[min(v, 255u)], 1u);
        }
        if (eq) atomicSub(&h[min(v0, 255u)], n);
        meta[(uint64_t)b * g.P + p] = eq ? (0x80000000u | v0) : 0u;
    }
    __syncthreads();
    if (h[threadIdx.x]) atomicAdd(&hist[256 * b + threadIdx.x], h[threadIdx.x]);
}

// One wave per block; lane l holds symbols 4l .. 4l+3. Writes the block's
// 256 u16 frequencies into the container, enc[s] = f | c << 16 (c the
// cumulative start), and usable = a RANS stream may use the table.
__global__ __launch_bounds__(64) void k_enc_table(const uint32_t *hist, uint16_t *table, uint32_t *enc,
                                                  uint8_t *usable) {
    const uint32_t b = blockIdx.x, lane = threadIdx.x;
    uint32_t h[4], f[4];
    uint32_t N = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        h[k] = hist[256 * b + 4 * lane + k];
        N += h[k];
    }
    N = wave_sum(N);  // at most 512 x 1024^2 values
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        f[k] = h[k] ? max(1u, (uint32_t)((uint64_t)h[k] * 4096u / N)) : 0u;
        sum += f[k];
    }
    sum = wave_sum(sum);
    // too many: decrement the largest f > 1, lowest symbol on ties
    while (sum > 4096u) {
        uint64_t key = 0;
#pragma unroll
        for (int k = 0; k < 4; k++)
            if (f[k] > 1) key = max(key, ((uint64_t)f[k] << 8) | (255u - (4 * lane + k)));
        key = wave_max64(key);
        const uint32_t s = 255u - (uint32_t)(key & 255u);
        if (s / 4 == lane) f[s % 4]--;
        sum--;
    }
    // too few: the whole deficit goes to the largest h, lowest symbol on ties
    if (N && sum < 4096u) {
        uint64_t key = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) key = max(key, ((uint64_t)h[k] << 8) | (255u - (4 * lane + k)));
        key = wave_max64(key);
        const uint32_t s = 255u - (uint32_t)(key & 255u);
        if (s / 4 == lane) f[s % 4] += 4096u - sum;
    }
    // cumulative starts: the lane's own prefix, then an exclusive scan over lanes
    uint32_t local = f[0] + f[1] + f[2] + f[3], x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= (uint32_t)off) x += y;
    }
    uint32_t c = x - local;
    uint32_t nz = 0, full = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        table[256 * b + 4 * lane + k] = (uint16_t)f[k];
        enc[256 * b + 4 * lane + k] = f[k] | (c << 16);
        c += f[k];
        nz += f[k] != 0;
        full |= f[k] == 4096u;
    }
    nz = wave_sum(nz);
    full = wave_sum(full);
    if (lane == 0) usable[b] = nz > 0 && full == 0;
}

// The rANS coder over one stream in reverse (FORMAT 2.3): returns the number
// of pushed words; with WRITE, word k (in push order) goes to w[W - 1 - k]
// and the final state to st[0], st[1].
template <typename T, bool WRITE>
__device__ __forceinline__ uint32_t rans_stream(const T *data, const EncGeom &g, uint32_t b, uint32_t p, uint32_t n,
                                                const uint32_t *tab, uint16_t *st, uint32_t W) {
    uint32_t x = kRansL, k = 0;
    uint16_t *w = st + 2;
    for (int j = (int)n - 1; j >= 0; j--) {
        const uint32_t v = value_at(data, g, b, (uint32_t)j, p);
        uint32_t s = v;
        if (sizeof(T) == 2 && v >= 255u) {  // escape: the literal is pushed first
            if (WRITE) w[W - 1 - k] = (uint16_t)v;
            k++;
            s = 255u;
        }
        const uint32_t e = tab[s], f = e & 0xFFFFu, c = e >> 16;
        if ((uint64_t)x >= ((uint64_t)f << 20)) {
            if (WRITE) w[W - 1 - k] = (uint16_t)x;
            k++;
            x >>= 16;
        }
        x = ((x / f) << 12) + (x % f) + c;
    }
    if (WRITE) {
        st[0] = (uint16_t)x;
        st[1] = (uint16_t)(x >> 16);
    }
    return k;
}

// size[b][p] = mode << 16 | stream bytes (header included)
template <typename T>
__global__ __launch_bounds__(kWG) void k_enc_size(const T *data, EncGeom g, const uint32_t *enc,
                                                  const uint8_t *usable, const uint32_t *meta, uint32_t *size) {
    __shared__ uint32_t tab[256];
    const uint32_t b = blockIdx.y, p = blockIdx.x * kWG + threadIdx.x, n = block_scans(g, b);
    tab[threadIdx.x] = enc[256 * b + threadIdx.x];
    __syncthreads();
    if (p >= g.P) return;
    const uint64_t i = (uint64_t)b * g.P + p;
    const uint32_t raw = raw_bytes(n, sizeof(T) == 2);
    uint32_t out;
    if (meta[i] >> 31) {
        out = (R_CONST << 16) | 4u;
    } else if (!usable[b]) {
        out = (R_RAW << 16) | raw;
    } else {
        const uint32_t bytes = 2 + 2 * (2 + rans_stream<T, false>(data, g, b, p, n, tab, nullptr, 0));
        out = bytes < raw ? ((R_RANS << 16) | bytes) : ((R_RAW << 16) | raw);
    }
    size[i] = out;
}

// One 1024-thread workgroup per block: stream offsets within the block
// (soff), the grouped offsets written into the container, and the block size.
__global__ __launch_bounds__(1024) void k_enc_offsets(EncGeom g, const uint32_t *size, uint32_t *soff,
                                                      uint32_t *gbase, uint16_t *rel, uint64_t *bbytes) {
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t last_gb;
    const uint32_t b = blockIdx.x, tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint32_t running = 0;
    for (uint32_t base = 0; base < g.P; base += 1024) {
        const uint32_t p = base + tid;
        const uint32_t sz = p < g.P ? size[(uint64_t)b * g.P + p] & 0xFFFFu : 0u;
        uint32_t x = sz;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= (uint32_t)off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        uint32_t before = running, all = running;
#pragma unroll
        for (uint32_t w = 0; w < 16; w++) {
            before += w < wave ? wsum[w] : 0u;
            all += wsum[w];
        }
        const uint32_t start = before + x - sz;
        const uint32_t gb = __shfl(start, lane & ~31u);  // the group's first stream (groups of 32 never straddle a wave)
        if (p < g.P) {
            soff[(uint64_t)b * g.P + p] = start;
            const uint64_t gi = (uint64_t)b * g.G + p / 32;
            if ((p & 31u) == 0) gbase[gi] = start;
            rel[gi * 32 + (p & 31u)] = (uint16_t)(start - gb);
            if (p / 32 == g.G - 1) last_gb = gb;
        }
        __syncthreads();
        running = all;
    }
    // the unused entries of a final partial group point at the group's end
    const uint32_t used = g.P - 32 * (g.G - 1);
    if (tid >= used && tid < 32) rel[((uint64_t)b * g.G + g.G - 1) * 32 + tid] = (uint16_t)(running - last_gb);
    if (tid == 0) bbytes[b] = running;
}

// One 1024-thread workgroup: block bases (a prefix over the block sizes), the
// block directory, and the payload size.
__global__ __launch_bounds__(1024) void k_enc_dir(EncGeom g, const uint64_t *bbytes, uint8_t *dir, uint64_t *bbase,
                                                  uint64_t *total) {
    __shared__ uint64_t wsum[16];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    uint64_t running = 0;
    for (uint32_t base = 0; base < g.nb; base += 1024) {
        const uint32_t b = base + tid;
        const uint64_t sz = b < g.nb ? bbytes[b] : 0;
        uint64_t x = sz;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint64_t y = ((uint64_t)(uint32_t)__shfl_up((int)(uint32_t)(x >> 32), off) << 32) |
                               (uint32_t)__shfl_up((int)(uint32_t)x, off);
            if (lane >= (uint32_t)off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        uint64_t before = running, all = running;
#pragma unroll
        for (uint32_t w = 0; w < 16; w++) {
            before += w < wave ? wsum[w] : 0;
            all += wsum[w];
        }
        if (b < g.nb) {
            const uint64_t start = before + x - sz;
            bbase[b] = start;
            *reinterpret_cast<uint64_t *>(dir + 16ull * b) = start;
            *reinterpret_cast<uint32_t *>(dir + 16ull * b + 8) = block_scans(g, b);
            *reinterpret_cast<uint32_t *>(dir + 16ull * b + 12) = (uint32_t)sz;
        }
        __syncthreads();
        running = all;
    }
    if (tid == 0) *total = running;
}

// Header and payload of every stream (FORMAT 2.4), at payload + its block base
// + its offset in the block; all streams start 2-byte aligned.
template <typename T>
__global__ __launch_bounds__(kWG) void k_enc_write(const T *data, EncGeom g, const uint32_t *enc,
                                                   const uint32_t *meta, const uint32_t *size, const uint32_t *soff,
                                                   const uint64_t *bbase, uint8_t *payload) {
    __shared__ uint32_t tab[256];
    const uint32_t b = blockIdx.y, p = blockIdx.x * kWG + threadIdx.x, n = block_scans(g, b);
    tab[threadIdx.x] = enc[256 * b + threadIdx.x];
    __syncthreads();
    if (p >= g.P) return;
    const uint64_t i = (uint64_t)b * g.P + p;
    const uint32_t mode = size[i] >> 16, bytes = size[i] & 0xFFFFu;
    uint8_t *dst = payload + bbase[b] + soff[i];
    uint16_t *d16 = reinterpret_cast<uint16_t *>(dst);
    d16[0] = (uint16_t)mode;
    if (mode == R_CONST) {
        d16[1] = (uint16_t)(meta[i] & 0xFFFFu);
    } else if (mode == R_RAW) {
        if (sizeof(T) == 2) {
            for (uint32_t j = 0; j < n; j++) d16[1 + j] = (uint16_t)value_at(data, g, b, j, p);
        } else {
            for (uint32_t j = 0; j < n; j++) dst[2 + j] = (uint8_t)value_at(data, g, b, j, p);
            if (n & 1u) dst[2 + n] = 0;
        }
    } else {
        rans_stream<T, true>(data, g, b, p, n, tab, d16 + 1, (bytes - 6) / 2);
    }
}

// ------------------------------------------------------------------ paired tANS (FORMAT 3)
// Device copy of the pair models' encode tables.
struct PairDev {
    uint16_t n[kModels][256];
    uint16_t first[kModels][257];
    uint16_t states[kModels][kTansL];
    uint16_t cost[kModels][256];
    uint32_t a0[kModels], use[kModels];
};

__device__ __forceinline__ uint32_t wsym(uint32_t v, uint32_t a0, uint32_t use) {
    const uint32_t d = v - a0;
    return (v >= a0 && d < 15 && ((use >> d) & 1u)) ? d : 15u;
}

// smallest k with (x >> k) < 2 n (x < 2048, n >= 1)
__device__ __forceinline__ uint32_t tans_shift(uint32_t x, uint32_t n) {
    uint32_t k = 0;
    while ((x >> k) >= 2 * n) k++;
    return k;
}

// size[b][p] = mode << 16 | bytes; aux[b][p] = model | code bits << 8 (PAIRED)
template <typename T>
__global__ __launch_bounds__(kWG) void k_penc_size(const T *data, EncGeom g, const PairDev *pd, uint32_t *size,
                                                   uint32_t *aux) {
    __shared__ uint16_t cost[kModels * 256];
    __shared__ uint32_t a0s[kModels], uses[kModels];
    for (uint32_t i = threadIdx.x; i < kModels * 256; i += kWG) cost[i] = pd->cost[i / 256][i % 256];
    if (threadIdx.x < kModels) {
        a0s[threadIdx.x] = pd->a0[threadIdx.x];
        uses[threadIdx.x] = pd->use[threadIdx.x];
    }
    __syncthreads();
    const uint32_t b = blockIdx.y, p = blockIdx.x * kWG + threadIdx.x;
    if (p >= g.P) return;
    const uint64_t i = (uint64_t)b * g.P + p;
    const bool wide = sizeof(T) == 2;
    const uint32_t lit = wide ? 16 : 8;
    const uint32_t v0 = value_at(data, g, b, 0, p);
    uint32_t nnz = 0;
    bool eq = true;
    for (uint32_t j = 0; j < kBlock; j++) {
        const uint32_t v = value_at(data, g, b, j, p);
        eq &= v == v0;
        nnz += v != 0;
    }
    if (nnz == 0) {
        size[i] = (P_EMPTY << 16) | 2u;
        return;
    }
    if (eq) {
        size[i] = (P_CONST << 16) | 4u;
        return;
    }
    const uint32_t sparse = 4 + 2 * nnz + (wide ? 2 * nnz : nnz + (nnz & 1u));
    // static cost of every model (1/256 bits), lowest model on ties
    uint32_t c[kModels];
#pragma unroll
    for (uint32_t m = 0; m < kModels; m++) c[m] = 0;
    for (uint32_t t = 0; t < 256; t++) {
        const uint32_t x0 = value_at(data, g, b, 2 * t, p), x1 = value_at(data, g, b, 2 * t + 1, p);
#pragma unroll
        for (uint32_t m = 0; m < kModels; m++) {
            const uint32_t a = wsym(x0, a0s[m], uses[m]), e = wsym(x1, a0s[m], uses[m]);
            c[m] += cost[m * 256 + a * 16 + e] + (a == 15 ? 256 * lit : 0) + (e == 15 ? 256 * lit : 0);
        }
    }
    uint32_t best = 0, best_c = c[0];
#pragma unroll
    for (uint32_t m = 1; m < kModels; m++)
        if (c[m] < best_c) {
            best_c = c[m];
            best = m;
        }
    // exact code bits of the chosen model: the coder in reverse
    const uint32_t a0 = a0s[best], use = uses[best];
    uint32_t x = kTansL, bits = 10;
    for (int t = 255; t >= 0; t--) {
        const uint32_t x0 = value_at(data, g, b, 2 * t, p), x1 = value_at(data, g, b, 2 * t + 1, p);
        const uint32_t a = wsym(x0, a0, use), e = wsym(x1, a0, use), s = a * 16 + e;
        const uint32_t ns = pd->n[best][s], k = tans_shift(x, ns);
        bits += k + (a == 15 ? lit : 0) + (e == 15 ? lit : 0);
        x = kTansL + pd->states[best][pd->first[best][s] + ((x >> k) - ns)];
    }
    const uint32_t paired = 2 + (bits + 15) / 16 * 2;
    uint32_t mode = P_SPARSE, bytes = sparse;
    if (sparse >= paired + 2) {
        mode = P_PAIRED;
        bytes = paired;
    }
    const uint32_t raw = raw_bytes(kBlock, wide);
    if (raw < bytes) {
        mode = P_RAW;
        bytes = raw;
    }
    size[i] = (mode << 16) | bytes;
    aux[i] = best | (bits << 8);
}

// Code section writer that runs backwards: bits are prepended below the
// buffer, and each completed 16-bit word at its top is stored.
struct BackBits {
    uint16_t *words;  // the code section
    uint64_t acc;     // buffered bits, lowest = the lowest buffered position
    uint32_t nb, top; // buffered bit count; position just above the buffer
    __device__ __forceinline__ void put(uint32_t v, uint32_t k) {
        acc = (acc << k) | v;
        nb += k;
        while (nb >= 32) flush16();
    }
    __device__ __forceinline__ void flush16() {
        words[(top - 16) / 16] = (uint16_t)(acc >> (nb - 16));
        top -= 16;
        nb -= 16;
        acc &= (1ull << nb) - 1;
    }
};

template <typename T>
__global__ __launch_bounds__(kWG) void k_penc_write(const T *data, EncGeom g, const PairDev *pd, const uint32_t *size,
                                                    const uint32_t *aux, const uint32_t *soff, const uint64_t *bbase,
                                                    uint8_t *payload) {
    const uint32_t b = blockIdx.y, p = blockIdx.x * kWG + threadIdx.x;
    if (p >= g.P) return;
    const uint64_t i = (uint64_t)b * g.P + p;
    const bool wide = sizeof(T) == 2;
    const uint32_t mode = size[i] >> 16;
    uint8_t *dst = payload + bbase[b] + soff[i];
    uint16_t *d16 = reinterpret_cast<uint16_t *>(dst);
    if (mode == P_EMPTY) {
        d16[0] = P_EMPTY;
    } else if (mode == P_CONST) {
        d16[0] = P_CONST;
        d16[1] = (uint16_t)value_at(data, g, b, 0, p);
    } else if (mode == P_RAW) {
        d16[0] = P_RAW;
        if (wide)
            for (uint32_t j = 0; j < kBlock; j++) d16[1 + j] = (uint16_t)value_at(data, g, b, j, p);
        else
            for (uint32_t j = 0; j < kBlock; j++) dst[2 + j] = (uint8_t)value_at(data, g, b, j, p);
    } else if (mode == P_SPARSE) {
        d16[0] = P_SPARSE;
        uint32_t nnz = 0;
        for (uint32_t j = 0; j < kBlock; j++)
            if (value_at(data, g, b, j, p)) d16[2 + nnz++] = (uint16_t)j;
        d16[1] = (uint16_t)nnz;
        uint8_t *vals = dst + 4 + 2 * nnz;
        uint32_t k = 0;
        for (uint32_t j = 0; j < kBlock; j++) {
            const uint32_t v = value_at(data, g, b, j, p);
            if (!v) continue;
            if (wide)
                reinterpret_cast<uint16_t *>(vals)[k++] = (uint16_t)v;
            else
                vals[k++] = (uint8_t)v;
        }
        if (!wide && (nnz & 1u)) vals[nnz] = 0;
    } else {
        const uint32_t m = aux[i] & 0xFFu, bits = aux[i] >> 8, lit = wide ? 16 : 8;
        d16[0] = (uint16_t)(P_PAIRED | (m << 3));
        const uint32_t a0 = pd->a0[m], use = pd->use[m];
        const uint32_t padded = (bits + 15) / 16 * 16;
        BackBits w{d16 + 1, 0, padded - bits, padded};  // the zero padding is buffered first
        uint32_t x = kTansL;
        for (int t = 255; t >= 0; t--) {
            const uint32_t x0 = value_at(data, g, b, 2 * t, p), x1 = value_at(data, g, b, 2 * t + 1, p);
            const uint32_t a = wsym(x0, a0, use), e = wsym(x1, a0, use), s = a * 16 + e;
            const uint32_t ns = pd->n[m][s], k = tans_shift(x, ns);
            // pair t reads: state bits, then the first literal, then the second
            if (e == 15) w.put(x1, lit);
            if (a == 15) w.put(x0, lit);
            w.put(x & ((1u << k) - 1u), k);
            x = kTansL + pd->states[m][pd->first[m][s] + ((x >> k) - ns)];
        }
        w.put(x - kTansL, 10);
        while (w.nb) w.flush16();
    }
}

template <typename T>
hipError_t encode_rans(const T *data, const EncGeom &g, const Sections &s0, uint8_t *blob, uint32_t *hist,
                       uint32_t *enc, uint8_t *usable, uint32_t *meta, uint32_t *size, uint32_t *soff,
                       uint64_t *bbytes, uint64_t *bbase, uint64_t *total, hipStream_t st) {
    const dim3 grid((g.P + kWG - 1) / kWG, g.nb);
    hipLaunchKernelGGL(k_enc_scan<T>, grid, dim3(kWG), 0, st, data, g, hist, meta);
    hipLaunchKernelGGL(k_enc_table, dim3(g.nb), dim3(64), 0, st, hist,
                       reinterpret_cast<uint16_t *>(blob + s0.table), enc, usable);
    hipLaunchKernelGGL(k_enc_size<T>, grid, dim3(kWG), 0, st, data, g, enc, usable, meta, size);
    hipLaunchKernelGGL(k_enc_offsets, dim3(g.nb), dim3(1024), 0, st, g, size, soff,
                       reinterpret_cast<uint32_t *>(blob + s0.gbase), reinterpret_cast<uint16_t *>(blob + s0.rel),
                       bbytes);
    hipLaunchKernelGGL(k_enc_dir, dim3(1), dim3(1024), 0, st, g, bbytes, blob + s0.dir, bbase, total);
    return hipGetLastError();
}

template <typename T>
hipError_t write_rans(const T *data, const EncGeom &g, const Sections &s0, uint8_t *blob, const uint32_t *enc,
                      const uint32_t *meta, const uint32_t *size, const uint32_t *soff, const uint64_t *bbase,
                      hipStream_t st) {
    const dim3 grid((g.P + kWG - 1) / kWG, g.nb);
    hipLaunchKernelGGL(k_enc_write<T>, grid, dim3(kWG), 0, st, data, g, enc, meta, size, soff, bbase,
                       blob + s0.payload);
    return hipGetLastError();
}

template <typename T>
hipError_t encode_paired(const T *data, const EncGeom &g, const Sections &s0, uint8_t *blob, const PairDev *pd,
                         uint32_t *size, uint32_t *aux, uint32_t *soff, uint64_t *bbytes, uint64_t *bbase,
                         uint64_t *total, hipStream_t st) {
    const dim3 grid((g.P + kWG - 1) / kWG, g.nb);
    hipLaunchKernelGGL(k_penc_size<T>, grid, dim3(kWG), 0, st, data, g, pd, size, aux);
    hipLaunchKernelGGL(k_enc_offsets, dim3(g.nb), dim3(1024), 0, st, g, size, soff,
                       reinterpret_cast<uint32_t *>(blob + s0.gbase), reinterpret_cast<uint16_t *>(blob + s0.rel),
                       bbytes);
    hipLaunchKernelGGL(k_enc_dir, dim3(1), dim3(1024), 0, st, g, bbytes, blob + s0.dir, bbase, total);
    return hipGetLastError();
}

template <typename T>
hipError_t write_paired(const T *data, const EncGeom &g, const Sections &s0, uint8_t *blob, const PairDev *pd,
                        const uint32_t *size, const uint32_t *aux, const uint32_t *soff, const uint64_t *bbase,
                        hipStream_t st) {
    const dim3 grid((g.P + kWG - 1) / kWG, g.nb);
    hipLaunchKernelGGL(k_penc_write<T>, grid, dim3(kWG), 0, st, data, g, pd, size, aux, soff, bbase,
                       blob + s0.payload);
    return hipGetLastError();
}

// Host copy of the pair models' encode tables in the device layout.
const PairDev &pair_dev() {
    static const PairDev t = [] {
        PairDev d{};
        const PairModels &pm = pair_models();
        const PairEncodeTables &pt = pair_encode_tables();
        for (uint32_t m = 0; m < kModels; m++) {
            for (uint32_t i = 0; i < 256; i++) {
                d.n[m][i] = pm.n[m][i];
                d.cost[m][i] = (uint16_t)pt.cost[m][i];  // at most 256 * 10
            }
            for (uint32_t i = 0; i < 257; i++) d.first[m][i] = pt.first[m][i];
            for (uint32_t X = 0; X < kTansL; X++) d.states[m][X] = pt.states[m][X];
            d.a0[m] = pm.a0[m];
            d.use[m] = pm.in_use[m];
        }
        return d;
    }();
    return t;
}

// Device workspace of one encode, carved from a single allocation.
struct Workspace {
    void *base = nullptr;
    uint32_t *hist = nullptr, *enc = nullptr, *meta = nullptr, *size = nullptr, *soff = nullptr, *bad = nullptr;
    uint8_t *usable = nullptr;
    uint64_t *bbytes = nullptr, *bbase = nullptr, *total = nullptr;
    unsigned long long *lo = nullptr, *hi = nullptr;
    double *calib = nullptr;
    uint16_t *codes = nullptr;
    PairDev *pair = nullptr;
    ~Workspace() {
        if (base) (void)hipFree(base);
    }
    hipError_t alloc(const Geometry &g) {
        const uint64_t nb = g.n_blocks(), P = g.P();
        uint64_t off = 0;
        auto take = [&](uint64_t bytes) {
            const uint64_t o = off;
            off += (bytes + 255) / 256 * 256;
            return o;
        };
        const uint64_t o_hist = take(4 * 256 * nb), o_enc = take(4 * 256 * nb), o_usable = take(nb);
        const uint64_t o_meta = take(4 * nb * P), o_size = take(4 * nb * P), o_soff = take(4 * nb * P);
        const uint64_t o_bbytes = take(8 * nb), o_bbase = take(8 * nb), o_total = take(8), o_bad = take(4);
        const uint64_t o_lo = take(8 * nb), o_hi = take(8 * nb), o_calib = take(16 * nb);
        const uint64_t o_codes = g.scaled ? take(2 * g.S() * P) : 0;
        const uint64_t o_pair = g.layout == 1 ? take(sizeof(PairDev)) : 0;
        hipError_t e = hipMalloc(&base, off);
        if (e != hipSuccess) {
            base = nullptr;
            return e;
        }
        uint8_t *b8 = static_cast<uint8_t *>(base);
        hist = reinterpret_cast<uint32_t *>(b8 + o_hist);
        enc = reinterpret_cast<uint32_t *>(b8 + o_enc);
        usable = b8 + o_usable;
        meta = reinterpret_cast<uint32_t *>(b8 + o_meta);
        size = reinterpret_cast<uint32_t *>(b8 + o_size);
        soff = reinterpret_cast<uint32_t *>(b8 + o_soff);
        bbytes = reinterpret_cast<uint64_t *>(b8 + o_bbytes);
        bbase = reinterpret_cast<uint64_t *>(b8 + o_bbase);
        total = reinterpret_cast<uint64_t *>(b8 + o_total);
        bad = reinterpret_cast<uint32_t *>(b8 + o_bad);
        lo = reinterpret_cast<unsigned long long *>(b8 + o_lo);
        hi = reinterpret_cast<unsigned long long *>(b8 + o_hi);
        calib = reinterpret_cast<double *>(b8 + o_calib);
        codes = g.scaled ? reinterpret_cast<uint16_t *>(b8 + o_codes) : nullptr;
        pair = g.layout == 1 ? reinterpret_cast<PairDev *>(b8 + o_pair) : nullptr;
        return hipSuccess;
    }
};

qsc_status hip_status(hipError_t e) { return e == hipErrorOutOfMemory ? QSC_ERR_OOM : QSC_ERR_HIP; }

}  // namespace

extern "C" {

qsc_status qsc_encode_device_bound(const qsc_geometry *geom, uint64_t *nbytes) {
    if (!geom || !nbytes) return QSC_ERR_INVALID_ARG;
    Geometry g;
    g.scan_rows = geom->scan_rows;
    g.scan_cols = geom->scan_cols;
    g.det_rows = geom->det_rows;
    g.det_cols = geom->det_cols;
    g.dtype = geom->dtype;
    g.layout = geom->layout;
    g.scaled = geom->scaled;
    if (!check_geometry(g).empty()) return QSC_ERR_INVALID_ARG;
    // every stream RAW: its raw bytes are the most any mode takes
    uint64_t pay = 0;
    for (uint32_t b = 0; b < g.n_blocks(); b++) {
        const uint64_t n = std::min<uint64_t>(kBlock, g.S() - uint64_t(b) * kBlock);
        pay += uint64_t(g.P()) * (g.dtype == 2 ? 2 + 2 * n : 2 + n + (n & 1));
    }
    *nbytes = layout_sections(g, pay).total;
    return QSC_OK;
}

qsc_status qsc_encode_device(const qsc_geometry *geom, const void *d_data, void *d_blob, uint64_t capacity,
                             uint64_t *nbytes, void *hip_stream) {
    if (!geom || !d_data || !d_blob || !nbytes) return QSC_ERR_INVALID_ARG;
    Geometry g;
    g.scan_rows = geom->scan_rows;
    g.scan_cols = geom->scan_cols;
    g.det_rows = geom->det_rows;
    g.det_cols = geom->det_cols;
    g.dtype = geom->dtype;
    g.layout = geom->layout;
    g.scaled = geom->scaled;
    if (!check_geometry(g).empty()) return QSC_ERR_INVALID_ARG;
    const Sections s0 = layout_sections(g, 0);
    if (capacity < s0.payload) return QSC_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    uint8_t *blob = static_cast<uint8_t *>(d_blob);
    const EncGeom eg{g.S(), g.P(), g.G(), g.n_blocks()};
    Workspace ws;
    hipError_t e = ws.alloc(g);
    if (e != hipSuccess) return hip_status(e);
    // header, directory, tables and offsets sections start zeroed (gaps stay 0)
    if ((e = hipMemsetAsync(blob, 0, s0.payload, st)) != hipSuccess) return hip_status(e);
    if ((e = hipMemsetAsync(ws.hist, 0, 4 * 256ull * eg.nb, st)) != hipSuccess) return hip_status(e);
    const void *src = d_data;
    if (g.scaled) {
        if ((e = hipMemsetAsync(ws.lo, 0xFF, 8ull * eg.nb, st)) != hipSuccess) return hip_status(e);
        if ((e = hipMemsetAsync(ws.hi, 0, 8ull * eg.nb, st)) != hipSuccess) return hip_status(e);
        if ((e = hipMemsetAsync(ws.bad, 0, 4, st)) != hipSuccess) return hip_status(e);
        const float *x = static_cast<const float *>(d_data);
        const uint32_t chunk = 1u << 16;
        const uint64_t per_block = uint64_t(kBlock) * eg.P;
        hipLaunchKernelGGL(k_cal_minmax, dim3((uint32_t)((per_block + chunk - 1) / chunk), eg.nb), dim3(kWG), 0, st, x,
                           eg, chunk, ws.lo, ws.hi, ws.bad);
        hipLaunchKernelGGL(k_cal_params, dim3((eg.nb + 255) / 256), dim3(256), 0, st, x, eg, ws.lo, ws.hi, ws.calib);
        const uint64_t n = eg.S * eg.P;
        hipLaunchKernelGGL(k_cal_codes, dim3((uint32_t)std::min<uint64_t>(65536, (n + kWG - 1) / kWG)), dim3(kWG), 0,
                           st, x, eg, ws.calib, ws.codes);
        src = ws.codes;
    }
    if (g.layout == 1) {
        // the 32 pair models' counts are the table section
        const PairDev &pd = pair_dev();
        if ((e = hipMemcpyAsync(ws.pair, &pd, sizeof(PairDev), hipMemcpyHostToDevice, st)) != hipSuccess)
            return hip_status(e);
        if ((e = hipMemcpyAsync(blob + s0.table, pair_models().n, sizeof(pair_models().n), hipMemcpyHostToDevice,
                                st)) != hipSuccess)
            return hip_status(e);
        if (g.dtype == 2)
            e = encode_paired(static_cast<const uint16_t *>(src), eg, s0, blob, ws.pair, ws.size, ws.meta, ws.soff,
                              ws.bbytes, ws.bbase, ws.total, st);
        else
            e = encode_paired(static_cast<const uint8_t *>(src), eg, s0, blob, ws.pair, ws.size, ws.meta, ws.soff,
                              ws.bbytes, ws.bbase, ws.total, st);
    } else if (g.dtype == 2 || g.scaled) {
        e = encode_rans(static_cast<const uint16_t *>(src), eg, s0, blob, ws.hist, ws.enc, ws.usable, ws.meta,
                        ws.size, ws.soff, ws.bbytes, ws.bbase, ws.total, st);
    } else {
        e = encode_rans(static_cast<const uint8_t *>(src), eg, s0, blob, ws.hist, ws.enc, ws.usable, ws.meta,
                        ws.size, ws.soff, ws.bbytes, ws.bbase, ws.total, st);
    }
    if (e != hipSuccess) return hip_status(e);
    uint64_t pay = 0;
    uint32_t bad = 0;
    if ((e = hipMemcpyAsync(&pay, ws.total, 8, hipMemcpyDeviceToHost, st)) != hipSuccess) return hip_status(e);
    if (g.scaled && (e = hipMemcpyAsync(&bad, ws.bad, 4, hipMemcpyDeviceToHost, st)) != hipSuccess)
        return hip_status(e);
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_status(e);
    if (bad) return QSC_ERR_INVALID_ARG;  // NaN or infinite input
    const Sections s = layout_sections(g, pay);
    *nbytes = s.total;
    if (s.total > capacity) return QSC_ERR_INVALID_ARG;
    if (g.layout == 1) {
        if (g.dtype == 2)
            e = write_paired(static_cast<const uint16_t *>(src), eg, s0, blob, ws.pair, ws.size, ws.meta, ws.soff,
                             ws.bbase, st);
        else
            e = write_paired(static_cast<const uint8_t *>(src), eg, s0, blob, ws.pair, ws.size, ws.meta, ws.soff,
                             ws.bbase, st);
    } else if (g.dtype == 2 || g.scaled) {
        e = write_rans(static_cast<const uint16_t *>(src), eg, s0, blob, ws.enc, ws.meta, ws.size, ws.soff, ws.bbase,
                       st);
    } else {
        e = write_rans(static_cast<const uint8_t *>(src), eg, s0, blob, ws.enc, ws.meta, ws.size, ws.soff, ws.bbase,
                       st);
    }
    if (e != hipSuccess) return hip_status(e);
    if (g.scaled) {
        const uint64_t end = s.payload + s.payload_bytes;
        if ((e = hipMemsetAsync(blob + end, 0, s.calib - end, st)) != hipSuccess) return hip_status(e);
        if ((e = hipMemcpyAsync(blob + s.calib, ws.calib, 16ull * eg.nb, hipMemcpyDeviceToDevice, st)) != hipSuccess)
            return hip_status(e);
    }
    uint8_t hdr[kHeaderBytes];
    write_header(g, s, hdr);
    if ((e = hipMemcpyAsync(blob, hdr, kHeaderBytes, hipMemcpyHostToDevice, st)) != hipSuccess) return hip_status(e);
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_status(e);
    return QSC_OK;
}

}  // extern "C"
