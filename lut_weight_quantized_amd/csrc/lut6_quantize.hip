// LUT-6 table fitting on gfx950: one 64-entry FP16 table per 16 output
// channels by one-dimensional k-means, then the packed indices (page
// "Clef-Flash-ANE-LUT6", section "LUT-6 text weights").  The page fixes the
// round count, 40, and the starting centres: 32 at quantiles of the group's
// values, 32 at even steps from its smallest to its largest value.
//
// Everything finer is a reading:
//   - FP16 weights, all finite; a group is rows 16g .. 16g + 15, n = 16 K
//     values;
//   - starting centres: the values of rank floor((2i + 1) n / 64) in the
//     sorted group (i = 0..31) and min + (max - min) * j / 31 (j = 0..31), in
//     FP64, sorted;
//   - a round: boundaries b_i = (c_i + c_{i+1}) / 2; a value v <= b_i and
//     > b_{i-1} belongs to cluster i; each centre becomes its cluster's mean,
//     an empty cluster's centre stays; the centres are sorted again;
//   - sums are exact: FP16 values are integer multiples of 2^-24, so a sum
//     is a 64-bit count of 2^-24 units and a mean is (double)sum / count *
//     2^-24;
//   - the table is the last centres rounded to FP16 (nearest, ties to even),
//     sorted (-0 before +0); each weight's index is its nearest entry by the
//     same boundary rule on the FP16 entries.
//
// One workgroup per group (a grid of at most Q_MAX_WG workgroups walks the
// groups).  In one dimension k-means needs no per-value work per round: with
// the group's values as a histogram over the 65,536 FP16 bit patterns, kept
// in order-preserving key order, and inclusive prefix counts P and prefix
// sums S over it, the values <= b are the keys up to the largest key whose
// value is <= b.  That key is computed from b alone (FP16 values are whole
// numbers of 2^-24 units: b rounded down onto them), so a round costs one
// load of P and one of S per boundary, in one wave.  The histogram is counted in LDS, 32,768 keys per pass (one
// pass covers every FP16 value in [-0.5, 0.5]); P and S go to a library
// workspace slot of 768 KB per workgroup, written and read back by that
// workgroup alone, so plain loads see them (a CU's waves share its vector
// cache).  Agent-scope atomics and loads on that scratch, the first design,
// went past the per-XCD L2 on every access and took about 1.2 ms per group.
//
// Compiled for gfx950 only.  No FP contraction in this file: every FP64 step
// rounds once, as written.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "lut6.h"

#pragma clang fp contract(off)

namespace {

constexpr int Q_THREADS = 256;
constexpr int Q_KEYS = 65536;
constexpr int Q_ROUNDS = 40;
constexpr int Q_ENTRIES = 64;
constexpr int Q_MAX_WG = 256;
constexpr int Q_CHUNK = 32768;      // histogram keys per LDS pass
constexpr int Q_WAVE_KEYS = Q_CHUNK / (Q_THREADS / 64);   // keys per wave in the scan
// one workspace slot: P (u32) then S (i64) over the 65,536 keys
constexpr size_t Q_SLOT_BYTES = (size_t)Q_KEYS * 4 + (size_t)Q_KEYS * 8;

// Order-preserving key of an FP16 bit pattern: negative values reversed
// below 0x8000, positive values above (-0 just below +0).
__device__ __forceinline__ uint32_t q_key(uint32_t h)
{
    return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ uint32_t q_bits(uint32_t key)
{
    return (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
}
// A finite FP16 value in units of 2^-24 (|result| < 2^41).
__device__ __forceinline__ int64_t q_units(uint32_t h)
{
    const int e = (h >> 10) & 31, m = h & 1023;
    const int64_t u = e == 0 ? (int64_t)m : ((int64_t)(1024 + m) << (e - 1));
    return (h & 0x8000u) ? -u : u;
}
// The value of a finite FP16 pattern as a double (-0 stays -0).
__device__ __forceinline__ double q_value(uint32_t h)
{
    const int e = (h >> 10) & 31, m = h & 1023;
    const double mag = e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
    return (h & 0x8000u) ? -mag : mag;
}
// Pattern of the FP16 magnitude nearest to u (a whole number of 2^-24 units,
// 0 <= u <= 65,504 * 2^24) from below (up = false) or from above (up = true).
// Below 1,024 units (the subnormals) every whole number is a value; above,
// the binade of u has 1,024 values spaced 2^(ex - 11) units apart, ex being
// frexp's exponent of u, and rounding up from its last value reaches the
// first value of the next binade.
__device__ __forceinline__ uint32_t q_mag_bits(double u, bool up)
{
    if (u < 1024.0) return (uint32_t)u;
    int ex;
    (void)frexp(u, &ex);
    const double mq = up ? ceil(ldexp(u, 11 - ex)) : floor(ldexp(u, 11 - ex));
    return mq == 2048.0 ? (uint32_t)(ex - 9) << 10 : ((uint32_t)(ex - 10) << 10) | ((uint32_t)mq - 1024u);
}
// Largest key in [lo_key, hi_key] whose value is <= b, or lo_key - 1 if none
// (every key in the range is a finite value, increasing with the key).  The
// FP16 values are whole numbers of 2^-24 units, so the largest one <= b is
// b's units rounded down onto that grid: the magnitude truncated for b >= 0
// (-0 included: +0 is the larger key of value 0), rounded up for b < 0.
__device__ __forceinline__ int q_floor_key(double b, int lo_key, int hi_key)
{
    const double F16_MAX_UNITS = 65504.0 * 16777216.0;
    const double t = ldexp(b, 24);                      // exact
    uint32_t h;
    if (t >= 0.0) {
        h = q_mag_bits(fmin(floor(t), F16_MAX_UNITS), false);
    } else {
        const double c = ceil(-t);
        if (c > F16_MAX_UNITS) return lo_key - 1;
        h = q_mag_bits(c, true) | 0x8000u;
    }
    const int k = (int)q_key(h);
    return k > hi_key ? hi_key : (k < lo_key ? lo_key - 1 : k);
}
// FP16 bit pattern nearest to c, ties to the even pattern; c lies within
// the values of keys [lo_key, hi_key] (a centre is a mean of the group's
// values, so it does).
__device__ __forceinline__ uint32_t q_round_f16(double c, int lo_key, int hi_key)
{
    if (c == 0.0) return __builtin_signbit(c) ? 0x8000u : 0u;
    const int k1 = q_floor_key(c, lo_key, hi_key);
    const uint32_t h1 = q_bits((uint32_t)k1);
    const double v1 = q_value(h1);
    if (v1 == c || k1 >= hi_key) return h1;
    const uint32_t h2 = q_bits((uint32_t)(k1 + 1));
    const double d1 = c - v1, d2 = q_value(h2) - c;   // exact: v1 < c < v2, neighbours
    if (d1 < d2) return h1;
    if (d2 < d1) return h2;
    return (h1 & 1u) ? h2 : h1;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// within each row of 16 lanes (lanes shifted in from outside the row add
// 0), then the last lane of row 0 into row 1 and of row 2 into row 3, then
// lane 31 into rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t q_dpp(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int64_t q_dpp64(int64_t x)
{
    const uint32_t lo = q_dpp<CTRL, ROWS>((uint32_t)x), hi = q_dpp<CTRL, ROWS>((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t q_wave_scan(uint32_t x)
{
    x += q_dpp<0x111, 0xf>(x);      // row_shr:1
    x += q_dpp<0x112, 0xf>(x);      // row_shr:2
    x += q_dpp<0x114, 0xf>(x);      // row_shr:4
    x += q_dpp<0x118, 0xf>(x);      // row_shr:8
    x += q_dpp<0x142, 0xa>(x);      // row_bcast:15 into rows 1 and 3
    x += q_dpp<0x143, 0xc>(x);      // row_bcast:31 into rows 2 and 3
    return x;
}
__device__ __forceinline__ int64_t q_wave_scan64(int64_t x)
{
    x += q_dpp64<0x111, 0xf>(x);
    x += q_dpp64<0x112, 0xf>(x);
    x += q_dpp64<0x114, 0xf>(x);
    x += q_dpp64<0x118, 0xf>(x);
    x += q_dpp64<0x142, 0xa>(x);
    x += q_dpp64<0x143, 0xc>(x);
    return x;
}
// A wave's values moved one lane up (lane i gets lane i - 1's, lane 0 gets 0)
// or down (lane i gets lane i + 1's, lane 63 gets 0): whole-wave DPP shifts.
__device__ __forceinline__ uint64_t q_up1(uint64_t x)
{
    return ((uint64_t)q_dpp<0x138, 0xf>((uint32_t)(x >> 32)) << 32) | q_dpp<0x138, 0xf>((uint32_t)x);
}
__device__ __forceinline__ uint64_t q_down1(uint64_t x)
{
    return ((uint64_t)q_dpp<0x130, 0xf>((uint32_t)(x >> 32)) << 32) | q_dpp<0x130, 0xf>((uint32_t)x);
}
__device__ __forceinline__ uint32_t q_lane63(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ int64_t q_lane63_64(int64_t x)
{
    const uint32_t lo = q_lane63((uint32_t)x), hi = q_lane63((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Orders one wave's LDS accesses before and after it (the lanes of a wave
// run in step; this keeps the compiler from moving accesses across).
__device__ __forceinline__ void q_wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sort 64 doubles in LDS (ascending; of equal values -0 first, then by
// position): each of 64 threads computes its element's rank.
__device__ __forceinline__ void q_rank_sort(const double* src, double* dst, int tid)
{
    if (tid < Q_ENTRIES) {
        const double v = src[tid];
        const bool vneg = __builtin_signbit(v);
        int rank = 0;
#pragma unroll
        for (int j = 0; j < Q_ENTRIES; ++j) {
            const double u = src[j];
            const bool before = u < v || (u == v && ((__builtin_signbit(u) && !vneg) ||
                                                     (__builtin_signbit(u) == vneg && j < tid)));
            rank += before ? 1 : 0;
        }
        dst[rank] = v;
    }
}

__global__ void __launch_bounds__(Q_THREADS)
lut6_quantize_kernel(const uint16_t* __restrict__ w, uint8_t* __restrict__ packed,
                     uint16_t* __restrict__ tables, int N, int K, uint8_t* __restrict__ work)
{
    // 128 KB: a histogram chunk (u32) during the scan, then the key -> index
    // map of the final table (u8)
    __shared__ __attribute__((aligned(16))) uint32_t lds_buf[Q_CHUNK];
    uint32_t* const hist = lds_buf;
    uint8_t* const map = (uint8_t*)lds_buf;
    __shared__ double cen[Q_ENTRIES], tmp[Q_ENTRIES], bnd[Q_ENTRIES];
    __shared__ uint32_t cle[Q_ENTRIES];
    __shared__ int fkey[Q_ENTRIES];
    __shared__ int64_t sle[Q_ENTRIES];
    __shared__ uint32_t part_c[Q_THREADS];
    __shared__ int64_t part_s[Q_THREADS];
    __shared__ int key_lo, key_hi;

    const int tid = threadIdx.x;
    uint32_t* const P = (uint32_t*)(work + (size_t)blockIdx.x * Q_SLOT_BYTES);
    int64_t* const S = (int64_t*)(work + (size_t)blockIdx.x * Q_SLOT_BYTES + (size_t)Q_KEYS * 4);
    const int groups = N / 16;
    const int64_t n = 16 * (int64_t)K;
    const int row_bytes = K / 4 * 3;

    for (int g = blockIdx.x; g < groups; g += gridDim.x) {
        const uint16_t* const wg = w + (size_t)g * 16 * K;

        // 1. the smallest and largest key present
        if (tid == 0) { key_lo = Q_KEYS; key_hi = -1; }
        __syncthreads();
        const uint4* const wg16 = (const uint4*)wg;       // 8 values per load
        const int n8 = (int)(n / 8);
        {
            int mn = Q_KEYS, mx = -1;
            for (int i0 = tid; i0 < n8; i0 += 4 * Q_THREADS) {
                uint4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = i0 + u * Q_THREADS < n8 ? wg16[i0 + u * Q_THREADS] : wg16[i0];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int key = (int)q_key((wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                        mn = min(mn, key);
                        mx = max(mx, key);
                    }
                }
            }
            atomicMin(&key_lo, mn);
            atomicMax(&key_hi, mx);
        }
        __syncthreads();
        const int klo = key_lo, khi = key_hi;

        // 2. histogram (in LDS, Q_CHUNK keys at a time) and the inclusive
        //    prefix counts P and exact prefix sums S over keys [klo, khi]
        uint32_t carry_c = 0;
        int64_t carry_s = 0;
        for (int c0 = klo; c0 <= khi; c0 += Q_CHUNK) {
            for (int i = tid; i < Q_CHUNK / 4; i += Q_THREADS) ((uint4*)hist)[i] = make_uint4(0, 0, 0, 0);
            __syncthreads();
            for (int i0 = tid; i0 < n8; i0 += 4 * Q_THREADS) {
                uint4 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = i0 + u * Q_THREADS < n8 ? wg16[i0 + u * Q_THREADS] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (i0 + u * Q_THREADS >= n8) continue;
                    const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int rel = (int)q_key((wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) - c0;
                        if (rel >= 0 && rel < Q_CHUNK) atomicAdd(&hist[rel], 1u);
                    }
                }
            }
            __syncthreads();
            // wave w takes keys [w Q_WAVE_KEYS, (w + 1) Q_WAVE_KEYS) of the
            // chunk in blocks of 64, lane l key l of a block: first each
            // wave's totals, then the inclusive prefixes block by block (an
            // in-wave scan plus the running carry), stored coalesced.  The
            // sums are integers, so any order gives the same P and S.
            const int wave = tid >> 6, lane = tid & 63;
            uint32_t wc = 0;
            int64_t wsum = 0;
            for (int b = 0; b < Q_WAVE_KEYS; b += 64) {
                const int rel = wave * Q_WAVE_KEYS + b + lane;
                const uint32_t c = hist[rel];
                wc += c;
                wsum += (int64_t)c * q_units(q_bits((uint32_t)min(c0 + rel, Q_KEYS - 1)));
            }
            wc = q_wave_scan(wc);
            wsum = q_wave_scan64(wsum);
            if (lane == 63) {
                part_c[wave] = wc;
                part_s[wave] = wsum;
            }
            __syncthreads();
            uint32_t run_c = carry_c;
            int64_t run_s = carry_s;
            for (int v = 0; v < wave; ++v) {
                run_c += part_c[v];
                run_s += part_s[v];
            }
            for (int b = 0; b < Q_WAVE_KEYS && c0 + wave * Q_WAVE_KEYS + b <= khi; b += 64) {
                const int rel = wave * Q_WAVE_KEYS + b + lane;
                const int key = c0 + rel;
                const uint32_t c = hist[rel];
                const uint32_t x = q_wave_scan(c);
                const int64_t y = q_wave_scan64((int64_t)c * q_units(q_bits((uint32_t)min(key, Q_KEYS - 1))));
                if (key <= khi) {
                    P[key] = run_c + x;
                    S[key] = run_s + y;
                }
                run_c += q_lane63(x);
                run_s += q_lane63_64(y);
            }
            for (int v = 0; v < Q_THREADS / 64; ++v) {
                carry_c += part_c[v];
                carry_s += part_s[v];
            }
            __syncthreads();
        }

        // 3. starting centres: 32 quantiles and 32 evenly spread values
        if (tid < 32) {
            // smallest key with P > rank
            const int64_t rank = ((int64_t)(2 * tid + 1) * n) / 64;
            int lo = klo, hi = khi;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((int64_t)P[mid] > rank) hi = mid;
                else lo = mid + 1;
            }
            tmp[tid] = q_value(q_bits((uint32_t)lo));
        } else if (tid < 64) {
            const double vlo = q_value(q_bits((uint32_t)klo)), vhi = q_value(q_bits((uint32_t)khi));
            const double span = vhi - vlo;
            const double step = span * (double)(tid - 32);
            tmp[tid] = vlo + step / 31.0;
        }
        __syncthreads();
        q_rank_sort(tmp, cen, tid);
        __syncthreads();

        // 4. Lloyd rounds, all in wave 0: lane i holds centre i, its
        //    neighbours come by whole-wave DPP shifts.  The new centres are already in
        //    the sort's order whenever each comes after its left neighbour
        //    (a mean lies between its cluster's boundaries, an empty cluster
        //    keeps its centre); then the rank sort would leave them in place
        //    and is skipped.  Otherwise (equal zeros of opposite sign) they go
        //    through it in LDS.
        if (tid < Q_ENTRIES) {
            double c = cen[tid];
            const int64_t s_all = S[khi];
            for (int round = 0; round < Q_ROUNDS; ++round) {
                const double c_next = __builtin_bit_cast(double, q_down1(__builtin_bit_cast(uint64_t, c)));
                uint32_t cnt = (uint32_t)n;
                int64_t sum = s_all;
                if (tid < Q_ENTRIES - 1) {
                    const int k = q_floor_key((c + c_next) * 0.5, klo, khi);
                    // P and S are zero below the smallest key present
                    cnt = k >= klo ? P[k] : 0u;
                    sum = k >= klo ? S[k] : 0;
                }
                const uint32_t cnt_prev = q_dpp<0x138, 0xf>(cnt);           // 0 in lane 0
                const int64_t sum_prev = (int64_t)q_up1((uint64_t)sum);
                const uint32_t num = cnt - cnt_prev;
                const double v = num ? ldexp((double)(sum - sum_prev) / (double)num, -24) : c;
                const double u = __builtin_bit_cast(double, q_up1(__builtin_bit_cast(uint64_t, v)));
                const bool after = tid == 0 || u < v ||
                                   (u == v && !(!__builtin_signbit(u) && __builtin_signbit(v)));
                if (__all(after)) {
                    c = v;
                } else {
                    tmp[tid] = v;
                    q_wave_sync();
                    q_rank_sort(tmp, cen, tid);
                    q_wave_sync();
                    c = cen[tid];
                    q_wave_sync();
                }
            }
            cen[tid] = c;
        }
        __syncthreads();

        // 5. the FP16 table, sorted, and the final boundaries
        if (tid < Q_ENTRIES) tmp[tid] = q_value(q_round_f16(cen[tid], klo, khi));
        __syncthreads();
        q_rank_sort(tmp, bnd, tid);
        __syncthreads();
        if (tid < Q_ENTRIES) {
            const double t = bnd[tid];
            const uint32_t h = t == 0.0 ? (__builtin_signbit(t) ? 0x8000u : 0u) : q_round_f16(t, klo, khi);
            tables[(size_t)g * Q_ENTRIES + tid] = (uint16_t)h;
            tmp[tid] = t;
        }
        __syncthreads();
        if (tid < Q_ENTRIES - 1) bnd[tid] = (tmp[tid] + tmp[tid + 1]) * 0.5;
        __syncthreads();

        // 6. key -> index: a key's value exceeds boundary i exactly when the
        //    key is above the boundary's floor key, so the index of a key is
        //    the number of floor keys below it; each thread walks a
        //    contiguous range of keys
        if (tid < Q_ENTRIES - 1) fkey[tid] = q_floor_key(bnd[tid], klo, khi);
        __syncthreads();
        {
            const int span = khi - klo + 1;
            const int per = (span + Q_THREADS - 1) / Q_THREADS;
            const int k0 = klo + tid * per, k1 = min(khi + 1, k0 + per);
            if (k0 < k1) {
                int idx = 0;                           // floor keys below k0
                while (idx < Q_ENTRIES - 1 && fkey[idx] < k0) ++idx;
                int next = idx < Q_ENTRIES - 1 ? fkey[idx] : Q_KEYS;
                for (int key = k0; key < k1; ++key) {
                    while (next < key) {
                        ++idx;
                        next = idx < Q_ENTRIES - 1 ? fkey[idx] : Q_KEYS;
                    }
                    map[key] = (uint8_t)idx;
                }
            }
        }
        __syncthreads();

        // 7. pack: 16 consecutive weights of a row -> 12 bytes (three words)
        const int units_per_row = K / 16;
        for (int u = tid; u < 16 * units_per_row; u += Q_THREADS) {
            const int r = u / units_per_row, c = u % units_per_row;
            const uint16_t* src = wg + (size_t)r * K + 16 * c;
            uint32_t out[3] = {0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t word = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) word |= (uint32_t)map[q_key(src[4 * q + t])] << (6 * t);
                // 24-bit little-endian word q at byte 3q of the 12
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int byte = 3 * q + b;
                    out[byte >> 2] |= ((word >> (8 * b)) & 0xFFu) << (8 * (byte & 3));
                }
            }
            uint32_t* dst = (uint32_t*)(packed + (size_t)(16 * g + r) * row_bytes + 12 * c);
            dst[0] = out[0];
            dst[1] = out[1];
            dst[2] = out[2];
        }
        __syncthreads();
    }
}

struct QWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_qws_mutex;
std::map<std::tuple<int, uintptr_t>, QWorkspace> g_qws;   // key: (device, stream)

int q_workspace(hipStream_t stream, size_t bytes, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LUT6_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_qws_mutex);
    QWorkspace& ws = g_qws[std::make_tuple(dev, (uintptr_t)stream)];
    if (ws.bytes < bytes) {
        // grown in stream order (no host synchronisation): the old buffer is
        // released after the work already enqueued on this stream
        if (ws.ptr) {
            if (hipFreeAsync(ws.ptr, stream) != hipSuccess) return LUT6_E_DEVICE;
            ws.ptr = nullptr;
            ws.bytes = 0;
        }
        void* p = nullptr;
        if (hipMallocAsync(&p, bytes, stream) != hipSuccess) return LUT6_E_DEVICE;
        ws.ptr = p;
        ws.bytes = bytes;
    }
    *out = ws.ptr;
    return LUT6_OK;
}

bool q_overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// int8 code selection (page "clef-flash — Core AI", section "Precision":
// int8 per block of 32, symmetric with clipping, weights only).  One thread
// per block of 32 inputs of one row (four lanes per block, each taking a
// quarter, was slower on a weight larger than the last-level cache):
//   - the block's largest magnitude a (on the bit patterns with the sign
//     cleared, which order finite FP16 magnitudes);
//   - scale s = fp16(a / 127): the FP32 quotient rounded to FP16 equals the
//     single rounding of a / 127 (FP32 has more than twice FP16's 11 bits,
//     plus two, so the double rounding is innocuous);
//   - code = w / s in FP32 (correctly rounded), rounded to nearest even and
//     clamped to -127..127; a scale of zero gives zero codes.
// Reads 64 bytes and writes 34 per block: bound by HBM.
typedef uint32_t q_u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256)
lut6_int8_quantize_kernel(const uint16_t* __restrict__ w, int8_t* __restrict__ q, uint16_t* __restrict__ qs,
                          int64_t nblocks)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const q_u32x4 x = *(const q_u32x4*)(w + b * 32 + 8 * i);
        v[4 * i] = x[0];
        v[4 * i + 1] = x[1];
        v[4 * i + 2] = x[2];
        v[4 * i + 3] = x[3];
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = max(mx, max(v[i] & 0x7fffu, (v[i] >> 16) & 0x7fffu));
    const float a = (float)__builtin_bit_cast(_Float16, (uint16_t)mx);
    const _Float16 sh = (_Float16)(a / 127.0f);
    qs[b] = __builtin_bit_cast(uint16_t, sh);
    const float s = (float)sh;
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * i + e;
            const uint16_t hb = (uint16_t)((v[j >> 1] >> (16 * (j & 1))) & 0xffffu);
            int code = 0;
            if (s != 0.0f) {
                const float r = __builtin_rintf((float)__builtin_bit_cast(_Float16, hb) / s);
                code = r > 127.0f ? 127 : r < -127.0f ? -127 : (int)r;
            }
            word |= ((uint32_t)code & 0xffu) << (8 * e);
        }
        out[i] = word;
    }
    *(q_u32x4*)(q + b * 32) = q_u32x4{out[0], out[1], out[2], out[3]};
    *(q_u32x4*)(q + b * 32 + 16) = q_u32x4{out[4], out[5], out[6], out[7]};
}

}  // namespace

extern "C" int lut6_quantize(const void* w, uint8_t* packed, void* tables, int64_t N, int64_t K,
                             hipStream_t stream)
{
    if (!w || !packed || !tables) return LUT6_E_NULL;
    if (N <= 0 || K <= 0 || N % 16 || K % 64 || 16 * K > (1 << 22) || N > INT32_MAX) return LUT6_E_SHAPE;
    if (((uintptr_t)w | (uintptr_t)packed | (uintptr_t)tables) & 15u) return LUT6_E_ALIGN;
    const size_t wb = (size_t)N * K * 2, pb = (size_t)N * (K / 4 * 3), tb = (size_t)(N / 16) * 128;
    if (q_overlaps(packed, pb, w, wb) || q_overlaps(tables, tb, w, wb) || q_overlaps(packed, pb, tables, tb))
        return LUT6_E_ALIAS;
    const int groups = (int)(N / 16);
    const int wgs = groups < Q_MAX_WG ? groups : Q_MAX_WG;
    void* work = nullptr;
    const int st = q_workspace(stream, (size_t)wgs * Q_SLOT_BYTES, &work);
    if (st != LUT6_OK) return st;
    hipLaunchKernelGGL(lut6_quantize_kernel, dim3((unsigned)wgs), dim3(Q_THREADS), 0, stream,
                       (const uint16_t*)w, packed, (uint16_t*)tables, (int)N, (int)K, (uint8_t*)work);
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}

extern "C" int lut6_int8_quantize(const void* w, int8_t* q, void* scales, int64_t N, int64_t K,
                                  hipStream_t stream)
{
    if (!w || !q || !scales) return LUT6_E_NULL;
    if (N <= 0 || K <= 0 || K % 32 || N > INT64_MAX / K) return LUT6_E_SHAPE;
    const int64_t nblocks = N * (K / 32);
    if ((nblocks + 255) / 256 > INT32_MAX) return LUT6_E_SHAPE;
    if ((((uintptr_t)w | (uintptr_t)q) & 15u) || ((uintptr_t)scales & 1u)) return LUT6_E_ALIGN;
    const size_t wb = (size_t)N * K * 2, qb = (size_t)N * K, sb = (size_t)nblocks * 2;
    if (q_overlaps(q, qb, w, wb) || q_overlaps(scales, sb, w, wb) || q_overlaps(q, qb, scales, sb))
        return LUT6_E_ALIAS;
    hipLaunchKernelGGL(lut6_int8_quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, stream,
                       (const uint16_t*)w, q, (uint16_t*)scales, nblocks);
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}

namespace lut6_detail {
// Free the table-fitting workspaces (lut6_release calls this), after
// synchronising the devices that hold one.
int quantize_release()
{
    std::lock_guard<std::mutex> lock(g_qws_mutex);
    int status = LUT6_OK;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_qws) {
        if (!kv.second.ptr) continue;
        if (hipSetDevice(std::get<0>(kv.first)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            status = LUT6_E_DEVICE;
        if (hipFreeAsync(kv.second.ptr, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            status = LUT6_E_DEVICE;
    }
    g_qws.clear();
    (void)hipSetDevice(cur);
    return status;
}
}  // namespace lut6_detail
