// LUT-6 dequant-GEMM for AMD Instinct MI355X (gfx950, CDNA4).
//
// What it computes (page "Clef-Flash-ANE-LUT6", sections "Weight precision"
// and "LUT-6 text weights"):
//     W[n, k]  = table[n / 16][index(n, k)]          (one FP16 table per 16 channels)
//     xs       = fp16(x * s)                          (s = in_scale, a power of two <= 16)
//     a[l, n]  = (sum_k xs[l, k] * W[n, k]) / s       (FP32 accumulation)
//     y        = epilogue(a): FP32, FP16, or silu(gate) * up in FP16.
//
// Mapping onto the hardware (one MI355X: 256 CUs in 8 XCDs, 4 SIMDs per CU)
//   * Every contraction runs on v_mfma_f32_32x32x16_f16 (FP16 operands,
//     FP32 accumulation): the weight is the MFMA "A" operand (32 channels x
//     16 k), the activations the "B" operand (16 k x 32 tokens).  The k order
//     inside an MFMA is free as long as A and B agree; lane group h = lane /
//     32 takes k in [32h, 32h + 32) of a 64-k chunk, so its 32 indices are
//     24 contiguous packed bytes (a 192-bit little-endian word).
//   * Tables sit in LDS, 128 bytes each; a lookup is one shift or funnel
//     shift, one v_and_or_b32 into an LDS byte offset and one ds_read_u16,
//     a bit copy (dequantisation is exact).  The streaming kernel uses
//     4096-word pair tables instead (two consecutive k per lookup).
//   * Three paths by token count (lut6_linear_path):
//       - L <= 192, lut6_stream_kernel: each weight serves few tokens;
//         64-token x 32-channel tiles over the whole K range (one kernel,
//         outputs finished in place), K split into slices added by a second
//         kernel in a fixed order only when the tiles are too few to fill
//         the CUs (no atomics, bit-identical run to run).
//       - 192 < L < 1024, lut6_tile256_kernel: 256 x 256 tiles, four waves
//         (one per SIMD, 64 x 256 accumulators each); packed words go
//         straight to registers, activations through three LDS stages, and
//         the table lookups are spread over the MFMA stream.
//       - L >= 1024, lut6_expand_kernel + lut6_expanded_gemm_kernel: the
//         fused kernel repeats every lookup once per 256-token tile, and one
//         wave per SIMD cannot issue those lookups and keep the matrix unit
//         fed; with many tokens the weight is expanded once per call into
//         FP16 MFMA fragments (1 KB each, contiguous) and the GEMM loads them
//         straight into registers.
//   * Tiles are remapped from the round-robin XCD dispatch to contiguous
//     ranges per XCD and grouped by 4 token tiles, so the workgroups resident
//     on one XCD share activation and weight tiles in its L2.
//   * Outputs go through LDS so that each store instruction writes whole
//     rows; the input scale is applied to the FP16 activation fragments
//     (exactly fp16(x * s)) and undone on the FP32 sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <tuple>
#include <type_traits>
#include <mutex>
#include <utility>

#include "lut6.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;          // k per main-loop step (two MFMA k-steps of 32)
constexpr int NUM_XCD = 8;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Round-robin XCD dispatch -> contiguous tile ranges per XCD.
__device__ __forceinline__ int xcd_remap(int b, int nb)
{
    const int xcd = b % NUM_XCD, local = b / NUM_XCD;
    const int q = nb / NUM_XCD, r = nb % NUM_XCD;
    return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
}

// Sixteen consecutive 6-bit indices, held as the little-endian 96-bit word
// d0 | d1 << 32 | d2 << 64 (index t = bits 6t .. 6t+5), looked up in one
// 64-entry table; entries 0..7 go to `lo`, 8..15 to `hi`.
__device__ __forceinline__ void gather16(uint32_t d0, uint32_t d1, uint32_t d2,
                                         const uint16_t* __restrict__ tab,
                                         f16x8& lo, f16x8& hi)
{
    uint32_t e[16];
    e[0] = d0 & 63u;
    e[1] = (d0 >> 6) & 63u;
    e[2] = (d0 >> 12) & 63u;
    e[3] = (d0 >> 18) & 63u;
    e[4] = (d0 >> 24) & 63u;
    e[5] = __builtin_amdgcn_alignbit(d1, d0, 30) & 63u;
    e[6] = (d1 >> 4) & 63u;
    e[7] = (d1 >> 10) & 63u;
    e[8] = (d1 >> 16) & 63u;
    e[9] = (d1 >> 22) & 63u;
    e[10] = __builtin_amdgcn_alignbit(d2, d1, 28) & 63u;
    e[11] = (d2 >> 2) & 63u;
    e[12] = (d2 >> 8) & 63u;
    e[13] = (d2 >> 14) & 63u;
    e[14] = (d2 >> 20) & 63u;
    e[15] = d2 >> 26;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = (uint32_t)tab[e[2 * i]] | ((uint32_t)tab[e[2 * i + 1]] << 16);
    u32x4 a = {w[0], w[1], w[2], w[3]};
    u32x4 b = {w[4], w[5], w[6], w[7]};
    lo = __builtin_bit_cast(f16x8, a);
    hi = __builtin_bit_cast(f16x8, b);
}

// Workgroup barrier for the main loops: each wave has already waited for its
// own LDS copies (vmcnt), and LDS needs no cache maintenance, so the LDS
// fence that __syncthreads() adds (a wait for every outstanding LDS read,
// including the prefetches of the next step) is not needed.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float silu_f32(float g)
{
    // g / (1 + e^-g); e^-g = 2^(-g log2 e) on the hardware exp2
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g / (1.0f + e);
}

struct GemmArgs {
    const uint16_t* x;        // FP16 [L, K]
    const uint8_t* packed;    // [N, 3K/4]
    const uint16_t* tables;   // FP16 [N/16, 64]
    void* y;                  // output (epilogue layout) when not split
    float* partial;           // FP32 [splits, L, N] when split
    const uint16_t* w16;      // FP16 [N, K], the expanded weight (two-pass path)
    int L, K, N;
    int k_chunks_per_split;   // BK-chunks per split
    int tiles_m;              // token tiles
    int n_tiles;              // total (token x channel) tiles
    _Float16 scale;           // in_scale as FP16 (exact)
    float inv_scale;          // 1 / in_scale (exact)
};

// ---------------------------------------------------------------------------
// Large-tile kernel: 256 channels x 256 tokens per workgroup, four waves.
//   Wave w owns channels [64w, 64w + 64) of the tile as two 32-row MFMA "A"
//   fragments and all 256 tokens as eight 32-token "B" fragments, contracted
//   with v_mfma_f32_32x32x16_f16 (the FP16 shape with the most work per
//   operand byte on gfx950).  2 x 8 accumulators of 16 floats = 256
//   accumulation registers per lane.
//   Over a 64-wide k tile, lane group h = lane / 32 takes k in [32h, 32h + 32),
//   eight per MFMA step, so its 32 indices are 24 contiguous packed bytes
//   (a 192-bit little-endian word, index i at bits 6i .. 6i + 5), loaded from
//   global memory straight into registers two tiles ahead.
//   A 32-row fragment spans two tables: lanes whose row is in the upper 16
//   read the second.
//   Memory pipeline: three LDS stages of activations (256 rows x 128 bytes,
//   XOR-swizzled), filled by buffer loads that write LDS directly (no
//   staging registers), issued two tiles ahead.
//   Compute pipeline (one wave per SIMD, so the MFMA unit only stays busy if
//   nothing the wave issues has to wait): each step of 16 MFMAs also reads
//   the B fragments of the next step, gathers the A entries of the step after
//   it, and packs the entries gathered one step earlier into the next step's
//   A fragments, all spread evenly over the step (two gathers, one B read and
//   one pack per MFMA pair), so every LDS read has a whole step to land.  The
//   barrier sits before the last step of a tile, which reads the first B
//   fragments of the next tile.
// ---------------------------------------------------------------------------
constexpr int T2 = 256;                        // tile channels and tokens
constexpr int T2_XBYTES = T2 * BK * 2;         // activation tile (32 KB)
constexpr int T2_NSTAGE = 3;
constexpr int T2_TABLES = 2048;                // 16 tables of 128 bytes
constexpr int T2_LDS = T2_TABLES + T2_NSTAGE * T2_XBYTES;
constexpr int T2_GROUP_M = 4;                  // token tiles per scheduling group
constexpr int RAW_BUFFER_WORD3 = 0x00020000;   // gfx9 raw buffer descriptor word 3
// s_waitcnt immediate that waits for vmcnt = 0 and leaves the other counters
// alone (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int VMCNT0 = 0x0F70;
// vmcnt <= 16 (bits 3:0 = 0, bits 15:14 = 1), other counters not waited for
constexpr int VMCNT16 = 0x4F70;
// lgkmcnt = 0, other counters not waited for
constexpr int LGKMCNT0 = 0xC07F;
// lgkmcnt <= 12 (bits 11:8), other counters not waited for
constexpr int LGKMCNT12 = 0xCC7F;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS byte offset of 16-byte chunk c (0..7) of activation row r.  Rows are
// 128 bytes; the chunk is XOR-swizzled with (r >> 1) & 7 so that sixteen
// consecutive rows read at one chunk cover all 64 four-byte banks once (a
// 16-byte read serves 16 lanes per cycle).
__device__ __forceinline__ int xswz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// (v & 0x7e) | base in one instruction (LLVM would otherwise split the mask
// and merge into an and plus an add).
__device__ __forceinline__ uint32_t and_or_7e(uint32_t v, uint32_t base)
{
#if __HIP_DEVICE_COMPILE__
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(0x7eu), "v"(base));
    return r;
#else
    return (v & 0x7eu) | base;   // the host pass only parses device code
#endif
}

// Byte offset of table entry "index I" (I = 0..31 of the 192-bit
// little-endian word p, index I at bits 6I .. 6I + 5) in a 128-byte-aligned
// LDS table at byte offset tab: the field is shifted to bits 1..6 (one shift
// or funnel shift), then masked and merged with the table offset.
template <int I>
__device__ __forceinline__ uint32_t entry_off(const uint32_t (&p)[6], uint32_t tab)
{
    constexpr int bit = 6 * I, w = bit >> 5, o = bit & 31;
    uint32_t v;
    if constexpr (o == 0 && w == 0)
        v = p[0] << 1;
    else if constexpr (o == 0)
        v = __builtin_amdgcn_alignbit(p[w], p[w - 1], 31);
    else if constexpr (o <= 26)
        v = p[w] >> (o - 1);
    else
        v = __builtin_amdgcn_alignbit(p[w + 1], p[w], o - 1);
    return and_or_7e(v, tab);
}

// (v & 0x3ffc) | base in one instruction.
__device__ __forceinline__ uint32_t and_or_3ffc(uint32_t v, uint32_t base)
{
#if __HIP_DEVICE_COMPILE__
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(0x3ffcu), "v"(base));
    return r;
#else
    return (v & 0x3ffcu) | base;
#endif
}

// Byte offset of a pair-table word in a 16 KB-aligned LDS pair table at
// byte offset tab.  The word for the 12-bit field at bit B of the 192-bit
// little-endian word p (indices i0 at bits B .. B+5 and i1 at B+6 .. B+11,
// two consecutive k) is entry i0 | i1 << 6, holding T[i0] in its low half
// and T[i1] in its high half: the field is shifted to bits 2 .. 13 (one
// shift or funnel shift), then masked and merged with the table offset.
template <int B>
__device__ __forceinline__ uint32_t pair_off(const uint32_t (&p)[6], uint32_t tab)
{
    constexpr int w = B >> 5, o = B & 31;
    uint32_t v;
    if constexpr (o == 0 && w == 0)
        v = p[0] << 2;
    else if constexpr (o == 0)
        v = __builtin_amdgcn_alignbit(p[w], p[w - 1], 30);
    else if constexpr (o <= 20)
        v = p[w] >> (o - 2);
    else
        v = __builtin_amdgcn_alignbit(p[w + 1], p[w], o - 2);
    return and_or_3ffc(v, tab);
}

// Global weight row of tile row t (0..255) of channel tile tn.  Tile row
// t = 64w + 32f + r is row r of fragment f of wave w.  Rows past the end are
// clamped (computed on a copy of the last row and never stored).
template <int EPI>
__device__ __forceinline__ int tile_row(int t, int tn, int N)
{
    if constexpr (EPI == 2) {
        // fragment 0 of each wave: gate rows, fragment 1: the matching up rows
        const int w = t >> 6, f = (t >> 5) & 1, r = t & 31;
        const int j = min(tn * 128 + 32 * w + r, N / 2 - 1);
        return f ? N / 2 + j : j;
    } else {
        return min(tn * 256 + t, N - 1);
    }
}

// Split-K partial sums through LDS: each wave writes the raw FP32 sums of
// its 64 accumulator channels (for silu(gate) * up: 32 gate then the 32
// matching up channels) of 32 * JP tokens into an LDS block with padded rows,
// then stores whole row segments: 16 bytes per lane, so each store
// instruction covers whole 128-byte lines (storing straight from the
// accumulators wrote 32-byte pieces of 32 rows per instruction, and with
// every workgroup writing its partials at the same moment that took twice
// as long).  Partial plane ks is [L, N] with the gate columns at [0, N/2)
// and the up columns at [N/2, N).  The caller has synchronised the
// workgroup: the pipeline stages are free.
template <int EPI, int NJ, int JP>
__device__ __forceinline__ void tile_store_partial(const GemmArgs& a, const f32x16 (&acc)[2][NJ], int tok0,
                                                   int tn, int w, int lane, uint8_t* lds, int ks)
{
    constexpr int ROWB = 64 * 4;                  // one token's 64 sums
    constexpr int PITCH = ROWB + 16;
    constexpr int LPR = ROWB / 16;                // lanes per row when reading back
    constexpr int NREAD = 32 * JP * ROWB / 1024;  // read/store instructions per pass
    const int r32 = lane & 31, h = lane >> 5;
    uint8_t* const wl = lds + w * (32 * JP * PITCH);
    const int L = a.L, N = a.N;
    float* const plane = a.partial + (size_t)ks * L * N;
#pragma unroll
    for (int p = 0; p < NJ / JP; ++p) {
        // one pass at a time: hoisting every pass's accumulator reads would
        // take nearly every register
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
            const int j = JP * p + jj;
            uint8_t* const row = wl + (32 * jj + r32) * PITCH;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(f32x4*)(row + (32 * f + 8 * q + 4 * h) * 4) =
                        f32x4{acc[f][j][4 * q], acc[f][j][4 * q + 1], acc[f][j][4 * q + 2], acc[f][j][4 * q + 3]};
        }
#pragma unroll
        for (int i = 0; i < NREAD; ++i) {
            const int idx = i * 64 + lane, r = idx / LPR, seg = idx % LPR;
            const u32x4 v = *(const u32x4*)(wl + r * PITCH + seg * 16);
            const int tok = tok0 + 32 * JP * p + r;
            int col;
            bool ok;
            if constexpr (EPI == 2) {
                // segments 0..7: gate channels, 8..15: the matching up channels
                const int jcol = tn * 128 + 32 * w + (seg & 7) * 4;
                ok = jcol < N / 2;
                col = seg < 8 ? jcol : N / 2 + jcol;
            } else {
                col = tn * 256 + 64 * w + seg * 4;
                ok = col < N;
            }
            if (tok < L && ok) *(u32x4*)(plane + (size_t)tok * N + col) = v;
        }
    }
}

// Epilogue through LDS (not split): each wave writes its 64 output channels
// (32 for silu(gate) * up) of 64 tokens at a time into an LDS block with
// padded rows (16 spare bytes per row: the 32 lanes of one fragment write
// 32 different rows without bank conflicts), then reads whole row segments
// back and stores them, 16 bytes per lane, so every store instruction
// writes whole cache lines (instead of 16-byte pieces of 32 rows).  The
// caller has synchronised the workgroup: the pipeline stages are free.
// NJ 32-token fragments per wave, JP of them per pass; the wave's channels
// are tile rows 64w + [0, 64), its tokens start at tok0, its LDS block is
// number slot.
template <int EPI, int NJ, int JP>
__device__ __forceinline__ void tile_store_rows(const GemmArgs& a, const f32x16 (&acc)[2][NJ], int tok0, int tn,
                                               int w, int slot, int lane, uint8_t* lds)
{
    constexpr int OUTC = EPI == 2 ? 32 : 64;      // output channels per wave
    constexpr int ESZ = EPI == 0 ? 4 : 2;         // output element bytes
    constexpr int ROWB = OUTC * ESZ;              // one token's bytes
    constexpr int PITCH = ROWB + 16;
    constexpr int LPR = ROWB / 16;                // lanes per row when reading back
    constexpr int NREAD = 32 * JP * ROWB / 1024;  // read/store instructions per pass
    const int r32 = lane & 31, h = lane >> 5;
    uint8_t* const wl = lds + slot * (32 * JP * PITCH);
    const int L = a.L;
    const int ncols = EPI == 2 ? a.N / 2 : a.N;
    const int n0 = EPI == 2 ? tn * 128 + 32 * w : tn * 256 + 64 * w;
#pragma unroll
    for (int p = 0; p < NJ / JP; ++p) {
        // one pass at a time: the pass's fragments are taken out of the
        // accumulator registers here (the empty asm pins them there until
        // now), so the reads of every pass are not hoisted together, which
        // would take nearly every register
        f32x16 fr[2][JP];
#pragma unroll
        for (int jj = 0; jj < JP; ++jj)
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                fr[f][jj] = acc[f][JP * p + jj];
                asm volatile("" : "+a"(fr[f][jj]));
            }
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
            uint8_t* const row = wl + (32 * jj + r32) * PITCH;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (EPI == 2) {
                    f16x4 hv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float gv = fr[0][jj][4 * q + e] * a.inv_scale;
                        const float uv = fr[1][jj][4 * q + e] * a.inv_scale;
                        hv[e] = (_Float16)(silu_f32(gv) * uv);
                    }
                    *(f16x4*)(row + (8 * q + 4 * h) * 2) = hv;
                } else {
#pragma unroll
                    for (int f = 0; f < 2; ++f) {
                        f32x4 v = {fr[f][jj][4 * q], fr[f][jj][4 * q + 1], fr[f][jj][4 * q + 2], fr[f][jj][4 * q + 3]};
                        v *= a.inv_scale;
                        const int col = 32 * f + 8 * q + 4 * h;
                        if constexpr (EPI == 0) {
                            *(f32x4*)(row + col * 4) = v;
                        } else {
                            const f16x4 hv = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                            *(f16x4*)(row + col * 2) = hv;
                        }
                    }
                }
            }
        }
        // the wave reads back what its own lanes wrote (LDS executes a
        // wave's accesses in order)
#pragma unroll
        for (int i = 0; i < NREAD; ++i) {
            const int idx = i * 64 + lane, r = idx / LPR, seg = idx % LPR;
            const u32x4 v = *(const u32x4*)(wl + r * PITCH + seg * 16);
            const int tok = tok0 + 32 * JP * p + r, col = n0 + seg * (16 / ESZ);
            if (tok < L && col < ncols)
                *(u32x4*)((uint8_t*)a.y + ((size_t)tok * ncols + col) * ESZ) = v;
        }
    }
}

template <int EPI, bool SCALED, bool SPLIT>
__global__ void __launch_bounds__(256, 1)
lut6_tile256_kernel(GemmArgs a)
{
    // one LDS block: 16 tables at offset 0 (gather addresses need no base),
    // then three activation stages
    __shared__ __attribute__((aligned(1024))) uint8_t lds[T2_LDS];
    _Float16* const tl = (_Float16*)lds;
    const uint8_t* const tlb = lds;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, h = lane >> 5;
    const int K = a.K, N = a.N, L = a.L;
    const int row_bytes = K / 4 * 3;

    // tile: XCD-contiguous ranges, then groups of T2_GROUP_M token tiles so
    // the workgroups resident on one XCD share activation and weight tiles
    const int tiles_n = a.n_tiles / a.tiles_m;
    const int t = xcd_remap(blockIdx.x, a.n_tiles);
    const int group = t / (T2_GROUP_M * tiles_n);
    const int first_m = group * T2_GROUP_M;
    const int gm = min(a.tiles_m - first_m, T2_GROUP_M);
    const int within = t - group * T2_GROUP_M * tiles_n;
    const int tm = first_m + within % gm, tn = within / gm;
    const int m0 = tm * T2;
    const int kc_begin = blockIdx.y * a.k_chunks_per_split;
    const int kc_end = min(K / BK, kc_begin + a.k_chunks_per_split);

    // tables: slot s = t / 16 holds the table of tile rows 16s .. 16s + 15
    for (int i = tid; i < 16 * 64; i += 256)
        tl[i] = ((const _Float16*)a.tables)[(tile_row<EPI>(16 * (i >> 6), tn, N) / 16) * 64 + (i & 63)];
    // byte offsets (128-aligned) of this lane's two tables
    const uint32_t tab0 = (uint32_t)((4 * wave + 0 + (r32 >> 4)) * 128);
    const uint32_t tab1 = (uint32_t)((4 * wave + 2 + (r32 >> 4)) * 128);

    // buffer descriptors (31-bit byte offsets; sizes checked on the host)
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, (int)((size_t)L * K * 2), RAW_BUFFER_WORD3);
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.packed, (short)0, (int)((size_t)N * row_bytes), RAW_BUFFER_WORD3);

    // Activation DMA: each instruction writes 1 KB of LDS, 16 bytes per lane
    // in lane order; instruction i of wave w fills rows 32i + 8w .. +8 (slot
    // = lane & 7 of row 32i + 8w + lane / 8).
    const int xrow = 8 * wave + (lane >> 3);
    const int xchunk = (lane & 7) ^ ((xrow >> 1) & 7);
    int xgoff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        xgoff[i] = min(m0 + 32 * i + xrow, L - 1) * (K * 2) + xchunk * 16;
    // this lane's packed words: 24 bytes at tile offset 24h of weight rows
    // 64w + r32 (fragment 0) and 64w + 32 + r32 (fragment 1)
    int pgoff[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) pgoff[f] = tile_row<EPI>(64 * wave + 32 * f + r32, tn, N) * row_bytes + 24 * h;

    // this lane's B-fragment offsets inside a stage, per MFMA step
    int xoff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xoff[s] = xswz(r32, 4 * h + s);

    f32x16 acc[2][8];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[f][j][e] = 0.f;

    // packed words of three tiles (tile kc_begin + i in set i % 3), operands
    // by step parity: step s multiplies X[s & 1], W[s & 1] while X[~s & 1]
    // and W[~s & 1] are refilled and G[s & 1] gathers for step s + 2
    uint32_t PC[3][2][6];
    f16x8 X[2][8];
    f16x8 W[2][2];
    uint32_t G[2][16];
    // LDS byte offsets of the gathers of a step, computed one step earlier
    // (by step parity), so a gather never waits for its own address
    uint32_t GA[2][16];
    f16x8 XS[2];

    // buffer -> LDS copies of the activations of tile kc into stage st
    auto issue_x = [&](int st, int kc) {
        uint8_t* const sp = lds + T2_TABLES + st * T2_XBYTES;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (lds_ptr_t)(sp + i * 4096 + wave * 1024), 16, xgoff[i], kc * (BK * 2), 0, 0);
    };
    // packed words of tile kc into set PS (a constant)
    auto load_pc = [&](auto ps_c, int kc) {
        constexpr int PS = decltype(ps_c)::value;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(pr, pgoff[f], kc * 48, 0);
            const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(pr, pgoff[f] + 16, kc * 48, 0);
            PC[PS][f][0] = v[0];
            PC[PS][f][1] = v[1];
            PC[PS][f][2] = v[2];
            PC[PS][f][3] = v[3];
            PC[PS][f][4] = u[0];
            PC[PS][f][5] = u[1];
        }
    };
    auto read_xf = [&](int so, int s, int j) -> f16x8 {
        return *(const f16x8*)(lds + so + xoff[s] + j * 4096);
    };
    // unit u (0..3) of load_pc: fragment u / 2, the 16-byte part (u even) or
    // the 8-byte part
    auto load_pc_unit = [&](auto ps_c, int kc, int u) {
        constexpr int PS = decltype(ps_c)::value;
        const int f = u >> 1;
        if (u & 1) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(pr, pgoff[f] + 16, kc * 48, 0);
            PC[PS][f][4] = v[0];
            PC[PS][f][5] = v[1];
        } else {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(pr, pgoff[f], kc * 48, 0);
            PC[PS][f][0] = v[0];
            PC[PS][f][1] = v[1];
            PC[PS][f][2] = v[2];
            PC[PS][f][3] = v[3];
        }
    };
    auto issue_x1 = [&](int st, int kc, int i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (lds_ptr_t)(lds + T2_TABLES + st * T2_XBYTES + i * 4096 + wave * 1024), 16, xgoff[i],
            kc * (BK * 2), 0, 0);
    };

    // gather q (0..15) of step NS from packed set PS: fragment q / 8, index
    // 8 NS + q % 8 of the lane's 32
#define LUT6_GATHER(GP, PS, NS, Q)                                                     \
    G[GP][Q] = *(const uint16_t*)(tlb + entry_off<8 * (NS) + (Q) % 8>(PC[PS][(Q) / 8], (Q) / 8 ? tab1 : tab0))
#define LUT6_ADDR(AP, PS, NS, Q)                                                       \
    GA[AP][Q] = entry_off<8 * (NS) + (Q) % 8>(PC[PS][(Q) / 8], (Q) / 8 ? tab1 : tab0)
#define LUT6_LOAD(GP, Q) G[GP][Q] = *(const uint16_t*)(tlb + GA[GP][Q])
    // pack c (0..7) of the A fragments of the next step: fragment c / 4,
    // dword c % 4 from gathers 2c, 2c + 1
#define LUT6_PACK(GP, C) wn[(C) / 4][(C) % 4] = G[GP][2 * (C)] | (G[GP][2 * (C) + 1] << 16)
    // with SCALED the B fragment of pair J was scaled during pair J - 1 (into
    // XS[J & 1]), so the MFMAs never wait for their own multiplies; pair 7
    // scales the next step's first fragment, read in this step's pair 0
#define LUT6_MMA(P, J)                                                                 \
    do {                                                                               \
        const f16x8 xj = SCALED ? XS[(J) & 1] : X[P][J];                               \
        acc[0][J] = __builtin_amdgcn_mfma_f32_32x32x16_f16(W[P][0], xj, acc[0][J], 0, 0, 0); \
        acc[1][J] = __builtin_amdgcn_mfma_f32_32x32x16_f16(W[P][1], xj, acc[1][J], 0, 0, 0); \
        if constexpr (SCALED)                                                          \
            XS[((J) + 1) & 1] = ((J) < 7 ? X[P][((J) + 1) & 7] : X[1 - (P)][0]) * a.scale; \
    } while (0)
    // One step: MFMAs on parity P; B fragments of the next step from stage
    // byte offset SN (step NB of its tile); the gathers whose addresses the
    // previous step computed (entries of the step after next); the addresses
    // of the next step's gathers (step NA of the tile whose packed words are
    // in set PA); packs of the entries gathered one step ago.
    // sched_barrier(0) keeps each MFMA pair with its share of the other work:
    // left alone the scheduler clusters the LDS reads.
#define LUT6_PAIR(P, SN, NB, PA, NA, J)                                                \
    do {                                                                               \
        LUT6_MMA(P, J);                                                                \
        X[1 - (P)][J] = read_xf(SN, NB, J);                                            \
        LUT6_LOAD(P, 2 * (J));                                                         \
        LUT6_LOAD(P, 2 * (J) + 1);                                                     \
        LUT6_ADDR(1 - (P), PA, NA, 2 * (J));                                           \
        LUT6_ADDR(1 - (P), PA, NA, 2 * (J) + 1);                                       \
        LUT6_PACK(1 - (P), J);                                                         \
        __builtin_amdgcn_sched_barrier(0);                                             \
    } while (0)
#define LUT6_STEP(P, SN, NB, PA, NA)                                                   \
    do {                                                                               \
        uint32_t wn[2][4];                                                             \
        LUT6_PAIR(P, SN, NB, PA, NA, 0);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 1);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 2);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 3);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 4);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 5);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 6);                                               \
        LUT6_PAIR(P, SN, NB, PA, NA, 7);                                               \
        W[1 - (P)][0] = __builtin_bit_cast(f16x8, u32x4{wn[0][0], wn[0][1], wn[0][2], wn[0][3]}); \
        W[1 - (P)][1] = __builtin_bit_cast(f16x8, u32x4{wn[1][0], wn[1][1], wn[1][2], wn[1][3]}); \
    } while (0)
    // the same step with one extra memory instruction per MFMA pair: MEM(J)
#define LUT6_PAIR_M(P, SN, NB, PA, NA, J, MEM)                                         \
    do {                                                                               \
        LUT6_MMA(P, J);                                                                \
        X[1 - (P)][J] = read_xf(SN, NB, J);                                            \
        LUT6_LOAD(P, 2 * (J));                                                         \
        LUT6_LOAD(P, 2 * (J) + 1);                                                     \
        LUT6_ADDR(1 - (P), PA, NA, 2 * (J));                                           \
        LUT6_ADDR(1 - (P), PA, NA, 2 * (J) + 1);                                       \
        LUT6_PACK(1 - (P), J);                                                         \
        MEM(J);                                                                        \
        __builtin_amdgcn_sched_barrier(0);                                             \
    } while (0)
#define LUT6_STEP_M(P, SN, NB, PA, NA, MEM)                                            \
    do {                                                                               \
        uint32_t wn[2][4];                                                             \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 0, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 1, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 2, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 3, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 4, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 5, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 6, MEM);                                        \
        LUT6_PAIR_M(P, SN, NB, PA, NA, 7, MEM);                                        \
        W[1 - (P)][0] = __builtin_bit_cast(f16x8, u32x4{wn[0][0], wn[0][1], wn[0][2], wn[0][3]}); \
        W[1 - (P)][1] = __builtin_bit_cast(f16x8, u32x4{wn[1][0], wn[1][1], wn[1][2], wn[1][3]}); \
    } while (0)

    // prologue: activations and packed words of the first two tiles in
    // flight; the first tile's step-0 operands in registers and its step-1
    // entries gathered
    const int last = kc_end - 1;
    issue_x(0, kc_begin);
    load_pc(std::integral_constant<int, 0>{}, kc_begin);
    issue_x(1, min(kc_begin + 1, last));
    load_pc(std::integral_constant<int, 1>{}, min(kc_begin + 1, last));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    {
        constexpr int so = T2_TABLES;
#pragma unroll
        for (int j = 0; j < 8; ++j) X[0][j] = read_xf(so, 0, j);
        if constexpr (SCALED) XS[0] = X[0][0] * a.scale;
        uint32_t wn[2][4];
#define LUT6_PRO(Q)                                                                    \
    do {                                                                               \
        LUT6_GATHER(0, 0, 0, Q);                                                       \
        LUT6_GATHER(1, 0, 1, Q);                                                       \
    } while (0)
        LUT6_PRO(0); LUT6_PRO(1); LUT6_PRO(2); LUT6_PRO(3); LUT6_PRO(4); LUT6_PRO(5); LUT6_PRO(6); LUT6_PRO(7);
        LUT6_PRO(8); LUT6_PRO(9); LUT6_PRO(10); LUT6_PRO(11); LUT6_PRO(12); LUT6_PRO(13); LUT6_PRO(14); LUT6_PRO(15);
#undef LUT6_PRO
        LUT6_PACK(0, 0); LUT6_PACK(0, 1); LUT6_PACK(0, 2); LUT6_PACK(0, 3);
        LUT6_PACK(0, 4); LUT6_PACK(0, 5); LUT6_PACK(0, 6); LUT6_PACK(0, 7);
        // addresses of the first step's gathers (step 2 of the first tile)
#define LUT6_PRO_A(Q) LUT6_ADDR(0, 0, 2, Q)
        LUT6_PRO_A(0); LUT6_PRO_A(1); LUT6_PRO_A(2); LUT6_PRO_A(3); LUT6_PRO_A(4); LUT6_PRO_A(5);
        LUT6_PRO_A(6); LUT6_PRO_A(7); LUT6_PRO_A(8); LUT6_PRO_A(9); LUT6_PRO_A(10); LUT6_PRO_A(11);
        LUT6_PRO_A(12); LUT6_PRO_A(13); LUT6_PRO_A(14); LUT6_PRO_A(15);
#undef LUT6_PRO_A
        W[0][0] = __builtin_bit_cast(f16x8, u32x4{wn[0][0], wn[0][1], wn[0][2], wn[0][3]});
        W[0][1] = __builtin_bit_cast(f16x8, u32x4{wn[1][0], wn[1][1], wn[1][2], wn[1][3]});
    }

    // One tile: tile kc in stage ST (a constant; its packed words in set ST).
    // Past the end, tiles are fetched again (valid memory, into a stage and a
    // set that are no longer read).  Memory instructions go one per MFMA
    // pair: step 0 loads tile kc + 2's packed words into set (ST + 2) % 3
    // (tile kc - 1's, last read by its step 1's gathers), step 3 copies tile
    // kc + 2's activations into stage (ST + 2) % 3.  (Issued as a burst of
    // twelve per wave after the barrier they held up the MFMAs behind them:
    // about 3,300 cycles per 64-k chunk against 2,850 spread out.)  The
    // barrier before step 3 waits for every load of this wave (copies of
    // tile kc + 1, packed words of tile kc + 2); after it, all of tile kc + 1
    // is in LDS and every read of the stage that tile kc + 2 refills (tile
    // kc - 1's) has completed.
    auto tile_step = [&](auto st_c, int kc) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int S1 = (ST + 1) % T2_NSTAGE, S2 = (ST + 2) % T2_NSTAGE;
        constexpr int so = T2_TABLES + ST * T2_XBYTES;
        constexpr int sn = T2_TABLES + S1 * T2_XBYTES;
        const int kn = min(kc + 2, last);
#define LUT6_MEM_PC(J) do { if ((J) < 4) load_pc_unit(std::integral_constant<int, S2>{}, kn, (J)); } while (0)
#define LUT6_MEM_X(J) issue_x1(S2, kn, (J))
        // steps 0..3 gather entries of (ST, 2), (ST, 3), (S1, 0), (S1, 1) and
        // compute the addresses of the next step's: (ST, 3), (S1, 0), (S1, 1)
        // and (S1, 2), the first step of tile kc + 1
        LUT6_STEP_M(0, so, 1, ST, 3, LUT6_MEM_PC);
        LUT6_STEP(1, so, 2, S1, 0);
        LUT6_STEP(0, so, 3, S1, 1);
        __builtin_amdgcn_s_waitcnt(VMCNT0);
        lds_barrier();
        LUT6_STEP_M(1, sn, 0, S1, 2, LUT6_MEM_X);
#undef LUT6_MEM_PC
#undef LUT6_MEM_X
    };
    int kc = kc_begin;
    for (; kc + T2_NSTAGE <= kc_end; kc += T2_NSTAGE) {
        tile_step(std::integral_constant<int, 0>{}, kc);
        tile_step(std::integral_constant<int, 1>{}, kc + 1);
        tile_step(std::integral_constant<int, 2>{}, kc + 2);
    }
    if (kc < kc_end) tile_step(std::integral_constant<int, 0>{}, kc);
    if (kc + 1 < kc_end) tile_step(std::integral_constant<int, 1>{}, kc + 1);
#undef LUT6_STEP_M
#undef LUT6_PAIR_M
#undef LUT6_STEP
#undef LUT6_PAIR
#undef LUT6_MMA
#undef LUT6_PACK
#undef LUT6_LOAD
#undef LUT6_ADDR
#undef LUT6_GATHER
    // the last tiles' refetches are still in flight
    __builtin_amdgcn_s_waitcnt(0);

    if constexpr (SPLIT) {
        __syncthreads();
        tile_store_partial<EPI, 8, 2>(a, acc, m0, tn, wave, lane, lds, blockIdx.y);
    } else {
        __syncthreads();
        tile_store_rows<EPI, 8, 2>(a, acc, m0, tn, wave, wave, lane, lds);
    }
}

// ---------------------------------------------------------------------------
// Two-pass path for many tokens.  The fused kernel above gathers every weight
// once per 256-token tile, so at L = 16,384 each weight is looked up 64
// times, and each lookup costs an LDS gather and about three VALU
// instructions per MFMA: with one wave per SIMD (all 512 registers of a lane
// go to one wave so that it can hold 64 x 256 accumulators) the wave's issue
// slots, not the matrix unit, set the pace.  For many tokens the weight is
// therefore expanded once per call (lut6_expand_kernel: the same unpack and
// table lookup, FP16 [N, K] into a library workspace) and the contraction
// reads both operands as FP16 tiles.
//
// The GEMM keeps the large-tile kernel's shape: 256 channels x 256 tokens per
// workgroup, wave w owning channels [64w, 64w + 64) as two 32-row A fragments
// and all 256 tokens as eight B fragments of v_mfma_f32_32x32x16_f16.  A
// pipeline stage holds one 64-k tile of the activations and one of the
// expanded weight (each 256 rows x 128 bytes, XOR-swizzled), filled by
// buffer -> LDS copies; two stages.  Per MFMA pair a wave issues one B read
// and, twice per step, one A read: about 0.6 LDS reads per MFMA instead of
// the fused kernel's 1.5 LDS and 2.5 VALU instructions.  The barrier sits
// before the last step of a tile: every wave then has its operands of that
// step in registers, so the stage it read is refilled with the tile after
// next right away.
// ---------------------------------------------------------------------------
// Token counts from which the two-pass path runs.  Below them the fused
// kernel is as fast or faster: one expansion pass costs about as much as the
// fused kernel's extra LDS and VALU work over that many tokens, and for a
// deep K (a down-projection) the fused kernel keeps up to about 3000 tokens.
constexpr int EXPAND_MIN_L = 1536;
constexpr int EXPAND_MIN_L_DEEP_K = 3072;
constexpr int DEEP_K = 8192;

template <int EPI, bool SCALED, bool SPLIT>
__global__ void __launch_bounds__(256, 1)
lut6_expanded_gemm_kernel(GemmArgs a)
{
    // Persistent: workgroup g computes tiles g, g + G, g + 2G, ... (G =
    // gridDim.x); tile v is (K slice v / n_tiles, channel x token tile
    // xcd_remap(v % n_tiles)), so with G a multiple of 8 each workgroup stays
    // on the tiles its XCD would have run and the tiles in flight at one time
    // are the same sets as with one workgroup per tile.  Three activation
    // stages; FP16 and SiLU outputs are staged for the epilogue in a region
    // of their own, so the next tile's first two chunks are in flight while
    // this tile's outputs are written (FP32 outputs and split partials stage
    // in the pipeline region, after which the next tile's loads are issued).
    constexpr bool OWN_EPI = !SPLIT && EPI != 0;
    constexpr int EPI_BYTES = OWN_EPI ? 4 * 64 * ((EPI == 2 ? 64 : 128) + 16) : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[T2_NSTAGE * T2_XBYTES + EPI_BYTES];
    uint8_t* const epi_lds = OWN_EPI ? lds + T2_NSTAGE * T2_XBYTES : lds;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, h = lane >> 5;
    const int K = a.K, N = a.N, L = a.L;
    const int chunks = K / BK;
    const int splits = (chunks + a.k_chunks_per_split - 1) / a.k_chunks_per_split;
    const int total = a.n_tiles * splits;
    const int tiles_n = a.n_tiles / a.tiles_m;

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, (int)((size_t)L * K * 2), RAW_BUFFER_WORD3);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.w16, (short)0, (int)((size_t)tiles_n * 8 * (chunks + 1) * 4096), RAW_BUFFER_WORD3);
    const int bstride = (chunks + 1) * 4096;   // one fragment block (see lut6_expand_kernel)

    // per tile: first token, channel tile, K slice and its chunks (uniform)
    int m0, tn, ks, kc_begin, kc_end, last;
    auto set_tile = [&](int v) {
        ks = v / a.n_tiles;
        const int t = xcd_remap(v - ks * a.n_tiles, a.n_tiles);
        const int group = t / (T2_GROUP_M * tiles_n);
        const int first_m = group * T2_GROUP_M;
        const int gm = min(a.tiles_m - first_m, T2_GROUP_M);
        const int within = t - group * T2_GROUP_M * tiles_n;
        m0 = (first_m + within % gm) * T2;
        tn = within / gm;
        kc_begin = ks * a.k_chunks_per_split;
        kc_end = min(chunks, kc_begin + a.k_chunks_per_split);
        last = kc_end - 1;
    };
    // per lane: global offsets of the copies and A-fragment loads, and the
    // B-fragment offsets inside a stage.  Recomputed from an opaque copy of
    // the lane id whenever needed, so that none of them stays live through
    // an epilogue (whose accumulator reads need nearly every register).
    //  - activation copies: instruction i of wave w fills rows 32i + 8w .. +8
    //    of the tile (slot lane & 7 of row 32i + 8w + lane / 8);
    //  - A fragments come straight from the expanded weight, stored in
    //    fragment order by lut6_expand_kernel: fragment (tile tn, wave w,
    //    fragment f, chunk kc, step s) is 1 KB, 16 bytes per lane in lane
    //    order, so each load is contiguous;
    //  - B fragments: token r32 of each 32-token block, pieces 4h + s.
    int xgoff[8], wgoff[2], xoff[4];
    auto set_lane_offsets = [&]() {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int xrow = 8 * wave + (ln >> 3);
        const int xchunk = (ln & 7) ^ ((xrow >> 1) & 7);
#pragma unroll
        for (int i = 0; i < 8; ++i) xgoff[i] = min(m0 + 32 * i + xrow, L - 1) * (K * 2) + xchunk * 16;
#pragma unroll
        for (int f = 0; f < 2; ++f) wgoff[f] = ((tn * 4 + wave) * 2 + f) * bstride + ln * 16;
#pragma unroll
        for (int s = 0; s < 4; ++s) xoff[s] = xswz(ln & 31, 4 * (ln >> 5) + s);
    };

    f32x16 acc[2][8];
    // B fragments by step parity; A fragments of three tiles (tile
    // kc_begin + i in set i % 3), [step][fragment]
    f16x8 X[2][8];
    f16x8 WA[3][4][2];

    auto issue_x = [&](int st, int kc, int i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (lds_ptr_t)(lds + st * T2_XBYTES + i * 4096 + wave * 1024), 16, xgoff[i], kc * (BK * 2), 0, 0);
    };
    auto load_w = [&](auto ws_c, int kc) {
        constexpr int WS = decltype(ws_c)::value;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int f = 0; f < 2; ++f)
                WA[WS][s][f] = __builtin_bit_cast(
                    f16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, wgoff[f] + 1024 * s, kc * 4096, 0));
    };
    auto read_x = [&](int so, int s, int j) -> f16x8 { return *(const f16x8*)(lds + so + xoff[s] + j * 4096); };
    // activations (into LDS) and A fragments (into registers) of the tile's
    // first two chunks in flight
    auto prologue_x = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) issue_x(0, kc_begin, i);
#pragma unroll
        for (int i = 0; i < 8; ++i) issue_x(1, min(kc_begin + 1, last), i);
    };
    auto prologue_w = [&]() {
        load_w(std::integral_constant<int, 0>{}, kc_begin);
        load_w(std::integral_constant<int, 1>{}, min(kc_begin + 1, last));
    };

#define E_MMA(P, WS, S, J)                                                             \
    do {                                                                               \
        f16x8 xj = X[P][J];                                                            \
        if constexpr (SCALED) xj = xj * a.scale;                                       \
        acc[0][J] = __builtin_amdgcn_mfma_f32_32x32x16_f16(WA[WS][S][0], xj, acc[0][J], 0, 0, 0); \
        acc[1][J] = __builtin_amdgcn_mfma_f32_32x32x16_f16(WA[WS][S][1], xj, acc[1][J], 0, 0, 0); \
    } while (0)
    // MFMA pair J of step S (parity P, A fragments of set WS), then the B
    // fragment J of the next step (step NB of the tile in stage SN)
#define E_PAIR(P, WS, S, SN, NB, J)                                                    \
    do {                                                                               \
        E_MMA(P, WS, S, J);                                                            \
        X[1 - (P)][J] = read_x(SN, NB, J);                                             \
        __builtin_amdgcn_sched_barrier(0);                                             \
    } while (0)
#define E_STEP(P, WS, S, SN, NB)                                                       \
    do {                                                                               \
        E_PAIR(P, WS, S, SN, NB, 0); E_PAIR(P, WS, S, SN, NB, 1);                      \
        E_PAIR(P, WS, S, SN, NB, 2); E_PAIR(P, WS, S, SN, NB, 3);                      \
        E_PAIR(P, WS, S, SN, NB, 4); E_PAIR(P, WS, S, SN, NB, 5);                      \
        E_PAIR(P, WS, S, SN, NB, 6); E_PAIR(P, WS, S, SN, NB, 7);                      \
    } while (0)
    // the first step of a tile also loads the A fragments of tile KN into
    // set S2 (step J / 2, fragment J % 2), the last step issues the copies of
    // tile KN into stage S2: one memory instruction per MFMA pair.  (Eight
    // loads per wave in a row, 32 per CU at once, held up the MFMAs queued
    // behind them; two per pair, loads and copies in the same step, too.)
#define E_PAIR_LOADW(P, WS, S, SN, NB, J, S2, KN)                                      \
    do {                                                                               \
        E_MMA(P, WS, S, J);                                                            \
        X[1 - (P)][J] = read_x(SN, NB, J);                                             \
        WA[S2][(J) / 2][(J) % 2] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128( \
            wr, wgoff[(J) % 2] + 1024 * ((J) / 2), (KN) * 4096, 0));                   \
        __builtin_amdgcn_sched_barrier(0);                                             \
    } while (0)
#define E_PAIR_ISSUE(P, WS, S, SN, NB, J, S2, KN)                                      \
    do {                                                                               \
        E_MMA(P, WS, S, J);                                                            \
        X[1 - (P)][J] = read_x(SN, NB, J);                                             \
        issue_x(S2, KN, J);                                                            \
        __builtin_amdgcn_sched_barrier(0);                                             \
    } while (0)

    // One 64-k chunk: chunk kc in stage ST, its A fragments in set ST
    // (constants).  Step 0 loads the A fragments of chunk kc + 2 into set
    // (ST + 2) % 3, which chunk kc - 1 used.  The barrier before step 3: every
    // load of this wave is complete (the copies of chunk kc + 1, issued a
    // chunk ago, and the A fragments of chunk kc + 2), so after the barrier
    // all of chunk kc + 1 is in LDS; and every wave has read its step-3
    // operands of stage ST, so the copies of chunk kc + 2 can go to stage
    // (ST + 2) % 3.  The wait is for every outstanding load, not for all but
    // the youngest: register loads issued after copies into LDS can complete
    // before them (waiting for all but the eight youngest let the barrier pass
    // early on cold data).
    auto tile_step = [&](auto st_c, int kc) {
        constexpr int ST = decltype(st_c)::value;
        constexpr int S1 = (ST + 1) % T2_NSTAGE, S2 = (ST + 2) % T2_NSTAGE;
        constexpr int so = ST * T2_XBYTES, sn = S1 * T2_XBYTES;
        const int kn = min(kc + 2, last);
        E_PAIR_LOADW(0, ST, 0, so, 1, 0, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 1, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 2, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 3, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 4, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 5, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 6, S2, kn);
        E_PAIR_LOADW(0, ST, 0, so, 1, 7, S2, kn);
        E_STEP(1, ST, 1, so, 2);
        E_STEP(0, ST, 2, so, 3);
        __builtin_amdgcn_s_waitcnt(VMCNT0);
        lds_barrier();
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 0, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 1, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 2, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 3, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 4, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 5, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 6, S2, kn);
        E_PAIR_ISSUE(1, ST, 3, sn, 0, 7, S2, kn);
    };

    int v = blockIdx.x;
    set_tile(v);
    set_lane_offsets();
    prologue_x();
    prologue_w();
    for (;;) {
        // wait for the tile's first copies (the second chunk's and the A
        // fragments may still be in flight; on later tiles also the previous
        // epilogue's stores)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) X[0][j] = read_x(0, 0, j);
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[f][j][e] = 0.f;

        int kc = kc_begin;
        for (; kc + T2_NSTAGE <= kc_end; kc += T2_NSTAGE) {
            tile_step(std::integral_constant<int, 0>{}, kc);
            tile_step(std::integral_constant<int, 1>{}, kc + 1);
            tile_step(std::integral_constant<int, 2>{}, kc + 2);
        }
        if (kc < kc_end) tile_step(std::integral_constant<int, 0>{}, kc);
        if (kc + 1 < kc_end) tile_step(std::integral_constant<int, 1>{}, kc + 1);
        // every copy and load of this tile has landed, and after the barrier
        // every wave is done reading the stages
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        const int t_m0 = m0, t_tn = tn, t_ks = ks;
        const int vn = v + (int)gridDim.x;
        const bool more = vn < total;
        if constexpr (OWN_EPI) {
            // the next tile's copies go out first (they need no registers
            // while the accumulators are stored), its A fragments after
            if (more) {
                set_tile(vn);
                set_lane_offsets();
                prologue_x();
            }
            tile_store_rows<EPI, 8, 2>(a, acc, t_m0, t_tn, wave, wave, lane, epi_lds);
            if (more) {
                set_lane_offsets();
                prologue_w();
            }
        } else {
            if constexpr (SPLIT)
                tile_store_partial<EPI, 8, 2>(a, acc, t_m0, t_tn, wave, lane, lds, t_ks);
            else
                tile_store_rows<EPI, 8, 2>(a, acc, t_m0, t_tn, wave, wave, lane, lds);
            if (more) {
                __syncthreads();          // the staging reads are done
                set_tile(vn);
                set_lane_offsets();
                prologue_x();
                prologue_w();
            }
        }
        if (!more) break;
        v = vn;
    }
#undef E_PAIR_ISSUE
#undef E_PAIR_LOADW
#undef E_STEP
#undef E_PAIR
#undef E_MMA
}

// Weight expansion for the two-pass path, written in the order the GEMM
// reads its A fragments: for channel tile tn, wave w, fragment f (tile rows
// 64w + 32f + r, r = lane % 32, as chosen by tile_row), 64-k chunk kc and
// MFMA step s, lane l holds the FP16 weights k = 64 kc + 32 (l / 32) + 8s ..
// +8 of its row: 16 bytes, lanes in order, 1 KB per fragment.  The chunks of
// one (tn, w, f) form a block of K / 64 + 1 chunks of 4 KB: the spare chunk
// keeps the blocks that concurrent workgroups read from sitting a power of
// two apart, which would map them onto the same memory channels.
// Workgroup (tn, g) expands chunks [2g, 2g + 2) of the 256 rows of channel
// tile tn (small workgroups, so that even a 4096 x 4096 weight spreads over
// 512 of them); a thread takes up to four (w, f, chunk, lane) units: 24
// contiguous packed bytes (32 indices) in, four 16-byte stores (one per
// step) out, each store instruction contiguous across the wave.  All four
// units' packed bytes are loaded before the first lookup.
constexpr int X_CHUNKS = 2;                       // chunks per expansion workgroup
constexpr int X_UNITS = 8 * X_CHUNKS * 64 / 256;  // units per thread

template <int EPI>
__global__ void __launch_bounds__(256)
lut6_expand_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ tables,
                   uint16_t* __restrict__ w16, int N, int K)
{
    __shared__ __attribute__((aligned(16))) uint16_t tab[16 * 64];
    const int tn = blockIdx.x, g = blockIdx.y;
    const int chunks = K / BK;
    const int row_bytes = K / 4 * 3;
    // the 16 tables of the tile: slot s = tile row / 16 (four entries per
    // thread, all loaded before the first store)
    uint16_t tv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = threadIdx.x + 256 * j;
        tv[j] = tables[(tile_row<EPI>(16 * (i >> 6), tn, N) / 16) * 64 + (i & 63)];
    }
    const int nch = min(X_CHUNKS, chunks - g * X_CHUNKS);
    // unit u = threadIdx.x + 256 i: lane u % 64, chunk (u / 64) % nch of the
    // group, fragment wf = (u / 64) / nch; past 512 nch units a thread
    // re-reads unit 0's bytes and stores nothing
    u32x2 q[X_UNITS][3];
    int trow[X_UNITS], dsto[X_UNITS];
#pragma unroll
    for (int i = 0; i < X_UNITS; ++i) {
        const int uu = threadIdx.x + 256 * i;
        const int u = uu < 8 * nch * 64 ? uu : 0;
        const int lane = u & 63, kl = (u >> 6) % nch, wf = (u >> 6) / nch;
        const int kc = g * X_CHUNKS + kl;
        trow[i] = 64 * (wf >> 1) + 32 * (wf & 1) + (lane & 31);
        const int row = tile_row<EPI>(trow[i], tn, N);
        const uint8_t* src = packed + (size_t)row * row_bytes + 48 * kc + 24 * (lane >> 5);
        // 8-byte aligned (rows are 48-byte multiples, the offset 48 kc + 24h)
        const u32x2* const qp = (const u32x2*)__builtin_assume_aligned(src, 8);
        q[i][0] = qp[0];
        q[i][1] = qp[1];
        q[i][2] = qp[2];
        dsto[i] = uu < 8 * nch * 64 ? (int)(((size_t)(tn * 8 + wf) * (chunks + 1) + kc) * 2048 + lane * 8) : -1;
    }
    // the table entries go to LDS once every load is in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) tab[threadIdx.x + 256 * j] = tv[j];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < X_UNITS; ++i) {
        if (dsto[i] < 0) continue;
        const uint32_t pw[6] = {q[i][0][0], q[i][0][1], q[i][1][0], q[i][1][1], q[i][2][0], q[i][2][1]};
        const uint16_t* const t = tab + 64 * (trow[i] >> 4);
        uint16_t* const dst = w16 + (size_t)dsto[i];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // indices 8 st .. 8 st + 7 of the 192-bit word
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int bit = 6 * (8 * st + j), wd = bit >> 5, o = bit & 31;
                const uint32_t lo = pw[wd] >> o;
                const uint32_t hi = (o > 26 && wd + 1 < 6) ? (pw[wd + 1] << (32 - o)) : 0u;
                e[j] = (lo | hi) & 63u;
            }
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = (uint32_t)t[e[2 * j]] | ((uint32_t)t[e[2 * j + 1]] << 16);
            *(u32x4*)(dst + st * 512) = out;
        }
    }
}

// int8 weight-only variant: the same fragment-order FP16 buffer as
// lut6_expand_kernel, from an int8 weight q [N, K] and one FP16 scale per
// row and block of 32 along K (qs [N, K/32]).  A unit (row, 64-k chunk, lane
// group h) is exactly one block: 32 int8 values and one scale, written as
// the FP16 value nearest to q * scale (exact in FP32: 8 by 11 significant
// bits, so the conversion to FP16 is the only rounding).
template <int EPI>
__global__ void __launch_bounds__(256)
lut6_int8_expand_kernel(const int8_t* __restrict__ q, const uint16_t* __restrict__ qs,
                        uint16_t* __restrict__ w16, int N, int K)
{
    const int tn = blockIdx.x, g = blockIdx.y;
    const int chunks = K / BK;
    const int nch = min(X_CHUNKS, chunks - g * X_CHUNKS);
    u32x4 v[X_UNITS][2];
    uint16_t sc[X_UNITS];
    int dsto[X_UNITS];
#pragma unroll
    for (int i = 0; i < X_UNITS; ++i) {
        const int uu = threadIdx.x + 256 * i;
        const int u = uu < 8 * nch * 64 ? uu : 0;
        const int lane = u & 63, kl = (u >> 6) % nch, wf = (u >> 6) / nch;
        const int kc = g * X_CHUNKS + kl;
        const int row = tile_row<EPI>(64 * (wf >> 1) + 32 * (wf & 1) + (lane & 31), tn, N);
        const int k0 = BK * kc + 32 * (lane >> 5);
        const u32x4* const src = (const u32x4*)(q + (size_t)row * K + k0);   // 32-byte aligned
        v[i][0] = src[0];
        v[i][1] = src[1];
        sc[i] = qs[(size_t)row * (K / 32) + k0 / 32];
        dsto[i] = uu < 8 * nch * 64 ? (int)(((size_t)(tn * 8 + wf) * (chunks + 1) + kc) * 2048 + lane * 8) : -1;
    }
#pragma unroll
    for (int i = 0; i < X_UNITS; ++i) {
        if (dsto[i] < 0) continue;
        const float s = (float)__builtin_bit_cast(_Float16, sc[i]);
        const uint32_t wd[8] = {v[i][0][0], v[i][0][1], v[i][0][2], v[i][0][3],
                                v[i][1][0], v[i][1][1], v[i][1][2], v[i][1][3]};
        uint16_t* const dst = w16 + (size_t)dsto[i];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            // values 8 st .. 8 st + 7 of the block: words 2 st, 2 st + 1
            u32x4 out;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t word = wd[2 * st + (j >> 1)];
                const int sh = 16 * (j & 1);
                const float a = (float)(int8_t)((word >> sh) & 0xFFu) * s;
                const float b = (float)(int8_t)((word >> (sh + 8)) & 0xFFu) * s;
                out[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
            }
            *(u32x4*)(dst + st * 512) = out;
        }
    }
}

// int8 weight-only variant, few tokens (L <= 192): the weight streams once
// from HBM straight into MFMA A fragments, with no expanded copy.  A
// workgroup owns 32 output rows (for silu(gate) * up: 16 gate rows and the
// matching 16 up rows) and 64 tokens over the whole K range; its four waves
// take a quarter of the 64-k chunks each and meet in LDS.  In a chunk, lane
// half h takes the 32 contiguous codes k0 + 32 h .. + 31 of its row, which
// are exactly one scale block, and step j of the four MFMA steps uses codes
// 8 j .. 8 j + 7 of them; the B fragments read the activations with the
// same k order from a per-wave LDS tile filled by whole-row loads (a
// fragment loaded straight from memory touches 32 rows per instruction).  A code becomes FP16 exactly (0x6400 | (q + 128) is
// 1152 + q; subtracting 1152 is exact) and one FP16 multiply by the scale
// rounds q * scale once, as the format defines.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 i8x4_to_f16x4(uint32_t w, f16x2_t sc)
{
    const uint32_t t = w ^ 0x80808080u;                     // q + 128 in each byte
    const uint32_t lo = (t & 0xFFu) | ((t & 0xFF00u) << 8) | 0x64006400u;
    const uint32_t hi = ((t >> 16) & 0xFFu) | ((t >> 8) & 0xFF0000u) | 0x64006400u;
    const f16x2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const f16x2_t a = (__builtin_bit_cast(f16x2_t, lo) - bias) * sc;
    const f16x2_t b = (__builtin_bit_cast(f16x2_t, hi) - bias) * sc;
    return u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

template <int EPI, bool SCALED>
__global__ void __launch_bounds__(256)
lut6_int8_stream_kernel(const uint16_t* __restrict__ x, const int8_t* __restrict__ q,
                        const uint16_t* __restrict__ qs, void* __restrict__ y, int L, int K, int N,
                        float in_scale, float inv_scale)
{
    __shared__ __attribute__((aligned(16))) float red[3][2][16][64];
    // per wave, two stages of a 64-token x 64-k activation tile (rows padded
    // to 144 B so that a fragment's 32 rows start on distinct banks)
    __shared__ __attribute__((aligned(16))) uint16_t xs[4][2][64][72];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, rl = lane & 31;
    const int tn = blockIdx.x, tm = blockIdx.y;
    // the lane's weight row
    int row;
    if constexpr (EPI == 2) {
        const int j = min(tn * 16 + (rl & 15), N / 2 - 1);
        row = rl < 16 ? j : N / 2 + j;
    } else {
        row = min(tn * 32 + rl, N - 1);
    }
    const int8_t* const qrow = q + (size_t)row * K + 32 * h;
    const uint16_t* const srow = qs + (size_t)row * (K / 32) + h;
    // activation pieces of this lane: token (lane + 64 i) / 8, 16 bytes at
    // k offset 8 ((lane + 64 i) % 8) of each chunk (whole 128-byte rows per
    // instruction)
    const uint16_t* xrow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        xrow[i] = x + (size_t)min(tm * 64 + ((lane + 64 * i) >> 3), L - 1) * K + 8 * (lane & 7);
    const int chunks = K / 64;
    const int c0 = wave * chunks / 4, c1 = (wave + 1) * chunks / 4;
    f32x16 acc[2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[f][r] = 0.0f;
    const _Float16 sh = (_Float16)in_scale;                        // a power of two: exact
    const f16x8 s8 = {sh, sh, sh, sh, sh, sh, sh, sh};
    // two register sets: chunk kc + 1's loads are in flight while chunk kc
    // is converted and multiplied
    struct Chunk {
        u32x4 w[2];
        u32x4 xr[8];
        uint16_t sc;
    };
    auto load = [&](Chunk& c, int kc) {
        c.w[0] = *(const u32x4*)(qrow + 64 * kc);
        c.w[1] = *(const u32x4*)(qrow + 64 * kc + 16);
        c.sc = srow[2 * kc];
#pragma unroll
        for (int i = 0; i < 8; ++i) c.xr[i] = *(const u32x4*)(xrow[i] + 64 * kc);
    };
    // the wave's own LDS tile: LDS instructions of one wave complete in
    // order, so no barrier is needed between its writes and reads
    auto stage = [&](const Chunk& c, int b) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4*)(&xs[wave][b][(lane + 64 * i) >> 3][8 * (lane & 7)]) = c.xr[i];
    };
    auto compute = [&](const Chunk& c, int b) {
        const _Float16 sc = __builtin_bit_cast(_Float16, c.sc);
        const f16x2_t sc2 = {sc, sc};
        const uint32_t wd[8] = {c.w[0][0], c.w[0][1], c.w[0][2], c.w[0][3],
                                c.w[1][0], c.w[1][1], c.w[1][2], c.w[1][3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x2 a0 = i8x4_to_f16x4(wd[2 * j], sc2), a1 = i8x4_to_f16x4(wd[2 * j + 1], sc2);
            const u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                f16x8 bv = *(const f16x8*)(&xs[wave][b][32 * f + rl][32 * h + 8 * j]);
                if constexpr (SCALED) bv = bv * s8;                  // fp16(x * s), exact or inf
                acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av), bv, acc[f],
                                                                0, 0, 0);
            }
        }
    };
    // chunks in pairs with no branch inside the loop (the load of the chunk
    // after next is clamped to the last one: at most one spare load per
    // wave), an odd last chunk after it.  (With the second chunk's work
    // under a branch, the accumulators went through vector registers and
    // back on every pass.)
    Chunk ca, cb;
    if (c0 < c1) {
        load(ca, c0);
        int kc = c0;
        for (; kc + 1 < c1; kc += 2) {
            load(cb, kc + 1);
            stage(ca, 0);
            compute(ca, 0);
            load(ca, min(kc + 2, c1 - 1));
            stage(cb, 1);
            compute(cb, 1);
        }
        if (kc < c1) {
            stage(ca, 0);
            compute(ca, 0);
        }
    }
    // waves 1..3 hand their sums to wave 0, which adds them in wave order
    if (wave > 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[wave - 1][f][r][lane] = acc[f][r];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[f][r] += red[w][f][r][lane];
    // accumulator (f, r) of this lane: row 8 (r / 4) + 4 h + r % 4 of the
    // tile, token tm * 64 + 32 f + rl
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int tok = tm * 64 + 32 * f + rl;
        if (tok >= L) continue;
        if constexpr (EPI == 2) {
            const int n_out = N / 2;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int ch = tn * 16 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (ch < n_out)
                    ((_Float16*)y)[(size_t)tok * n_out + ch] =
                        (_Float16)(silu_f32(acc[f][r] * inv_scale) * (acc[f][r + 8] * inv_scale));
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ch = tn * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (ch >= N) continue;
                const float v = acc[f][r] * inv_scale;
                if constexpr (EPI == 0) ((float*)y)[(size_t)tok * N + ch] = v;
                else ((_Float16*)y)[(size_t)tok * N + ch] = (_Float16)v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for few tokens (L <= 192).  Every weight serves at
// most 192 tokens here, so streaming the packed weight once from HBM, and
// the activations from L2, bound the kernel.  A workgroup owns 32 channels
// (one A fragment: two tables) x 64 tokens (two B fragments) over the whole
// K range, so that the outputs leave the kernel finished: no partial sums,
// no second kernel (a launch costs more than the whole weight read at this
// size).  With 64 tokens per tile the activation re-reads from L2 (one per
// 32 channels) stay within what 256 CUs draw from their L2s while the packed
// weight streams once, and the A fragment of each MFMA step serves two
// MFMAs.  The four waves split K four ways and meet in LDS at the end.
//
// Lookups use pair tables: entry i0 | i1 << 6 of a 4096-word LDS table holds
// T[i0] and T[i1], so two consecutive k of one channel cost one 12-bit field
// extraction (shift, v_and_or_b32) and one ds_read_b32, and the word is
// already the packed FP16 pair an MFMA fragment takes.  Activations go
// through per-wave LDS rings by buffer->LDS copies (whole 128-byte rows per
// instruction), four 64-k chunks in flight per wave; each ring slot is its
// own LDS array, so the compiler's wait for a slot's copy does not also wait
// for the copies into the other slots.
//
// Few tiles (small N or L) split K into slices with FP32 partial planes
// added by lut6_reduce_kernel in a fixed order.
// ---------------------------------------------------------------------------
constexpr int S_BN = 32, S_BM = 64;
constexpr int S_WAVE_SLOT = 8192;        // one 64-k chunk of 64 token rows
constexpr int S_SLOT = 4 * S_WAVE_SLOT;  // one ring slot of all four waves
constexpr int S_MIN_CHUNKS = 16;         // fewest 64-k chunks per K slice

template <int EPI, bool SCALED, bool SPLIT, bool F16>
__global__ void __launch_bounds__(256, 1)
lut6_stream_kernel(GemmArgs a)
{
    // F16: every wave has exactly 16 chunks (K slice of 4096); all their
    // packed words are loaded up front, so that the copies of activations,
    // which hit in L2, never wait behind a packed-word load from HBM in
    // the wave's in-order load queue.
    //
    // pair tables (slot s: tile rows 16s .. 16s+15), then the four ring slots
    // (the largest alignment: the pair tables go first, at LDS address 0, so
    // a lookup's offset is its address and needs no add)
    __shared__ __attribute__((aligned(16384))) uint8_t s_pair[2 * 16384];
    __shared__ __attribute__((aligned(1024))) uint8_t s_x0[S_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t s_x1[S_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t s_x2[S_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t s_x3[S_SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, h = lane >> 5;
    const int K = a.K, N = a.N, L = a.L;
    const int row_bytes = K / 4 * 3;

    // one-dimensional grid; after the remap consecutive indices (one XCD)
    // are the token tiles, then the K slices, of one channel tile
    const int splits = gridDim.x / a.n_tiles;
    const int r = xcd_remap(blockIdx.x, gridDim.x);
    const int t = r / splits, split = r % splits;
    const int tm = t % a.tiles_m, tn = t / a.tiles_m;
    const int m0 = tm * S_BM;
    const int kc_begin = split * a.k_chunks_per_split;
    const int kc_end = min(K / BK, kc_begin + a.k_chunks_per_split);
    const int per_wave = (kc_end - kc_begin + 3) / 4;
    // k quarter of this wave, rotated by tile so that the workgroups of one
    // XCD do not all read the same activation chunk at the same time
    const int quarter = (wave + r) & 3;
    const int w_begin = min(kc_begin + quarter * per_wave, kc_end);
    const int nch = F16 ? 16 : min(w_begin + per_wave, kc_end) - w_begin;
    const int kc_last = max(w_begin + nch - 1, 0);

    // global weight row of tile row i (clamped into range; such rows are
    // computed on a copy of the last row and never stored): for SiLU, rows
    // 0..15 are gate channels and 16..31 the matching up channels
    auto trow = [&](int i) -> int {
        if constexpr (EPI == 2) {
            const int j = min(tn * (S_BN / 2) + (i & 15), N / 2 - 1);
            return i >= 16 ? N / 2 + j : j;
        } else {
            return min(tn * S_BN + i, N - 1);
        }
    };

    // Table entries for the pair tables, loaded first: this thread builds
    // words 16 tid .. 16 tid + 15 of both slots, whose low halves are
    // entries 16 (tid % 4) .. +15 and whose high half is entry tid / 4.
    u32x4 tlo[2][2];
    uint32_t thi[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint16_t* T = a.tables + (size_t)(trow(16 * s) / 16) * 64;
        tlo[s][0] = *(const u32x4*)(T + 16 * (tid & 3));
        tlo[s][1] = *(const u32x4*)(T + 16 * (tid & 3) + 8);
        thi[s] = T[tid >> 2];
    }

    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.x, (short)0, (int)((size_t)L * K * 2), RAW_BUFFER_WORD3);
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)a.packed, (short)0, (int)((size_t)N * row_bytes), RAW_BUFFER_WORD3);
    const int poff = trow(r32) * row_bytes + 24 * h;
    // activation copies: instruction i fills ring rows 8i .. 8i+7, lane l
    // row 8i + l / 8, position l % 8, which holds the row's 16-byte piece
    // (l % 8) ^ ((row >> 1) & 7)
    int xg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * i + (lane >> 3);
        xg[i] = min(m0 + row, L - 1) * (K * 2) + (((lane & 7) ^ ((row >> 1) & 7)) << 4);
    }
    // this lane's B-fragment pieces: token 32j + r32, piece 4h + s (lane
    // group h takes k 32h .. 32h + 31 of the chunk, as for the weights)
    int xo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xo[s] = wave * S_WAVE_SLOT + r32 * 128 + (((4 * h + s) ^ ((r32 >> 1) & 7)) << 4);

    auto slot_base = [&](auto sc) -> uint8_t* {
        constexpr int SL = decltype(sc)::value;
        return SL == 0 ? s_x0 : SL == 1 ? s_x1 : SL == 2 ? s_x2 : s_x3;
    };
    // copies and packed words of chunk ch; past the range (only in the
    // prologue) a valid chunk is re-read and never used
    auto copy_x = [&](int ch, auto sc) {
        uint8_t* const st = slot_base(sc) + wave * S_WAVE_SLOT;
        const int kc = min(w_begin + ch, kc_last);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(st + i * 1024), 16, xg[i],
                                                     kc * (BK * 2), 0, 0);
    };
    uint32_t PW[4][6];
    auto load_pw = [&](int ch, auto sc) {
        constexpr int SL = decltype(sc)::value;
        const int kc = min(w_begin + ch, kc_last);
        const u32x4 q4 = __builtin_amdgcn_raw_buffer_load_b128(pr, poff, kc * 48, 0);
        const u32x2 q2 = __builtin_amdgcn_raw_buffer_load_b64(pr, poff + 16, kc * 48, 0);
        PW[SL][0] = q4[0]; PW[SL][1] = q4[1]; PW[SL][2] = q4[2]; PW[SL][3] = q4[3];
        PW[SL][4] = q2[0]; PW[SL][5] = q2[1];
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    // F16: packed words of all 16 chunks, then the copies of chunks 0..3
    uint32_t P16[F16 ? 16 : 1][6];
    auto load_p16 = [&](auto cc) {
        constexpr int C = decltype(cc)::value;
        const int kc = w_begin + C;
        const u32x4 q4 = __builtin_amdgcn_raw_buffer_load_b128(pr, poff, kc * 48, 0);
        const u32x2 q2 = __builtin_amdgcn_raw_buffer_load_b64(pr, poff + 16, kc * 48, 0);
        P16[C][0] = q4[0]; P16[C][1] = q4[1]; P16[C][2] = q4[2]; P16[C][3] = q4[3];
        P16[C][4] = q2[0]; P16[C][5] = q2[1];
    };
    if constexpr (F16) {
        // the first four chunks' words and copies lead, so the loop can
        // start while the other twelve chunks' words stream in behind them
        load_p16(std::integral_constant<int, 0>{});  load_p16(std::integral_constant<int, 1>{});
        load_p16(std::integral_constant<int, 2>{});  load_p16(std::integral_constant<int, 3>{});
        copy_x(0, C0{});
        copy_x(1, C1{});
        copy_x(2, C2{});
        copy_x(3, C3{});
        load_p16(std::integral_constant<int, 4>{});  load_p16(std::integral_constant<int, 5>{});
        load_p16(std::integral_constant<int, 6>{});  load_p16(std::integral_constant<int, 7>{});
        load_p16(std::integral_constant<int, 8>{});  load_p16(std::integral_constant<int, 9>{});
        load_p16(std::integral_constant<int, 10>{}); load_p16(std::integral_constant<int, 11>{});
        load_p16(std::integral_constant<int, 12>{}); load_p16(std::integral_constant<int, 13>{});
        load_p16(std::integral_constant<int, 14>{}); load_p16(std::integral_constant<int, 15>{});
    } else {
        // every prologue load is unconditional, so the main loop is entered
        // with the same loads in flight, in the same order, as it leaves
        // each iteration (the compiler's waits stay exact)
        load_pw(0, C0{});
        copy_x(0, C0{});
        load_pw(1, C1{});
        copy_x(1, C1{});
        load_pw(2, C2{});
        copy_x(2, C2{});
        load_pw(3, C3{});
        copy_x(3, C3{});
    }

    // pair tables: word p of slot s = T[p % 64] | T[p / 64] << 16
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t hi = thi[s] << 16;
        uint32_t wv[16];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const uint32_t lo2 = tlo[s][d >> 2][d & 3];
            wv[2 * d] = (lo2 & 0xffffu) | hi;
            wv[2 * d + 1] = (lo2 >> 16) | hi;
        }
        u32x4* dst = (u32x4*)(s_pair + s * 16384 + tid * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = u32x4{wv[4 * q], wv[4 * q + 1], wv[4 * q + 2], wv[4 * q + 3]};
    }
    // the pair tables are the only LDS data shared between waves (each wave
    // waits for its own ring copies): a plain barrier after the stores
    __builtin_amdgcn_s_waitcnt(LGKMCNT0);
    lds_barrier();

    // pair table of this lane's channel row
    const uint32_t tab = (uint32_t)((r32 >> 4) * 16384);
    // A fragment of step S from packed words P
    auto gather = [&](const uint32_t (&p)[6], auto stc) -> f16x8 {
        constexpr int S = decltype(stc)::value;
        const u32x4 d = {*(const uint32_t*)(s_pair + pair_off<48 * S + 0>(p, tab)),
                         *(const uint32_t*)(s_pair + pair_off<48 * S + 12>(p, tab)),
                         *(const uint32_t*)(s_pair + pair_off<48 * S + 24>(p, tab)),
                         *(const uint32_t*)(s_pair + pair_off<48 * S + 36>(p, tab))};
        return __builtin_bit_cast(f16x8, d);
    };

    f32x16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

    if constexpr (F16) {
        // chunk C computes on fragments read during chunk C - 1 (register
        // set C % 2).  Its four MFMA steps each carry a share of the next
        // chunk's reads (B fragments in steps 0 and 1, then each step's A
        // gathers) and two of the copies of chunk C + 4 into its slot, so
        // the MFMAs run while the reads and copies are in flight.  At the
        // start of chunk C its B reads are complete (LDS returns in order:
        // at most the twelve gathers issued after them are outstanding), so
        // its slot can be refilled.
        f16x8 A[2][4], B[2][2][4];
        auto fetch = [&](auto cc) __attribute__((always_inline)) {
            constexpr int C = decltype(cc)::value, RS = C & 1;
            const uint8_t* const st = slot_base(std::integral_constant<int, C & 3>{});
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) B[RS][j][s] = *(const f16x8*)(st + 4096 * j + xo[s]);
            A[RS][0] = gather(P16[C], C0{});
            A[RS][1] = gather(P16[C], C1{});
            A[RS][2] = gather(P16[C], C2{});
            A[RS][3] = gather(P16[C], C3{});
        };
        // B fragments of steps 2h, 2h + 1 of chunk C
        auto fetch_b = [&](auto cc, auto hc) __attribute__((always_inline)) {
            constexpr int C = decltype(cc)::value, RS = C & 1, H = decltype(hc)::value;
            const uint8_t* const st = slot_base(std::integral_constant<int, C & 3>{});
#pragma unroll
            for (int s = 2 * H; s < 2 * H + 2; ++s)
#pragma unroll
                for (int j = 0; j < 2; ++j) B[RS][j][s] = *(const f16x8*)(st + 4096 * j + xo[s]);
        };
        // copies i and i + 1 of chunk ch into slot SL
        auto copy_x2 = [&](int ch, auto sc, int i) __attribute__((always_inline)) {
            uint8_t* const st = slot_base(sc) + wave * S_WAVE_SLOT;
            const int kc = min(w_begin + ch, kc_last);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(st + (i + u) * 1024), 16, xg[i + u],
                                                         kc * (BK * 2), 0, 0);
        };
        auto scale_b = [&](auto rc, int s) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;
#pragma unroll
            for (int j = 0; j < 2; ++j) B[R][j][s] = B[R][j][s] * a.scale;
        };
        auto step16 = [&](auto cc) __attribute__((always_inline)) {
            constexpr int C = decltype(cc)::value, RS = C & 1, NX = (C + 1) & 1;
            constexpr bool NEXT = C + 1 < 16, COPY = C + 4 < 16;
            using SL = std::integral_constant<int, C & 3>;
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(LGKMCNT12);
            __builtin_amdgcn_sched_barrier(0);
            auto mma = [&](int s) __attribute__((always_inline)) {
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[RS][s], B[RS][0][s], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[RS][s], B[RS][1][s], acc[1], 0, 0, 0);
            };
            // step 0
            mma(0);
            if constexpr (SCALED) scale_b(std::integral_constant<int, RS>{}, 1);
            if constexpr (NEXT) fetch_b(std::integral_constant<int, C + 1>{}, C0{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (NEXT) A[NX][0] = gather(P16[NEXT ? C + 1 : C], C0{});
            if constexpr (COPY) copy_x2(C + 4, SL{}, 0);
            __builtin_amdgcn_sched_barrier(0);
            // step 1
            mma(1);
            if constexpr (SCALED) scale_b(std::integral_constant<int, RS>{}, 2);
            if constexpr (NEXT) fetch_b(std::integral_constant<int, C + 1>{}, C1{});
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (NEXT) A[NX][1] = gather(P16[NEXT ? C + 1 : C], C1{});
            if constexpr (COPY) copy_x2(C + 4, SL{}, 2);
            __builtin_amdgcn_sched_barrier(0);
            // step 2
            mma(2);
            if constexpr (SCALED) scale_b(std::integral_constant<int, RS>{}, 3);
            if constexpr (NEXT) A[NX][2] = gather(P16[NEXT ? C + 1 : C], C2{});
            if constexpr (COPY) copy_x2(C + 4, SL{}, 4);
            __builtin_amdgcn_sched_barrier(0);
            // step 3
            mma(3);
            if constexpr (SCALED && NEXT) scale_b(std::integral_constant<int, NX>{}, 0);
            if constexpr (NEXT) A[NX][3] = gather(P16[NEXT ? C + 1 : C], C3{});
            if constexpr (COPY) copy_x2(C + 4, SL{}, 6);
        };
        fetch(C0{});
        if constexpr (SCALED) scale_b(std::integral_constant<int, 0>{}, 0);
        step16(std::integral_constant<int, 0>{});  step16(std::integral_constant<int, 1>{});
        step16(std::integral_constant<int, 2>{});  step16(std::integral_constant<int, 3>{});
        step16(std::integral_constant<int, 4>{});  step16(std::integral_constant<int, 5>{});
        step16(std::integral_constant<int, 6>{});  step16(std::integral_constant<int, 7>{});
        step16(std::integral_constant<int, 8>{});  step16(std::integral_constant<int, 9>{});
        step16(std::integral_constant<int, 10>{}); step16(std::integral_constant<int, 11>{});
        step16(std::integral_constant<int, 12>{}); step16(std::integral_constant<int, 13>{});
        step16(std::integral_constant<int, 14>{}); step16(std::integral_constant<int, 15>{});
    } else {
    // chunk c on ring slot SL = c % 4: its B fragments leave the slot, which
    // then takes chunk c + 4 when PF; its A fragments are gathered one MFMA
    // step ahead (step 0 during the previous chunk's step 3, from the next
    // slot's packed words, possibly of a chunk past the range: a harmless
    // lookup); once its steps are gathered, the packed words of chunk c + 4
    // (clamped) replace it
    f16x8 Wc = gather(PW[0], C0{});
    auto chunk = [&](int c, auto sc, auto pf) __attribute__((always_inline)) {
        constexpr int SL = decltype(sc)::value, NS = (SL + 1) & 3;
        const uint8_t* const st = slot_base(sc);
        __builtin_amdgcn_sched_barrier(0);
        f16x8 X[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int s = 0; s < 4; ++s) X[j][s] = *(const f16x8*)(st + 4096 * j + xo[s]);
        if constexpr (decltype(pf)::value) {
            // the slot's reads have completed before the copy may land
            __builtin_amdgcn_s_waitcnt(LGKMCNT0);
            copy_x(c + 4, sc);
        }
        if constexpr (SCALED) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int s = 0; s < 4; ++s) X[j][s] = X[j][s] * a.scale;
        }
        // the scheduling barriers keep each step's lookups in that step, so
        // no lookup (and its wait for packed words) is hoisted ahead
        f16x8 Wn;
#define S8_STEP(S, NEXT)                                                                 \
        __builtin_amdgcn_sched_barrier(0);                                               \
        Wn = NEXT;                                                                       \
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Wc, X[0][S], acc[0], 0, 0, 0);   \
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Wc, X[1][S], acc[1], 0, 0, 0);   \
        Wc = Wn;
        S8_STEP(0, gather(PW[SL], C1{}));
        S8_STEP(1, gather(PW[SL], C2{}));
        S8_STEP(2, gather(PW[SL], C3{}));
        S8_STEP(3, gather(PW[NS], C0{}));
#undef S8_STEP
        __builtin_amdgcn_sched_barrier(0);
        load_pw(c + 4, sc);
        __builtin_amdgcn_sched_barrier(0);
    };
    using Y = std::true_type;
    using Nn = std::false_type;
    // G groups of four chunks, then R more: the groups before the last copy
    // all four successors, the last one only the R that exist
    const int G = nch >> 2, R = nch & 3;
    for (int g = 0; g + 1 < G; ++g) {
        chunk(4 * g + 0, C0{}, Y{});
        chunk(4 * g + 1, C1{}, Y{});
        chunk(4 * g + 2, C2{}, Y{});
        chunk(4 * g + 3, C3{}, Y{});
    }
    if (G > 0) {
        const int c = 4 * (G - 1);
        switch (R) {
        case 0: chunk(c, C0{}, Nn{}); chunk(c + 1, C1{}, Nn{}); chunk(c + 2, C2{}, Nn{}); chunk(c + 3, C3{}, Nn{}); break;
        case 1: chunk(c, C0{}, Y{}); chunk(c + 1, C1{}, Nn{}); chunk(c + 2, C2{}, Nn{}); chunk(c + 3, C3{}, Nn{}); break;
        case 2: chunk(c, C0{}, Y{}); chunk(c + 1, C1{}, Y{}); chunk(c + 2, C2{}, Nn{}); chunk(c + 3, C3{}, Nn{}); break;
        default: chunk(c, C0{}, Y{}); chunk(c + 1, C1{}, Y{}); chunk(c + 2, C2{}, Y{}); chunk(c + 3, C3{}, Nn{}); break;
        }
    }
    {
        const int c = 4 * G;
        switch (R) {
        case 1: chunk(c, C0{}, Nn{}); break;
        case 2: chunk(c, C0{}, Nn{}); chunk(c + 1, C1{}, Nn{}); break;
        case 3: chunk(c, C0{}, Nn{}); chunk(c + 1, C1{}, Nn{}); chunk(c + 2, C2{}, Nn{}); break;
        default: break;
        }
    }
    }

    // k quarters meet in slot 0 of the ring, [token fragment j][group q]
    // [k quarter][lane] of f32x4; wave 2j + (q & 1) owns (j, q) and adds the
    // four quarters in k order.  Every copy has landed and every wave is
    // done with its ring before the exchange.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x4* const xa = (f32x4*)s_x0;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (2 * j + (q & 1) != wave)
                xa[((j * 4 + q) * 4 + quarter) * 64 + lane] =
                    f32x4{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
    __syncthreads();
    auto finish = [&](auto wc) {
        constexpr int w = decltype(wc)::value, j = w >> 1, q0 = w & 1;
        f32x4 v[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = q0 + 2 * u;
            const f32x4 own = {acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const f32x4 o = kq == quarter ? own : xa[((j * 4 + q) * 4 + kq) * 64 + lane];
                v[u] = kq == 0 ? o : v[u] + o;
            }
        }
        // v[u]: rows 8 (q0 + 2u) + 4h + 0..3 of the fragment, token 32j + r32
        const int tok = m0 + 32 * j + r32;
        if (tok >= L) return;
        if constexpr (EPI == 2) {
            const int c = tn * (S_BN / 2) + 8 * q0 + 4 * h;   // gate rows, up rows 16 further
            if constexpr (SPLIT) {
                float* const pp = a.partial + (size_t)split * L * N + (size_t)tok * N;
                *(f32x4*)(pp + c) = v[0];
                *(f32x4*)(pp + N / 2 + c) = v[1];
            } else {
                f16x4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hv[e] = (_Float16)(silu_f32(v[0][e] * a.inv_scale) * (v[1][e] * a.inv_scale));
                *(f16x4*)((_Float16*)a.y + (size_t)tok * (N / 2) + c) = hv;
            }
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int c = tn * S_BN + 8 * (q0 + 2 * u) + 4 * h;
                if (c >= N) continue;
                if constexpr (SPLIT) {
                    *(f32x4*)(a.partial + (size_t)split * L * N + (size_t)tok * N + c) = v[u];
                } else if constexpr (EPI == 0) {
                    *(f32x4*)((float*)a.y + (size_t)tok * N + c) = v[u] * a.inv_scale;
                } else {
                    const f32x4 o = v[u] * a.inv_scale;
                    *(f16x4*)((_Float16*)a.y + (size_t)tok * N + c) =
                        f16x4{(_Float16)o[0], (_Float16)o[1], (_Float16)o[2], (_Float16)o[3]};
                }
            }
        }
    };
    switch (wave) {
    case 0: finish(std::integral_constant<int, 0>{}); break;
    case 1: finish(std::integral_constant<int, 1>{}); break;
    case 2: finish(std::integral_constant<int, 2>{}); break;
    default: finish(std::integral_constant<int, 3>{}); break;
    }
}

// Fixed-order sum of split-K partials, then the epilogue.  One thread per
// four consecutive output columns.
template <int EPI>
__global__ void __launch_bounds__(256)
lut6_reduce_kernel(const float* __restrict__ partial, void* __restrict__ y, int L, int N,
                   int splits, float inv_scale)
{
    const int n_out = EPI == 2 ? N / 2 : N;
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total4 = (int64_t)L * n_out / 4;
    if (i4 >= total4) return;
    const int tok = (int)(i4 / (n_out / 4));
    const int c = (int)(i4 % (n_out / 4)) * 4;
    const size_t plane = (size_t)L * N;
    // slices four at a time, loaded before the adds (one wait per four);
    // past the last slice a valid re-read, for which zero is added
    auto sum = [&](size_t off) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; s += 4) {
            f32x4 b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                b[i] = *(const f32x4*)(partial + (size_t)min(s + i, splits - 1) * plane + off);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) v += s + i < splits ? b[i] : z;
        }
        return v;
    };
    if constexpr (EPI == 2) {
        f32x4 g = sum((size_t)tok * N + c), u = sum((size_t)tok * N + N / 2 + c);
        g *= inv_scale;
        u *= inv_scale;
        f16x4 h;
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = (_Float16)(silu_f32(g[r]) * u[r]);
        *(f16x4*)((_Float16*)y + (size_t)tok * n_out + c) = h;
    } else {
        f32x4 v = sum((size_t)tok * N + c);
        v *= inv_scale;
        if constexpr (EPI == 0) {
            *(f32x4*)((float*)y + (size_t)tok * N + c) = v;
        } else {
            f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
            *(f16x4*)((_Float16*)y + (size_t)tok * N + c) = h;
        }
    }
}

// Dequantize 16 channels (one table) per workgroup: w[n, k] = T[n/16][idx].
__global__ void __launch_bounds__(256)
lut6_dequant_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ tables,
                    uint16_t* __restrict__ w, int N, int K)
{
    __shared__ __attribute__((aligned(16))) uint16_t tab[64];
    const int grp = blockIdx.x;
    if (threadIdx.x < 64) tab[threadIdx.x] = tables[grp * 64 + threadIdx.x];
    __syncthreads();
    const int per_row = K / 16;
    const int row_bytes = K / 4 * 3;
    for (int item = threadIdx.x; item < 16 * per_row; item += 256) {
        const int n = grp * 16 + item / per_row;
        const int j = item % per_row;
        const uint32_t* q = (const uint32_t*)(packed + (size_t)n * row_bytes + 12 * j);
        f16x8 lo, hi;
        gather16(q[0], q[1], q[2], tab, lo, hi);
        f16x8* dst = (f16x8*)(w + (size_t)n * K + 16 * j);
        dst[0] = lo;
        dst[1] = hi;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};

// workspace kinds: split-K partial sums, expanded FP16 weight (2: the
// attention's key-split partials, lut6_attention.hip)
enum { WS_PARTIAL = 0, WS_EXPANDED = 1 };

std::mutex g_ws_mutex;
std::map<std::tuple<int, uintptr_t, int>, Workspace> g_ws;   // key: (device, stream, kind)

int workspace_for(hipStream_t stream, int kind, size_t bytes, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LUT6_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& w = g_ws[std::make_tuple(dev, (uintptr_t)stream, kind)];
    if (w.bytes < bytes) {
        // grown in stream order, without stopping the host: the old buffer
        // is released once the work already enqueued on this stream (which
        // may still use it) is done, and the new one is valid for the work
        // enqueued after this call
        if (w.ptr) {
            if (hipFreeAsync(w.ptr, stream) != hipSuccess) return LUT6_E_DEVICE;
            w.ptr = nullptr;
            w.bytes = 0;
        }
        void* p = nullptr;
        if (hipMallocAsync(&p, bytes, stream) != hipSuccess) return LUT6_E_DEVICE;
        w.ptr = p;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return LUT6_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

struct Plan {
    int kind;      // 0 = small-L split-K tiles, 1 = large tiles
    int splits;
};

int launch_reduce(const GemmArgs& a, int epi, int splits, hipStream_t stream)
{
    const int n_out = epi == 2 ? a.N / 2 : a.N;
    const int64_t total4 = (int64_t)a.L * n_out / 4;
    dim3 rgrid((unsigned)((total4 + 255) / 256));
    switch (epi) {
    case 0: hipLaunchKernelGGL(lut6_reduce_kernel<0>, rgrid, dim3(256), 0, stream, a.partial, a.y, a.L, a.N, splits, a.inv_scale); break;
    case 1: hipLaunchKernelGGL(lut6_reduce_kernel<1>, rgrid, dim3(256), 0, stream, a.partial, a.y, a.L, a.N, splits, a.inv_scale); break;
    default: hipLaunchKernelGGL(lut6_reduce_kernel<2>, rgrid, dim3(256), 0, stream, a.partial, a.y, a.L, a.N, splits, a.inv_scale); break;
    }
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}

// Workgroups of the persistent expanded GEMM: one per CU (a multiple of the
// 8 XCDs, so each workgroup keeps its XCD's tiles).
constexpr int PERSIST_WGS = 256;

// Launch the 256 x 256 tile kernel, fused (grid: tiles x K slices) or on the
// expanded weight (persistent: at most PERSIST_WGS workgroups walk the tiles).
template <bool SPLIT>
void launch_tiles_t(const GemmArgs& a, bool two_pass, int epilogue, bool scaled, dim3 grid, hipStream_t stream)
{
    const dim3 block(256);
    const int sel = epilogue * 2 + (scaled ? 1 : 0);
    if (two_pass) {
        const int64_t total = (int64_t)grid.x * grid.y;
        grid = dim3((unsigned)(total < PERSIST_WGS ? total : PERSIST_WGS));
        switch (sel) {
        case 0: hipLaunchKernelGGL((lut6_expanded_gemm_kernel<0, false, SPLIT>), grid, block, 0, stream, a); break;
        case 1: hipLaunchKernelGGL((lut6_expanded_gemm_kernel<0, true, SPLIT>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((lut6_expanded_gemm_kernel<1, false, SPLIT>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((lut6_expanded_gemm_kernel<1, true, SPLIT>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((lut6_expanded_gemm_kernel<2, false, SPLIT>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((lut6_expanded_gemm_kernel<2, true, SPLIT>), grid, block, 0, stream, a); break;
        }
    } else {
        switch (sel) {
        case 0: hipLaunchKernelGGL((lut6_tile256_kernel<0, false, SPLIT>), grid, block, 0, stream, a); break;
        case 1: hipLaunchKernelGGL((lut6_tile256_kernel<0, true, SPLIT>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((lut6_tile256_kernel<1, false, SPLIT>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((lut6_tile256_kernel<1, true, SPLIT>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((lut6_tile256_kernel<2, false, SPLIT>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((lut6_tile256_kernel<2, true, SPLIT>), grid, block, 0, stream, a); break;
        }
    }
}

void launch_tiles(const GemmArgs& a, bool two_pass, int epilogue, bool scaled, bool split, dim3 grid,
                  hipStream_t stream)
{
    if (split) launch_tiles_t<true>(a, two_pass, epilogue, scaled, grid, stream);
    else launch_tiles_t<false>(a, two_pass, epilogue, scaled, grid, stream);
}

// Which kernels lut6_linear runs for a (valid) shape: the weight-streaming
// kernel for few tokens, the fused tile kernel, or weight expansion plus the
// FP16 GEMM for many tokens (when the expanded weight fits 31-bit offsets).
constexpr int STREAM_MAX_L = 192;   // the weight-streaming kernels up to this many tokens

int choose_path(int64_t L, int64_t K, int64_t N, int epilogue)
{
    if (L <= STREAM_MAX_L) return LUT6_PATH_STREAM;
    if (L < (K >= DEEP_K ? EXPAND_MIN_L_DEEP_K : EXPAND_MIN_L)) return LUT6_PATH_FUSED;
    const int64_t n_half = epilogue == 2 ? N / 2 : N;
    const int64_t bn_cov = epilogue == 2 ? 128 : 256;
    const int64_t tiles_n = (n_half + bn_cov - 1) / bn_cov;
    const size_t w16_bytes = (size_t)tiles_n * 8 * (K / BK + 1) * 4096;
    return w16_bytes <= (size_t)INT32_MAX ? LUT6_PATH_EXPANDED : LUT6_PATH_FUSED;
}

}  // namespace

extern "C" int lut6_linear_path(int64_t L, int64_t K, int64_t N, int epilogue)
{
    if (L < 0 || K <= 0 || N <= 0 || K % 64 || N % 16) return -LUT6_E_SHAPE;
    if (L > INT32_MAX || K > INT32_MAX || N > INT32_MAX) return -LUT6_E_SHAPE;
    if (epilogue < 0 || epilogue > 2) return -LUT6_E_EPILOGUE;
    if (epilogue == LUT6_EPI_SILU_MUL_F16 && N % 32) return -LUT6_E_SHAPE;
    if ((size_t)L * K * 2 >= ((size_t)1 << 31) || (size_t)N * (K / 4 * 3) >= ((size_t)1 << 31))
        return -LUT6_E_SHAPE;
    return choose_path(L, K, N, epilogue);
}

namespace {

// Everything lut6_linear decides for one valid shape before it launches.
struct LinearPlan {
    int path;                 // lut6_path
    int splits;               // K slices (1: none)
    int tiles, tiles_m, tiles_n;
    int k_chunks_per_split;
    bool f16;                 // stream path: every wave holds exactly 16 chunks
    size_t w16_bytes;         // expanded weight (0 unless LUT6_PATH_EXPANDED)
    size_t partial_bytes;     // split-K partial sums (0 unless splits > 1)
};

// Host checks of lut6_linear, in the order the header lists them.
int check_linear(const void* x, const uint8_t* packed, const void* tables, void* y, int64_t L,
                 int64_t K, int64_t N, float in_scale, int epilogue)
{
    if (!x || !packed || !tables || !y) return LUT6_E_NULL;
    if (L < 0 || K <= 0 || N <= 0 || K % 64 || N % 16) return LUT6_E_SHAPE;
    if (L > INT32_MAX || K > INT32_MAX || N > INT32_MAX) return LUT6_E_SHAPE;
    if (epilogue < 0 || epilogue > 2) return LUT6_E_EPILOGUE;
    if (epilogue == LUT6_EPI_SILU_MUL_F16 && N % 32) return LUT6_E_SHAPE;
    if (!(in_scale == 1.0f || in_scale == 2.0f || in_scale == 4.0f || in_scale == 8.0f ||
          in_scale == 16.0f))
        return LUT6_E_SCALE;
    if (!aligned16(x) || !aligned16(packed) || !aligned16(tables) || !aligned16(y))
        return LUT6_E_ALIGN;
    const size_t x_bytes = (size_t)L * K * 2, p_bytes = (size_t)N * (K / 4 * 3),
                 t_bytes = (size_t)(N / 16) * 128;
    const size_t y_bytes = (size_t)L * (epilogue == 0 ? N * 4 : epilogue == 1 ? N * 2 : N);
    // activation and packed-weight byte sizes must fit 31-bit buffer offsets
    if (x_bytes >= ((size_t)1 << 31) || p_bytes >= ((size_t)1 << 31)) return LUT6_E_SHAPE;
    if (L == 0) return LUT6_OK;
    if (overlaps(y, y_bytes, x, x_bytes) || overlaps(y, y_bytes, packed, p_bytes) ||
        overlaps(y, y_bytes, tables, t_bytes))
        return LUT6_E_ALIAS;
    return LUT6_OK;
}

// Path, tiles and K split for a shape check_linear accepted with L > 0.
int plan_linear(int64_t L, int64_t K, int64_t N, int epilogue, LinearPlan& p)
{
    p = LinearPlan{};
    const int chunks = (int)(K / BK);
    p.path = choose_path(L, K, N, epilogue);
    const int n_half = epilogue == 2 ? (int)N / 2 : (int)N;
    if (p.path == LUT6_PATH_STREAM) {
        // weight-streaming regime: 64-token x 32-channel tiles over the whole
        // K range; K is split into slices (partial planes, fixed-order sum)
        // only when the tiles would leave most of the 256 CUs idle
        const int bn_cov = epilogue == 2 ? S_BN / 2 : S_BN;
        p.tiles_m = (int)((L + S_BM - 1) / S_BM);
        p.tiles_n = (n_half + bn_cov - 1) / bn_cov;
        p.tiles = p.tiles_n * p.tiles_m;
        int splits = 1;
        if (p.tiles < 192) {
            splits = (256 + p.tiles - 1) / p.tiles;
            const int max_splits = chunks / S_MIN_CHUNKS > 0 ? chunks / S_MIN_CHUNKS : 1;
            if (splits > max_splits) splits = max_splits;
        }
        p.k_chunks_per_split = (chunks + splits - 1) / splits;
        p.splits = (chunks + p.k_chunks_per_split - 1) / p.k_chunks_per_split;
        if ((int64_t)p.tiles * p.splits > INT32_MAX) return LUT6_E_SHAPE;
        p.f16 = p.k_chunks_per_split == 64 && chunks % 64 == 0;
    } else {
        // compute regime: 256 x 256 tiles; split K (fixed-order reduction)
        // when the tiles cannot fill most of the 256 CUs
        const int bn_cov = epilogue == 2 ? 128 : 256;
        p.tiles_m = (int)((L + T2 - 1) / T2);
        p.tiles_n = (n_half + bn_cov - 1) / bn_cov;
        p.tiles = p.tiles_n * p.tiles_m;
        int splits = 1;
        if (p.tiles < 192) {
            splits = (256 + p.tiles - 1) / p.tiles;
            const int max_splits = chunks / 8 > 0 ? chunks / 8 : 1;
            if (splits > max_splits) splits = max_splits;
        }
        p.k_chunks_per_split = (chunks + splits - 1) / splits;
        p.splits = (chunks + p.k_chunks_per_split - 1) / p.k_chunks_per_split;
        if (p.path == LUT6_PATH_EXPANDED)   // whole tiles, fragment order
            p.w16_bytes = (size_t)p.tiles_n * 8 * (chunks + 1) * 4096;
    }
    p.partial_bytes = p.splits > 1 ? (size_t)p.splits * L * N * sizeof(float) : 0;
    return LUT6_OK;
}

// Enqueue the kernels of a plan.  w16 and partial are device buffers of at
// least p.w16_bytes and p.partial_bytes (unused when those are 0).
int launch_linear(const LinearPlan& p, const void* x, const uint8_t* packed, const void* tables,
                  void* y, int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                  void* w16, float* partial, hipStream_t stream)
{
    GemmArgs a{};
    a.x = (const uint16_t*)x;
    a.packed = packed;
    a.tables = (const uint16_t*)tables;
    a.y = y;
    a.L = (int)L;
    a.K = (int)K;
    a.N = (int)N;
    a.scale = (_Float16)in_scale;
    a.inv_scale = 1.0f / in_scale;
    a.tiles_m = p.tiles_m;
    a.n_tiles = p.tiles;
    a.k_chunks_per_split = p.k_chunks_per_split;
    a.partial = p.splits > 1 ? partial : nullptr;
    const bool scaled = in_scale != 1.0f;
    const int splits = p.splits;
    if (p.path == LUT6_PATH_STREAM) {
        const dim3 grid((unsigned)(p.tiles * splits)), block(256);
        switch (((epilogue * 2 + (scaled ? 1 : 0)) * 2 + (splits > 1 ? 1 : 0)) * 2 + (p.f16 ? 1 : 0)) {
#define S8_CASE(I, E, S, P)                                                                                   \
        case 2 * (I): hipLaunchKernelGGL((lut6_stream_kernel<E, S, P, false>), grid, block, 0, stream, a); break; \
        case 2 * (I) + 1: hipLaunchKernelGGL((lut6_stream_kernel<E, S, P, true>), grid, block, 0, stream, a); break;
        S8_CASE(0, 0, false, false) S8_CASE(1, 0, false, true) S8_CASE(2, 0, true, false) S8_CASE(3, 0, true, true)
        S8_CASE(4, 1, false, false) S8_CASE(5, 1, false, true) S8_CASE(6, 1, true, false) S8_CASE(7, 1, true, true)
        S8_CASE(8, 2, false, false) S8_CASE(9, 2, false, true) S8_CASE(10, 2, true, false) S8_CASE(11, 2, true, true)
#undef S8_CASE
        default: return LUT6_E_EPILOGUE;
        }
        if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
        return splits > 1 ? launch_reduce(a, epilogue, splits, stream) : LUT6_OK;
    }
    const dim3 grid(p.tiles, splits), block(256);
    // many tokens: expand the weight once, then the FP16 GEMM; otherwise the
    // fused kernel
    const bool two_pass = p.path == LUT6_PATH_EXPANDED;
    if (two_pass) {
        const int chunks = (int)(K / BK);
        const dim3 xgrid((unsigned)p.tiles_n, (unsigned)((chunks + X_CHUNKS - 1) / X_CHUNKS));
        switch (epilogue) {
        case 2: hipLaunchKernelGGL(lut6_expand_kernel<2>, xgrid, dim3(256), 0, stream,
                                   packed, (const uint16_t*)tables, (uint16_t*)w16, (int)N, (int)K); break;
        default: hipLaunchKernelGGL(lut6_expand_kernel<0>, xgrid, dim3(256), 0, stream,
                                    packed, (const uint16_t*)tables, (uint16_t*)w16, (int)N, (int)K); break;
        }
        if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
        a.w16 = (const uint16_t*)w16;
    }
    launch_tiles(a, two_pass, epilogue, scaled, splits > 1, grid, stream);
    if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
    return splits > 1 ? launch_reduce(a, epilogue, splits, stream) : LUT6_OK;
}

}  // namespace

extern "C" int lut6_linear(const void* x, const uint8_t* packed, const void* tables, void* y,
                           int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                           hipStream_t stream)
{
    int st = check_linear(x, packed, tables, y, L, K, N, in_scale, epilogue);
    if (st != LUT6_OK || L == 0) return st;
    LinearPlan p;
    st = plan_linear(L, K, N, epilogue, p);
    if (st != LUT6_OK) return st;
    void* w16 = nullptr;
    float* partial = nullptr;
    if (p.w16_bytes) {
        st = workspace_for(stream, WS_EXPANDED, p.w16_bytes, &w16);
        if (st != LUT6_OK) return st;
    }
    if (p.partial_bytes) {
        st = workspace_for(stream, WS_PARTIAL, p.partial_bytes, (void**)&partial);
        if (st != LUT6_OK) return st;
    }
    return launch_linear(p, x, packed, tables, y, L, K, N, in_scale, epilogue, w16, partial, stream);
}

// ---------------------------------------------------------------------------
// lut6_linear_noalloc: the same plan and kernels, with the expanded weight and
// the split-K partials carved from one static device array per GPU, so that
// no call allocates.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LUT6_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mutex;
std::map<int, void*> g_scratch_addr;   // device -> device address of `scratch`

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.  The host-side symbol is only a
// stand-in: kernels and copies get this address, never the symbol.
int scratch_address(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LUT6_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    auto it = g_scratch_addr.find(dev);
    if (it == g_scratch_addr.end()) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LUT6_E_DEVICE;
        it = g_scratch_addr.emplace(dev, p).first;
    }
    *out = it->second;
    return LUT6_OK;
}
}  // namespace

extern "C" int lut6_linear_noalloc(const void* x, const uint8_t* packed, const void* tables, void* y,
                                   int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                                   hipStream_t stream)
{
    int st = check_linear(x, packed, tables, y, L, K, N, in_scale, epilogue);
    if (st != LUT6_OK || L == 0) return st;
    LinearPlan p;
    st = plan_linear(L, K, N, epilogue, p);
    if (st != LUT6_OK) return st;
    // expanded weight first, partial sums after it on a 256-byte boundary
    const size_t w16_span = (p.w16_bytes + 255) & ~(size_t)255;
    if (w16_span + p.partial_bytes > LUT6_NOALLOC_SCRATCH_BYTES) return LUT6_E_SCRATCH;
    void* base = nullptr;
    if (p.w16_bytes || p.partial_bytes) {
        st = scratch_address(&base);
        if (st != LUT6_OK) return st;
    }
    void* w16 = p.w16_bytes ? base : nullptr;
    float* partial = p.partial_bytes ? (float*)((unsigned char*)base + w16_span) : nullptr;
    return launch_linear(p, x, packed, tables, y, L, K, N, in_scale, epilogue, w16, partial, stream);
}

extern "C" int lut6_int8_linear(const void* x, const int8_t* q, const void* scales, void* y,
                                int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                                hipStream_t stream)
{
    if (!x || !q || !scales || !y) return LUT6_E_NULL;
    if (L < 0 || K <= 0 || N <= 0 || K % 64 || N % 16) return LUT6_E_SHAPE;
    if (L > INT32_MAX || K > INT32_MAX || N > INT32_MAX) return LUT6_E_SHAPE;
    if (epilogue < 0 || epilogue > 2) return LUT6_E_EPILOGUE;
    if (epilogue == LUT6_EPI_SILU_MUL_F16 && N % 32) return LUT6_E_SHAPE;
    if (!(in_scale == 1.0f || in_scale == 2.0f || in_scale == 4.0f || in_scale == 8.0f ||
          in_scale == 16.0f))
        return LUT6_E_SCALE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(scales) || !aligned16(y)) return LUT6_E_ALIGN;
    const size_t x_bytes = (size_t)L * K * 2, q_bytes = (size_t)N * K, s_bytes = (size_t)N * (K / 32) * 2;
    const size_t y_bytes = (size_t)L * (epilogue == 0 ? N * 4 : epilogue == 1 ? N * 2 : N);
    if (x_bytes >= ((size_t)1 << 31) || q_bytes >= ((size_t)1 << 31)) return LUT6_E_SHAPE;
    if (L == 0) return LUT6_OK;
    if (overlaps(y, y_bytes, x, x_bytes) || overlaps(y, y_bytes, q, q_bytes) || overlaps(y, y_bytes, scales, s_bytes))
        return LUT6_E_ALIAS;

    if (L <= STREAM_MAX_L) {
        // few tokens: stream the codes straight into the products
        const int n_tiles = epilogue == 2 ? (int)(N / 32) : (int)((N + 31) / 32);
        const dim3 grid((unsigned)n_tiles, (unsigned)((L + 63) / 64));
        const bool sc = in_scale != 1.0f;
        const float inv = 1.0f / in_scale;
#define I8S(E, S) hipLaunchKernelGGL((lut6_int8_stream_kernel<E, S>), grid, dim3(256), 0, stream, \
                                     (const uint16_t*)x, q, (const uint16_t*)scales, y, (int)L, (int)K, \
                                     (int)N, in_scale, inv)
        switch (epilogue * 2 + (sc ? 1 : 0)) {
        case 0: I8S(0, false); break;
        case 1: I8S(0, true); break;
        case 2: I8S(1, false); break;
        case 3: I8S(1, true); break;
        case 4: I8S(2, false); break;
        default: I8S(2, true); break;
        }
#undef I8S
        return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
    }

    GemmArgs a{};
    a.x = (const uint16_t*)x;
    a.y = y;
    a.L = (int)L;
    a.K = (int)K;
    a.N = (int)N;
    a.scale = (_Float16)in_scale;
    a.inv_scale = 1.0f / in_scale;
    // many tokens: weight expansion, then the FP16 GEMM
    // (split K when the 256 x 256 tiles cannot fill most CUs)
    const int chunks = (int)(K / BK);
    const int n_half = epilogue == 2 ? (int)N / 2 : (int)N;
    const int bn_cov = epilogue == 2 ? 128 : 256;
    const int tiles_m = (int)((L + T2 - 1) / T2);
    const int tiles_n = (n_half + bn_cov - 1) / bn_cov;
    const int tiles = tiles_n * tiles_m;
    int splits = 1;
    if (tiles < 192) {
        splits = (256 + tiles - 1) / tiles;
        const int max_splits = chunks / 8 > 0 ? chunks / 8 : 1;
        if (splits > max_splits) splits = max_splits;
    }
    a.tiles_m = tiles_m;
    a.n_tiles = tiles;
    a.k_chunks_per_split = (chunks + splits - 1) / splits;
    splits = (chunks + a.k_chunks_per_split - 1) / a.k_chunks_per_split;
    const size_t w16_bytes = (size_t)tiles_n * 8 * (chunks + 1) * 4096;
    if (w16_bytes > (size_t)INT32_MAX) return LUT6_E_SHAPE;
    void* w16 = nullptr;
    int st = workspace_for(stream, WS_EXPANDED, w16_bytes, &w16);
    if (st != LUT6_OK) return st;
    const dim3 xgrid((unsigned)tiles_n, (unsigned)((chunks + X_CHUNKS - 1) / X_CHUNKS));
    if (epilogue == 2)
        hipLaunchKernelGGL(lut6_int8_expand_kernel<2>, xgrid, dim3(256), 0, stream, q,
                           (const uint16_t*)scales, (uint16_t*)w16, (int)N, (int)K);
    else
        hipLaunchKernelGGL(lut6_int8_expand_kernel<0>, xgrid, dim3(256), 0, stream, q,
                           (const uint16_t*)scales, (uint16_t*)w16, (int)N, (int)K);
    if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
    a.w16 = (const uint16_t*)w16;
    if (splits > 1) {
        st = workspace_for(stream, WS_PARTIAL, (size_t)splits * L * N * sizeof(float), (void**)&a.partial);
        if (st != LUT6_OK) return st;
    }
    launch_tiles(a, true, epilogue, in_scale != 1.0f, splits > 1, dim3(tiles, splits), stream);
    if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
    return splits > 1 ? launch_reduce(a, epilogue, splits, stream) : LUT6_OK;
}

extern "C" int lut6_dequant(const uint8_t* packed, const void* tables, void* w, int64_t N,
                            int64_t K, hipStream_t stream)
{
    if (!packed || !tables || !w) return LUT6_E_NULL;
    if (N <= 0 || K <= 0 || K % 64 || N % 16 || N > INT32_MAX || K > INT32_MAX)
        return LUT6_E_SHAPE;
    if ((size_t)N * K >= ((size_t)1 << 40)) return LUT6_E_SHAPE;
    if (!aligned16(packed) || !aligned16(tables) || !aligned16(w)) return LUT6_E_ALIGN;
    if (overlaps(w, (size_t)N * K * 2, packed, (size_t)N * (K / 4 * 3)) ||
        overlaps(w, (size_t)N * K * 2, tables, (size_t)(N / 16) * 128))
        return LUT6_E_ALIAS;
    hipLaunchKernelGGL(lut6_dequant_kernel, dim3((unsigned)(N / 16)), dim3(256), 0, stream,
                       packed, (const uint16_t*)tables, (uint16_t*)w, (int)N, (int)K);
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}

namespace lut6_detail {
int quantize_release();   // lut6_quantize.hip

// the per-(device, stream) workspaces for the other sources (kinds from 2 up)
int workspace(hipStream_t stream, int kind, size_t bytes, void** out)
{
    return workspace_for(stream, kind, bytes, out);
}
}

extern "C" int lut6_release(void)
{
    int status = lut6_detail::quantize_release();
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_ws) {
        if (!kv.second.ptr) continue;
        const int dev = std::get<0>(kv.first);
        if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            status = LUT6_E_DEVICE;
        // stream-ordered allocations, freed on the null stream (the stream
        // they were made on may no longer exist), the device idle
        if (hipFreeAsync(kv.second.ptr, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            status = LUT6_E_DEVICE;
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
    return status;
}
