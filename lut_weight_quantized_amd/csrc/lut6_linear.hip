// LUT-6 dequant-GEMM for AMD Instinct MI355X (gfx950, CDNA4).
//
// What it computes (page "Clef-Flash-ANE-LUT6", sections "Weight precision"
// and "LUT-6 text weights"):
//     W[n, k]  = table[n / 16][index(n, k)]          (one FP16 table per 16 channels)
//     xs       = fp16(x * s)                          (s = in_scale, a power of two <= 16)
//     a[l, n]  = (sum_k xs[l, k] * W[n, k]) / s       (FP32 accumulation)
//     y        = epilogue(a): FP32, FP16, or silu(gate) * up in FP16.
//
// Mapping onto the hardware
//   * The contraction runs on v_mfma_f32_16x16x32_f16 (FP16 inputs, FP32
//     accumulate).  The weight is the MFMA "A" operand (16 output channels x
//     32 k) and the activations the "B" operand (32 k x 16 tokens), so each
//     accumulator lane holds four consecutive channels of one token and the
//     store is a 16-byte (FP32) or 8-byte (FP16) vector per lane.
//   * A 16-channel fragment uses exactly one table, because fragments are
//     16-aligned.  The tables of a workgroup's channels sit in LDS (128 bytes
//     each: one table spans the 32 four-byte banks once, so a wave's lookups
//     into one table never conflict).
//   * Index tiles are never materialised: each lane loads the 12 packed bytes
//     that hold 16 consecutive indices of one channel (three aligned dwords,
//     a 96-bit little-endian word whose field t is index t), extracts each
//     6-bit field and gathers its table entry from LDS straight into the
//     FP16 fragment registers.  Workgroup waves own disjoint channels, so
//     every weight is dequantised once per workgroup.
//   * The sum over k is insensitive to the order of k inside one MFMA as long
//     as A and B agree; lane group g (= lane / 16) takes k0+16g .. k0+16g+15
//     for a pair of MFMAs, which keeps its 12 packed bytes contiguous.
//   * Activation tiles (BM tokens x 64 k) are double-buffered in LDS with a
//     16-byte row pad (144-byte rows), which keeps the 16-byte fragment reads
//     conflict-free.  The input scale is applied while staging, in FP16
//     (one rounding, exactly as fp16(x * s)).
//   * Small token counts split K across workgroups; partial sums go to a
//     workspace and a second kernel adds them in a fixed order (no atomics),
//     so results are bit-identical run to run.
//   * Workgroups are dispatched round-robin over the 8 XCDs; the tile index
//     is remapped so that consecutive tiles (which share a weight tile) run
//     on the same XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
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
constexpr int XROW = BK + 8;    // LDS activation row, in halves (144 bytes)
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
    int L, K, N;
    int k_chunks_per_split;   // BK-chunks per split
    int tiles_m;              // token tiles
    int n_tiles;              // total (token x channel) tiles
    _Float16 scale;           // in_scale as FP16 (exact)
    float inv_scale;          // 1 / in_scale (exact)
};

// ---------------------------------------------------------------------------
// The GEMM kernel.
//   BN x BM tile of (channels x tokens); WN_W x WM_W waves; each wave owns
//   BN/WN_W channels (FN fragments of 16) and BM/WM_W tokens (FM of 16).
//   EPI: 0 = FP32, 1 = FP16, 2 = SiLU(gate) * up FP16.  SPLIT: write FP32
//   partial sums instead of the epilogue.
//   For EPI 2 a tile covers gate channels [j0, j0 + BN/2) and the matching
//   up channels [N/2 + j0, ...); wave fragments f < FN/2 are gate, the rest up,
//   so each lane holds both operands of its outputs.
// ---------------------------------------------------------------------------
template <int BN, int BM, int WN_W, int WM_W, int EPI, bool SPLIT>
__global__ void __launch_bounds__(64 * WN_W * WM_W)
lut6_gemm_kernel(GemmArgs a)
{
    constexpr int NT = 64 * WN_W * WM_W;
    constexpr int WN = BN / WN_W, WM = BM / WM_W;
    constexpr int FN = WN / 16, FM = WM / 16;
    constexpr int XCH = BM * BK / 8;            // 16-byte chunks per activation tile
    constexpr int XPT = (XCH + NT - 1) / NT;    // chunks per thread
    static_assert(BN % (16 * WN_W) == 0 && BM % (16 * WM_W) == 0, "tile shape");
    static_assert(EPI != 2 || FN % 2 == 0, "SiLU needs an even fragment count");

    __shared__ __attribute__((aligned(16))) _Float16 xs_lds[2][BM * XROW];
    __shared__ __attribute__((aligned(16))) uint16_t tab_lds[BN / 16 * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN_W, wm = wave / WN_W;
    const int r16 = lane & 15, g4 = lane >> 4;

    const int tile = xcd_remap(blockIdx.x, a.n_tiles);
    const int tm = tile % a.tiles_m, tn = tile / a.tiles_m;
    const int m0 = tm * BM;
    const int K = a.K, N = a.N, L = a.L;
    const int kc_begin = blockIdx.y * a.k_chunks_per_split;
    const int kc_end = min(K / BK, kc_begin + a.k_chunks_per_split);
    const int row_bytes = K / 4 * 3;

    // First channel of fragment f of wave w (may be >= the valid range:
    // such fragments are computed on a clamped row and never stored).
    auto frag_row = [&](int w, int f) -> int {
        if constexpr (EPI == 2) {
            const int j = tn * (BN / 2) + w * (WN / 2) + 16 * (f % (FN / 2));
            return f < FN / 2 ? j : N / 2 + j;
        } else {
            return tn * BN + w * WN + 16 * f;
        }
    };
    auto frag_valid = [&](int w, int f) -> bool {
        if constexpr (EPI == 2) return tn * (BN / 2) + w * (WN / 2) + 16 * (f % (FN / 2)) < N / 2;
        else return frag_row(w, f) < N;
    };

    // tables of this workgroup's fragments -> LDS (slot = wave * FN + f)
    for (int i = tid; i < BN / 16 * 64; i += NT) {
        const int s = i / 64, w = s / FN, f = s % FN;
        const int row = frag_valid(w, f) ? frag_row(w, f) : 0;
        tab_lds[i] = a.tables[(row / 16) * 64 + (i % 64)];
    }

    // per-lane packed-byte pointers for each fragment
    const uint8_t* prow[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
        const int row = (frag_valid(wn, f) ? frag_row(wn, f) : 0) + r16;
        prow[f] = a.packed + (size_t)row * row_bytes + 12 * g4;
    }

    f32x4 acc[FN][FM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int m = 0; m < FM; ++m) acc[f][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bool scaled = a.scale != (_Float16)1.0f;

    // activation chunk c of k-step kc -> registers
    auto load_x = [&](int kc, u32x4 (&xr)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int c = tid + i * NT;
            const int r = c / (BK / 8), cc = c % (BK / 8);
            const int tok = m0 + r;
            if (c < XCH && tok < L)
                xr[i] = *(const u32x4*)(a.x + (size_t)tok * K + kc * BK + cc * 8);
            else
                xr[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_x = [&](int buf, u32x4 (&xr)[XPT]) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int c = tid + i * NT;
            if (c < XCH) {
                const int r = c / (BK / 8), cc = c % (BK / 8);
                u32x4 v = xr[i];
                if (scaled) {
                    f16x8 h = __builtin_bit_cast(f16x8, v);
                    h = h * a.scale;
                    v = __builtin_bit_cast(u32x4, h);
                }
                *(u32x4*)(&xs_lds[buf][r * XROW + cc * 8]) = v;
            }
        }
    };
    auto load_p = [&](int kc, uint32_t (&p)[FN][3]) {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const uint32_t* q = (const uint32_t*)(prow[f] + (size_t)kc * (BK / 4 * 3));
            p[f][0] = q[0];
            p[f][1] = q[1];
            p[f][2] = q[2];
        }
    };

    u32x4 xr[XPT];
    uint32_t pk[FN][3], pn[FN][3];
    if (kc_begin < kc_end) {
        load_x(kc_begin, xr);
        load_p(kc_begin, pk);
        store_x(0, xr);
    }
    __syncthreads();

    const uint16_t* tab_w = tab_lds + wn * FN * 64;
    for (int kc = kc_begin; kc < kc_end; ++kc) {
        const int cur = (kc - kc_begin) & 1;
        const bool more = kc + 1 < kc_end;
        if (more) {
            load_x(kc + 1, xr);
            load_p(kc + 1, pn);
        }
        // activation fragments of this wave: token r16 of each 16-token block
        f16x8 xb[FM][2];
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            const _Float16* src = &xs_lds[cur][(wm * WM + 16 * m + r16) * XROW + 16 * g4];
            xb[m][0] = *(const f16x8*)(src);
            xb[m][1] = *(const f16x8*)(src + 8);
        }
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            f16x8 w0, w1;
            gather16(pk[f][0], pk[f][1], pk[f][2], tab_w + f * 64, w0, w1);
#pragma unroll
            for (int m = 0; m < FM; ++m) {
                acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w0, xb[m][0], acc[f][m], 0, 0, 0);
                acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w1, xb[m][1], acc[f][m], 0, 0, 0);
            }
        }
        if (more) {
            store_x(cur ^ 1, xr);
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                pk[f][0] = pn[f][0];
                pk[f][1] = pn[f][1];
                pk[f][2] = pn[f][2];
            }
        }
        __syncthreads();
    }

    // epilogue: lane holds channels frag_row + 4*g4 + (0..3) of token r16
#pragma unroll
    for (int m = 0; m < FM; ++m) {
        const int tok = m0 + wm * WM + 16 * m + r16;
        if (tok >= L) continue;
        if constexpr (SPLIT) {
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                if (!frag_valid(wn, f)) continue;
                const int n = frag_row(wn, f) + 4 * g4;
                float* dst = a.partial + ((size_t)blockIdx.y * L + tok) * N + n;
                *(f32x4*)dst = acc[f][m];
            }
        } else if constexpr (EPI == 0) {
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                if (!frag_valid(wn, f)) continue;
                const int n = frag_row(wn, f) + 4 * g4;
                *(f32x4*)((float*)a.y + (size_t)tok * N + n) = acc[f][m] * a.inv_scale;
            }
        } else if constexpr (EPI == 1) {
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                if (!frag_valid(wn, f)) continue;
                const int n = frag_row(wn, f) + 4 * g4;
                const f32x4 v = acc[f][m] * a.inv_scale;
                f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
                *(f16x4*)((_Float16*)a.y + (size_t)tok * N + n) = h;
            }
        } else {
#pragma unroll
            for (int f = 0; f < FN / 2; ++f) {
                if (!frag_valid(wn, f)) continue;
                const int j = frag_row(wn, f) + 4 * g4;
                const f32x4 gv = acc[f][m] * a.inv_scale;
                const f32x4 uv = acc[f + FN / 2][m] * a.inv_scale;
                f16x4 h;
#pragma unroll
                for (int r = 0; r < 4; ++r) h[r] = (_Float16)(silu_f32(gv[r]) * uv[r]);
                *(f16x4*)((_Float16*)a.y + (size_t)tok * (N / 2) + j) = h;
            }
        }
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
    if constexpr (EPI == 2) {
        f32x4 g = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s) {
            g += *(const f32x4*)(partial + s * plane + (size_t)tok * N + c);
            u += *(const f32x4*)(partial + s * plane + (size_t)tok * N + N / 2 + c);
        }
        g *= inv_scale;
        u *= inv_scale;
        f16x4 h;
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = (_Float16)(silu_f32(g[r]) * u[r]);
        *(f16x4*)((_Float16*)y + (size_t)tok * n_out + c) = h;
    } else {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < splits; ++s)
            v += *(const f32x4*)(partial + s * plane + (size_t)tok * N + c);
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
    float* ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;   // key: (device, stream)

int workspace_for(hipStream_t stream, size_t bytes, float** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LUT6_E_DEVICE;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& w = g_ws[std::make_pair(dev, (uintptr_t)stream)];
    if (w.bytes < bytes) {
        if (w.ptr) {
            // a previous launch on this stream may still use the old buffer
            if (hipStreamSynchronize(stream) != hipSuccess) return LUT6_E_DEVICE;
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        void* p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) return LUT6_E_DEVICE;
        w.ptr = (float*)p;
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

template <int BN, int BM, int WN_W, int WM_W>
int launch_tiles(GemmArgs a, int epi, int splits, hipStream_t stream)
{
    const int n_half = epi == 2 ? a.N / 2 : a.N;
    const int bn_cov = epi == 2 ? BN / 2 : BN;
    const int tiles_n = (n_half + bn_cov - 1) / bn_cov;
    a.tiles_m = (a.L + BM - 1) / BM;
    a.n_tiles = a.tiles_m * tiles_n;
    const int chunks = a.K / BK;
    a.k_chunks_per_split = (chunks + splits - 1) / splits;
    splits = (chunks + a.k_chunks_per_split - 1) / a.k_chunks_per_split;
    dim3 grid(a.n_tiles, splits), block(64 * WN_W * WM_W);
    if (splits > 1) {
        const size_t bytes = (size_t)splits * a.L * a.N * sizeof(float);
        const int st = workspace_for(stream, bytes, &a.partial);
        if (st != LUT6_OK) return st;
        switch (epi) {
        case 0: hipLaunchKernelGGL((lut6_gemm_kernel<BN, BM, WN_W, WM_W, 0, true>), grid, block, 0, stream, a); break;
        case 1: hipLaunchKernelGGL((lut6_gemm_kernel<BN, BM, WN_W, WM_W, 1, true>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((lut6_gemm_kernel<BN, BM, WN_W, WM_W, 2, true>), grid, block, 0, stream, a); break;
        }
        if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
        const int n_out = epi == 2 ? a.N / 2 : a.N;
        const int64_t total4 = (int64_t)a.L * n_out / 4;
        dim3 rgrid((unsigned)((total4 + 255) / 256));
        switch (epi) {
        case 0: hipLaunchKernelGGL(lut6_reduce_kernel<0>, rgrid, dim3(256), 0, stream, a.partial, a.y, a.L, a.N, splits, a.inv_scale); break;
        case 1: hipLaunchKernelGGL(lut6_reduce_kernel<1>, rgrid, dim3(256), 0, stream, a.partial, a.y, a.L, a.N, splits, a.inv_scale); break;
        default: hipLaunchKernelGGL(lut6_reduce_kernel<2>, rgrid, dim3(256), 0, stream, a.partial, a.y, a.L, a.N, splits, a.inv_scale); break;
        }
    } else {
        switch (epi) {
        case 0: hipLaunchKernelGGL((lut6_gemm_kernel<BN, BM, WN_W, WM_W, 0, false>), grid, block, 0, stream, a); break;
        case 1: hipLaunchKernelGGL((lut6_gemm_kernel<BN, BM, WN_W, WM_W, 1, false>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((lut6_gemm_kernel<BN, BM, WN_W, WM_W, 2, false>), grid, block, 0, stream, a); break;
        }
    }
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}

}  // namespace

extern "C" int lut6_linear(const void* x, const uint8_t* packed, const void* tables, void* y,
                           int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                           hipStream_t stream)
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
    if ((size_t)L * K >= ((size_t)1 << 40) || (size_t)N * K >= ((size_t)1 << 40))
        return LUT6_E_SHAPE;
    if (L == 0) return LUT6_OK;
    if (overlaps(y, y_bytes, x, x_bytes) || overlaps(y, y_bytes, packed, p_bytes) ||
        overlaps(y, y_bytes, tables, t_bytes))
        return LUT6_E_ALIAS;

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

    const int chunks = (int)(K / BK);
    if (L <= 192) {
        // weight-streaming regime: 128-channel x 128-token tiles, K split so
        // that about 512 workgroups stream the weight at once
        const int n_half = epilogue == 2 ? (int)N / 2 : (int)N;
        const int bn_cov = epilogue == 2 ? 64 : 128;
        const int tiles = ((n_half + bn_cov - 1) / bn_cov) * (int)((L + 127) / 128);
        int splits = (512 + tiles - 1) / tiles;
        splits = splits < 1 ? 1 : splits;
        splits = splits > chunks / 2 ? (chunks / 2 > 0 ? chunks / 2 : 1) : splits;
        return launch_tiles<128, 128, 4, 1>(a, epilogue, splits, stream);
    }
    // compute regime: 256-channel x 128-token tiles, split K only when the
    // tile count cannot fill the 256 CUs
    const int n_half = epilogue == 2 ? (int)N / 2 : (int)N;
    const int bn_cov = epilogue == 2 ? 128 : 256;
    const int tiles = ((n_half + bn_cov - 1) / bn_cov) * (int)((L + 127) / 128);
    int splits = 1;
    if (tiles < 256) {
        splits = (512 + tiles - 1) / tiles;
        if (splits > chunks / 8) splits = chunks / 8 > 0 ? chunks / 8 : 1;
    }
    return launch_tiles<256, 128, 4, 1>(a, epilogue, splits, stream);
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

extern "C" int lut6_release(void)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int status = LUT6_OK;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_ws) {
        if (!kv.second.ptr) continue;
        const int dev = kv.first.first;
        if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
            status = LUT6_E_DEVICE;
        (void)hipFree(kv.second.ptr);
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
    return status;
}
