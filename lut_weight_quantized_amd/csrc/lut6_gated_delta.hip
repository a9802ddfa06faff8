// Gated DeltaNet recurrence of the linear-attention layers on gfx950 (page
// "Clef-Flash-ANE-LUT6", section "Model architecture": 16 key and 32 value
// heads of size 128; page "clef-flash — Core AI", the decoder states: one
// recurrent state [32, 128, 128] per layer, carried between calls; page
// "clef-flash-LiteRT", section "Provenance, conversion and license": the
// recurrence runs as a chunked kernel of 64 positions).
//
// The pages name the layer, not its update; the reading is the gated delta
// rule.  Per value head h (key head h / (Hv / Hk)), state S (dk x dv, FP32),
// for each token t in order:
//   S <- exp(g_t) S;   d = beta_t (v_t - S^T k_t);   S <- S + k_t d^T;
//   o_t = S^T q_t / sqrt(dk)   (rounded once to FP16)
//
// Chunked form (L >= 64), an evaluation order of the same rule.  Within a
// chunk of 64 positions, with G_t = g_1 + .. + g_t (inclusive, FP64),
// gamma_t = e^G_t, S0 the state before the chunk:
//   A[t][s] = beta_t e^(G_t - G_s) k_t.k_s  (s < t),   T = (I + A)^-1,
//   D = T (diag(beta) V - diag(beta gamma) K S0)        (the d_t as rows),
//   O = (diag(gamma) Q S0 + P D) / sqrt(dk),  P[t][s] = e^(G_t - G_s) q_t.k_s (s <= t),
//   S  = gamma_63 S0 + K^T diag(eta) D,       eta_s = e^(G_63 - G_s).
// lut6_gdn_prep_kernel computes T, P and the decay vectors of every (chunk,
// head) in parallel: K K^T and Q K^T on v_mfma_f32_16x16x32_f16 (the FP16
// inputs give exact products and FP32 sums), T by substitution.
// lut6_gdn_chunk_kernel then walks the chunks in order, one workgroup per
// (head, 16 state columns): every product with the state on
// v_mfma_f32_16x16x4f32, the state's FP32 columns held in the waves'
// accumulators and mirrored in LDS as the next chunk's operand.
//
// Token-sequential form (L < 64): column j of a head's state evolves on its
// own (it needs only its own S^T k and S^T q entries), so 16 lanes own one
// column, 8 rows each, in registers; the two 128-term dot products per
// token are 8 FMAs per lane and a 4-step DPP reduction over the 16 lanes.
// A workgroup holds 16 columns of one head (256 workgroups for 32 heads, one
// per CU).  Tokens go through LDS 64 at a time in two stages: k and q of the
// key head (converted to FP32 once there), v of the workgroup's columns, g
// and beta; the next chunk is loaded into registers while the current one
// is processed, and outputs leave through LDS as 16-byte rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lut6.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int DK = 128, DV = 128;
constexpr int COLS = 16;              // state columns per workgroup
constexpr int T = 64;                 // tokens per LDS stage

struct GdnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    uint16_t* o;
    float* state;                     // [Hv][DK][DV], read at the start, written at the end
    int64_t ldq, ldk, ldv, ldg, ldo;
    int L, Hv, grp;
};

// sum over the 16 lanes of a row (xor 1, xor 2 inside quads, then the
// mirrored lane of the other quad, then of the other half-row)
__device__ __forceinline__ float row16_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

__global__ void __launch_bounds__(256) lut6_gated_delta_kernel(GdnArgs a)
{
    // per stage: k then q [T][DK] in FP32 (converted once while staging),
    // v [T][COLS] halves, g and beta [T]
    __shared__ __attribute__((aligned(16))) float kq[2][T][2 * DK];
    __shared__ __attribute__((aligned(16))) uint16_t vs[2][T][COLS];
    __shared__ float gb[2][2][T];
    __shared__ __attribute__((aligned(16))) uint16_t os[2][T][COLS];

    const int tid = threadIdx.x;
    const int h = blockIdx.x / (DV / COLS), c0 = (blockIdx.x % (DV / COLS)) * COLS;
    const int kh = h / a.grp;
    const int cl = tid >> 4, r = tid & 15;       // column c0 + cl, rows 8 r .. 8 r + 7
    const float scale = 0.08838834764831845f;    // 1 / sqrt(128)

    float S[8];
    float* const sp = a.state + ((size_t)h * DK + 8 * r) * DV + c0 + cl;
#pragma unroll
    for (int e = 0; e < 8; ++e) S[e] = sp[(size_t)e * DV];

    // staging: k and q as 2,048 16-byte pieces (8 per thread); v as 128
    // pieces (threads 0..127); g and beta (threads 128..255).  Tokens past L
    // re-read token L - 1 and are never used.
    u32x4 kqr[8], vr = {0u, 0u, 0u, 0u};
    float gbr = 0.0f;
    auto load_chunk = [&](int ch) {
        const int t0 = ch * T;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = tid + 256 * u, tt = idx >> 5, part = (idx >> 4) & 1, piece = idx & 15;
            const int t = min(t0 + tt, a.L - 1);
            const uint16_t* src = part ? a.q + (size_t)t * a.ldq : a.k + (size_t)t * a.ldk;
            kqr[u] = *(const u32x4*)(src + (size_t)kh * DK + piece * 8);
        }
        if (tid < 128) {
            const int tt = tid >> 1, half = tid & 1;
            const int t = min(t0 + tt, a.L - 1);
            vr = *(const u32x4*)(a.v + (size_t)t * a.ldv + (size_t)h * DV + c0 + 8 * half);
        } else {
            const int tt = (tid - 128) & 63;
            const int t = min(t0 + tt, a.L - 1);
            gbr = tid < 192 ? a.g[(size_t)t * a.ldg + h] : a.beta[(size_t)t * a.ldg + h];
        }
    };
    auto store_chunk = [&](int b) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = tid + 256 * u, tt = idx >> 5, part = (idx >> 4) & 1, piece = idx & 15;
            const f16x8 hv = __builtin_bit_cast(f16x8, kqr[u]);
            float* const dst = &kq[b][tt][part * DK + piece * 8];
            *(float4*)dst = float4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
            *(float4*)(dst + 4) = float4{(float)hv[4], (float)hv[5], (float)hv[6], (float)hv[7]};
        }
        if (tid < 128) *(u32x4*)(&vs[b][tid >> 1][8 * (tid & 1)]) = vr;
        else gb[b][tid < 192 ? 0 : 1][(tid - 128) & 63] = gbr;
    };

    const int nch = (a.L + T - 1) / T;
    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    if (nch > 1) load_chunk(1);
    for (int ch = 0; ch < nch; ++ch) {
        const int b = ch & 1;
        const int n = min(T, a.L - ch * T);
        for (int tt = 0; tt < n; ++tt) {
            const float al = __expf(gb[b][0][tt]);
            const float be = gb[b][1][tt];
            const float4 k0 = *(const float4*)(&kq[b][tt][8 * r]);
            const float4 k1 = *(const float4*)(&kq[b][tt][8 * r + 4]);
            const float4 q0 = *(const float4*)(&kq[b][tt][DK + 8 * r]);
            const float4 q1 = *(const float4*)(&kq[b][tt][DK + 8 * r + 4]);
            const float kf[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
            const float qf[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            float kv = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) kv = __builtin_fmaf(S[e], kf[e], kv);
            kv = row16_sum(kv);
            const float vv = (float)__builtin_bit_cast(_Float16, vs[b][tt][cl]);
            const float d = be * (vv - al * kv);
            float ov = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                S[e] = __builtin_fmaf(kf[e], d, al * S[e]);
                ov = __builtin_fmaf(S[e], qf[e], ov);
            }
            ov = row16_sum(ov);
            if (r == 0) os[b][tt][cl] = __builtin_bit_cast(uint16_t, (_Float16)(ov * scale));
        }
        if (ch + 1 < nch) store_chunk(b ^ 1);
        __syncthreads();
        // outputs of this chunk: 16 columns of n tokens, 16 bytes per thread
        if (tid < 2 * n) {
            const int tt = tid >> 1, half = tid & 1;
            *(u32x4*)(a.o + (size_t)(ch * T + tt) * a.ldo + (size_t)h * DV + c0 + 8 * half) =
                *(const u32x4*)(&os[b][tt][8 * half]);
        }
        if (ch + 2 < nch) load_chunk(ch + 2);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sp[(size_t)e * DV] = S[e];
}

// ---------------------------------------------------------------------------
// chunked form
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;                            // positions per chunk
constexpr int CB = 16;                            // state columns per recurrence workgroup
constexpr int WS_T = 0, WS_P = CH * CH;           // workspace layout per (head, chunk), floats
constexpr int WS_GAMMA = 2 * CH * CH, WS_ETA = WS_GAMMA + CH, WS_BETA = WS_ETA + CH;
constexpr int WS_PAD = WS_BETA + CH;              // 256 bytes never read
constexpr int WS_FLOATS = 2 * CH * CH + 4 * CH;   // T, P, gamma, eta, beta, pad
constexpr int WS_GDN = 3;                         // library workspace kind
constexpr int64_t MAX_WINDOW_CHUNKS = 128;        // chunks per prep + recurrence launch pair
constexpr size_t WS_BUDGET = (size_t)160 << 20;   // workspace bytes, at most
constexpr int64_t MAX_LD = int64_t(1) << 24;      // largest row stride, elements (32-bit lane offsets)

struct ChunkArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    uint16_t* o;
    float* state;                     // [Hv][DK][DV]
    float* ws;                        // [Hv][n_chunks][WS_FLOATS]
    int64_t ldq, ldk, ldv, ldg, ldo;
    int L;                            // tokens of the call
    int t_begin;                      // first token of this window
    int n_chunks;                     // chunks in this window
    int Hv, grp;
};

__device__ __forceinline__ float quad_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ float half_at(const u32x4& w, int i)
{
    const uint32_t word = w[i >> 1];
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? word >> 16 : word & 0xffffu));
}

// One (chunk, value head): T = (I + A)^-1, P and the decay vectors.
__global__ void __launch_bounds__(256) lut6_gdn_prep_kernel(ChunkArgs a)
{
    // the k and q rows (FP16) while K K^T and Q K^T are formed, then T and
    // per-wave block products
    __shared__ __attribute__((aligned(16))) union {
        struct {
            uint16_t k[CH][DK + 8];
            uint16_t q[CH][DK + 8];
        } rows;
        struct {
            float t[CH][CH + 4];
            float u[4][16][20];
        } inv;
    } sh;
    uint16_t (&kh)[CH][DK + 8] = sh.rows.k;
    uint16_t (&qh)[CH][DK + 8] = sh.rows.q;
    float (&ts)[CH][CH + 4] = sh.inv.t;
    float (&us)[4][16][20] = sh.inv.u;
    __shared__ float as[CH][CH + 4];                                    // A (zero on and above the diagonal)
    __shared__ double gl[CH];                                           // G_t
    __shared__ float bs[CH];                                            // beta_t

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lo = lane & 15, hi = lane >> 4;
    const int c = blockIdx.x, h = blockIdx.y, kq = h / a.grp;
    const int t0 = a.t_begin + c * CH;
    float* const ws = a.ws + ((size_t)h * a.n_chunks + c) * WS_FLOATS;

    // k and q rows of the key head, zero past L: the eight loads go out
    // together (rows past L re-read row L - 1 and are zeroed on the way to
    // LDS; under a branch each pair of loads waited for the one before)
    {
        u32x4 kv[4], qv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u, row = idx >> 4, piece = idx & 15;
            const size_t t = (size_t)min(t0 + row, a.L - 1);
            kv[u] = *(const u32x4*)(a.k + t * a.ldk + (size_t)kq * DK + piece * 8);
            qv[u] = *(const u32x4*)(a.q + t * a.ldq + (size_t)kq * DK + piece * 8);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u, row = idx >> 4, piece = idx & 15;
            const uint32_t m = t0 + row < a.L ? 0xffffffffu : 0u;
            *(u32x4*)&kh[row][piece * 8] = kv[u] & m;
            *(u32x4*)&qh[row][piece * 8] = qv[u] & m;
        }
    }
    for (int i = tid; i < CH * (CH + 4); i += 256) (&as[0][0])[i] = 0.0f;
    // the log-decay prefix in FP64 and beta (g = beta = 0 past L)
    if (wave == 0) {
        const int t = t0 + lane;
        double x = 0.0;
        float be = 0.0f;
        if (t < a.L) {
            x = (double)a.g[(size_t)t * a.ldg + h];
            be = a.beta[(size_t)t * a.ldg + h];
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        gl[lane] = x;
        bs[lane] = be;
        const double last = __shfl(x, 63);
        ws[WS_GAMMA + lane] = expf((float)x);
        ws[WS_ETA + lane] = expf((float)(last - x));
        ws[WS_BETA + lane] = be;
    }
    __syncthreads();

    // K K^T (tiles on and below the diagonal, into A) and Q K^T (into P):
    // 20 tiles of 16 x 16, five per wave.  All five tiles' products first,
    // then per tile its decays from one read of the four G_t and beta_t and
    // stores without per-element branches (entries of A on or above the
    // diagonal get the zero they already hold): with a branch around each
    // element, each decay waited for its own LDS round trips.
    f32x4 acc[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int job = wave + 4 * j;                       // 0..9: K K^T, 10..19: Q K^T
        const bool isq = job >= 10;
        const int tri = isq ? job - 10 : job;               // lower-triangle tile index
        const int rt = tri >= 6 ? 3 : tri >= 3 ? 2 : tri >= 1 ? 1 : 0;
        const int st_ = tri - rt * (rt + 1) / 2;
        const uint16_t (*xa)[DK + 8] = isq ? qh : kh;
        acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const f16x8 av = *(const f16x8*)&xa[16 * rt + lo][32 * kk + 8 * hi];
            const f16x8 bv = *(const f16x8*)&kh[16 * st_ + lo][32 * kk + 8 * hi];
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int job = wave + 4 * j;
        const bool isq = job >= 10;
        const int tri = isq ? job - 10 : job;
        const int rt = tri >= 6 ? 3 : tri >= 3 ? 2 : tri >= 1 ? 1 : 0;
        const int st_ = tri - rt * (rt + 1) / 2;
        const int s = 16 * st_ + lo, tb = 16 * rt + 4 * hi;
        const double gs = gl[s];
        float dec[4], bt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dec[e] = expf((float)(gl[tb + e] - gs));
            bt[e] = bs[tb + e];
        }
        if (isq) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ws[WS_P + (tb + e) * CH + s] = s <= tb + e ? dec[e] * acc[j][e] : 0.0f;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) as[tb + e][s] = s < tb + e ? bt[e] * dec[e] * acc[j][e] : 0.0f;
        }
    }
    // P above its diagonal tiles is zero
    for (int i = tid; i < 6 * 256; i += 256) {
        const int tile = i >> 8, r = (i >> 4) & 15, cc = i & 15;
        const int rt = tile < 3 ? 0 : tile < 5 ? 1 : 2;
        const int st_ = tile < 3 ? tile + 1 : tile < 5 ? tile - 1 : 3;
        ws[WS_P + (16 * rt + r) * CH + 16 * st_ + cc] = 0.0f;
    }
    __syncthreads();

    // T = (I + A)^-1 in 16 x 16 blocks T_ij (unit lower triangular, like
    // I + A).  The diagonal blocks are (I + A_ii)^-1, wave i by substitution
    // down each column (column lane / 4, its rows split over four lanes by
    // row % 4, a quad reduction per row); wave i also clears the blocks
    // right of its diagonal one.  Row block i of (I + A) T = I then gives,
    // below the diagonal, T_ij = -T_ii sum_{j <= m < i} A_im T_mj: level
    // i - j = 1, 2, 3 in turn, one block per wave, on the FP32 matrix unit.
    {
        const int j = lane >> 2, p = lane & 3, b0 = 16 * wave;
        float tc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tc[i] = (4 * i + p == j) ? 1.0f : 0.0f;
#pragma unroll
        for (int t = 1; t < 16; ++t) {
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i <= (t - 1) / 4; ++i) sum = __builtin_fmaf(as[b0 + t][b0 + 4 * i + p], tc[i], sum);
            sum = quad_sum(sum);
            if (p == (t & 3) && t > j) tc[t >> 2] = -sum;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ts[b0 + 4 * i + p][b0 + j] = tc[i];
        for (int cb = wave + 1; cb < 4; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e) ts[b0 + j][16 * cb + 4 * p + e] = 0.0f;
    }
    __syncthreads();
    // C += X Y for 16 x 16 blocks (X, Y row-major with leading dimensions);
    // lane holds C[4 hi + e][lo]
    auto mm = [&](const float* x, int ldx, const float* y, int ldy, f32x4 acc) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[lo * ldx + 4 * kk + hi], y[(4 * kk + hi) * ldy + lo], acc, 0,
                                                     0, 0);
        return acc;
    };
    for (int lvl = 1; lvl < 4; ++lvl) {
        const bool act = wave < 4 - lvl;
        const int bi = wave + lvl, bj = wave;
        if (act) {
            f32x4 u = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int m = bj; m < bi; ++m) u = mm(&as[16 * bi][16 * m], CH + 4, &ts[16 * m][16 * bj], CH + 4, u);
#pragma unroll
            for (int e = 0; e < 4; ++e) us[wave][4 * hi + e][lo] = u[e];
        }
        __syncthreads();
        if (act) {
            const f32x4 t = mm(&ts[16 * bi][16 * bi], CH + 4, &us[wave][0][0], 20, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int e = 0; e < 4; ++e) ts[16 * bi + 4 * hi + e][16 * bj + lo] = -t[e];
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = tid + 256 * u, r = idx >> 4, c4 = idx & 15;
        *(f32x4*)(ws + WS_T + r * CH + 4 * c4) = *(const f32x4*)&ts[r][4 * c4];
    }
}

// The recurrence over the chunks of a window: one workgroup per (value head,
// 16 state columns), eight waves, two per SIMD.  Wave w has the role p = w / 4
// (0: K, 1: Q) on the row block r = w % 4 of the chunk: per chunk a K wave
// takes rows 16 r .. 16 r + 15 of K S0, then of R = beta (v - gamma K S0) and
// D = T R; a Q wave the same rows of Q S0, then of the output O = gamma Q S0
// + P D; and every wave one 16-row tile of the state update (tile w).  Both
// roles run the same loads and the same first product on their own rows (k
// and T rows, or q and P rows), so the compiler's counts of loads in flight
// are exact on both, and the two waves on a SIMD fill each other's stalls.
// A chunk's operands are loaded into registers while the chunk before it is
// computed, with the two operand sets swapped every chunk.
__global__ void __launch_bounds__(512) lut6_gdn_chunk_kernel(ChunkArgs a)
{
    __shared__ __attribute__((aligned(16))) float st[CB][DK + 4];     // S^T of the block
    // k rows of the chunk; column c of row i is stored at c ^ 4 ((i / 4) % 4):
    // the stride suits the state update's reads (rows 4 m + hi, columns
    // 16 w + lo: one bank per lane), and the swizzle spreads the row writes,
    // whose 16 lanes (rows 16 r + lo) would otherwise share four 16-byte
    // bank groups
    __shared__ __attribute__((aligned(16))) float ks[CH][DK + 16];
    __shared__ __attribute__((aligned(16))) float rt[CB][CH + 4];     // R^T, R = beta (v - gamma K S)
    __shared__ __attribute__((aligned(16))) float dt[CB][CH + 4];     // D^T
    __shared__ __attribute__((aligned(16))) float dh[CB][CH + 4];     // (eta D)^T, like D^T
    __shared__ float vec[2][3][CH];                                   // gamma, eta, beta (two chunks)

    const int tid = threadIdx.x, lane = tid & 63, lo = lane & 15, hi = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = w >> 2, r = w & 3;
    // the 8 column blocks of a head share its chunk data: keep them on one
    // XCD (dispatch is round-robin over the 8 XCDs)
    const int h = blockIdx.x % a.Hv, jb = blockIdx.x / a.Hv;
    const int kq = h / a.grp;
    const int col0 = h * DV + jb * CB;
    float* const sp = a.state + (size_t)h * DK * DV + jb * CB;
    const float rsq = 0.08838834764831845f;           // 1 / sqrt(128)
    // this wave's row operand: k rows and T rows (K waves), q rows and P rows
    // (Q waves)
    const uint16_t* const xbase = (role ? a.q : a.k) + (size_t)kq * DK;
    const int64_t ldx = role ? a.ldq : a.ldk;
    const int wsm = role ? WS_P : WS_T;
    float* const wsh = a.ws + (size_t)h * a.n_chunks * WS_FLOATS;
    const int trow = 16 * r + lo;                     // this lane's A-operand row of the tiles

    // S^T tile w: lane holds S[16 w + lo][4 hi + e]
    f32x4 sacc;
    {
        const int i = 16 * w + lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sacc[e] = sp[(size_t)i * DV + 4 * hi + e];
            st[4 * hi + e][i] = sacc[e];
        }
    }

    // one chunk's register operands: the lane's k or q row pieces (row trow,
    // k = 32 z + 8 hi + i), its T or P row pieces (columns 16 z + 4 hi + j),
    // v of its R rows (16 r + 4 hi + e; used by K waves) and one
    // decay-vector entry (threads < 192).  In each row load the four lane
    // groups hi = 0..3 of a row read 64 contiguous bytes, so one instruction
    // touches 16 row segments.
    struct Ops {
        u32x4 xr[4];
        f32x4 mv[4];
        uint32_t vr[4];
        float vc;
    };
    // Every load and store address is a uniform base, formed per chunk on
    // the scalar unit, plus one of these lane byte offsets, formed once
    // (32-bit: the host bounds the row strides): k or q row, T or P row, the
    // four v rows, the decay entry, the four o rows and the pad slot.
    uint32_t ox = 2u * ((uint32_t)trow * (uint32_t)ldx + 8u * (uint32_t)hi);
    uint32_t om = 4u * (uint32_t)(trow * CH + 4 * hi);
    uint32_t oc = 4u * (uint32_t)(WS_GAMMA + (tid < 3 * CH ? tid : 0));
    uint32_t opad = 4u * (uint32_t)WS_PAD + 2u * (uint32_t)lane;
    uint32_t ov[4], os[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t row = (uint32_t)(16 * r + 4 * hi + e);
        ov[e] = 2u * (row * (uint32_t)a.ldv + (uint32_t)lo);
        os[e] = 2u * (row * (uint32_t)a.ldo + (uint32_t)lo);
    }
    // Every load is unconditional (rows past L re-read row L - 1): with
    // loads under branches the compiler cannot count the ones in flight, and
    // its wait for this chunk's operands then also waited for the next
    // chunk's, a full memory latency per chunk.  Only the call's last chunk
    // can hold rows past L, so the row offsets are pulled back once, when it
    // is the next chunk to load.  Rows past L are zeroed where the chunk is
    // consumed, not here: any arithmetic on a loaded register makes the wave
    // wait for that load in the iteration that issued it.
    bool clamped = false;
    auto clamp_tail = [&](int c) {
        const int t0 = a.t_begin + c * CH;
        if (!clamped && t0 + CH > a.L) {
            ox -= 2u * (uint32_t)max(t0 + trow - (a.L - 1), 0) * (uint32_t)ldx;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ov[e] -= 2u * (uint32_t)max(t0 + 16 * r + 4 * hi + e - (a.L - 1), 0) * (uint32_t)a.ldv;
            clamped = true;
        }
    };
    auto load_ops = [&](int c, Ops& op) {
        const int t0 = a.t_begin + c * CH;
        const char* const xb = (const char*)(xbase + (size_t)t0 * ldx);
        const char* const mb = (const char*)(wsh + (size_t)c * WS_FLOATS + wsm);
        const char* const vb = (const char*)(a.v + (size_t)t0 * a.ldv + col0);
        const char* const gb = (const char*)(wsh + (size_t)c * WS_FLOATS);
#pragma unroll
        for (int z = 0; z < 4; ++z) op.xr[z] = *(const u32x4*)(xb + ox + 64 * z);
#pragma unroll
        for (int z = 0; z < 4; ++z) op.mv[z] = *(const f32x4*)(mb + om + 64 * z);
#pragma unroll
        for (int e = 0; e < 4; ++e) op.vr[e] = *(const uint16_t*)(vb + ov[e]);
        op.vc = *(const float*)(gb + oc);
    };

    // A chunk's outputs are stored during the next chunk, after its loads:
    // stores count in the same in-order counter as loads, so stores issued
    // just before the barrier made the wait for the next operands also wait
    // for the write acknowledgements.  Every path stores four times: K
    // waves, the empty store of chunk 0 and rows past L go to the unused pad
    // of a workspace block.
    uint16_t ob[4] = {0, 0, 0, 0};
    auto store_o = [&](int cc, bool real) {
        const int t0c = a.t_begin + cc * CH;
        if (real && role == 1 && t0c + CH <= a.L) {
            char* const orow = (char*)(a.o + (size_t)t0c * a.ldo + col0);
#pragma unroll
            for (int e = 0; e < 4; ++e) *(uint16_t*)(orow + os[e]) = ob[e];
        } else if (real && role == 1) {
            uint16_t* const pad = (uint16_t*)(wsh + (size_t)cc * WS_FLOATS + WS_PAD) + lane;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tg = t0c + 16 * r + 4 * hi + e;
                // both addresses are formed first so that the choice is a
                // select, not a branch around the multiply
                uint16_t* const row = a.o + (size_t)min(tg, a.L - 1) * a.ldo + col0 + lo;
                *(tg < a.L ? row : pad) = ob[e];
            }
        } else {
            char* const pad = (char*)(wsh + (size_t)cc * WS_FLOATS);
#pragma unroll
            for (int e = 0; e < 4; ++e) *(uint16_t*)(pad + opad) = ob[e];
        }
    };

    // chunk c from the operands in cur while the next chunk's are loaded
    // into nxt (the loop runs two chunks per pass with the two sets swapped,
    // so that no set is copied)
    auto chunk = [&](int c, const Ops& cur, Ops& nxt) {
        const int t0 = a.t_begin + c * CH, b = c & 1;
        const int cn = c + 1 < a.n_chunks ? c + 1 : c;
        // (opaque per chunk: hoisted, the offsets were widened to 64 bits
        // once and every access then added them on the vector unit)
        asm volatile("" : "+v"(om), "+v"(oc), "+v"(opad), "+v"(os[0]), "+v"(os[1]), "+v"(os[2]), "+v"(os[3]));
        asm volatile("" : "+v"(ox), "+v"(ov[0]), "+v"(ov[1]), "+v"(ov[2]), "+v"(ov[3]));
        clamp_tail(cn);
        load_ops(cn, nxt);

        // stage 1: rows 16 r .. 16 r + 15 of K S0 (K waves) or Q S0 (Q
        // waves), step n taking k = 32 (n / 8) + 8 hi + n % 8; K waves then
        // put the k row in LDS for the state update and R in LDS
        f32x4 x;
        {
            float xf[32];
            // rows past L read as zero (a select, not a branch: the next
            // chunk's loads above and these products must stay in one
            // scheduling region for their pacing)
            const uint32_t km = t0 + trow < a.L ? 0xffffffffu : 0u;
#pragma unroll
            for (int z = 0; z < 4; ++z)
#pragma unroll
                for (int i = 0; i < 8; ++i) xf[8 * z + i] = half_at(cur.xr[z] & km, i);
            x = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            // each group's S0 column piece is read one group ahead, so that
            // no product waits for an LDS round trip
            f32x4 bv[2];
            bv[0] = *(const f32x4*)&st[lo][8 * hi];
#pragma unroll
            for (int m4 = 0; m4 < 8; ++m4) {
                if (m4 + 1 < 8)
                    bv[(m4 + 1) & 1] = *(const f32x4*)&st[lo][32 * ((m4 + 1) >> 1) + 8 * hi + 4 * ((m4 + 1) & 1)];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    x = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[4 * m4 + mm], bv[m4 & 1][mm], x, 0, 0, 0);
            }
            // pace the next chunk's 8 row loads (k or q, T or P) one per four
            // of the 32 matrix instructions: issued back to back they fill
            // the vector memory path, and the in-order wave then stalls at
            // each further load while its matrix work waits behind it.  The
            // S0 pieces are read one group of 4 products ahead (left to
            // itself the compiler reads each just before its products).
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            // the previous chunk's outputs (after the loads, so no wait for
            // this chunk's operands waits for a write acknowledgement)
            store_o(c > 0 ? c - 1 : 0, c > 0);
            if (role == 0) {
#pragma unroll
                for (int z = 0; z < 8; ++z)
                    *(f32x4*)&ks[trow][32 * (z >> 1) + ((8 * hi + 4 * (z & 1)) ^ (4 * ((lo >> 2) & 3)))] =
                        f32x4{xf[4 * z], xf[4 * z + 1], xf[4 * z + 2], xf[4 * z + 3]};
                f32x4 r4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * r + 4 * hi + e;
                    const uint16_t vb = t0 + t < a.L ? (uint16_t)cur.vr[e] : (uint16_t)0;
                    const float vv = (float)__builtin_bit_cast(_Float16, vb);
                    r4[e] = vec[b][2][t] * (vv - vec[b][0][t] * x[e]);
                }
                *(f32x4*)&rt[lo][16 * r + 4 * hi] = r4;
            }
        }
        __syncthreads();
        // stage 2 (K waves): D rows 16 r .. 16 r + 15 = T R (step m takes s =
        // 16 (m / 4) + 4 hi + m % 4).  R and D are kept transposed in LDS, so
        // a lane's four entries of one step group are one 16-byte read; two
        // accumulation chains (even and odd steps).
        if (role == 0) {
            f32x4 d2[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
            // all four R pieces are read before the first product
            f32x4 rv[4];
#pragma unroll
            for (int z = 0; z < 4; ++z) rv[z] = *(const f32x4*)&rt[lo][16 * z + 4 * hi];
#pragma unroll
            for (int z = 0; z < 4; ++z)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    d2[j & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.mv[z][j], rv[z][j], d2[j & 1], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
            const f32x4 d = d2[0] + d2[1];
            *(f32x4*)&dt[lo][16 * r + 4 * hi] = d;
            f32x4 dhe;
#pragma unroll
            for (int e = 0; e < 4; ++e) dhe[e] = vec[b][1][16 * r + 4 * hi + e] * d[e];
            *(f32x4*)&dh[lo][16 * r + 4 * hi] = dhe;
        }
        __syncthreads();

        // stage 3: the state rows 16 w .. 16 w + 15, S^T = gamma_63 S0^T +
        // (eta D)^T K (contraction s = 4 m + hi); then (Q waves) the output
        // rows 16 r .. 16 r + 15, O = (gamma Q S0 + P D) / sqrt(128)
        {
            const float gt = vec[b][0][CH - 1];
            f32x4 acc = sacc * gt;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int s = 4 * m + hi;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(dh[lo][s], ks[s][16 * w + (lo ^ (4 * (m & 3)))], acc, 0,
                                                           0, 0);
            }
            sacc = acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[4 * hi + e][16 * w + lo] = acc[e];
            if (role == 1) {
                f32x4 o2[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
                for (int e = 0; e < 4; ++e) o2[0][e] = vec[b][0][16 * r + 4 * hi + e] * x[e];
                // all four D pieces are read before the first product
                f32x4 dv[4];
#pragma unroll
                for (int z = 0; z < 4; ++z) dv[z] = *(const f32x4*)&dt[lo][16 * z + 4 * hi];
#pragma unroll
                for (int z = 0; z < 4; ++z)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        o2[j & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.mv[z][j], dv[z][j], o2[j & 1], 0, 0, 0);
                const f32x4 o = o2[0] + o2[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) ob[e] = __builtin_bit_cast(uint16_t, (_Float16)(o[e] * rsq));
            }
        }
        // the next chunk's decay vectors (that buffer was last read before
        // the previous barrier)
        if (tid < 3 * CH) vec[b ^ 1][tid >> 6][tid & 63] = nxt.vc;
        __syncthreads();
    };

    Ops opa, opb;
    clamp_tail(0);
    load_ops(0, opa);
    if (tid < 3 * CH) vec[0][tid >> 6][tid & 63] = opa.vc;
    __syncthreads();
    for (int c = 0; c < a.n_chunks; c += 2) {
        chunk(c, opa, opb);
        if (c + 1 < a.n_chunks) chunk(c + 1, opb, opa);
    }
    store_o(a.n_chunks - 1, true);
    {
        const int i = 16 * w + lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[(size_t)i * DV + 4 * hi + e] = sacc[e];
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

namespace lut6_detail {
int workspace(hipStream_t stream, int kind, size_t bytes, void** out);   // lut6_linear.hip
}

extern "C" int lut6_gated_delta(const void* q, int64_t ldq, const void* k, int64_t ldk,
                                const void* v, int64_t ldv, const float* g, const float* beta,
                                int64_t ldg, void* o, int64_t ldo, float* state, int64_t L,
                                int64_t n_k_heads, int64_t n_v_heads, int64_t dk, int64_t dv,
                                hipStream_t stream)
{
    if (!q || !k || !v || !g || !beta || !o || !state) return LUT6_E_NULL;
    if (dk != DK || dv != DV || n_k_heads <= 0 || n_v_heads <= 0 || n_v_heads % n_k_heads ||
        n_v_heads > 4096 || L < 0 || L > INT32_MAX - T)
        return LUT6_E_SHAPE;
    if (ldq < n_k_heads * DK || ldk < n_k_heads * DK || ldv < n_v_heads * DV || ldo < n_v_heads * DV ||
        ldg < n_v_heads)
        return LUT6_E_SHAPE;
    if (ldq > MAX_LD || ldk > MAX_LD || ldv > MAX_LD || ldo > MAX_LD) return LUT6_E_SHAPE;
    if (ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8) return LUT6_E_ALIGN;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)g & 3) ||
        ((uintptr_t)beta & 3) || ((uintptr_t)state & 3))
        return LUT6_E_ALIGN;
    if (L == 0) return LUT6_OK;
    const size_t ob = ((size_t)(L - 1) * ldo + n_v_heads * DV) * 2;
    const size_t sb = (size_t)n_v_heads * DK * DV * 4;
    const size_t qb = ((size_t)(L - 1) * ldq + n_k_heads * DK) * 2;
    const size_t kb = ((size_t)(L - 1) * ldk + n_k_heads * DK) * 2;
    const size_t vb = ((size_t)(L - 1) * ldv + n_v_heads * DV) * 2;
    const size_t gbb = ((size_t)(L - 1) * ldg + n_v_heads) * 4;
    if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, vb) ||
        overlaps(o, ob, g, gbb) || overlaps(o, ob, beta, gbb) || overlaps(o, ob, state, sb) ||
        overlaps(state, sb, q, qb) || overlaps(state, sb, k, kb) || overlaps(state, sb, v, vb) ||
        overlaps(state, sb, g, gbb) || overlaps(state, sb, beta, gbb))
        return LUT6_E_ALIAS;

    GdnArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.g = g;
    a.beta = beta;
    a.o = (uint16_t*)o;
    a.state = state;
    a.ldq = ldq;
    a.ldk = ldk;
    a.ldv = ldv;
    a.ldg = ldg;
    a.ldo = ldo;
    a.L = (int)L;
    a.Hv = (int)n_v_heads;
    a.grp = (int)(n_v_heads / n_k_heads);
    if (L < CH) {
        hipLaunchKernelGGL(lut6_gated_delta_kernel, dim3((unsigned)(n_v_heads * (DV / COLS))), dim3(256), 0,
                           stream, a);
        return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
    }
    // chunked: windows of chunks, each a prep launch then a recurrence launch
    const int64_t chunks = (L + CH - 1) / CH;
    const size_t per_chunk = (size_t)n_v_heads * WS_FLOATS * sizeof(float);
    int64_t win = (int64_t)(WS_BUDGET / per_chunk);
    win = win < 1 ? 1 : win > MAX_WINDOW_CHUNKS ? MAX_WINDOW_CHUNKS : win;
    if (win > chunks) win = chunks;
    void* ws = nullptr;
    const int st = lut6_detail::workspace(stream, WS_GDN, (size_t)win * per_chunk, &ws);
    if (st != LUT6_OK) return st;
    ChunkArgs ca;
    ca.q = a.q;
    ca.k = a.k;
    ca.v = a.v;
    ca.g = g;
    ca.beta = beta;
    ca.o = a.o;
    ca.state = state;
    ca.ws = (float*)ws;
    ca.ldq = ldq;
    ca.ldk = ldk;
    ca.ldv = ldv;
    ca.ldg = ldg;
    ca.ldo = ldo;
    ca.L = (int)L;
    ca.Hv = (int)n_v_heads;
    ca.grp = a.grp;
    for (int64_t c0 = 0; c0 < chunks; c0 += win) {
        const int64_t nc = chunks - c0 < win ? chunks - c0 : win;
        ca.t_begin = (int)(c0 * CH);
        ca.n_chunks = (int)nc;
        hipLaunchKernelGGL(lut6_gdn_prep_kernel, dim3((unsigned)nc, (unsigned)n_v_heads), dim3(256), 0, stream, ca);
        hipLaunchKernelGGL(lut6_gdn_chunk_kernel, dim3((unsigned)(n_v_heads * (DV / CB))), dim3(512), 0, stream, ca);
        if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
    }
    return LUT6_OK;
}
