// Gated DeltaNet recurrence of the linear-attention layers on gfx950 (page
// "Clef-Flash-ANE-LUT6", section "Model architecture": 16 key and 32 value
// heads of size 128; page "clef-flash — Core AI", the decoder states: one
// recurrent state [32, 128, 128] per layer, carried between calls).
//
// The pages name the layer, not its update; the reading is the gated delta
// rule.  Per value head h (key head h / (Hv / Hk)), state S (dk x dv, FP32),
// for each token t in order:
//   S <- exp(g_t) S;   d = beta_t (v_t - S^T k_t);   S <- S + k_t d^T;
//   o_t = S^T q_t / sqrt(dk)   (rounded once to FP16)
//
// Design (token-sequential): column j of a head's state evolves on its own
// (it needs only its own S^T k and S^T q entries), so 16 lanes own one
// column, 8 rows each, in registers; the two 128-term dot products per
// token are 8 FMAs per lane and a 4-step DPP reduction over the 16 lanes.
// A workgroup holds 16 columns of one head (256 workgroups for 32 heads, one
// per CU).  Tokens go through LDS 64 at a time in two stages: k and q of the
// key head (converted to FP32 once there), v of the workgroup's columns, g
// and beta; the next chunk is loaded into registers while the current one
// is processed, and outputs leave through LDS as 16-byte rows.  The chunked form (products over 64
// positions on the matrix cores) is not built.
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

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

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
    hipLaunchKernelGGL(lut6_gated_delta_kernel, dim3((unsigned)(n_v_heads * (DV / COLS))), dim3(256), 0,
                       stream, a);
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}
