// Full attention of the attention layers on gfx950, FP16 in and out, with
// the probabilities scaled by 16 before they are rounded to FP16 (page
// "Clef-Flash-ANE-LUT6", section "Model architecture": 16 query and 4
// key-value heads of size 256, full attention over the context; section
// "LUT-6 text weights": attention probabilities are scaled up by 16 in FP16
// and scaled back afterwards).
//
// What one call computes (readings where the page is silent):
//   - the L queries are the last L positions of the Lk keys: query i sees
//     keys 0 .. Lk - L + i (causal, one chunk of a prefill over a cache);
//   - query head h reads key-value head h / (Hq / Hkv);
//   - softmax scale 1 / sqrt(256) = 1/16;
//   - o = (sum_j fp16(16 p_j) v_j) / (16 l), p_j = exp(s_j - m) in FP32, l
//     the FP32 sum of the p_j; one FP16 rounding of o.
//
// Design: one workgroup per (query head, 128 queries), four waves of 32
// queries.  Keys go by blocks of 32, two workgroups per CU (of 64, one per
// CU, for small launches and key splits), through two LDS stages, K and V
// both row-major and copied straight from global memory into LDS: a block is
// computed from one stage while the next block is copied into the other;
// one barrier per block.  Short query chunks over a long cache split the
// keys over several workgroups, whose partial sums a second kernel combines.
// Per block a wave computes S^T = K Q^T (keys x queries, so that each lane
// holds one query and its softmax needs a single cross-lane exchange), the
// online-softmax update, and O^T += V^T P^T, all on
// v_mfma_f32_32x32x16_f16; the V^T fragments come from row-major V through
// the transposing LDS read.  The P^T values never leave registers: the
// accumulator layout of S^T, with its k slots read in the same key order
// from V^T, is the B operand of the second product.  Every address in the
// key loop is a uniform base plus a lane offset computed once (the K
// fragment offsets from a single base by XOR), so that the loop's vector
// instructions go to the softmax, and the K and V fragments are read two
// products ahead of their use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lut6.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int HD = 256;               // head size
constexpr int BQ = 128;               // queries per workgroup
constexpr int BKEY = 64;              // keys per block (key splits and fewer workgroups)
constexpr int BKEY_SMALL = 32;        // keys per block with two workgroups per CU
// Launches of at least this many workgroups (and no key split) use 32-key
// blocks: 64 KB of LDS and at most 256 registers per lane, so two
// workgroups share a CU and each SIMD runs two waves.  Measured from 128
// workgroups up (1,024 queries with 16 heads, chunks over a longer cache
// included) that form is as fast or faster; below, the 64-key form.
constexpr int64_t SMALL_BLOCK_MIN_WGS = 128;
constexpr int64_t MAX_KV_LD = int64_t(1) << 24;   // largest k / v row stride, elements
constexpr int WS_ATTENTION = 2;       // library workspace kind of the key-split partials

struct AttArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* part_o;                    // key splits: [split][L][Hq][256] unnormalised sums
    float* part_ml;                   // key splits: [split][L][Hq][2] (max, sum)
    int64_t ldq, ldk, ldv, ldo;       // elements between consecutive token rows
    int L, Lk, Hq, grp, nqb;
    int kb_per_split;                 // key blocks per split (key splits only)
};

// A row's running maximum is raised only when a block's maximum passes it
// by more than TAU (base-2 units): softmax does not depend on the shift, the
// probabilities against the older maximum stay below 2^TAU (16 p < 2^12 in
// FP16), and the 128 accumulators are rescaled only on those blocks.
constexpr float TAU = 8.0f;

__device__ __forceinline__ uint32_t pack_f16(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// one LDS stage: K [BK][256], then V [BK][256], both row-major.  Rows are
// copied straight from global memory (64 lanes x 16 bytes, two rows per
// instruction), so instead of padding, the 16-byte pieces of a row are
// XOR-swizzled: piece p (dims 8 p .. 8 p + 7) of key row r sits in slot
//   K: p ^ (r & 15): a K-fragment read's 16 lanes per cycle take 16 rows at
//      one piece, which land on 16 distinct 4-bank groups;
//   V: p ^ 4 (r & 3): a transposing read's 16 lanes take 4 rows x 4 pieces,
//      also 16 distinct groups.
constexpr int VMCNT0 = 0x0F70;        // s_waitcnt: vmcnt = 0, other counters not waited for
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <bool SPLIT, int BK>
__global__ void __launch_bounds__(256, BK == BKEY_SMALL ? 2 : 1) lut6_attention_kernel(AttArgs a)
{
    constexpr int NST = BK / 32;                   // 32-key tiles per block
    constexpr int NCOPY = BK / 4;                  // copies per wave and block (K and V)
    constexpr int TILE_HALVES = BK * HD;           // one K or V tile in LDS, unpadded
    constexpr int STAGE_HALVES = 2 * TILE_HALVES;
    // the two stages are separate arrays: the compiler then sees that a copy
    // into one cannot overwrite what is being read from the other, and does
    // not drain the outstanding LDS reads before each copy
    __shared__ __attribute__((aligned(16))) uint16_t lds0[STAGE_HALVES];
    __shared__ __attribute__((aligned(16))) uint16_t lds1[STAGE_HALVES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, c = lane & 31;
    // the query blocks with the most keys start first
    const int hq = blockIdx.x % a.Hq;
    const int qb = a.nqb - 1 - (int)(blockIdx.x / a.Hq);
    const int kh = hq / a.grp;
    const int q0 = qb * BQ;
    const int qrow = q0 + 32 * wave + c;
    const int off = a.Lk - a.L;                                // position of query 0
    const int pos = off + qrow;                                // this lane's query position
    const int last = off + min(q0 + BQ - 1, a.L - 1);          // last key the workgroup needs
    int kb0 = 0, kb1 = last / BK + 1;
    if constexpr (SPLIT) {
        kb0 = min((int)blockIdx.y * a.kb_per_split, kb1);
        kb1 = min(kb0 + a.kb_per_split, kb1);
    }

    f32x16 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
    float m = -__builtin_inff(), l = 0.0f;

    if (kb0 < kb1) {
        // Q as B fragments of K Q^T: dims 16 j + 8 h .. + 7 of the lane's
        // query (rows past L read row L - 1 and are never stored)
        u32x4 qf[16];
        {
            const uint16_t* qp = a.q + (size_t)min(qrow, a.L - 1) * a.ldq + (size_t)hq * HD + 8 * h;
#pragma unroll
            for (int j = 0; j < 16; ++j) qf[j] = *(const u32x4*)(qp + 16 * j);
        }

        // staging: wave w's copy i fills rows 2 (C w + i) and 2 (C w + i) + 1
        // of the K and of the V tile (C = NCOPY / 2 copies per wave and
        // tile); lane L writes slot L % 32 of row 2 (C w + i) + L / 32, so it
        // reads the piece that belongs there.  A copy's address is a uniform
        // base (the block's first row) plus the lane's byte offset kco / vco
        // (32-bit: the host bounds the row strides).  Keys past Lk re-read
        // key Lk - 1 (they are masked): only the last block can hold such
        // keys, so the offsets are pulled back once, when that block is the
        // next one to copy.
        uint32_t kco[NCOPY / 2], vco[NCOPY / 2];
#pragma unroll
        for (int i = 0; i < NCOPY / 2; ++i) {
            const int r = 2 * (NCOPY / 2 * wave + i) + h;
            kco[i] = 2u * ((uint32_t)r * (uint32_t)a.ldk + 8u * (uint32_t)(c ^ (r & 15)));
            vco[i] = 2u * ((uint32_t)r * (uint32_t)a.ldv + 8u * (uint32_t)(c ^ ((r & 3) << 2)));
        }
        bool clamped = false;
        auto clamp_tail = [&](int kb) {
            if (!clamped && kb * BK + BK > a.Lk) {
#pragma unroll
                for (int i = 0; i < NCOPY / 2; ++i) {
                    const int r = 2 * (NCOPY / 2 * wave + i) + h;
                    const uint32_t d = (uint32_t)max(kb * BK + r - (a.Lk - 1), 0);
                    kco[i] -= 2u * d * (uint32_t)a.ldk;
                    vco[i] -= 2u * d * (uint32_t)a.ldv;
                }
                clamped = true;
            }
        };
        // copy n (0..NCOPY-1): K (n even) or V (n odd) rows of wave copy i = n / 2
        auto issue_kv = [&](int kb, uint16_t* kst, int n) {
            const int i = n >> 1;
            // (the offset goes through a local: with the array element
            // written inside the builtin's argument, the host pass of this
            // compiler emitted no launch stub for the kernel)
            const uint32_t lo = (n & 1) ? vco[i] : kco[i];
            const size_t row0 = (size_t)kb * BK;
            if ((n & 1) == 0)
                __builtin_amdgcn_global_load_lds((const char*)(a.k + row0 * a.ldk + (size_t)kh * HD) + lo,
                                                 (lds_ptr_t)(kst + (NCOPY / 2 * wave + i) * 512), 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((const char*)(a.v + row0 * a.ldv + (size_t)kh * HD) + lo,
                                                 (lds_ptr_t)(kst + TILE_HALVES + (NCOPY / 2 * wave + i) * 512), 16, 0, 0);
        };
        // LDS byte offsets of the lane's fragments within a stage, whose
        // other parts are immediates.  K: row c of a 32-key tile at piece
        // (2 j + h) ^ (c & 15); for j = 0..7 that is kfo0 ^ 32 j (the piece
        // bits lie between the row's and the lane half's), and j + 8 is 256
        // bytes further.  V: the transposing read for dims 32 dt .. with
        // dt = 0..3 (dt + 4: 256 bytes further), key rows 4 h + i / 4
        // (i = lane % 16).
        uint32_t vfo[4];
        const uint32_t kfo0 = 2u * (uint32_t)(c * HD + 8 * (h ^ (c & 15)));
        {
            const int gi = lane & 15, vr = 4 * h + (gi >> 2);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const int vp = 4 * dt + 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);
                vfo[dt] = 2u * (uint32_t)(vr * HD + 8 * (vp ^ ((vr & 3) << 2)) + 4 * (gi & 1));
            }
        }

        const float cl = 1.4426950408889634f / 16.0f;          // log2(e) / sqrt(256)
        clamp_tail(kb0);
#pragma unroll
        for (int n = 0; n < NCOPY; ++n) issue_kv(kb0, lds0, n);
        __builtin_amdgcn_s_waitcnt(VMCNT0);
        __syncthreads();
        // block kb from stage ks while the next block is copied into nst
        auto block = [&](int kb, const uint16_t* ks, uint16_t* nst) {
            const uint16_t* const vs = ks + TILE_HALVES;
            // the next block goes into the other stage (last read before the
            // previous barrier), its NCOPY copies spread evenly over the S^T
            // products below; the last block again on the last iteration
            const int kn = min(kb + 1, kb1 - 1);
            clamp_tail(kn);
            // (an opaque copy: the seven other K offsets are formed per block
            // by one XOR each, not kept in registers through the loop; a
            // lane needs every register it can keep for the prefetches)
            uint32_t k0 = kfo0;
            asm volatile("" : "+v"(k0));

            // S^T for keys 32 st .. 32 st + 31 of the block: lane (c, h),
            // value r is key 8 (r / 4) + 4 h + r % 4 of the tile, query c
            // (with two tiles their products alternate, so that no product
            // waits for the one before it to finish)
            f32x16 s[NST];
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[st][r] = 0.0f;
            // (issued back to back, the copies fill the vector memory path
            // and the in-order wave stalls at the later ones with its
            // products waiting behind them; the copies write LDS, so the
            // compiler keeps them where they are written)
            // The K fragments are read two steps ahead: the compiler does
            // not move an LDS read above a copy into LDS.
            auto kfrag = [&](int j, int st) {
                return *(const f16x8*)((const char*)ks + (k0 ^ (32u * (j & 7))) + 256 * (j >> 3) + 2 * 32 * HD * st);
            };
            f16x8 ka[3][NST];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int st = 0; st < NST; ++st) ka[j][st] = kfrag(j, st);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (j + 2 < 16)
#pragma unroll
                    for (int st = 0; st < NST; ++st) ka[(j + 2) % 3][st] = kfrag(j + 2, st);
#pragma unroll
                for (int st = 0; st < NST; ++st)
                    s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[j % 3][st], __builtin_bit_cast(f16x8, qf[j]),
                                                                   s[st], 0, 0, 0);
                if (j % (16 / NCOPY) == 0) issue_kv(kn, nst, j / (16 / NCOPY));
            }

            // online softmax (base 2) on the raw scores: masked keys get
            // -inf, only in blocks that reach past the workgroup's first
            // query; the block maximum is scaled after the max (cl > 0)
            float bm = -__builtin_inff();
            if (kb * BK + BK - 1 > off + q0) {
#pragma unroll
                for (int st = 0; st < NST; ++st)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb * BK + 32 * st + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (key > pos) s[st][r] = -__builtin_inff();
                    }
            }
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int r = 0; r < 16; ++r) bm = fmaxf(bm, s[st][r]);
            {
                // the other half's maximum (lanes L and L ^ 32 hold the same
                // query), exchanged in registers rather than through LDS
                const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, bm),
                                                                 __builtin_bit_cast(uint32_t, bm), false, false);
                bm = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1])) * cl;
            }
            const bool raise = bm > m + TAU;                   // also the first finite maximum
            if (__any(raise)) {
                const float mn = raise ? bm : m;
                const float alpha = raise ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                m = mn;
            }
            const float mu = m == -__builtin_inff() ? 0.0f : m;
            const float sh = 4.0f - mu;                        // 16 p = 2^(cl s - mu + 4)
            // per 32-key tile and half jj: P^T x 16 in FP16 as the B fragment
            // (values r = 8 jj .. 8 jj + 7: keys 16 jj + 4 h + 0..3 and
            // 16 jj + 8 + 4 h + 0..3), then O^T (dims x queries) += V^T P^T
            // with the A slots on the same keys; a half's exponentials come
            // just before its eight products, so fewer values are live.
            // V^T fragments by transposing reads: in each 16-lane group
            // (g = lane / 16, i = lane % 16) lane i points at 4 dims of key
            // K0 + i / 4 and receives keys K0 .. K0 + 3 of dim
            // 32 dt + 16 (g % 2) + i; K0 = 32 st + 16 jj + 4 h, and + 8 for
            // the second half of the fragment.  Fragment n = (st, jj, dt) in
            // product order; they are read two products ahead, the first two
            // before the exponentials.
            auto vfrag = [&](int n) {
                const int st = n >> 4, jj = (n >> 3) & 1, dt = n & 7;
                const char* vp = (const char*)vs + vfo[dt & 3] + 256 * (dt >> 2) + 2 * (32 * st + 16 * jj) * HD;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)vp);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(vp + 2 * 8 * HD));
                const u32x4 va = {__builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 0, 1)),
                                  __builtin_bit_cast(uint32_t, __builtin_shufflevector(lo, lo, 2, 3)),
                                  __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 0, 1)),
                                  __builtin_bit_cast(uint32_t, __builtin_shufflevector(hi, hi, 2, 3))};
                return __builtin_bit_cast(f16x8, va);
            };
            constexpr int NV = 16 * NST;
            f16x8 vb[3];
            vb[0] = vfrag(0);
            vb[1] = vfrag(1);
            __builtin_amdgcn_sched_barrier(0);
            float sum = 0.0f;
#pragma unroll
            for (int st = 0; st < NST; ++st) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    u32x4 pf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 8 * jj + 2 * e;
                        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][r], cl, sh));
                        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][r + 1], cl, sh));
                        sum += p0 + p1;
                        pf[e] = pack_f16(p0, p1);
                    }
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt) {
                        const int n = 16 * st + 8 * jj + dt;
                        if (n + 2 < NV) vb[(n + 2) % 3] = vfrag(n + 2);
                        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[n % 3], __builtin_bit_cast(f16x8, pf),
                                                                       o[dt], 0, 0, 0);
                    }
                }
            }
            l += sum * 0.0625f;                                // sum holds 16 p

            // this wave's copies of the next block have landed; after the
            // barrier, everyone's have
            __builtin_amdgcn_s_waitcnt(VMCNT0);
            __syncthreads();
        };
        for (int kb = kb0; kb < kb1; kb += 2) {
            block(kb, lds0, lds1);
            if (kb + 1 < kb1) block(kb + 1, lds1, lds0);
        }
    }

    const float lt = l + __shfl_xor(l, 32);                    // both lane halves
    if (qrow >= a.L) return;
    if constexpr (SPLIT) {
        // unnormalised sums, the row maximum and the probability sum
        const size_t row = ((size_t)blockIdx.y * a.L + qrow) * a.Hq + hq;
        float* op = a.part_o + row * HD + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 w = {o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]};
                *(float4*)(op + dt * 32 + 8 * g) = w;
            }
        if (h == 0) *(float2*)(a.part_ml + 2 * row) = float2{m, lt};
    } else {
        // scale back: o / (16 l)
        const float inv = 1.0f / (16.0f * lt);
        uint16_t* op = a.o + (size_t)qrow * a.ldo + (size_t)hq * HD + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 w = {pack_f16(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                                 pack_f16(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
                *(u32x2*)(op + dt * 32 + 8 * g) = w;
            }
    }
}

// Key splits: o = sum_s 2^(m_s - m) o_s / (16 sum_s 2^(m_s - m) l_s), m the
// largest m_s; a split that saw no visible key has m_s = -inf, l_s = 0.
// One thread per (row, head, 4 dims).
__global__ void __launch_bounds__(256) lut6_attention_combine_kernel(AttArgs a, int splits)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rows = (int64_t)a.L * a.Hq;
    if (t >= rows * (HD / 4)) return;
    const int64_t row = t / (HD / 4);
    const int d4 = (int)(t % (HD / 4));
    float mx = -__builtin_inff();
    for (int s = 0; s < splits; ++s) mx = fmaxf(mx, a.part_ml[2 * (s * rows + row)]);
    float w = 0.0f;
    float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < splits; ++s) {
        const float2 ml = *(const float2*)(a.part_ml + 2 * (s * rows + row));
        const float f = __builtin_amdgcn_exp2f(ml.x - mx);
        w += f * ml.y;
        const float4 v = *(const float4*)(a.part_o + (s * rows + row) * HD + 4 * d4);
        acc.x += f * v.x;
        acc.y += f * v.y;
        acc.z += f * v.z;
        acc.w += f * v.w;
    }
    const float inv = 1.0f / (16.0f * w);
    const int64_t qrow = row / a.Hq, hq = row % a.Hq;
    const u32x2 out = {pack_f16(acc.x * inv, acc.y * inv), pack_f16(acc.z * inv, acc.w * inv)};
    *(u32x2*)(a.o + qrow * a.ldo + hq * HD + 4 * d4) = out;
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

extern "C" int lut6_attention(const void* q, int64_t ldq, const void* k, int64_t ldk,
                              const void* v, int64_t ldv, void* o, int64_t ldo, int64_t L,
                              int64_t Lk, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                              hipStream_t stream)
{
    if (!q || !k || !v || !o) return LUT6_E_NULL;
    if (head_dim != HD || n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads) return LUT6_E_SHAPE;
    if (n_heads > 4096 || L < 0 || Lk < L || Lk > (int64_t)INT32_MAX - BKEY) return LUT6_E_SHAPE;
    if (ldq < n_heads * HD || ldo < n_heads * HD || ldk < n_kv_heads * HD || ldv < n_kv_heads * HD)
        return LUT6_E_SHAPE;
    // the key loop's copy offsets are 32-bit: up to 63 rows of k and v
    if (ldk > MAX_KV_LD || ldv > MAX_KV_LD) return LUT6_E_SHAPE;
    if (ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8) return LUT6_E_ALIGN;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LUT6_E_ALIGN;
    if (L == 0) return LUT6_OK;
    const size_t qb = ((size_t)(L - 1) * ldq + n_heads * HD) * 2;
    const size_t ob = ((size_t)(L - 1) * ldo + n_heads * HD) * 2;
    const size_t kb = ((size_t)(Lk - 1) * ldk + n_kv_heads * HD) * 2;
    const size_t vb = ((size_t)(Lk - 1) * ldv + n_kv_heads * HD) * 2;
    if (overlaps(o, ob, q, qb) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, vb)) return LUT6_E_ALIAS;

    AttArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
    a.ldq = ldq;
    a.ldk = ldk;
    a.ldv = ldv;
    a.ldo = ldo;
    a.L = (int)L;
    a.Lk = (int)Lk;
    a.Hq = (int)n_heads;
    a.grp = (int)(n_heads / n_kv_heads);
    a.nqb = (int)((L + BQ - 1) / BQ);
    const int64_t blocks = (int64_t)a.nqb * n_heads;
    if (blocks > INT32_MAX) return LUT6_E_SHAPE;
    // few workgroups (short query chunks over a long cache): split the keys
    // so that about 256 workgroups run, each over at least 4 key blocks
    const int nkb = (int)((Lk - 1) / BKEY + 1);
    int splits = 1;
    if (blocks < 128 && nkb >= 8) {
        splits = (int)((256 + blocks - 1) / blocks);
        if (splits > nkb / 4) splits = nkb / 4;
    }
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.kb_per_split = nkb;
    if (splits > 1) {
        a.kb_per_split = (nkb + splits - 1) / splits;
        splits = (nkb + a.kb_per_split - 1) / a.kb_per_split;
        const size_t rows = (size_t)L * n_heads * splits;
        void* ws = nullptr;
        const int st = lut6_detail::workspace(stream, WS_ATTENTION, rows * (HD + 2) * sizeof(float), &ws);
        if (st != LUT6_OK) return st;
        a.part_o = (float*)ws;
        a.part_ml = a.part_o + rows * HD;
        hipLaunchKernelGGL((lut6_attention_kernel<true, BKEY>), dim3((unsigned)blocks, (unsigned)splits), dim3(256),
                           0, stream, a);
        if (hipGetLastError() != hipSuccess) return LUT6_E_DEVICE;
        const int64_t threads = (int64_t)L * n_heads * (HD / 4);
        hipLaunchKernelGGL(lut6_attention_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, stream, a, splits);
    } else if (blocks >= SMALL_BLOCK_MIN_WGS) {
        hipLaunchKernelGGL((lut6_attention_kernel<false, BKEY_SMALL>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL((lut6_attention_kernel<false, BKEY>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? LUT6_OK : LUT6_E_DEVICE;
}
