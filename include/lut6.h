/*
 * lut6.h -- C ABI of the LUT-6 weight-quantized linear layer on AMD
 * Instinct MI355X (gfx950).
 *
 * The format (page "Clef-Flash-ANE-LUT6", section "Weight precision"): a
 * linear layer's weight W[N, K] (N output channels, K input features) is
 * stored as one 6-bit index per weight plus one table of 64 FP16 values per
 * 16 consecutive output channels; W[n, k] = table[n / 16][index(n, k)].
 * Section "LUT-6 text weights": four 6-bit indices are packed into three
 * bytes, little-endian, so that with its tables a layer with 4,096 inputs
 * takes about 6.02 bits per weight; activations are FP16, and the MLP
 * down-projection input is scaled up (by at most 16x) and the result scaled
 * back.
 *
 * Layouts (the readings this library takes where the page is silent):
 *   idx     uint8 [N, K] row-major, every value in 0..63 (host only).
 *   packed  uint8 [N, 3K/4] row-major.  Input columns 4j..4j+3 of row n form
 *           the 24-bit word w = i0 | i1<<6 | i2<<12 | i3<<18 (i0 = column
 *           4j), stored as bytes 3j, 3j+1, 3j+2 = w & 0xff, (w>>8) & 0xff,
 *           w >> 16.
 *   tables  FP16 [N/16, 64] row-major (128 bytes per table); table g serves
 *           output channels 16g..16g+15; entry = table[index], no offset.
 *   x       FP16 [L, K] row-major (L tokens).
 *   y       FP32 [L, N], FP16 [L, N] or FP16 [L, N/2] by epilogue.
 *
 * Ownership: the caller allocates, owns and frees every buffer.  Pointers
 * passed to lut6_linear / lut6_dequant are device pointers of the current
 * HIP device; pointers passed to lut6_pack / lut6_unpack are host pointers.
 * The library keeps no per-call state.  It owns lazily created device
 * workspaces, one of each kind per (device, stream): split-K partial sums,
 * and the expanded FP16 weight of the many-token path (see
 * lut6_linear_path); each is created on the first call that needs it and
 * grown when a later call needs more, both in stream order
 * (hipMallocAsync, and hipFreeAsync of the smaller buffer after the work
 * already enqueued on that stream: the host is not stopped), and freed by
 * lut6_release().
 *
 * Errors: every function returns LUT6_OK (0) or a named status, and launches
 * nothing on error.  Arguments are checked on the host; nothing is silently
 * truncated or padded.  Device-side failures of an enqueued launch surface
 * as LUT6_E_DEVICE when the launch itself fails, and otherwise at the
 * caller's next synchronisation, as usual in HIP.
 */
#ifndef LUT6_H
#define LUT6_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LUT6_OK = 0,
    LUT6_E_NULL = 1,         /* a required pointer is NULL                       */
    LUT6_E_SHAPE = 2,        /* sizes break a rule below                         */
    LUT6_E_ALIGN = 3,        /* a device pointer is not 16-byte aligned          */
    LUT6_E_SCALE = 4,        /* in_scale is not 1, 2, 4, 8 or 16                 */
    LUT6_E_EPILOGUE = 5,     /* unknown epilogue code                            */
    LUT6_E_INDEX_RANGE = 6,  /* lut6_pack: an index is above 63                  */
    LUT6_E_DEVICE = 7,       /* a HIP call or kernel launch failed               */
    LUT6_E_ALIAS = 8,        /* the output overlaps an input                     */
    LUT6_E_SCRATCH = 9       /* lut6_linear_noalloc: the shape needs more scratch
                              * than LUT6_NOALLOC_SCRATCH_BYTES                  */
} lut6_status;

typedef enum {
    /* y FP32 [L, N]: y = (sum_k fp16(x*s)[l,k] * W[n,k]) / s, rounded once  */
    LUT6_EPI_STORE_F32 = 0,
    /* y FP16 [L, N]: the same value rounded once to FP16 (nearest even)    */
    LUT6_EPI_STORE_F16 = 1,
    /* y FP16 [L, N/2]: rows [0, N/2) of W are the MLP gate, rows [N/2, N)
     * the up projection (tables likewise); y[l, j] = silu(a[l, j]) *
     * a[l, j + N/2] with a the scaled-back FP32 sum and
     * silu(g) = g / (1 + exp(-g)), rounded once to FP16                   */
    LUT6_EPI_SILU_MUL_F16 = 2
} lut6_epilogue;

/* Bytes of a packed [N, K] index matrix: N * 3K/4 (0 if K % 4 or a size
 * is not positive).                                                       */
size_t lut6_packed_bytes(int64_t N, int64_t K);

/* Bytes of the tables of an N-channel weight: (N/16) * 64 * 2 (0 if N % 16
 * or N is not positive).                                                  */
size_t lut6_table_bytes(int64_t N);

/* Pack idx [N, K] (host) into packed [N, 3K/4] (host), layout above.
 * N > 0, K > 0, K % 4 == 0 (else LUT6_E_SHAPE); an index above 63 is
 * refused with LUT6_E_INDEX_RANGE, never masked (packed is then
 * unspecified).  Synchronous.                                             */
int lut6_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K);

/* Inverse of lut6_pack: packed [N, 3K/4] (host) -> idx [N, K] (host).
 * Every byte string is a valid packing.  Synchronous.                     */
int lut6_unpack(const uint8_t* packed, uint8_t* idx, int64_t N, int64_t K);

/* The LUT-6 linear layer (page "Clef-Flash-ANE-LUT6", sections "Weight
 * precision" and "LUT-6 text weights"):
 *     xs = fp16(x * in_scale)          (round to nearest even, +-inf on overflow)
 *     a[l, n] = (sum_k xs[l, k] * W[n, k]) / in_scale,  FP32 accumulation
 *     y = epilogue(a)
 * Device pointers x (FP16 [L, K]), packed ([N, 3K/4]), tables (FP16
 * [N/16, 64]), y (see lut6_epilogue); all 16-byte aligned (LUT6_E_ALIGN).
 * Rules (LUT6_E_SHAPE): L >= 0, K > 0, N > 0, K % 64 == 0, N % 16 == 0, and
 * N % 32 == 0 for LUT6_EPI_SILU_MUL_F16; L, K, N at most 2^31 - 1, and
 * x (2LK bytes) and packed (3NK/4 bytes) each smaller than 2^31 bytes.
 * L == 0 is a no-op.
 * in_scale must be exactly 1, 2, 4, 8 or 16 (LUT6_E_SCALE), so the scaling
 * is exact.  y must not overlap x, packed or tables (LUT6_E_ALIAS).
 * Enqueues the work on `stream` (0 = null stream) and returns; results are
 * deterministic run to run (no floating-point atomics).                   */
int lut6_linear(const void* x, const uint8_t* packed, const void* tables, void* y,
                int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                hipStream_t stream);

/* Size of the static device array behind lut6_linear_noalloc: 256 MiB per
 * GPU, held from the library's load until the process ends.               */
#define LUT6_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* lut6_linear for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, rules, statuses, kernels and results as lut6_linear (the
 * same path and K split for every shape, so the output is bit-identical);
 * it never calls hipMalloc or hipFree and never synchronises.  The expanded
 * weight (LUT6_PATH_EXPANDED) and the split-K partial sums live in one
 * static device array of LUT6_NOALLOC_SCRATCH_BYTES per GPU instead of the
 * per-stream workspaces: expanded weight at offset 0, partial sums after it
 * on a 256-byte boundary.  A shape that needs more than that
 * (tiles_n * 8 * (K/64 + 1) * 4 KB for the expanded weight, rounded up to
 * 256 bytes, plus splits * L * N * 4 bytes of partial sums) is refused with
 * LUT6_E_SCRATCH before anything is launched.  Every shape of the 9B
 * model's projections fits, at any L.  Nothing in the array needs to start
 * at zero: each call writes what it reads.  All calls on one GPU share
 * its array, on any stream: two calls that overlap in time on one GPU race
 * and give unspecified results, so the caller orders them (one stream, or
 * events).                                                                */
int lut6_linear_noalloc(const void* x, const uint8_t* packed, const void* tables, void* y,
                        int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                        hipStream_t stream);

/* Kernel paths of lut6_linear (what lut6_linear_path returns).            */
typedef enum {
    /* L <= 192: the weight-streaming kernel (64-token x 32-channel tiles
     * over the whole K range; K split into slices, added by a second
     * kernel in a fixed order, only when the tiles are too few)           */
    LUT6_PATH_STREAM = 0,
    /* the fused kernel: 256 x 256 tiles, packed indices unpacked and looked
     * up in LDS per tile, FP16 MFMA                                       */
    LUT6_PATH_FUSED = 1,
    /* L >= 1536 (L >= 3072 when K >= 8192): the weight is expanded once
     * per call (the same unpack and lookup) into a workspace of
     * tiles_n * 8 * (K/64 + 1) * 4 KB, then an FP16 MFMA GEMM reads it
     * (tiles_n = ceil(N / 256); for LUT6_EPI_SILU_MUL_F16 a tile holds 128
     * gate|up row pairs, the same count); the fused kernel instead if that
     * workspace would reach 2 GB                                          */
    LUT6_PATH_EXPANDED = 2
} lut6_path;

/* The path lut6_linear takes for these sizes (a lut6_path value), or the
 * negated status lut6_linear would return for them (-LUT6_E_SHAPE,
 * -LUT6_E_EPILOGUE).  Host only; no device work.                          */
int lut6_linear_path(int64_t L, int64_t K, int64_t N, int epilogue);

/* Dequantize: w[n, k] = tables[n/16][index(n, k)] as FP16 bits [N, K] on
 * the device, with the same device unpack and lookup as lut6_linear.
 * N % 16 == 0, K % 64 == 0; 16-byte aligned pointers; enqueued on stream.
 * A bit copy: the result is exact.                                        */
int lut6_dequant(const uint8_t* packed, const void* tables, void* w,
                 int64_t N, int64_t K, hipStream_t stream);

/* int8 weight-only variant of lut6_linear (page "clef-flash — Core AI",
 * the bundle list at the top and section "Precision": int8 weights per
 * block of 32, weights only, activations FP16; the blocks are read as 32
 * consecutive inputs k of one output row).  The weight the layer uses is FP16, the value nearest
 * to q[n, k] * scales[n][k / 32]; everything else, including in_scale, the
 * epilogues and their rules, is as for lut6_linear.
 * q: device int8 [N, K], row-major; scales: device FP16 [N, K/32]; x, y as
 * for lut6_linear.  All 16-byte aligned (LUT6_E_ALIGN).  Same shape rules as
 * lut6_linear (LUT6_E_SHAPE); y must not overlap x, q or scales
 * (LUT6_E_ALIAS).  Up to 192 tokens the codes stream straight into the
 * products (no workspace); beyond, the weight is expanded into the
 * library's FP16 workspace and the FP16 GEMM reads it (split K when few
 * tiles, as lut6_linear).                                                 */
int lut6_int8_linear(const void* x, const int8_t* q, const void* scales, void* y,
                     int64_t L, int64_t K, int64_t N, float in_scale, int epilogue,
                     hipStream_t stream);

/* int8 code selection for lut6_int8_linear (page "clef-flash — Core AI",
 * section "Precision": int8 per block of 32, the mode named symmetric with
 * clipping, weights only).  The page names the mode only; read as: a block
 * is 32 consecutive inputs k of one row; scales[n][b] = the block's largest
 * magnitude / 127, rounded to FP16 (nearest, ties to even); q[n, k] = w / s
 * in FP32, rounded to nearest even and clamped to -127..127; a block whose
 * scale rounds to zero gets codes 0.  Weights must be finite (otherwise the
 * outputs are unspecified).
 * w: device FP16 [N, K], row-major, 16-byte aligned; q: device int8 [N, K],
 * 16-byte aligned; scales: device FP16 [N, K/32], 2-byte aligned
 * (LUT6_E_ALIGN); K % 32 == 0 (LUT6_E_SHAPE); no two overlapping
 * (LUT6_E_ALIAS).  Enqueued on stream; no workspace.                      */
int lut6_int8_quantize(const void* w, int8_t* q, void* scales, int64_t N, int64_t K,
                       hipStream_t stream);

/* Full attention of the attention layers, FP16 (page "Clef-Flash-ANE-LUT6",
 * section "Model architecture": query and key-value heads of size 256, full
 * attention; section "LUT-6 text weights": the probabilities are scaled up
 * by 16 in FP16 and scaled back afterwards).
 * The L queries are the last L of Lk positions: query i sees keys
 * 0 .. Lk - L + i.  Query head h reads key-value head h / (n_heads /
 * n_kv_heads).  o = softmax(q k^T / 16) v per head, computed as
 * (sum_j fp16(16 p_j) v_j) / (16 sum_j p_j) with p_j = exp(s_j - max) in
 * FP32, then rounded to FP16.
 * Layouts (device, FP16, row-major with element strides between token
 * rows): q [L, ldq] with head h at columns h*256 .. h*256+255; k and v
 * [Lk, ldk / ldv] with key-value head g at columns g*256 ..; o [L, ldo] like
 * q.  So the fused Q|K|V projection output can be passed in place (q = y,
 * k = y + 4096, v = y + 5120, ld = 6144).  The caller owns every buffer.
 * Rules: head_dim == 256, n_heads % n_kv_heads == 0, n_heads <= 4096,
 * 0 <= L <= Lk < 2^31 - 64, each ld >= its heads * 256, ldk and ldv at
 * most 2^24 (LUT6_E_SHAPE); pointers 16-byte aligned and every ld a
 * multiple of 8 (LUT6_E_ALIGN); o must not overlap q, k or v
 * (LUT6_E_ALIAS).  L == 0 is a no-op.  A call with fewer than 128
 * (query block of 128, head) pairs over at least 8 blocks of 64 keys
 * splits the keys over several workgroups; their partial sums go to a
 * library workspace of L x n_heads x splits x 1,032 bytes (splits <= 256),
 * created on the first call that needs it and kept until lut6_release.  */
int lut6_attention(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                   int64_t ldv, void* o, int64_t ldo, int64_t L, int64_t Lk, int64_t n_heads,
                   int64_t n_kv_heads, int64_t head_dim, hipStream_t stream);

/* Gated DeltaNet recurrence of the linear-attention layers (page
 * "Clef-Flash-ANE-LUT6", section "Model architecture": 16 key and 32 value
 * heads of size 128; page "clef-flash — Core AI", the decoder states: a
 * recurrent state [32, 128, 128] per layer, carried between calls).
 * The pages name the layer, not its update; read as the gated delta rule,
 * per value head h with key head h / (n_v_heads / n_k_heads), tokens in
 * order:  S <- exp(g_t) S;  d = beta_t (v_t - S^T k_t);  S <- S + k_t d^T;
 * o_t = S^T q_t / sqrt(128), rounded to FP16.  q and k are used as given
 * (any normalisation, convolution and gate computation come before).
 * Layouts (device): q, k FP16 [L, ldq / ldk], key head g at columns
 * g*128 ..; v FP16 [L, ldv] and o FP16 [L, ldo], value head h at columns
 * h*128 ..; g (log decay) and beta FP32 [L, ldg], head h at column h;
 * state FP32 [n_v_heads, 128, 128] (S[h][i][j], i over k, j over v), read
 * as the initial state and overwritten with the final one.  The caller
 * owns every buffer.
 * Rules: dk == dv == 128, n_v_heads % n_k_heads == 0, n_v_heads <= 4096,
 * 0 <= L < 2^31 - 64, each ld at least its row's width and ldq, ldk, ldv,
 * ldo at most 2^24 (LUT6_E_SHAPE); q,
 * k, v, o 16-byte aligned with ldq, ldk, ldv, ldo multiples of 8; g, beta,
 * state 4-byte aligned (LUT6_E_ALIGN); o and state must not overlap an
 * input or each other (LUT6_E_ALIAS).  L == 0 is a no-op.
 * From L = 64 the rule is evaluated in chunks of 64 positions counted from
 * the call's first token (page "clef-flash-LiteRT", section "Provenance,
 * conversion and license": a chunked kernel of 64 positions), on the matrix
 * cores; below 64, token by token.  The result is the same rule in either
 * order, within FP32 rounding; two calls with the state carried between
 * them give the bits of one call when the split falls on a multiple of 64
 * tokens (or both calls are shorter than 64).  The chunked form uses a
 * library workspace of n_v_heads x min(ceil(L/64), 128) x 33 KB (at most
 * 160 MB), created on the first call that needs it and kept until
 * lut6_release.                                                          */
int lut6_gated_delta(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                     int64_t ldv, const float* g, const float* beta, int64_t ldg, void* o,
                     int64_t ldo, float* state, int64_t L, int64_t n_k_heads, int64_t n_v_heads,
                     int64_t dk, int64_t dv, hipStream_t stream);

/* Fit the tables and write the packed indices of an FP16 weight [N, K]
 * (page "Clef-Flash-ANE-LUT6", section "LUT-6 text weights": one 64-entry
 * table per 16 output channels, from 40 rounds of one-dimensional k-means
 * started half at quantiles and half evenly between the group's minimum and
 * maximum).  The steps the page leaves open are fixed as follows, so that
 * the result is a function of the weight alone (bit for bit, on any run):
 *   - starting centres: the values of rank floor((2i + 1) n / 64),
 *     i = 0..31, of the group's n = 16 K values sorted, and
 *     min + (max - min) * j / 31, j = 0..31, in FP64, sorted;
 *   - a round assigns each value to its nearest centre (the lower one on a
 *     tie), replaces each centre by its cluster's mean (kept exactly: a sum
 *     of FP16 values in 2^-24 units, divided once in FP64), keeps the centre
 *     of an empty cluster, and sorts the centres;
 *   - tables[g] is the last centres rounded to FP16 (nearest, ties to
 *     even), sorted ascending (-0 before +0); each weight's index is its
 *     nearest entry (the lower one on a tie).
 * w: device FP16 [N, K], row-major; packed: device uint8 [N, 3K/4] (as
 * lut6_pack); tables: device FP16 [N/16, 64].  All three 16-byte aligned
 * (LUT6_E_ALIGN) and not overlapping (LUT6_E_ALIAS).  N % 16 == 0,
 * K % 64 == 0 and 16 K <= 2^22 (LUT6_E_SHAPE).  Every weight must be
 * finite; for a group holding inf or NaN the outputs are unspecified.
 * Enqueued on stream.  The first call allocates a library workspace of
 * 768 KB per workgroup (at most 256 workgroups: 192 MB), kept until
 * lut6_release.                                                           */
int lut6_quantize(const void* w, uint8_t* packed, void* tables, int64_t N, int64_t K,
                  hipStream_t stream);

/* Free the library's per-device workspaces (after synchronising the
 * devices that hold one): split-K partial sums and the expanded weight
 * (lut6_linear, lut6_int8_linear), the table-fitting scratch
 * (lut6_quantize), the key-split partials (lut6_attention) and the chunk
 * matrices of the recurrence (lut6_gated_delta).  Optional;
 * safe to call at any time when no call of the library is in flight.     */
int lut6_release(void);

/* Name of a status code ("LUT6_OK", "LUT6_E_SHAPE", ...); never NULL.     */
const char* lut6_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LUT6_H */
