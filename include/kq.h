/*
 * kq.h -- C ABI of libkq, an INT8 quantized linear layer for AMD Instinct
 * MI355X (gfx950).
 *
 * What the library computes (one linear layer, y = x W^T + bias, with both
 * operands quantized):
 *   - activations x (bf16, [M,K], one row per token) are quantized per token
 *     to int8 with an fp32 scale, inside the linear call;
 *   - weights W ([N,K], one row per output channel) are quantized offline,
 *     either to int8 with one fp32 scale per output channel, or to packed
 *     unsigned int4 with an fp16 scale and an fp16 offset per group of 64
 *     consecutive K;
 *   - an INT8 x INT8 -> INT32 matrix product runs on the MFMA units, and the
 *     dequantization (token scale x channel or group scale) and the bias add
 *     are fused into the same kernel's epilogue.
 *
 * Sources of the method (the pages are cited by title and section):
 *   [qlip]   "qlip-mlx" README (TheStageAI), the w8a8_linear / w4a8_linear
 *            feature bullets and "Quick start": W8A8 GEMM with per-token
 *            activation quantization inside the kernel, INT8xINT8->INT32
 *            matmul, dequant+bias fused into one node; quantize_weight_int8
 *            maps [N,K] fp weights to int8 plus fp32 scales; W4A8 keeps the
 *            same INT8 compute with weights stored as packed int4; calls with
 *            M <= 16 take a register-dequant GEMV.
 *   [mlx4722] MLX pull request 4722 (staged int8 affine quantized matmul),
 *            "Selector rules": affine weights, 2-D transposed [N,K] weight
 *            layout, K % 64 == 0, K/64 <= 1024, non-batched operands, group
 *            sizes 32/64/128 (this library: 64).
 *   [sage]   "qlip-mlx" README, sage_attention bullet, "Key features" and
 *            "Quick start": INT8 QK^T inside a flash-attention structure
 *            with exact online softmax; quantization touches only QK^T,
 *            with per-token / per-block scales; softmax and P.V stay in
 *            floating point; head dim 128, mask-free; q/k/v [B, heads, L,
 *            128] or tokens-first; scale 128^-0.5; fp16 output in the same
 *            layout.  The method is SageAttention's (published by Zhang et
 *            al.): K is smoothed by its mean over the tokens before the
 *            quantization.
 *   [kquant] mlx-kquant pull request 89 commit list: routes must not round
 *            beyond one weight and one output rounding; errors other than a
 *            declined route raise; the route decision is one tested function;
 *            a quantized matmul whose epilogue adds a gated residual.
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense, row-major, non-batched (callers flatten [B,L,K]
 *     to [M,K]).  Device pointers must be 16-byte aligned.
 *   - "device" pointers are HIP device allocations on the current device;
 *     "host" pointers are ordinary process memory.
 *   - The caller owns every buffer, the workspace included.  The library
 *     allocates no memory, keeps no pointer after a call returns, and never
 *     synchronizes: work is enqueued on `stream` (a hipStream_t; NULL means
 *     the null stream) and buffers must stay alive until it completes.
 *   - Every call returns a kq_status.  On failure nothing is enqueued (except
 *     KQ_ERR_LAUNCH) and kq_last_error() returns a message of the form
 *     "[kq_w4a8_linear] K=100 must be a multiple of 64".  No C++ exception
 *     and no abort crosses the ABI.
 *   - Shapes with M == 0 or N == 0 are valid and enqueue nothing.
 *   - Inputs must be finite.  Weights must satisfy |w| < 65504 for the int4
 *     format (its scale and offset are fp16).
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kq_status {
    KQ_SUCCESS = 0,
    KQ_ERR_INVALID_VALUE = 1, /* null pointer, negative size, misalignment */
    KQ_ERR_UNSUPPORTED = 2,   /* valid request outside the supported envelope */
    KQ_ERR_NO_DEVICE = 3,     /* no gfx950 device current */
    KQ_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
    KQ_ERR_LAUNCH = 5         /* the HIP runtime rejected a kernel launch */
} kq_status;

typedef enum kq_wformat {
    /* int8 codes [N,K], fp32 scale [N]; w ~= scale[n] * q[n,k]. */
    KQ_W8_PER_CHANNEL = 0,
    /* uint8 [N,K/2] with two 4-bit codes per byte (low nibble = even k),
     * fp16 scale [N,K/64] and fp16 offset [N,K/64];
     * w ~= scale[n,g] * q[n,k] + offset[n,g] with g = k / 64, q in [0,15]. */
    KQ_W4_AFFINE_G64 = 1
} kq_wformat;

/* Order of the activation codes within a row, for the entry points that
 * hand codes over (kq_quantize_act_ordered, kq_w4a8_gemm_ordered). */
typedef enum kq_code_order {
    KQ_CODES_NATURAL = 0, /* a[m,k] at byte m*K + k */
    /* each run of 8 codes k = 8j..8j+7 of a row stored as its even codes,
     * then its odd ones: bytes m*K + 8j + (0..7) hold k = 8j + {0, 2, 4, 6,
     * 1, 3, 5, 7}.  The order in which the int4 GEMM unpacks a packed
     * weight dword (low nibbles = even k, high nibbles = odd k), so its
     * weights need no reordering; K % 8 == 0. */
    KQ_CODES_SPLIT8 = 1
} kq_code_order;

typedef enum kq_dtype {
    KQ_DTYPE_F32 = 0,  /* fp32 output, rounded once from the exact result */
    KQ_DTYPE_BF16 = 1, /* bf16 output: the fp32 result rounded to nearest even */
    /* Debug output of the integer accumulators.  W8A8: int32 [M,N] holding
     * sum_k a[m,k]*q[n,k].  W4A8 / GEMV: int32 [K/64, M, N] holding, per
     * 64-wide K group g, P[g,m,n] = sum_{k in g} a[m,k]*q[n,k]. */
    KQ_DTYPE_I32 = 2
} kq_dtype;

typedef enum kq_route_kind {
    KQ_ROUTE_GEMM = 0, /* LDS-tiled MFMA GEMM */
    KQ_ROUTE_GEMV = 1, /* weight-streaming register-dequant kernels: 16x16 output
                          blocks over all of K (M <= 16, or thin N); M <= 2
                          with K <= 6144 takes kernels with 8 lanes per
                          output column (32 columns per workgroup, v_dot4
                          products; int4 and int8 weights), unless the
                          environment variable KQ_GEMV_LANE=0 */
    KQ_ROUTE_FUSED = 2 /* the linears' activation quantization inside the
                          product kernel, one launch and no codes stored
                          ([qlip] W8A8 bullet: quantization inside the
                          kernel), K <= 6144: M <= 4 on the GEMV kernel
                          (which quantizes its rows in its prologue), and
                          thin N (N <= 64) with M > 16 and M*N <= 2^19 (any M
                          for N <= 32), where one kernel quantizes 8 rows of
                          x in registers and computes all N columns of them */
} kq_route_kind;

/* Launch plan chosen for one linear call (see kq_route). */
typedef struct kq_route_info {
    int32_t kind;     /* kq_route_kind */
    int32_t tile_m;   /* output rows per workgroup */
    int32_t tile_n;   /* output columns per workgroup */
    int32_t threads;  /* threads per workgroup */
    int64_t grid;     /* workgroups in the main kernel */
    int32_t splits;   /* K slices of the GEMM (1: none).  With more, each
                         slice writes exact int32 partial sums [splits,M,N]
                         to the workspace and a fold kernel adds them and
                         applies the epilogue, so the result is the same,
                         bit for bit, as the unsplit product's. */
    int32_t reserved;
} kq_route_info;

/* Largest K the linears accept: 65536 * 127 * 127 < 2^31, so the int32
 * accumulator cannot overflow ([mlx4722] "Selector rules": K/64 <= 1024). */
#define KQ_MAX_K 65536
/* Largest M of the GEMV route ([qlip] W4A8 bullet: M <= 16). */
#define KQ_GEMV_MAX_M 16
/* Largest K of the GEMV route. */
#define KQ_GEMV_MAX_K 16384

/* 1 if the current HIP device is a gfx950 (MI355X class) GPU, else 0.
 * [qlip] "Key features": the package is a clean no-op where the INT8 matrix
 * hardware is missing (is_available() -> False).  Never fails. */
int kq_is_available(void);

/* Message of the last failed call on this thread ("" if none), in the
 * "[op] reason" form of the argument checks MLX pull request 3026 reviews
 * for its quantized SDPA (invalid arguments name the op and the bad value).
 * The string is owned by the library and valid until the next call on this
 * thread. */
const char* kq_last_error(void);

/* Bytes of device workspace a linear call with this shape and weight format
 * needs (MLX pull request 4722 stages a quantized matmul through int8
 * activations, "quantize_x", before the integer product; here that stage's
 * output lives in this caller-owned workspace): int8 activation codes
 * (M rounded up to 16, times K: where the route takes the MFMA GEMV the
 * codes are stored in its 16-row fragment order), fp32 token scales
 * (4*M), for the int4
 * format the per-group code sums (4*M*K/64), and when the route splits K
 * (kq_route_info.splits > 1) the int32 partial sums (4*splits*M*N), each
 * region 256-byte aligned.  The fused routes (KQ_ROUTE_FUSED) store no
 * codes and use only 4*M bytes of token scales at offset 0; the size
 * returned still covers the two-kernel route of the same shape, so one
 * workspace serves every linear entry point (kq_gemv_small_m included) and
 * KQ_FUSE setting.  Returns 0 for M == 0 or N == 0.  Pure host function; it
 * reads the same environment levers as the route. */
size_t kq_workspace_bytes(int64_t M, int64_t N, int64_t K, kq_wformat fmt);

/* Launch plan of a linear call; pure host function, no device access.
 * [kquant]: the route decision is one tested function.  Routing: with
 * K <= 6144, M <= 4 takes the GEMV with the activation quantization in its
 * prologue, and N <= 64 with M > 16 and M*N <= 2^19 (any M for N <= 32)
 * the fused thin-N kernel (one launch each; the environment variable
 * KQ_FUSE=0 turns both off).  Otherwise, with
 * K <= KQ_GEMV_MAX_K, M <= 16 or N <= 64 (thin N: the GEMM's tiles would
 * leave most of the GPU idle) takes the GEMV, and so does M <= 32 (two
 * 16-row blocks, measured faster than the GEMM at 5120 x 13824), unless
 * the environment
 * variable KQ_FORCE_ROUTE=gemm; KQ_FORCE_ROUTE=gemv forces the GEMV (and
 * fails for shapes it cannot take: M > 16 or K > KQ_GEMV_MAX_K).
 * An int8-weight GEMM whose tiles would leave more than half of the 256
 * CUs idle splits K into slices of at least 512 (at most 16 slices)
 * ([kquant] split-K: partials folded so the result rounds once); the
 * environment variable KQ_SPLIT=n forces n slices (1: never split).  The
 * kq_w8a8_gemm / kq_w4a8_gemm entry points, which take no workspace, never
 * split.
 * Returns KQ_ERR_INVALID_VALUE / KQ_ERR_UNSUPPORTED for shapes the linears
 * reject, with the same messages. */
kq_status kq_route(int64_t M, int64_t N, int64_t K, kq_wformat fmt,
                   kq_dtype y_dtype, kq_route_info* out /* host */);

/* Offline weight quantization ([qlip] "Quick start": quantize_weight_int8
 * maps [N,K] weights to int8 plus fp32 scales; [mlx4722]: affine 4-bit
 * weights with per-group scale and bias, group 64).
 *   w      device fp32 [N,K]
 *   KQ_W8_PER_CHANNEL: wq = int8 [N,K]; scale = fp32 [N]; gbias must be NULL.
 *     Per row n: amax = max_k |w|; if 127/amax overflows (amax == 0 or
 *     tiny) the row is all zero with scale 0; else inv = fp32(127/amax),
 *     q = clamp(rint(fp32(w*inv)), -127, 127), scale = fp32(amax/127).
 *   KQ_W4_AFFINE_G64: wq = uint8 [N,K/2]; scale = fp16 [N,K/64];
 *     gbias = fp16 [N,K/64]; K % 64 == 0.  Per group: lo = min, hi = max,
 *     scale = fp16(fp32((hi-lo)/15)), offset = fp16(lo); if scale == 0 the
 *     codes are 0, else q = clamp(rint(fp32(fp32(w-offset) * fp32(1/scale))),
 *     0, 15).
 * Rounding is IEEE round-to-nearest-even throughout; results are bit-exact
 * and deterministic. */
kq_status kq_quantize_weights(const float* w, int64_t N, int64_t K,
                              kq_wformat fmt, void* wq, void* scale,
                              void* gbias, void* stream);

/* Per-token activation quantization ([qlip] w8a8_linear bullet: activations
 * quantize dynamically per token; [mlx4722]: the activation-quantize kernel
 * handles K that is not a multiple of 32).
 *   x     device bf16 [M,K] (raw bf16 bit patterns), any K >= 1
 *   a     device int8 [M,K] codes      (output)
 *   sx    device fp32 [M] token scales (output)
 *   gsum  device int32 [M,K/64] sums of the codes of each 64-wide K group,
 *         or NULL; non-NULL requires K % 64 == 0 (output)
 * Same rule as the int8 weight rows: amax over the row, inv = fp32(127/amax),
 * codes = clamp(rint(fp32(x*inv)), -127, 127), sx = fp32(amax/127), and an
 * all-zero row (sx = 0) when 127/amax overflows.  Bit-exact. */
kq_status kq_quantize_act(const void* x, int64_t M, int64_t K, int8_t* a,
                          float* sx, int32_t* gsum, void* stream);

/* W8A8 linear ([qlip] w8a8_linear: per-token activation quantization,
 * INT8xINT8->INT32 matmul, dequant+bias fused).
 *   x     device bf16 [M,K]
 *   wq    device int8 [N,K], sw device fp32 [N] (from kq_quantize_weights)
 *   bias  device fp32 [N] or NULL
 *   y     device [M,N] of y_dtype:
 *           F32/BF16: y = sx[m]*sw[n]*acc[m,n] + bias[n], acc = sum_k a*q,
 *           computed in fp32 and rounded to y_dtype;
 *           I32: acc itself.
 *   ws    device workspace of at least kq_workspace_bytes(M,N,K,KQ_W8_...)
 * Requires 64 <= K <= KQ_MAX_K and K % 64 == 0.  M <= 16 routes to the GEMV
 * kernel (see kq_route). */
kq_status kq_w8a8_linear(const void* x, int64_t M, int64_t K, int64_t N,
                         const int8_t* wq, const float* sw, const float* bias,
                         void* y, kq_dtype y_dtype, void* ws, size_t ws_bytes,
                         void* stream);

/* W4A8 linear ([qlip] w4a8_linear: the same INT8 compute with weights
 * stored as packed int4; [mlx4722]: stage weights and activations as int8
 * instead of dequantizing).  Arguments as kq_w8a8_linear, with the int4
 * weights of kq_quantize_weights(KQ_W4_AFFINE_G64):
 *   wq4   device uint8 [N,K/2]; gscale, gbias device fp16 [N,K/64]
 *   y (F32/BF16) = sx[m] * sum_g (gscale[n,g]*P[g,m,n] + gbias[n,g]*A[m,g])
 *                  + bias[n], with P the per-group int8 products and A the
 *                  per-group code sums; y (I32) = P as int32 [K/64,M,N]. */
kq_status kq_w4a8_linear(const void* x, int64_t M, int64_t K, int64_t N,
                         const uint8_t* wq4, const void* gscale,
                         const void* gbias, const float* bias, void* y,
                         kq_dtype y_dtype, void* ws, size_t ws_bytes,
                         void* stream);

/* Linears on activations already quantized by kq_quantize_act: the same
 * kernels, routes and results as kq_w8a8_linear / kq_w4a8_linear, without
 * the activation pass.  One quantization can then feed several linears that
 * read the same activations (a DiT block's q/k/v projections, or its
 * modulation fan-out).
 *   a     device int8 [M,K] codes, sx device fp32 [M] scales
 *   gsum  device int32 [M,K/64] group sums (int4 weights only)
 * Other arguments, constraints and outputs as the corresponding linear; no
 * workspace is needed. */
kq_status kq_w8a8_gemm(const int8_t* a, const float* sx, int64_t M, int64_t K,
                       int64_t N, const int8_t* wq, const float* sw,
                       const float* bias, void* y, kq_dtype y_dtype,
                       void* stream);

kq_status kq_w4a8_gemm(const int8_t* a, const float* sx, const int32_t* gsum,
                       int64_t M, int64_t K, int64_t N, const uint8_t* wq4,
                       const void* gscale, const void* gbias,
                       const float* bias, void* y, kq_dtype y_dtype,
                       void* stream);

/* The same per-token quantization and int4 linear with the codes in a
 * chosen order ([qlip] w4a8_linear bullet: activations quantized once feed
 * the in-register int4 unpack; kq_code_order).  kq_quantize_act_ordered
 * with KQ_CODES_NATURAL is kq_quantize_act; with KQ_CODES_SPLIT8 it writes
 * the same codes, scales and group sums, the codes of each run of 8 in the
 * split order (K % 8 == 0, else KQ_ERR_UNSUPPORTED).
 * kq_w4a8_gemm_ordered reads codes in `order`: KQ_CODES_NATURAL is
 * kq_w4a8_gemm; KQ_CODES_SPLIT8 always takes the tiled int4 GEMM (the
 * kernel kq_w4a8_linear uses there: its weights then need no reordering),
 * for any M, with results identical to kq_w4a8_gemm on the natural codes
 * (the int32 group products are the same sums); KQ_FORCE_ROUTE=gemv with
 * split codes is KQ_ERR_UNSUPPORTED.  Other arguments as kq_quantize_act /
 * kq_w4a8_gemm; an unknown order is KQ_ERR_INVALID_VALUE. */
kq_status kq_quantize_act_ordered(const void* x, int64_t M, int64_t K,
                                  int8_t* a, float* sx, int32_t* gsum,
                                  kq_code_order order, void* stream);

kq_status kq_w4a8_gemm_ordered(const int8_t* a, const float* sx,
                               const int32_t* gsum, int64_t M, int64_t K,
                               int64_t N, const uint8_t* wq4,
                               const void* gscale, const void* gbias,
                               const float* bias, void* y, kq_dtype y_dtype,
                               kq_code_order order, void* stream);

/* Small-M GEMV ([qlip] w4a8_linear bullet: a register-dequant GEMV path for
 * M <= 16 runs decode-style calls at weight-bandwidth speed).  Same math and
 * arguments as kq_w4a8_linear (fmt = KQ_W4_AFFINE_G64: wq, scale, gbias as
 * there) or kq_w8a8_linear (fmt = KQ_W8_PER_CHANNEL: wq int8, scale fp32 [N],
 * gbias NULL), always on the GEMV kernel.  Requires 1 <= M <= 16 and
 * K <= KQ_GEMV_MAX_K (each wavefront keeps its K slice of the activations in
 * registers); the linears route larger K to the GEMM.  For M <= 4 and
 * K <= 6144 the GEMV quantizes x in its prologue (one launch, the same
 * results bit for bit), unless KQ_FUSE=0 or KQ_FORCE_ROUTE=gemv. */
kq_status kq_gemv_small_m(kq_wformat fmt, const void* x, int64_t M, int64_t K,
                          int64_t N, const void* wq, const void* scale,
                          const void* gbias, const float* bias, void* y,
                          kq_dtype y_dtype, void* ws, size_t ws_bytes,
                          void* stream);

/* Linear with the gated residual epilogue of a DiT block ([kquant]: a
 * quantized matmul with a gated residual epilogue; the pages give no
 * formula, and the reading taken is the DiT block's gated residual add):
 *   y[m,n] = residual[m,n] + gate[m / gate_rows, n] * lin[m,n]
 * where lin is what kq_w8a8_linear (fmt = KQ_W8_PER_CHANNEL) or
 * kq_w4a8_linear (fmt = KQ_W4_AFFINE_G64) computes in fp32, bias included.
 * The gate and residual terms are applied in the same kernel's epilogue as
 * one fp32 fma, and y is rounded once to y_dtype.
 *   wq, scale, gbias, bias   as the corresponding linear (gbias NULL for int8)
 *   residual  device bf16 [M,N] (16-byte aligned), or NULL for zero.  It may
 *             be y itself when y_dtype is BF16 (in place); any other
 *             overlap with y is rejected.
 *   gate      device fp32 [ceil(M/gate_rows), N] (4-byte aligned), or NULL
 *             for one.  One gate row serves gate_rows consecutive token rows
 *             (a DiT batch of B samples of L tokens each: gate_rows = L).
 *   gate_rows >= 1
 *   y_dtype   F32 or BF16 (I32 has no epilogue and is rejected)
 * Routes, workspace and the other constraints as the plain linears; with
 * residual and gate both NULL the result is the plain linear's, bit for
 * bit. */
kq_status kq_linear_gated(kq_wformat fmt, const void* x, int64_t M, int64_t K,
                          int64_t N, const void* wq, const void* scale,
                          const void* gbias, const float* bias,
                          const void* residual, const float* gate,
                          int64_t gate_rows, void* y, kq_dtype y_dtype,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * INT8 attention ([sage]).
 *
 * For each batch b and head h, with q [Lq,128], k and v [Lk,128] fp16:
 *   kmean = the mean of k over its Lk tokens, per channel: the exact sum
 *           (fp16 values as integers in units of 2^-24) converted to fp64,
 *           scaled by 2^-24, divided by Lk in fp64, rounded to fp32;
 *   ks    = fp32(k - kmean);
 *   qc, sq / kc, sk = int8 codes and per-token fp32 scales of q / ks, one
 *           absmax scale per block of q_block / k_block consecutive tokens
 *           (the linears' rule: inv = fp32(127/amax), codes =
 *           clamp(rint(fp32(v*inv)), +-127), scale = fp32(amax/127), 0 for
 *           an all-zero block);
 *   S     = scale * sq[i] * sk[j] * (qc[i] . kc[j])   (exact int32 dot);
 *   out   = softmax_j(S) v, in fp32 with P rounded to fp16 for the P.v
 *           product, rounded to fp16.
 * Codes, scales and kmean are bit-exact; out is within the rounding of P
 * and of the output (see the tests for the bound).
 *
 * Tensors: q, out [B,H,Lq,128] and k, v [B,H,Lk,128] fp16, dense, in the
 * layout given (KQ_LAYOUT_BHLD: heads-first, KQ_LAYOUT_BLHD: tokens-first
 * [B,L,H,128]), 16-byte aligned device memory.  Requirements: D = 128;
 * 1 <= q_block, k_block <= 128, powers of two; scale > 0 and finite;
 * B*H <= 65535; Lq, Lk <= 2^22; Lk >= 1 when Lq >= 1 (B, H or Lq = 0
 * enqueues nothing).  Inputs must be finite.
 * ------------------------------------------------------------------------ */
typedef enum kq_layout {
    KQ_LAYOUT_BHLD = 0,
    KQ_LAYOUT_BLHD = 1
} kq_layout;

/* Workspace of the attention: byte offsets of its regions and the total.
 * After kq_sage_prepare (or kq_sage_attention) it holds, with BH = B*H,
 * lq_pad / lk_pad = Lq / Lk rounded up to 128:
 *   qc    int8  [BH][lq_pad][128]  query codes (rows past Lq zero)
 *   sq    fp32  [BH][lq_pad]       per-token query scales (0 past Lq)
 *   kc    int8  [BH][lk_pad][128]  smoothed key codes
 *   sk    fp32  [BH][lk_pad]       per-token key scales
 *   vt    fp16  [BH][lk_pad/64][128][64]  v transposed per 64-key block,
 *                keys permuted within each 32-key half (slot 8g+i holds
 *                key 4g+i for i < 4, key 16+4g+(i-4) for i >= 4), zero
 *                past Lk
 *   kmean fp32  [BH][128]          the key means
 *   colsum int64 [BH][chunks][128] partial key sums (units of 2^-24)
 *   meta  int32 [4]                {k_block, q_block} of the preparation */
typedef struct kq_sage_workspace {
    int64_t lq_pad, lk_pad, chunks;
    size_t qc, sq, kc, sk, vt, kmean, colsum, meta, total;
} kq_sage_workspace;

kq_status kq_sage_workspace_layout(int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                   kq_sage_workspace* out /* host */);

/* The preparation pass alone: key means, codes and scales, transposed v,
 * written into the workspace. */
kq_status kq_sage_prepare(const void* q, const void* k, const void* v, int64_t B,
                          int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                          kq_layout layout, int64_t q_block, int64_t k_block,
                          void* ws, size_t ws_bytes, void* stream);

/* The attention alone, on a workspace kq_sage_prepare filled for the same
 * B, H, Lq and Lk.  k_block >= 64 asserts that every 64-key step shares one
 * key scale and takes the faster kernel for it.  The library keeps, per
 * workspace address, the shape and key block of the last kq_sage_prepare
 * this process issued on it, and returns KQ_ERR_INVALID_VALUE (nothing
 * enqueued) when the call's B, H, Lq or Lk differ from it, or when k_block
 * >= 64 meets a workspace prepared with a smaller k_block.  A workspace this
 * process never prepared is not checked on the host; for it, the kernel
 * compares the assertion with the key block the preparation wrote into the
 * workspace (meta) and, on a mismatch, writes NaN to every output element
 * instead of wrong values.  A k_block below 64 is correct on any prepared
 * workspace. */
kq_status kq_sage_attend(const void* ws, size_t ws_bytes, void* out, int64_t B,
                         int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                         kq_layout layout, float scale, int64_t k_block,
                         void* stream);

/* Both: out = INT8 attention of q, k, v. */
kq_status kq_sage_attention(const void* q, const void* k, const void* v, void* out,
                            int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                            kq_layout layout, float scale, int64_t q_block,
                            int64_t k_block, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's own device scratch on each GPU (64 MiB). */
#define KQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kq_w8a8_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus ws, ws_bytes),
 * routes, kernels and results, bit for bit, as kq_w8a8_linear; the
 * workspace is a fixed array of KQ_NOALLOC_SCRATCH_BYTES in the library's
 * device memory, one per GPU, held until the process ends.  The call
 * allocates nothing.
 *   Limit: kq_workspace_bytes(M, N, K, KQ_W8_PER_CHANNEL) must not exceed
 *   KQ_NOALLOC_SCRATCH_BYTES (e.g. M*K <= 64 MiB less the token scales);
 *   larger shapes return KQ_ERR_UNSUPPORTED and enqueue nothing.
 *   Concurrency: every call on one GPU shares that GPU's array, and it keeps
 *   the last call's contents (no kernel reads what it did not write in the
 *   same call, so nothing needs clearing).  Calls that may overlap on one
 *   GPU (several streams, several threads) race on it and must be
 *   serialized by the caller. */
kq_status kq_w8a8_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t N,
                                 const int8_t* wq, const float* sw,
                                 const float* bias, void* y, kq_dtype y_dtype,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Measurement probes: the machine's own floors beside its published peaks,
 * for roofline figures (mlx-kquant pull request 89 commit list: a DiT-shape
 * harness with a three-floor roofline).  They compute nothing of the
 * method.
 * ------------------------------------------------------------------------ */

/* Streaming read of `bytes` at src (device, 16-byte aligned, bytes a
 * multiple of 16), split into `grid` equal contiguous ranges, one per
 * workgroup of `threads` (64..1024, a multiple of 64) threads, with 16-byte
 * non-temporal loads.  sink: device uint32 [grid]; it is written only if a
 * data-dependent test that practically never holds succeeds, so the probe
 * moves the buffer's bytes and writes (almost surely) nothing.  Timing it
 * gives the HBM read rate a kernel with that grid can reach. */
kq_status kq_probe_read(const void* src, int64_t bytes, int64_t grid,
                        int32_t threads, uint32_t* sink, void* stream);

/* iters x 8 v_mfma_i32_16x16x64_i8 per wavefront on register operands, 8
 * wavefronts per workgroup, `grid` workgroups: 2^21 * iters * grid integer
 * operations (2^15 per instruction, a multiply-add counted as two) with no
 * memory traffic.
 * sink: device int32 [grid], written as for kq_probe_read. */
kq_status kq_probe_mfma_i8(int64_t iters, int64_t grid, int32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
