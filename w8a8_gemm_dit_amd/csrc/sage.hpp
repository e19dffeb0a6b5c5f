// Internal interface of the INT8 attention (SageAttention-style): the
// workspace layout shared by the host code and the kernels, and the
// launchers.  The method ("qlip-mlx" README, sage_attention bullet and "Key
// features"): K smoothed by its mean over the tokens, Q and the smoothed K
// quantized to int8 with one absmax scale per block of tokens, the scores
// from an INT8 x INT8 -> INT32 product, then an exact online softmax and
// P.V in floating point (fp16 P and V, fp32 accumulation), fp16 output.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kq {

constexpr int kSageD = 128;       // head dimension
constexpr int kSageQTile = 128;   // query rows per attention workgroup
constexpr int kSageKTile = 64;    // keys per attention step
constexpr int kSageRowTile = 128; // tokens per quantization workgroup
constexpr int kSageChunk = 256;   // tokens per key column-sum partial

// Element strides of a [B, H, L, 128] tensor whose 128 channels are
// contiguous (heads-first or tokens-first layouts).
struct SageStrides {
  int64_t b, h, l;
};

// Workspace regions (byte offsets, each 256-byte aligned).  BH = B*H,
// Lqp = Lq rounded up to 128, Lkp = Lk rounded up to 128.
//   qc     int8  [BH][Lqp][128]   query codes (padding rows zero)
//   sq     fp32  [BH][Lqp]        per-token query scales (block scale)
//   kc     int8  [BH][Lkp][128]   smoothed key codes
//   sk     fp32  [BH][Lkp]        per-token key scales
//   vt     fp16  [BH][Lkp/64][128][64]  V transposed per 64-key block: row d
//                holds the block's 64 values of channel d, keys permuted
//                within each 32-key half (slot 8g+i <- key 4g+i for i < 4,
//                key 16+4g+i-4 for i >= 4), which is the order the P.V
//                product consumes them in
//   kmean  fp32  [BH][128]        the key means
//   colsum int64 [BH][nchunk][128] per-chunk key column sums (units 2^-24)
//   meta   int32 [4]              {k_block, q_block} the preparation used
//                (the attention checks that the key blocks it assumes match)
struct SageLayout {
  int64_t BH, Lqp, Lkp, nchunk;
  size_t qc, sq, kc, sk, vt, kmean, colsum, meta, total;
};

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

inline SageLayout sage_layout(int64_t B, int64_t H, int64_t Lq, int64_t Lk) {
  SageLayout s{};
  s.BH = B * H;
  s.Lqp = round_up(Lq, kSageRowTile);
  s.Lkp = round_up(Lk, kSageRowTile);
  s.nchunk = (Lk + kSageChunk - 1) / kSageChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  s.qc = take((size_t)(s.BH * s.Lqp * kSageD));
  s.sq = take((size_t)(s.BH * s.Lqp * 4));
  s.kc = take((size_t)(s.BH * s.Lkp * kSageD));
  s.sk = take((size_t)(s.BH * s.Lkp * 4));
  s.vt = take((size_t)(s.BH * s.Lkp * kSageD * 2));
  s.kmean = take((size_t)(s.BH * kSageD * 4));
  s.colsum = take((size_t)(s.BH * s.nchunk * kSageD * 8));
  s.meta = take(16);
  s.total = off;
  return s;
}

// Preparation: key column sums, smoothed and quantized keys, quantized
// queries, transposed values (all into the workspace).  Returns the name of
// the last kernel.
const char* launch_sage_prepare(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                SageStrides sq, SageStrides sk, SageStrides sv, int64_t B,
                                int64_t H, int64_t Lq, int64_t Lk, int q_block, int k_block,
                                char* ws, const SageLayout& L, hipStream_t s);

// Attention on a prepared workspace; out fp16 with strides so.
// k_uniform: every 64-key step shares one key scale (k_block >= 64).
const char* launch_sage_attend(const char* ws, const SageLayout& L, uint16_t* out,
                               SageStrides so, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                               float scale, bool k_uniform, hipStream_t s);

}  // namespace kq
