// Quantization kernels of libkq.
//
// Activation rule ("qlip-mlx" README, w8a8_linear bullet: per-token
// activation quantization inside the kernel, no calibration), applied per
// row: amax = max |x|; inv = fp32(127/amax); codes = clamp(rint(x*inv),
// -127, 127); scale = fp32(amax/127); rows whose 127/amax overflows become
// zero with scale 0.  The same rule quantizes int8 weight rows ("qlip-mlx"
// README, "Quick start": quantize_weight_int8 gives int8 codes and fp32
// per-output-channel scales).  Int4 weights are min-max affine per 64-wide
// K group with fp16 scale and offset (MLX pull request 4722: affine 4-bit
// g64).  All arithmetic is IEEE fp32 with round-to-nearest-even and
// correctly rounded division, so results are bit-exact and deterministic.
//
// The activation kernel is HBM-bound (2 bytes in, 1 byte out per element):
// one wavefront per row, 16-byte coalesced non-temporal loads kept in
// registers, a wavefront max-reduction, then 8-byte code stores from the
// same registers.  The per-element VALU work is kept small because it runs
// after the row has arrived: the absmax on the bf16 bit patterns, rint by
// the 1.5*2^23 shift, codes packed with v_perm_b32, group sums with
// v_dot4_i32_i8.
#include <float.h>

#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

constexpr int kRowsPerBlock = 4;  // one wavefront per row, 4 waves per block
constexpr int64_t kWideMaxRows = 256;  // up to this many rows: a workgroup per row

// Quantize 8 bf16 values held in a uint4; returns 8 codes as uint2 and their
// sum (two signed 4-way byte dot products against ones).
__device__ __forceinline__ uint2 quant8(const uint4 v, float inv, int& sum) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const uint2 c = codes8_shift(w, inv);
  sum = __builtin_amdgcn_sdot4((int)c.y, 0x01010101, __builtin_amdgcn_sdot4((int)c.x, 0x01010101, 0, false),
                               false);
  return c;
}

// Running max of |x| over 8 bf16 values held in a uint4.
__device__ __forceinline__ u16x2 absmax8_bits(u16x2 m, const uint4 v) {
  m = absmax_bits2(m, v.x);
  m = absmax_bits2(m, v.y);
  m = absmax_bits2(m, v.z);
  return absmax_bits2(m, v.w);
}

// Sum over the 8 aligned lanes of a group (lanes 8q..8q+7).
__device__ __forceinline__ int group8_sum(int v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  return v;
}

// K % 8 == 0 and K <= 512*CH: the row stays in registers (CH chunks of 8
// values per lane; chunk c = lane + 64*j covers elements 8c..8c+7).
// FR: where the codes go: 0 row-major [M][K]; 1 and 2 the MFMA GEMV's
// fragment order for int8 and int4 weights (gemv_frag_offset); 3 row-major
// with every run of 8 codes stored as its even codes, then its odd ones
// (the order in which the int4 GEMM unpacks a packed weight dword).
template <int FR>
__device__ __forceinline__ uint2* code_slot(int8_t* a, int64_t row, int c, int K) {
  const int64_t off = FR == 0 || FR == 3 ? row * (int64_t)K + 8 * c
                                         : gemv_frag_offset(row, 8 * c, K, FR == 2);
  return reinterpret_cast<uint2*>(a + off);
}

// The 8 codes of a chunk (c0..c3 in .x, c4..c7 in .y) in FR's order.
template <int FR>
__device__ __forceinline__ uint2 order_codes(uint2 v) {
  if constexpr (FR != 3) return v;
  // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the first
  return make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),   // c0 c2 c4 c6
                    __builtin_amdgcn_perm(v.y, v.x, 0x07050301u));  // c1 c3 c5 c7
}

template <int CH, int FR>
__global__ __launch_bounds__(256) void quant_act_regs(
    const uint16_t* __restrict__ x, int64_t M, int K, int8_t* __restrict__ a,
    float* __restrict__ sx, int32_t* __restrict__ gsum) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nch = K >> 3;
  // x is read exactly once; non-temporal loads measured about 20% faster
  // than ordinary ones for this read-2-bytes/write-1-byte stream.
  const v4i* xr = reinterpret_cast<const v4i*>(x + row * (int64_t)K);
  uint4 v[CH];
  u16x2 mb = u16x2{0, 0};
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    v4i t = v4i{0, 0, 0, 0};
    if (c < nch) t = __builtin_nontemporal_load(xr + c);
    v[j] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
    mb = absmax8_bits(mb, v[j]);
  }
  const float amax = wave_max(absmax_bits_value(mb));
  float scale;
  const float inv = row_inv(amax, scale);
  if (lane == 0) sx[row] = scale;
  const int G = K >> 6;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = lane + 64 * j;
    int s;
    const uint2 codes = quant8(v[j], inv, s);
    if (c < nch) *code_slot<FR>(a, row, c, K) = order_codes<FR>(codes);
    if (gsum != nullptr) {
      s = group8_sum(s);
      if ((lane & 7) == 0 && c < nch) gsum[row * G + (c >> 3)] = s;
    }
  }
}

// Few rows (a GEMV's, a short sequence's): one workgroup of 8 wavefronts
// per row, so a row's loads are spread over 512 lanes and the kernel's
// latency is one load round trip, not one wavefront walking the row.  K %
// 8 == 0 and K <= 4096*CH; chunk c = tid + 512*j covers elements 8c..8c+7
// (the 8 chunks of a 64-group sit in 8 adjacent lanes).  The same
// per-element operations as quant_act_regs: identical codes and scales.
constexpr int kWideThreads = 512;

template <int CH, int FR>
__global__ __launch_bounds__(kWideThreads) void quant_act_wide(
    const uint16_t* __restrict__ x, int64_t M, int K, int8_t* __restrict__ a,
    float* __restrict__ sx, int32_t* __restrict__ gsum) {
  __shared__ float s_am[kWideThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nch = K >> 3;
  const v4i* xr = reinterpret_cast<const v4i*>(x + row * (int64_t)K);
  uint4 v[CH];
  u16x2 mb = u16x2{0, 0};
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = tid + kWideThreads * j;
    v4i t = v4i{0, 0, 0, 0};
    if (c < nch) t = __builtin_nontemporal_load(xr + c);
    v[j] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
    mb = absmax8_bits(mb, v[j]);
  }
  float amax = wave_max(absmax_bits_value(mb));
  if (lane == 0) s_am[wave] = amax;
  __syncthreads();
  amax = s_am[0];
#pragma unroll
  for (int w = 1; w < kWideThreads / 64; ++w) amax = fmaxf(amax, s_am[w]);
  float scale;
  const float inv = row_inv(amax, scale);
  if (tid == 0) sx[row] = scale;
  const int G = K >> 6;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = tid + kWideThreads * j;
    int s;
    const uint2 codes = quant8(v[j], inv, s);
    if (c < nch) *code_slot<FR>(a, row, c, K) = order_codes<FR>(codes);
    if (gsum != nullptr) {
      s = group8_sum(s);
      if ((lane & 7) == 0 && c < nch) gsum[row * G + (c >> 3)] = s;
    }
  }
}

// K % 8 == 0, any K: two passes over the row (the second hits the cache).
template <int FR>
__global__ __launch_bounds__(256) void quant_act_stream(
    const uint16_t* __restrict__ x, int64_t M, int K, int8_t* __restrict__ a,
    float* __restrict__ sx, int32_t* __restrict__ gsum) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * (int64_t)K);
  u16x2 mb = u16x2{0, 0};
  for (int c = lane; c < nch; c += 64) mb = absmax8_bits(mb, xr[c]);
  const float amax = wave_max(absmax_bits_value(mb));
  float scale;
  const float inv = row_inv(amax, scale);
  if (lane == 0) sx[row] = scale;
  const int G = K >> 6;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    int s = 0;
    uint2 codes = make_uint2(0, 0);
    if (c < nch) codes = quant8(xr[c], inv, s);
    if (c < nch) *code_slot<FR>(a, row, c, K) = order_codes<FR>(codes);
    if (gsum != nullptr) {
      s = group8_sum(s);
      if ((lane & 7) == 0 && c < nch) gsum[row * G + (c >> 3)] = s;
    }
  }
}

// Any K (not a multiple of 8): element-wise two-pass fallback, no group sums.
__global__ __launch_bounds__(256) void quant_act_scalar(
    const uint16_t* __restrict__ x, int64_t M, int K, int8_t* __restrict__ a,
    float* __restrict__ sx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint16_t* xr = x + row * (int64_t)K;
  float amax = 0.0f;
  for (int k = lane; k < K; k += 64) amax = fmaxf(amax, fabsf(bf16_to_f32(xr[k])));
  amax = wave_max(amax);
  float scale;
  const float inv = row_inv(amax, scale);
  if (lane == 0) sx[row] = scale;
  int8_t* ar = a + row * (int64_t)K;
  for (int k = lane; k < K; k += 64) ar[k] = (int8_t)quant_code(bf16_to_f32(xr[k]), inv);
}

// int8 weight rows from fp32: one wavefront per output channel.
__global__ __launch_bounds__(256) void quant_w8_rows(const float* __restrict__ w, int64_t N,
                                                     int K, int8_t* __restrict__ q,
                                                     float* __restrict__ sw) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= N) return;
  const float* wr = w + row * (int64_t)K;
  float amax = 0.0f;
  for (int k = lane; k < K; k += 64) amax = fmaxf(amax, fabsf(wr[k]));
  amax = wave_max(amax);
  float scale;
  const float inv = row_inv(amax, scale);
  if (lane == 0) sw[row] = scale;
  int8_t* qr = q + row * (int64_t)K;
  for (int k = lane; k < K; k += 64) qr[k] = (int8_t)quant_code(wr[k], inv);
}

// Affine int4 weights: one thread per (row n, 64-wide group g).
__global__ __launch_bounds__(256) void quant_w4_groups(const float* __restrict__ w, int64_t N,
                                                       int K, uint8_t* __restrict__ q4,
                                                       __half* __restrict__ gs,
                                                       __half* __restrict__ gb) {
  const int G = K >> 6;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= N * (int64_t)G) return;
  const int64_t n = id / G;
  const int g = (int)(id - n * G);
  const float4* src = reinterpret_cast<const float4*>(w + n * (int64_t)K + 64 * g);
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 t = src[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
  float lo = v[0], hi = v[0];
#pragma unroll
  for (int i = 1; i < 64; ++i) { lo = fminf(lo, v[i]); hi = fmaxf(hi, v[i]); }
  const __half s = __float2half_rn((hi - lo) / 15.0f);
  const __half b = __float2half_rn(lo);
  gs[id] = s;
  gb[id] = b;
  const float sf = __half2float(s);
  const float bf = __half2float(b);
  const float inv = (sf != 0.0f) ? 1.0f / sf : 0.0f;
  uint32_t out[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float t = rintf((v[8 * d + j] - bf) * inv);
      t = fminf(fmaxf(t, 0.0f), 15.0f);
      word |= ((uint32_t)t) << (4 * j);
    }
    out[d] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(q4 + n * (int64_t)(K / 2) + 32 * g);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

template <int FR>
const char* launch_act(const uint16_t* x, int64_t M, int K, int8_t* a, float* sx, int32_t* gsum,
                       hipStream_t s) {
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
  // Few rows: a workgroup per row (measured: 16 rows of 5120, one
  // wavefront per row took 4.7 us, latency-bound).
  const int wide = (K / 8 + kWideThreads - 1) / kWideThreads;  // chunks per lane
  if (M <= kWideMaxRows && K >= 1024 && wide <= 4) {
    const dim3 g1((unsigned)M), b1(kWideThreads);
    if (wide <= 1) { hipLaunchKernelGGL((quant_act_wide<1, FR>), g1, b1, 0, s, x, M, K, a, sx, gsum); return "quant_act_wide1"; }
    if (wide <= 2) { hipLaunchKernelGGL((quant_act_wide<2, FR>), g1, b1, 0, s, x, M, K, a, sx, gsum); return "quant_act_wide2"; }
    hipLaunchKernelGGL((quant_act_wide<4, FR>), g1, b1, 0, s, x, M, K, a, sx, gsum);
    return "quant_act_wide4";
  }
  const int need = (K / 8 + 63) / 64;  // chunks per lane
  const dim3 b(256);
#define KQ_REGS(ch)                                                                   \
  if (need <= ch) {                                                                   \
    hipLaunchKernelGGL((quant_act_regs<ch, FR>), grid, b, 0, s, x, M, K, a, sx, gsum); \
    return "quant_act_regs" #ch;                                                      \
  }
  KQ_REGS(1) KQ_REGS(2) KQ_REGS(4) KQ_REGS(6) KQ_REGS(8) KQ_REGS(12) KQ_REGS(16) KQ_REGS(24)
#undef KQ_REGS
  hipLaunchKernelGGL((quant_act_stream<FR>), grid, b, 0, s, x, M, K, a, sx, gsum);
  return "quant_act_stream";
}

}  // namespace

const char* launch_quant_act(const uint16_t* x, int64_t M, int K, int8_t* a, float* sx,
                             int32_t* gsum, hipStream_t s, int frag) {
  if (K % 8 != 0) {
    const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
    hipLaunchKernelGGL(quant_act_scalar, grid, dim3(256), 0, s, x, M, K, a, sx);
    return "quant_act_scalar";
  }
  if (frag == 1) return launch_act<1>(x, M, K, a, sx, gsum, s);
  if (frag == 2) return launch_act<2>(x, M, K, a, sx, gsum, s);
  if (frag == 3) return launch_act<3>(x, M, K, a, sx, gsum, s);
  return launch_act<0>(x, M, K, a, sx, gsum, s);
}

const char* launch_quant_w8(const float* w, int64_t N, int K, int8_t* q, float* sw,
                            hipStream_t s) {
  const dim3 grid((unsigned)((N + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(quant_w8_rows, grid, dim3(256), 0, s, w, N, K, q, sw);
  return "quant_w8_rows";
}

const char* launch_quant_w4(const float* w, int64_t N, int K, uint8_t* q4, void* gs, void* gb,
                            hipStream_t s) {
  const int64_t items = N * (int64_t)(K / 64);
  const dim3 grid((unsigned)((items + 255) / 256));
  hipLaunchKernelGGL(quant_w4_groups, grid, dim3(256), 0, s, w, N, K, q4,
                     reinterpret_cast<__half*>(gs), reinterpret_cast<__half*>(gb));
  return "quant_w4_groups";
}

}  // namespace kq
