// W4A8 GEMM of libkq:
//   y[m,n] = sx[m] * sum_g (gs[n,g]*P[g,m,n] + gb[n,g]*A[m,g]) + bias[n],
//   P[g,m,n] = sum_{k in group g} a[m,k]*q[n,k]   (exact int32),
//   A[m,g]   = sum_{k in group g} a[m,k]          (from the quantize kernel).
// This is x_hat . w_hat^T with w_hat = gs*q + gb per 64-group, regrouped so
// the K loop stays on INT8 MFMA ("qlip-mlx" README, w4a8_linear bullet: the
// same INT8 compute with packed int4 weights; MLX pull request 4722: stage
// weights and activations as int8 instead of dequantizing to fp16).
//
// gfx950 design: the W8A8 tile structure (2x2 wavefronts, 16x16x64 int8
// MFMA, weights as the MFMA A operand, XOR-swizzled double-buffered LDS),
// with three differences:
//   - the weight tile arrives packed (32 bytes per row per 64-group) and is
//     unpacked to int8 in registers (mask, shift, v_perm_b32) before the LDS
//     store, so every wavefront reads plain int8 fragments;
//   - one LDS stage is exactly one 64-group, so each stage's MFMA result is
//     the group's P and is rescaled at once into fp32 accumulators:
//     acc += gs*float(P) + gb*float(A), with the group's scales and offsets
//     (and the tile rows' code sums) staged in LDS alongside the operands;
//   - the epilogue is y = sx*acc + bias, rounded once to the output type.
#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

template <int BM, int BN>
struct Cfg4 {
  static constexpr int kThreads = 256;
  static constexpr int kWavesM = 2, kWavesN = 2;
  static constexpr int kWTM = BM / kWavesM;
  static constexpr int kWTN = BN / kWavesN;
  static constexpr int kTM = kWTM / 16;
  static constexpr int kTN = kWTN / 16;
  static constexpr int kChA = BM * 4;        // int8 activation chunks per stage
  static constexpr int kChB = BN * 4;        // unpacked int8 weight chunks per stage
  static constexpr int kChP = BN * 2;        // packed weight chunks per stage
  static constexpr int kLdA = (kChA + kThreads - 1) / kThreads;
  static constexpr int kLdP = (kChP + kThreads - 1) / kThreads;
};

__device__ __forceinline__ int swz4(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

template <int BM, int BN, int OUT>
__global__ __launch_bounds__(256) void gemm_w4a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int32_t* __restrict__ gsum,
    const uint8_t* __restrict__ W4, const __half* __restrict__ gs, const __half* __restrict__ gb,
    const float* __restrict__ bias, void* __restrict__ y, int M, int N, int K) {
  using C = Cfg4<BM, BN>;
  __shared__ int4 lds_a[2][C::kChA];
  __shared__ int4 lds_b[2][C::kChB];
  __shared__ float lds_gs[2][BN];
  __shared__ float lds_gb[2][BN];
  __shared__ float lds_as[2][BM];

  const int G = K / 64;
  const int tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::kWavesM;
  const int wn = wave / C::kWavesM;

  int64_t off_a[C::kLdA];
  int dst_a[C::kLdA];
#pragma unroll
  for (int i = 0; i < C::kLdA; ++i) {
    const int q = tid + i * C::kThreads;
    const int row = q >> 2, ch = q & 3;
    off_a[i] = (int64_t)min(m0 + row, M - 1) * K + ch * 16;
    dst_a[i] = (q < C::kChA) ? row : -1;
  }
  int64_t off_p[C::kLdP];
  int dst_p[C::kLdP];
#pragma unroll
  for (int i = 0; i < C::kLdP; ++i) {
    const int q = tid + i * C::kThreads;
    const int row = q >> 1, pc = q & 1;
    off_p[i] = (int64_t)min(n0 + row, N - 1) * (K / 2) + pc * 16;
    dst_p[i] = (q < C::kChP) ? row : -1;
  }
  // Per-group side data: thread t < BN stages the scale/offset of column
  // n0+t; thread t < BM stages the code sum of row m0+t.
  const int64_t side_n = (int64_t)min(n0 + tid, N - 1) * G;
  const int64_t side_m = (int64_t)min(m0 + tid, M - 1) * G;

  v4f acc[C::kTN][C::kTM];
#pragma unroll
  for (int i = 0; i < C::kTN; ++i)
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  int4 ra[C::kLdA];
  uint4 rp[C::kLdP];
  float r_gs = 0.f, r_gb = 0.f, r_as = 0.f;
  auto gload = [&](int g) {
#pragma unroll
    for (int i = 0; i < C::kLdA; ++i)
      if (dst_a[i] >= 0) ra[i] = *reinterpret_cast<const int4*>(A + off_a[i] + (int64_t)g * 64);
#pragma unroll
    for (int i = 0; i < C::kLdP; ++i)
      if (dst_p[i] >= 0) rp[i] = *reinterpret_cast<const uint4*>(W4 + off_p[i] + (int64_t)g * 32);
    if (tid < BN) {
      r_gs = __half2float(gs[side_n + g]);
      r_gb = __half2float(gb[side_n + g]);
    }
    if (tid < BM) r_as = (float)gsum[side_m + g];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLdA; ++i)
      if (dst_a[i] >= 0) {
        const int q = tid + i * C::kThreads;
        lds_a[buf][swz4(dst_a[i], q & 3)] = ra[i];
      }
#pragma unroll
    for (int i = 0; i < C::kLdP; ++i)
      if (dst_p[i] >= 0) {
        const int pc = (tid + i * C::kThreads) & 1;
        uint32_t u[8];
        unpack8_u4(rp[i].x, u[0], u[1]);
        unpack8_u4(rp[i].y, u[2], u[3]);
        unpack8_u4(rp[i].z, u[4], u[5]);
        unpack8_u4(rp[i].w, u[6], u[7]);
        lds_b[buf][swz4(dst_p[i], 2 * pc)] = make_int4(u[0], u[1], u[2], u[3]);
        lds_b[buf][swz4(dst_p[i], 2 * pc + 1)] = make_int4(u[4], u[5], u[6], u[7]);
      }
    if (tid < BN) {
      lds_gs[buf][tid] = r_gs;
      lds_gb[buf][tid] = r_gb;
    }
    if (tid < BM) lds_as[buf][tid] = r_as;
  };

  const int fr = lane & 15;
  const int fc = lane >> 4;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    if (g + 1 < G) gload(g + 1);
    v4i fa[C::kTM], fw[C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
      const int4 t = lds_a[buf][swz4(wm * C::kWTM + j * 16 + fr, fc)];
      fa[j] = v4i{t.x, t.y, t.z, t.w};
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int4 t = lds_b[buf][swz4(wn * C::kWTN + i * 16 + fr, fc)];
      fw[i] = v4i{t.x, t.y, t.z, t.w};
    }
    float af[C::kTM];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) af[j] = lds_as[buf][wm * C::kWTM + j * 16 + fr];
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int nb = wn * C::kWTN + i * 16 + fc * 4;
      const float4 s4 = *reinterpret_cast<const float4*>(&lds_gs[buf][nb]);
      const float4 b4 = *reinterpret_cast<const float4*>(&lds_gb[buf][nb]);
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int j = 0; j < C::kTM; ++j) {
        const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[i], fa[j], v4i{0, 0, 0, 0}, 0, 0, 0);
        if (OUT == kOutI32) {
          const int m = m0 + wm * C::kWTM + j * 16 + fr;
          const int n = n0 + nb;
          if (m < M) {
            int32_t* dst = reinterpret_cast<int32_t*>(y) + ((int64_t)g * M + m) * N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) dst[n + r] = p[r];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float t = fmaf(sv[r], (float)p[r], acc[i][j][r]);
            acc[i][j][r] = fmaf(bv[r], af[j], t);
          }
        }
      }
    }
    if (g + 1 < G) lstore(buf ^ 1);
    __syncthreads();
  }
  if (OUT == kOutI32) return;

  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int j = 0; j < C::kTM; ++j) {
    const int m = m0 + wm * C::kWTM + j * 16 + fr;
    if (m >= M) continue;
    const float s_m = sx[m];
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int n = n0 + wn * C::kWTN + i * 16 + fc * 4;
      if (n >= N) continue;
      const int valid = min(4, N - n);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float b = bias ? bias[min(n + r, N - 1)] : 0.0f;
        v[r] = fmaf(s_m, acc[i][j][r], b);
      }
      const int64_t idx = (int64_t)m * N + n;
      if (OUT == kOutF32) {
        float* p = reinterpret_cast<float*>(y) + idx;
        if (vec_ok && valid == 4) *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        else for (int r = 0; r < valid; ++r) p[r] = v[r];
      } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(y) + idx;
        if (vec_ok && valid == 4)
          *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        else for (int r = 0; r < valid; ++r) p[r] = (uint16_t)f32_to_bf16_rne(v[r]);
      }
    }
  }
}

template <int BM, int BN>
const char* launch_tile4(const int8_t* a, const float* sx, const int32_t* gsum, const uint8_t* q4,
                         const void* gs, const void* gb, const float* bias, void* y, int out, int M,
                         int N, int K, hipStream_t s, const char* name) {
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(256);
  const __half* hs = reinterpret_cast<const __half*>(gs);
  const __half* hb = reinterpret_cast<const __half*>(gb);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, kOutF32>), grid, block, 0, s, a, sx, gsum, q4, hs, hb, bias, y, M, N, K);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, kOutBF16>), grid, block, 0, s, a, sx, gsum, q4, hs, hb, bias, y, M, N, K);
  else
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, kOutI32>), grid, block, 0, s, a, sx, gsum, q4, hs, hb, bias, y, M, N, K);
  return name;
}

}  // namespace

const char* launch_gemm_w4a8(int tile, const int8_t* a, const float* sx, const int32_t* gsum,
                             const uint8_t* q4, const void* gs, const void* gb,
                             const float* bias, void* y, int out, int M, int N, int K,
                             hipStream_t s) {
  switch (tile) {
    case kTile256x256:
    case kTile256x128:
      return launch_tile4<256, 128>(a, sx, gsum, q4, gs, gb, bias, y, out, M, N, K, s, "gemm_w4a8_256x128");
    case kTile128x128:
      return launch_tile4<128, 128>(a, sx, gsum, q4, gs, gb, bias, y, out, M, N, K, s, "gemm_w4a8_128x128");
    default:
      return launch_tile4<64, 64>(a, sx, gsum, q4, gs, gb, bias, y, out, M, N, K, s, "gemm_w4a8_64x64");
  }
}

}  // namespace kq
