// W8A8 GEMM of libkq: y[m,n] = sx[m]*sw[n]*sum_k a[m,k]*q[n,k] + bias[n].
//
// "qlip-mlx" README, w8a8_linear bullet: INT8xINT8->INT32 matmul with
// dequant+bias fused into one node.  Both operands are K-contiguous ([M,K]
// codes and [N,K] weights, MLX pull request 4722 "Selector rules": 2-D
// transposed weights).
//
// gfx950 design:
//   - a workgroup computes a BM x BN output tile with 4 wavefronts in a 2x2
//     grid; each wavefront owns a (BM/2) x (BN/2) tile of int32
//     accumulators built from v_mfma_i32_16x16x64_i8 (16x16 outputs, K=64
//     per instruction);
//   - the weights are the MFMA "A" operand and the activations the "B"
//     operand, so each lane ends with 4 consecutive output columns of one
//     row (one 8- or 16-byte store per 16x16 tile);
//   - K advances 64 bytes per stage; both operand tiles are staged in LDS,
//     double buffered, rows of 64 bytes with the 16-byte chunk index XORed
//     with (row/4)%4 so that the 16 lanes of each ds_read_b128 phase hit 16
//     distinct bank groups;
//   - workgroup ids are remapped so each XCD (ids congruent mod 8) works on
//     a contiguous block of tiles, keeping operand panels in its own L2;
//   - the epilogue converts the accumulator to fp32, multiplies by
//     sx[m]*sw[n], adds the bias with one fma and rounds once to the output
//     type (fp32, or bf16 round-to-nearest-even).
#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

template <int BM, int BN>
struct Cfg {
  static constexpr int kThreads = 256;
  static constexpr int kWavesM = 2, kWavesN = 2;
  static constexpr int kWTM = BM / kWavesM;  // wave tile: rows (m)
  static constexpr int kWTN = BN / kWavesN;  // wave tile: columns (n)
  static constexpr int kTM = kWTM / 16;
  static constexpr int kTN = kWTN / 16;
  static constexpr int kChA = BM * 4;  // 16-byte chunks of one stage
  static constexpr int kChB = BN * 4;
  static constexpr int kLdA = (kChA + kThreads - 1) / kThreads;
  static constexpr int kLdB = (kChB + kThreads - 1) / kThreads;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

template <int OUT>
__device__ __forceinline__ void store_out(void* y, int64_t idx, const float v[4], const int32_t iv[4],
                                          int valid, bool vec_ok) {
  if (OUT == kOutI32) {
    int32_t* p = reinterpret_cast<int32_t*>(y) + idx;
    if (vec_ok && valid == 4) {
      *reinterpret_cast<int4*>(p) = make_int4(iv[0], iv[1], iv[2], iv[3]);
    } else {
      for (int i = 0; i < valid; ++i) p[i] = iv[i];
    }
  } else if (OUT == kOutF32) {
    float* p = reinterpret_cast<float*>(y) + idx;
    if (vec_ok && valid == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int i = 0; i < valid; ++i) p[i] = v[i];
    }
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(y) + idx;
    if (vec_ok && valid == 4) {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
      for (int i = 0; i < valid; ++i) p[i] = (uint16_t)f32_to_bf16_rne(v[i]);
    }
  }
}

template <int BM, int BN, int OUT>
__global__ __launch_bounds__(256) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const float* __restrict__ bias, void* __restrict__ y, int M,
    int N, int K) {
  using C = Cfg<BM, BN>;
  __shared__ int4 lds_a[2][C::kChA];
  __shared__ int4 lds_b[2][C::kChB];

  const int tiles_n = (N + BN - 1) / BN;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % C::kWavesM;
  const int wn = wave / C::kWavesM;

  // Global source of each 16-byte chunk this thread stages (rows past the
  // edge re-read the last row; their results are never stored).
  const int8_t* src_a[C::kLdA];
  const int8_t* src_b[C::kLdB];
  int dst_a[C::kLdA], dst_b[C::kLdB];
#pragma unroll
  for (int i = 0; i < C::kLdA; ++i) {
    const int q = tid + i * C::kThreads;
    const int row = q >> 2, ch = q & 3;
    const int gr = min(m0 + row, M - 1);
    src_a[i] = A + (int64_t)gr * K + ch * 16;
    dst_a[i] = (q < C::kChA) ? swz(row, ch) : -1;
  }
#pragma unroll
  for (int i = 0; i < C::kLdB; ++i) {
    const int q = tid + i * C::kThreads;
    const int row = q >> 2, ch = q & 3;
    const int gr = min(n0 + row, N - 1);
    src_b[i] = W + (int64_t)gr * K + ch * 16;
    dst_b[i] = (q < C::kChB) ? swz(row, ch) : -1;
  }

  v4i acc[C::kTN][C::kTM];
#pragma unroll
  for (int i = 0; i < C::kTN; ++i)
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  int4 ra[C::kLdA], rb[C::kLdB];
  auto gload = [&](int kt) {
    const int64_t off = (int64_t)kt * 64;
#pragma unroll
    for (int i = 0; i < C::kLdA; ++i)
      if (dst_a[i] >= 0) ra[i] = *reinterpret_cast<const int4*>(src_a[i] + off);
#pragma unroll
    for (int i = 0; i < C::kLdB; ++i)
      if (dst_b[i] >= 0) rb[i] = *reinterpret_cast<const int4*>(src_b[i] + off);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLdA; ++i)
      if (dst_a[i] >= 0) lds_a[buf][dst_a[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < C::kLdB; ++i)
      if (dst_b[i] >= 0) lds_b[buf][dst_b[i]] = rb[i];
  };

  const int fr = lane & 15;  // fragment row within a 16-row tile
  const int fc = lane >> 4;  // fragment 16-byte chunk
  const int KT = K / 64;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    v4i fa[C::kTM], fw[C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
      const int row = wm * C::kWTM + j * 16 + fr;
      const int4 t = lds_a[buf][swz(row, fc)];
      fa[j] = v4i{t.x, t.y, t.z, t.w};
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int row = wn * C::kWTN + i * 16 + fr;
      const int4 t = lds_b[buf][swz(row, fc)];
      fw[i] = v4i{t.x, t.y, t.z, t.w};
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i)
#pragma unroll
      for (int j = 0; j < C::kTM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[i], fa[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds D[n = nb + 4*(lane/16) + r][m = mb + lane%16], r = 0..3.
  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int j = 0; j < C::kTM; ++j) {
    const int m = m0 + wm * C::kWTM + j * 16 + fr;
    if (m >= M) continue;
    const float s_m = (OUT == kOutI32) ? 0.0f : sx[m];
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int n = n0 + wn * C::kWTN + i * 16 + fc * 4;
      if (n >= N) continue;
      const int valid = min(4, N - n);
      float v[4];
      int32_t iv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        iv[r] = acc[i][j][r];
        if (OUT != kOutI32) {
          const int nn = min(n + r, N - 1);
          const float b = bias ? bias[nn] : 0.0f;
          v[r] = fmaf(s_m * sw[nn], (float)iv[r], b);
        }
      }
      store_out<OUT>(y, (int64_t)m * N + n, v, iv, valid, vec_ok);
    }
  }
}

template <int BM, int BN>
const char* launch_tile(const int8_t* a, const float* sx, const int8_t* q, const float* sw,
                        const float* bias, void* y, int out, int M, int N, int K,
                        hipStream_t s, const char* name) {
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(256);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, kOutF32>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, kOutBF16>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K);
  else
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, kOutI32>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K);
  return name;
}

}  // namespace

const char* launch_gemm_w8a8(int tile, const int8_t* a, const float* sx, const int8_t* q,
                             const float* sw, const float* bias, void* y, int out, int M,
                             int N, int K, hipStream_t s) {
  switch (tile) {
    case kTile256x256:
      return launch_tile<256, 256>(a, sx, q, sw, bias, y, out, M, N, K, s, "gemm_w8a8_256x256");
    case kTile256x128:
      return launch_tile<256, 128>(a, sx, q, sw, bias, y, out, M, N, K, s, "gemm_w8a8_256x128");
    case kTile128x128:
      return launch_tile<128, 128>(a, sx, q, sw, bias, y, out, M, N, K, s, "gemm_w8a8_128x128");
    default:
      return launch_tile<64, 64>(a, sx, q, sw, bias, y, out, M, N, K, s, "gemm_w8a8_64x64");
  }
}

}  // namespace kq
