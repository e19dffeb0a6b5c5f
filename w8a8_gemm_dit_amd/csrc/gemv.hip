// Small-M GEMV of libkq (1 <= M <= 16): "qlip-mlx" README, w4a8_linear
// bullet -- a register-dequant GEMV path for small batches, so decode-style
// calls run at weight-bandwidth speed.  Same math as the GEMM routes:
//   int4: y = sx * sum_g (gs*P + gb*A) + bias,  int8: y = sx*sw*acc + bias.
//
// gfx950 design (HBM-bound: every weight byte is read once):
//   - a workgroup owns 32 output columns (two 16-column MFMA tiles) and its
//     4 wavefronts split the K groups between them (group g goes to wave
//     g % 4), so many independent weight loads are in flight per CU;
//   - weights go straight from global memory into MFMA operand registers
//     (8 bytes of packed int4 = 16 codes per lane per group, unpacked in
//     registers; or 16 int8 bytes), with no LDS staging; the M <= 16
//     activation rows ride in the MFMA's 16 columns (rows >= M read as 0);
//   - the group scales/offsets and code sums of the workgroup's columns and
//     rows are staged in LDS in 64-group chunks, transposed so that each
//     lane reads its 4 consecutive columns with one 16-byte LDS read;
//   - the 4 wavefronts' partial accumulators are summed through LDS, then
//     one wavefront applies the epilogue.
#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

constexpr int kCols = kGemvCols;  // 32
constexpr int kGC = 64;           // groups per LDS chunk
constexpr int kUnroll = 4;        // groups in flight per wave iteration

template <bool W4, int OUT>
__global__ __launch_bounds__(256) void gemv_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int32_t* __restrict__ gsum,
    const void* __restrict__ Wq, const void* __restrict__ gsv, const void* __restrict__ gbv,
    const float* __restrict__ bias, void* __restrict__ y, int M, int N, int K) {
  __shared__ float lds_gs[kGC][kCols];
  __shared__ float lds_gb[kGC][kCols];
  __shared__ float lds_as[kGC][16];
  __shared__ float lds_red[3][2][4][64];

  const int G = K / 64;
  const int n0 = blockIdx.x * kCols;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int fr = lane & 15;
  const int fc = lane >> 4;

  // Operand rows of this lane: weight rows n0 + 16*t + fr, activation row fr.
  const int ar = fr;
  const bool a_ok = ar < M;
  const int8_t* a_row = A + (int64_t)(a_ok ? ar : 0) * K + fc * 16;
  const uint8_t* w4_row[2];
  const int8_t* w8_row[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = min(n0 + 16 * t + fr, N - 1);
    w4_row[t] = reinterpret_cast<const uint8_t*>(Wq) + (int64_t)n * (K / 2) + fc * 8;
    w8_row[t] = reinterpret_cast<const int8_t*>(Wq) + (int64_t)n * K + fc * 16;
  }

  v4f facc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
  v4i iacc[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};

  for (int gc0 = 0; gc0 < G; gc0 += kGC) {
    const int gcn = min(kGC, G - gc0);
    if (W4) {
      __syncthreads();
      const __half* hs = reinterpret_cast<const __half*>(gsv);
      const __half* hb = reinterpret_cast<const __half*>(gbv);
      for (int e = tid; e < gcn * kCols; e += 256) {
        const int c = e / gcn, gl = e - c * gcn;  // consecutive threads walk one column's groups
        const int n = min(n0 + c, N - 1);
        lds_gs[gl][c] = __half2float(hs[(int64_t)n * G + gc0 + gl]);
        lds_gb[gl][c] = __half2float(hb[(int64_t)n * G + gc0 + gl]);
      }
      for (int e = tid; e < gcn * 16; e += 256) {
        const int r = e / gcn, gl = e - r * gcn;
        lds_as[gl][r] = (r < M) ? (float)gsum[(int64_t)r * G + gc0 + gl] : 0.0f;
      }
      __syncthreads();
    }
    for (int gb0 = wave; gb0 < gcn; gb0 += 4 * kUnroll) {
      v4i fa[kUnroll], fw[kUnroll][2];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int gl = gb0 + 4 * u;
        const int g = gc0 + (gl < gcn ? gl : 0);
        const int4 t = a_ok ? *reinterpret_cast<const int4*>(a_row + (int64_t)g * 64)
                            : make_int4(0, 0, 0, 0);
        fa[u] = v4i{t.x, t.y, t.z, t.w};
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          if (W4) {
            const uint2 p = *reinterpret_cast<const uint2*>(w4_row[t2] + (int64_t)g * 32);
            uint32_t u0, u1, u2, u3;
            unpack8_u4(p.x, u0, u1);
            unpack8_u4(p.y, u2, u3);
            fw[u][t2] = v4i{(int)u0, (int)u1, (int)u2, (int)u3};
          } else {
            const int4 w = *reinterpret_cast<const int4*>(w8_row[t2] + (int64_t)g * 64);
            fw[u][t2] = v4i{w.x, w.y, w.z, w.w};
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int gl = gb0 + 4 * u;
        if (gl >= gcn) break;
        const int g = gc0 + gl;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          if (W4) {
            const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[u][t2], fa[u], v4i{0, 0, 0, 0}, 0, 0, 0);
            if (OUT == kOutI32) {
              const int n = n0 + 16 * t2 + 4 * fc;
              if (fr < M) {
                int32_t* dst = reinterpret_cast<int32_t*>(y) + ((int64_t)g * M + fr) * N;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (n + r < N) dst[n + r] = p[r];
              }
            } else {
              const float4 s4 = *reinterpret_cast<const float4*>(&lds_gs[gl][16 * t2 + 4 * fc]);
              const float4 b4 = *reinterpret_cast<const float4*>(&lds_gb[gl][16 * t2 + 4 * fc]);
              const float af = lds_as[gl][fr];
              const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
              const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float t = fmaf(sv[r], (float)p[r], facc[t2][r]);
                facc[t2][r] = fmaf(bv[r], af, t);
              }
            }
          } else {
            iacc[t2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[u][t2], fa[u], iacc[t2], 0, 0, 0);
          }
        }
      }
    }
  }
  if (W4 && OUT == kOutI32) return;

  // Sum the 4 wavefronts' partials (fp32 for int4, exact int32 for int8).
  if (wave > 0) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lds_red[wave - 1][t2][r][lane] = W4 ? facc[t2][r] : __int_as_float(iacc[t2][r]);
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        if (W4) facc[t2][r] += lds_red[w][t2][r][lane];
        else iacc[t2][r] += __float_as_int(lds_red[w][t2][r][lane]);
      }

  const int m = fr;
  if (m >= M) return;
  const float s_m = (OUT == kOutI32) ? 0.f : sx[m];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const int n = n0 + 16 * t2 + 4 * fc;
    if (n >= N) continue;
    const int valid = min(4, N - n);
    const int64_t idx = (int64_t)m * N + n;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = min(n + r, N - 1);
      const float b = bias ? bias[nn] : 0.0f;
      if (W4) v[r] = fmaf(s_m, facc[t2][r], b);
      else if (OUT != kOutI32) v[r] = fmaf(s_m * reinterpret_cast<const float*>(gsv)[nn], (float)iacc[t2][r], b);
    }
    if (OUT == kOutI32) {
      int32_t* p = reinterpret_cast<int32_t*>(y) + idx;
      for (int r = 0; r < valid; ++r) p[r] = iacc[t2][r];
    } else if (OUT == kOutF32) {
      float* p = reinterpret_cast<float*>(y) + idx;
      for (int r = 0; r < valid; ++r) p[r] = v[r];
    } else {
      uint16_t* p = reinterpret_cast<uint16_t*>(y) + idx;
      for (int r = 0; r < valid; ++r) p[r] = (uint16_t)f32_to_bf16_rne(v[r]);
    }
  }
}

template <bool W4>
const char* launch_fmt(const int8_t* a, const float* sx, const int32_t* gsum, const void* q,
                       const void* gs, const void* gb, const float* bias, void* y, int out, int M,
                       int N, int K, hipStream_t s) {
  const dim3 grid((unsigned)((N + kCols - 1) / kCols)), block(256);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemv_kernel<W4, kOutF32>), grid, block, 0, s, a, sx, gsum, q, gs, gb, bias, y, M, N, K);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemv_kernel<W4, kOutBF16>), grid, block, 0, s, a, sx, gsum, q, gs, gb, bias, y, M, N, K);
  else
    hipLaunchKernelGGL((gemv_kernel<W4, kOutI32>), grid, block, 0, s, a, sx, gsum, q, gs, gb, bias, y, M, N, K);
  return W4 ? "gemv_w4a8" : "gemv_w8a8";
}

}  // namespace

const char* launch_gemv(bool w4, const int8_t* a, const float* sx, const int32_t* gsum,
                        const void* q, const void* gs, const void* gb, const float* bias,
                        void* y, int out, int M, int N, int K, hipStream_t s) {
  return w4 ? launch_fmt<true>(a, sx, gsum, q, gs, gb, bias, y, out, M, N, K, s)
            : launch_fmt<false>(a, sx, gsum, q, gs, gb, bias, y, out, M, N, K, s);
}

}  // namespace kq
