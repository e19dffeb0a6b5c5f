// Small-M GEMV of libkq: "qlip-mlx" README, w4a8_linear bullet -- a
// register-dequant GEMV path for small batches, so decode-style calls run at
// weight-bandwidth speed.  One workgroup computes 16 activation rows x 16
// output columns over all of K; the grid's second dimension walks 16-row
// blocks, so the same kernel also serves thin-N shapes (few output
// columns, many rows), which the tiled GEMM would spread over too few
// workgroups.  Same math as the GEMM routes:
//   int4: y = sx * sum_g (gs*P + gb*A) + bias,  int8: y = sx*sw*acc + bias,
// with P the exact int32 dot product of one 64-wide group and A the group
// sum of the activation codes.
//
// gfx950 design (HBM-bound: every weight byte is read once):
//   - a workgroup owns 16 output columns and its 8 wavefronts split the K
//     groups into 8 contiguous slices (rounded to whole 128-byte lines);
//   - each wavefront streams its slice through a private LDS chunk with
//     direct global->LDS buffer loads: one load instruction moves 8 rows x
//     one full 128-byte line, and the LDS layout is the MFMA fragment order,
//     so the fragment reads are contiguous and conflict-free.  A small chunk
//     (4 groups) keeps the LDS per workgroup low, so several workgroups per
//     CU keep loads in flight;
//   - the 16 columns' fp16 group scales and offsets are one contiguous run
//     per array; the workgroup stages them in LDS with coalesced loads
//     issued before the weight loads;
//   - v_mfma_i32_16x16x64_i8 with the activation codes as the A operand
//     (rows >= M zero) and the weights as B; a second MFMA against an
//     all-ones B gives the group sums A exactly, so no group-sum input is
//     read;
//   - the 8 partial sums are reduced through LDS (fp32 for int4 weights,
//     exact int32 for int8) and one wavefront applies the epilogue.
#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

constexpr int kWaves = 8;         // K slices per workgroup
constexpr int kChunk = 4;         // groups per LDS chunk of one wavefront
constexpr int kMaxG = kGemvMaxK / 64;

template <bool W4, int OUT>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx,
    const void* __restrict__ Wq, const void* __restrict__ gsv, const void* __restrict__ gbv,
    const float* __restrict__ bias, void* y, int Mtot, int N, int K, Epilogue ep) {
  // this workgroup's 16-row block of the activations
  const int m0 = blockIdx.y * 16;
  const int M = min(16, Mtot - m0);
  A += (int64_t)m0 * K;
  if (sx != nullptr) sx += m0;
  constexpr int UB = W4 ? 32 : 64;          // bytes of one weight row per group
  constexpr int LPR = UB / 16;              // DMA lanes per (row, group)
  constexpr int GPB = 128 / UB;             // groups per 128-byte line (one DMA block)
  constexpr int WLDS = kChunk * 16 * UB;    // LDS bytes of one wavefront's chunk
  constexpr bool kScales = W4 && OUT != kOutI32;
  static_assert(kChunk % GPB == 0, "a chunk is whole DMA blocks");
  __shared__ __attribute__((aligned(16))) int8_t lds_w[kWaves][WLDS];
  __shared__ float lds_red[kWaves - 1][4][64];
  extern __shared__ uint32_t lds_sb[];      // [G][16]: scale | offset << 16 (int4 only)

  const int G = K / 64;
  const int RB = W4 ? K / 2 : K;            // bytes per weight row
  const int n0 = blockIdx.x * 16;
  const int rows = min(16, N - n0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (readfirstlane): slice guards are scalar branches, the
  // LDS DMA bases stay scalar and every MFMA runs with the full EXEC mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15;  // MFMA A row m / B column of this lane
  const int fc = lane >> 4;  // MFMA 16-wide k chunk / output row block
  const int per = ((G + kWaves - 1) / kWaves + GPB - 1) / GPB * GPB;
  const int g0 = min(wave * per, G);
  const int gn = min(per, G - g0);  // 0 for trailing wavefronts of short K

  // 1. Scale/offset staging loads: rows n0..n0+rows-1 of the [N, G] arrays
  //    are one contiguous run of rows*G halves; issued first so that the LDS
  //    writes below wait for these loads only.
  constexpr int kSL = kScales ? kMaxG * 16 / (kWaves * 64) : 1;
  uint32_t sreg[kSL];
  if (kScales) {
    const uint16_t* hs = reinterpret_cast<const uint16_t*>(gsv) + (int64_t)n0 * G;
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(gbv) + (int64_t)n0 * G;
    const int lim = rows * G;
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = tid + j * kWaves * 64;
      uint32_t v = 0;
      if (e < lim) v = (uint32_t)hs[e] | ((uint32_t)hb[e] << 16);
      sreg[j] = v;
    }
  }

  // 2. Weight DMA.  The descriptor is rebased on row n0 with num_records =
  //    rows*RB: rows past N and groups past the matrix end read as zero.
  //    Block (r8, blk) = rows 8*r8..8*r8+7 x groups blk*GPB.. of the chunk;
  //    lane l moves 16 bytes: group l/(8*LPR), row (l/LPR)%8, piece l%LPR,
  //    into LDS byte 16*l of the block, which puts (row r, chunk group i) at
  //    (r/8)*kChunk*8*UB + i*8*UB + (r%8)*UB -- the fragment order.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(reinterpret_cast<const int8_t*>(Wq) + (int64_t)n0 * RB), 0,
      rows * RB, 0x00020000);
  const int d_gg = lane / (8 * LPR), d_rr = (lane / LPR) & 7, d_pc = lane % LPR;
  const int voff = d_rr * RB + d_gg * UB + d_pc * 16;
  auto issue = [&](int gs, int gc) {
#pragma unroll
    for (int blk = 0; blk < kChunk / GPB; ++blk) {
      if (blk * GPB < gc) {
#pragma unroll
        for (int r8 = 0; r8 < 2; ++r8) {
          lds_ptr_t dst = (lds_ptr_t)(&lds_w[wave][r8 * (kChunk * 8 * UB) + blk * 1024]);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, voff,
                                                   r8 * 8 * RB + (gs + blk * GPB) * UB, 0, 0);
        }
      }
    }
  };
  // 3. Activation fragments of a chunk: A row fr (< M), k chunk fc.
  v4i fa[kChunk];
  const int8_t* arow = A + (int64_t)fr * K + fc * 16;
  auto load_a = [&](int gs, int gc) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      int4 t = make_int4(0, 0, 0, 0);
      if (i < gc && fr < M) t = *reinterpret_cast<const int4*>(arow + (gs + i) * 64);
      fa[i] = v4i{t.x, t.y, t.z, t.w};
    }
  };
  issue(g0, min(gn, kChunk));
  load_a(g0, min(gn, kChunk));

  // Epilogue operands, loaded while the weights stream.
  const int nn = n0 + fr;
  const int nc = min(nn, N - 1);
  const float bv = bias ? bias[nc] : 0.0f;
  const float swn = (!W4 && OUT != kOutI32) ? reinterpret_cast<const float*>(gsv)[nc] : 0.0f;
  float sxm[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sxm[r] = (OUT != kOutI32) ? sx[min(4 * fc + r, M - 1)] : 0.0f;

  if (kScales) {
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = tid + j * kWaves * 64;
      if (e < 16 * G) {
        const int r = e / G, g = e - r * G;
        lds_sb[g * 16 + r] = sreg[j];
      }
    }
    wait_vm_lgkm0<63>();
    barrier_nofence();
  }

  v4f facc = v4f{0.f, 0.f, 0.f, 0.f};
  v4i iacc = v4i{0, 0, 0, 0};
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const int8_t* wl = &lds_w[wave][(fr >> 3) * (kChunk * 8 * UB) + (fr & 7) * UB + fc * (UB / 4)];
  for (int c0 = 0; c0 < gn; c0 += kChunk) {
    const int gc = min(kChunk, gn - c0);
    if (c0 > 0) {
      wait_vm_lgkm0<63>();  // fragment reads of the last chunk done before the DMA reuses it
      issue(g0 + c0, gc);
      load_a(g0 + c0, gc);
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (i < gc) {
        const int g = g0 + c0 + i;
        if (W4) {
          const uint2 wv = *reinterpret_cast<const uint2*>(wl + i * 8 * UB);
          uint32_t u0, u1, u2, u3;
          unpack8_u4(wv.x, u0, u1);
          unpack8_u4(wv.y, u2, u3);
          const v4i fw = v4i{(int)u0, (int)u1, (int)u2, (int)u3};
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fw, v4i{0, 0, 0, 0}, 0, 0, 0);
          if (OUT == kOutI32) {
            // debug output: P of every group, [G, M, N]; p[r] = P[g, 4*fc + r, n]
            if (nn < N) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int m = 4 * fc + r;
                if (m < M) reinterpret_cast<int32_t*>(y)[((int64_t)g * Mtot + m0 + m) * N + nn] = p[r];
              }
            }
          } else {
            const v4i as = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
            const uint32_t sb = lds_sb[g * 16 + fr];
            const float s = __half2float(__ushort_as_half((unsigned short)(sb & 0xffff)));
            const float b = __half2float(__ushort_as_half((unsigned short)(sb >> 16)));
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[r] = fmaf(b, (float)as[r], fmaf(s, (float)p[r], facc[r]));
          }
        } else {
          const int4 wv = *reinterpret_cast<const int4*>(wl + i * 8 * UB);
          iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], v4i{wv.x, wv.y, wv.z, wv.w}, iacc,
                                                       0, 0, 0);
        }
      }
    }
  }
  if (W4 && OUT == kOutI32) return;

  // Reduce the 8 partials: fp32 for int4 weights, exact int32 for int8.
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      lds_red[wave - 1][r][lane] = W4 ? facc[r] : __int_as_float(iacc[r]);
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (W4) facc[r] += lds_red[w][r][lane];
      else iacc[r] += __float_as_int(lds_red[w][r][lane]);
    }
  if (nn >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * fc + r;
    if (m >= M) continue;
    const int64_t idx = (int64_t)(m0 + m) * N + nn;
    if (OUT == kOutI32) {
      reinterpret_cast<int32_t*>(y)[idx] = iacc[r];
    } else {
      float v = W4 ? fmaf(sxm[r], facc[r], bv) : fmaf(sxm[r] * swn, (float)iacc[r], bv);
      if (ep.active()) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m0 + m, nn, N);
      if (OUT == kOutF32) reinterpret_cast<float*>(y)[idx] = v;
      else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <bool W4>
const char* launch_fmt(const int8_t* a, const float* sx, const void* q, const void* gs,
                       const void* gb, const float* bias, void* y, int out, int M, int N, int K,
                       hipStream_t s, const Epilogue& ep) {
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16)), block(kWaves * 64);
  const size_t sb = (W4 && out != kOutI32) ? (size_t)16 * (K / 64) * sizeof(uint32_t) : 0;
  if (out == kOutF32)
    hipLaunchKernelGGL((gemv_kernel<W4, kOutF32>), grid, block, sb, s, a, sx, q, gs, gb, bias, y, M, N, K, ep);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemv_kernel<W4, kOutBF16>), grid, block, sb, s, a, sx, q, gs, gb, bias, y, M, N, K, ep);
  else
    hipLaunchKernelGGL((gemv_kernel<W4, kOutI32>), grid, block, sb, s, a, sx, q, gs, gb, bias, y, M, N, K, ep);
  return W4 ? "gemv_w4a8" : "gemv_w8a8";
}

}  // namespace

const char* launch_gemv(bool w4, const int8_t* a, const float* sx, const int32_t* /*gsum*/,
                        const void* q, const void* gs, const void* gb, const float* bias,
                        void* y, int out, int M, int N, int K, hipStream_t s,
                        const Epilogue& ep) {
  return w4 ? launch_fmt<true>(a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep)
            : launch_fmt<false>(a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep);
}

}  // namespace kq
