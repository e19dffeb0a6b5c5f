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
// In-kernel quantization (XQ): at most kGemvXqRows rows and slices of at
// most kXqMaxGPW groups (K <= kFusedMaxK).
constexpr int kXqMaxGPW = 12;
constexpr int kXT = kXqMaxGPW / 2;  // 16-byte x loads per lane
static_assert(((int)(kFusedMaxK / 64) + kWaves - 1) / kWaves <= kXqMaxGPW &&
              kXqMaxGPW % kChunk == 0, "XQ slices");
static_assert(kGemvXqRows * 16 == 64, "XQ x loads: 16 lanes per row");

// XQ: A is unused and the kernel quantizes bf16 rows X itself (Mtot <=
// kGemvXqRows, one row block): the same absmax rule and rounding as the
// quantize kernel; the token scales go to sx_out (if not NULL).
template <bool W4, int OUT, bool XQ>
__global__ __launch_bounds__(kWaves * 64) void gemv_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx,
    const void* __restrict__ Wq, const void* __restrict__ gsv, const void* __restrict__ gbv,
    const float* __restrict__ bias, void* y, int Mtot, int N, int K, Epilogue ep,
    const uint16_t* __restrict__ X, float* __restrict__ sx_out) {
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
  __shared__ float s_xamax[XQ ? kWaves : 1][kGemvXqRows];
  __shared__ float s_xscale[kGemvXqRows];
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
    // Unconditional loads at a clamped index (lim >= 1): all of them issue
    // back to back (loads under a per-lane guard were each waited for
    // before the next one issued).
    uint16_t sl[kSL], bl[kSL];
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = min(tid + j * kWaves * 64, lim - 1);
      sl[j] = hs[e];
      bl[j] = hb[e];
    }
#pragma unroll
    for (int j = 0; j < kSL; ++j)
      sreg[j] = tid + j * kWaves * 64 < lim ? (uint32_t)sl[j] | ((uint32_t)bl[j] << 16) : 0u;
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
  // XQ: x with whole-line loads, issued before the weight DMA (load
  // counters retire in order, so the absmax below then waits for x alone).
  // Lane l takes row l/16 and, for t < kXT, the 16 bytes of values
  // 8*(l%8)..+7 of slice group 2t + (l%16)/8, so the 16 lanes of a row read
  // 256 contiguous bytes per instruction.
  const int xr = lane >> 4, xj = lane & 15;
  v4i xq[XQ ? kXT : 1];
  if constexpr (XQ) {
    const v4i* xrow = reinterpret_cast<const v4i*>(X + (int64_t)min(xr, Mtot - 1) * K + 8 * (xj & 7));
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      const int gi = 2 * t + (xj >> 3);
      xq[t] = v4i{0, 0, 0, 0};
      if (gi < gn && xr < Mtot) xq[t] = xrow[(g0 + gi) * 8];
    }
  }
  issue(g0, min(gn, kChunk));
  if (!XQ) load_a(g0, min(gn, kChunk));
  if constexpr (XQ) {
    // Row absmax on the bf16 bit patterns (for finite values the magnitude
    // bits order as |x|), over the row's 16 lanes, then the 8 slices.
    u16x2 mb = u16x2{0, 0};
#pragma unroll
    for (int t = 0; t < kXT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) mb = absmax_bits2(mb, (uint32_t)xq[t][j]);
    float am = absmax_bits_value(mb);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) am = fmaxf(am, __shfl_xor(am, off, kWave));
    if (xj == 0) s_xamax[wave][xr] = am;
  }

  // Epilogue operands, loaded while the weights stream.
  const int nn = n0 + fr;
  const int nc = min(nn, N - 1);
  const float bv = bias ? bias[nc] : 0.0f;
  const float swn = (!W4 && OUT != kOutI32) ? reinterpret_cast<const float*>(gsv)[nc] : 0.0f;
  float sxm[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sxm[r] = (OUT != kOutI32 && !XQ) ? sx[min(4 * fc + r, M - 1)] : 0.0f;

  if (kScales) {
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = tid + j * kWaves * 64;
      if (e < 16 * G) {
        const int r = e / G, g = e - r * G;
        lds_sb[g * 16 + r] = sreg[j];
      }
    }
  }
  if (kScales || XQ) {
    wait_vm_lgkm0<63>();  // LDS writes done; the weight DMA may still fly
    barrier_nofence();
  }
  // XQ: the codes (codes8_shift: the quantize kernel's rule); xc[t] holds
  // the 8 codes of the lane's load t, 4 per dword.
  int xc[XQ ? kXT : 1][2];
  if constexpr (XQ) {
    float am = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) am = fmaxf(am, s_xamax[w][xr]);
    float scale;
    const float inv = row_inv(am, scale);
    if (wave == 0 && xj == 0) {
      s_xscale[xr] = scale;
      if (sx_out != nullptr && xr < Mtot) sx_out[xr] = scale;
    }
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      const uint32_t w[4] = {(uint32_t)xq[t][0], (uint32_t)xq[t][1], (uint32_t)xq[t][2],
                             (uint32_t)xq[t][3]};
      const uint2 c = codes8_shift(w, inv);
      xc[t][0] = (int)c.x;
      xc[t][1] = (int)c.y;
    }
  }

  v4f facc = v4f{0.f, 0.f, 0.f, 0.f};
  v4i iacc = v4i{0, 0, 0, 0};
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const int8_t* wl = &lds_w[wave][(fr >> 3) * (kChunk * 8 * UB) + (fr & 7) * UB + fc * (UB / 4)];
  // One group's products: weight fragment i of the chunk in LDS, codes fa_g.
  auto group_product = [&](int i, int g, const v4i& fa_g) {
    if (W4) {
      const uint2 wv = *reinterpret_cast<const uint2*>(wl + i * 8 * UB);
      uint32_t u0, u1, u2, u3;
      unpack8_u4(wv.x, u0, u1);
      unpack8_u4(wv.y, u2, u3);
      const v4i fw = v4i{(int)u0, (int)u1, (int)u2, (int)u3};
      const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, fw, v4i{0, 0, 0, 0}, 0, 0, 0);
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
        const v4i as = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, ones, v4i{0, 0, 0, 0}, 0, 0, 0);
        const uint32_t sb = lds_sb[g * 16 + fr];
        const float s = __half2float(__ushort_as_half((unsigned short)(sb & 0xffff)));
        const float b = __half2float(__ushort_as_half((unsigned short)(sb >> 16)));
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[r] = fmaf(b, (float)as[r], fmaf(s, (float)p[r], facc[r]));
      }
    } else {
      const int4 wv = *reinterpret_cast<const int4*>(wl + i * 8 * UB);
      iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, v4i{wv.x, wv.y, wv.z, wv.w}, iacc, 0, 0, 0);
    }
  };
  if constexpr (XQ) {
    // Operand of slice group gi: lane fr + 16*fc (rows fr < 4) takes the
    // codes of values 16*fc..16*fc+15 from lanes 16*fr + 8*(gi%2) + 2*fc and
    // + 1 (their loads t = gi/2); rows 4-15 are zero.  Fully unrolled, so
    // the register of each load is known.
    const int src0 = 4 * (16 * (fr & 3) + 2 * fc);  // ds_bpermute byte address, gi even
#pragma unroll
    for (int c0 = 0; c0 < kXqMaxGPW; c0 += kChunk) {
      if (c0 >= gn) break;
      const int gc = min(kChunk, gn - c0);
      if (c0 > 0) {
        wait_vm_lgkm0<63>();  // fragment reads of the last chunk done before the DMA reuses it
        issue(g0 + c0, gc);
      }
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        if (i < gc) {
          const int gi = c0 + i;
          const int sa = src0 + 32 * (gi & 1);
          v4i f = v4i{__builtin_amdgcn_ds_bpermute(sa, xc[gi >> 1][0]),
                      __builtin_amdgcn_ds_bpermute(sa, xc[gi >> 1][1]),
                      __builtin_amdgcn_ds_bpermute(sa + 4, xc[gi >> 1][0]),
                      __builtin_amdgcn_ds_bpermute(sa + 4, xc[gi >> 1][1])};
          if (fr >= kGemvXqRows) f = v4i{0, 0, 0, 0};
          group_product(i, g0 + gi, f);
        }
      }
    }
  } else {
    for (int c0 = 0; c0 < gn; c0 += kChunk) {
      const int gc = min(kChunk, gn - c0);
      if (c0 > 0) {
        wait_vm_lgkm0<63>();  // fragment reads of the last chunk done before the DMA reuses it
        issue(g0 + c0, gc);
        load_a(g0 + c0, gc);
      }
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        if (i < gc) group_product(i, g0 + c0 + i, fa[i]);
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
  if (XQ && OUT != kOutI32) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sxm[r] = s_xscale[min(4 * fc + r, M - 1)];
  }
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

template <bool W4, bool XQ>
const char* launch_fmt(const int8_t* a, const float* sx, const void* q, const void* gs,
                       const void* gb, const float* bias, void* y, int out, int M, int N, int K,
                       hipStream_t s, const Epilogue& ep, const uint16_t* x, float* sx_out) {
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16)), block(kWaves * 64);
  const size_t sb = (W4 && out != kOutI32) ? (size_t)16 * (K / 64) * sizeof(uint32_t) : 0;
  if (out == kOutF32)
    hipLaunchKernelGGL((gemv_kernel<W4, kOutF32, XQ>), grid, block, sb, s, a, sx, q, gs, gb, bias, y, M, N, K, ep, x, sx_out);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemv_kernel<W4, kOutBF16, XQ>), grid, block, sb, s, a, sx, q, gs, gb, bias, y, M, N, K, ep, x, sx_out);
  else
    hipLaunchKernelGGL((gemv_kernel<W4, kOutI32, XQ>), grid, block, sb, s, a, sx, q, gs, gb, bias, y, M, N, K, ep, x, sx_out);
  if (XQ) return W4 ? "gemv_xq_w4a8" : "gemv_xq_w8a8";
  return W4 ? "gemv_w4a8" : "gemv_w8a8";
}

}  // namespace

const char* launch_gemv(bool w4, const int8_t* a, const float* sx, const int32_t* /*gsum*/,
                        const void* q, const void* gs, const void* gb, const float* bias,
                        void* y, int out, int M, int N, int K, hipStream_t s,
                        const Epilogue& ep, const uint16_t* x, float* sx_out) {
  if (x != nullptr)
    return w4 ? launch_fmt<true, true>(nullptr, nullptr, q, gs, gb, bias, y, out, M, N, K, s, ep, x, sx_out)
              : launch_fmt<false, true>(nullptr, nullptr, q, gs, gb, bias, y, out, M, N, K, s, ep, x, sx_out);
  return w4 ? launch_fmt<true, false>(a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, nullptr, nullptr)
            : launch_fmt<false, false>(a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, nullptr, nullptr);
}

}  // namespace kq
