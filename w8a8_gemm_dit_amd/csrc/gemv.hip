// Small-M GEMV of libkq: "qlip-mlx" README, w4a8_linear bullet -- a
// register-dequant GEMV path for small batches, so decode-style calls run at
// weight-bandwidth speed.  One workgroup computes 16 activation rows x 32
// output columns over all of K; the grid's second dimension walks 16-row
// blocks, so the same kernel also serves thin-N shapes (few output
// columns, many rows), which the tiled GEMM would spread over too few
// workgroups.  Same math as the GEMM routes:
//   int4: y = sx * sum_g (gs*P + gb*A) + bias,  int8: y = sx*sw*acc + bias,
// with P the exact int32 dot product of one 64-wide group and A the group
// sum of the activation codes.  M <= 2 with K <= 6144 takes the
// lane-per-column kernels further down instead (fewer instructions per
// weight byte where the 16-row MFMA tile would be mostly empty).
//
// gfx950 design (HBM-bound: every weight byte is read once):
//   - a workgroup owns 32 output columns (two MFMA column blocks) and its 8
//     wavefronts split the K groups into 8 contiguous slices; each
//     wavefront computes both column blocks of its slice, so one activation
//     operand serves two weight operands;
//   - the weights go straight to registers, already in MFMA operand order:
//     a load unit is 16 bytes a lane, lane (q, c) = (l/16, l%16) taking
//     bytes 16q..16q+15 of a 64-byte run of column c, so one instruction
//     moves 64 bytes of each of 16 columns (two int4 groups or one int8
//     group).  The units of a slice are issued D ahead of the arithmetic,
//     so the weight stream stays in flight while it runs;
//   - int4: lanes q = 0, 1 hold the first group of a unit and q = 2, 3 the
//     second; v_permlane32_swap exchanges the upper half of the first
//     operand with the lower half of the second, which leaves MFMA k chunk
//     q of one group with bytes {0, 16, 8, 24}[q] .. +8 of it (16 codes in
//     order), and the activation codes are read at the matching k offsets;
//   - the activation codes come either row-major (the entry points on
//     caller-given codes: 16 rows x 64 bytes per load) or in the fragment
//     order the linears' quantize kernel writes for this kernel (one
//     contiguous 1 KB per 16-row block and group: the load of a group's
//     operand reads 8 whole lines);
//   - buffer descriptors: rows past M, columns past N, groups past K and
//     units past a wavefront's share read as zero without touching memory;
//   - the 32 columns' fp16 group scales and offsets are one contiguous run
//     per array; the workgroup stages them in LDS with coalesced loads
//     issued before the weight loads;
//   - v_mfma_i32_16x16x64_i8 with the activation codes as the A operand and
//     the weights as B; a second MFMA against an all-ones B gives the group
//     sums A exactly, so no group-sum input is read;
//   - the 8 partial sums of each column block are reduced through LDS (fp32
//     for int4 weights, exact int32 for int8) and wavefronts 0 and 1 apply
//     the epilogue of one column block each.
#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

constexpr int kWaves = 8;         // K slices per workgroup
constexpr int kCB = 2;            // 16-column MFMA blocks per workgroup
static_assert(16 * kCB == kGemvCols, "GEMV columns per workgroup");
// In-kernel quantization (XQ): at most kGemvXqRows rows and slices of at
// most kXqMaxGPW groups (K <= kFusedMaxK).
constexpr int kXqMaxGPW = 12;
constexpr int kXT = kXqMaxGPW / 2;  // 16-byte x loads per lane
static_assert(((int)(kFusedMaxK / 64) + kWaves - 1) / kWaves <= kXqMaxGPW, "XQ slices");
static_assert(kGemvXqRows * 16 == 64, "XQ x loads: 16 lanes per row");

// XQ: A is unused and the kernel quantizes bf16 rows X itself (Mtot <=
// kGemvXqRows, one row block): the same absmax rule and rounding as the
// quantize kernel; the token scales go to sx_out (if not NULL).
// AF: A in the fragment order (gemv_frag_offset), else row-major.
// NU: load units a wavefront issues (its slice, rounded up; the units past
// its share read zero), D: units in flight ahead of the arithmetic.
template <int OUT, bool XQ, bool AF, int NU, int D>
__global__ __launch_bounds__(kWaves * 64) void gemv_w4_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ gsv,
    const uint16_t* __restrict__ gbv, const float* __restrict__ bias, void* y, int Mtot, int N,
    int K, Epilogue ep, const uint16_t* __restrict__ X, float* __restrict__ sx_out) {
  static_assert(D >= 1 && D <= NU, "pipeline depth");
  constexpr int GU = 2;                     // groups per load unit
  constexpr int UB = 32;                    // bytes of one weight column per group
  constexpr bool kScales = OUT != kOutI32;
  constexpr int kC = 16 * kCB;              // columns per workgroup
  static_assert(!XQ || NU * GU <= kXqMaxGPW, "XQ slices");
  // this workgroup's 16-row block of the activations
  const int m0 = blockIdx.y * 16;
  const int M = min(16, Mtot - m0);
  if (sx != nullptr) sx += m0;
  __shared__ float lds_red[kWaves][kCB][4][64];
  __shared__ float s_xamax[XQ ? kWaves : 1][kGemvXqRows];
  __shared__ float s_xscale[kGemvXqRows];
  extern __shared__ uint32_t lds_sb[];      // [G][kC]: scale | offset << 16 (int4 only)

  const int G = K / 64;
  const int RB = K / 2;                     // bytes per weight row
  const int n0 = blockIdx.x * kC;
  const int cols = min(kC, N - n0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (readfirstlane): slice guards are scalar branches and
  // every MFMA runs with the full EXEC mask.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15;  // MFMA A row m / B column of this lane
  const int fc = lane >> 4;  // MFMA 16-wide k chunk / output row block
  const int per = ((G + kWaves - 1) / kWaves + GU - 1) / GU * GU;
  const int g0 = min(wave * per, G);
  const int gn = min(per, G - g0);  // 0 for trailing wavefronts of short K
  const int nu = (gn + GU - 1) / GU;

  // 1. Scale/offset staging loads: columns n0..n0+cols-1 of the [N, G]
  //    arrays are one contiguous run of cols*G halves; issued first so that
  //    the LDS writes below wait for these loads only.
  constexpr int kSL = kScales ? (NU * GU * kWaves * kC + kWaves * 64 - 1) / (kWaves * 64) : 1;
  uint32_t sreg[kSL];
  if (kScales) {
    const uint16_t* hs = gsv + (int64_t)n0 * G;
    const uint16_t* hb = gbv + (int64_t)n0 * G;
    const int lim = cols * G;
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
  // XQ: x with whole-line loads, issued before the weights (load counters
  // retire in order, so the absmax below then waits for x alone).  Lane l
  // takes row l/16 and, for t < kXT, the 16 bytes of values 8*(l%8)..+7 of
  // slice group 2t + (l%16)/8, so the 16 lanes of a row read 256
  // contiguous bytes per instruction.
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
  // Epilogue operands of column block wave (< kCB), loaded ahead of the
  // weights.
  const int eb = min(wave, kCB - 1);
  const int nn = n0 + 16 * eb + fr;
  const int nc = min(nn, N - 1);
  const float bv = bias ? bias[nc] : 0.0f;
  float sxm[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sxm[r] = (OUT != kOutI32 && !XQ) ? sx[min(4 * fc + r, M - 1)] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);

  // 2. Weight and activation loads of unit u (groups g0 + GU*u ..).
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wq + (int64_t)n0 * RB), 0,
      __builtin_amdgcn_readfirstlane(cols * RB), 0x00020000);
  const int8_t* abase = XQ ? reinterpret_cast<const int8_t*>(X)
                      : AF ? A + (int64_t)blockIdx.y * G * 1024 : A + (int64_t)m0 * K;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(abase), 0,
      __builtin_amdgcn_readfirstlane(XQ ? 0 : AF ? G * 1024 : M * K), 0x00020000);
  const int woff = fr * RB + UB * g0 + 16 * fc;
  const int kc0 = ((fc & 1) << 5) | ((fc & 2) << 3);  // k of chunk fc: 0, 32, 16, 48
  const int aoff = AF ? 1024 * g0 + 16 * lane : fr * K + 64 * g0 + kc0;
  constexpr int AG = AF ? 1024 : 64;        // A bytes from one group to the next
  v4i wr[D][kCB];
  v4i ar[XQ ? 1 : D][GU];
  auto issue = [&](int u, int s) {
    const bool ok = u < nu;  // wave-uniform
    if constexpr (!XQ) {
#pragma unroll
      for (int j = 0; j < GU; ++j) {
        const int gi = GU * u + j;
        ar[s][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
            ra, ok && gi < gn ? aoff + AG * gi : 0x40000000, 0, 0));
      }
    }
#pragma unroll
    for (int b = 0; b < kCB; ++b)
      wr[s][b] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
          rw, ok ? woff + 16 * b * RB + UB * GU * u : 0x40000000, 0, 0));
  };
#pragma unroll
  for (int u = 0; u < D; ++u) issue(u, u);
  __builtin_amdgcn_sched_barrier(0);

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
  if (kScales) {
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = tid + j * kWaves * 64;
      if (e < kC * G) {
        const int r = e / G, g = e - r * G;
        lds_sb[g * kC + r] = sreg[j];
      }
    }
  }
  if (kScales || XQ) {
    wait_vm_lgkm0<63>();  // LDS writes done; the weights may still fly
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
  // XQ operand of slice group gi: lane fr + 16*fc (rows fr < 4) takes the
  // codes of values kc0..kc0+15 of the group from lanes 16*fr + 8*(gi%2) +
  // kc0/8 and + 1 (their loads t = gi/2); rows 4-15 are zero.
  const int xsrc = 4 * (16 * (fr & 3) + kc0 / 8);  // ds_bpermute byte address, gi even
  auto xq_operand = [&](int gi) {
    const int sa = xsrc + 32 * (gi & 1);
    v4i f = v4i{__builtin_amdgcn_ds_bpermute(sa, xc[gi >> 1][0]),
                __builtin_amdgcn_ds_bpermute(sa, xc[gi >> 1][1]),
                __builtin_amdgcn_ds_bpermute(sa + 4, xc[gi >> 1][0]),
                __builtin_amdgcn_ds_bpermute(sa + 4, xc[gi >> 1][1])};
    if (fr >= kGemvXqRows) f = v4i{0, 0, 0, 0};
    return f;
  };

  v4f facc[kCB];
#pragma unroll
  for (int b = 0; b < kCB; ++b) facc[b] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  // One int4 group's products for both column blocks: the weight operands
  // (two dwords of nibbles each) and the codes.
  auto group_w4 = [&](int gi, const uint32_t (&d)[kCB][2], const v4i& fa_g) {
    const int g = g0 + gi;
    v4i p[kCB];
#pragma unroll
    for (int b = 0; b < kCB; ++b) {
      uint32_t u0, u1, u2, u3;
      unpack8_u4(d[b][0], u0, u1);
      unpack8_u4(d[b][1], u2, u3);
      p[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, v4i{(int)u0, (int)u1, (int)u2, (int)u3},
                                                   v4i{0, 0, 0, 0}, 0, 0, 0);
    }
    if (OUT == kOutI32) {
      // debug output: P of every group, [G, M, N]; p[b][r] = P[g, 4*fc + r, n]
#pragma unroll
      for (int b = 0; b < kCB; ++b) {
        const int n = n0 + 16 * b + fr;
        if (n < N && gi < gn) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = 4 * fc + r;
            if (m < M) reinterpret_cast<int32_t*>(y)[((int64_t)g * Mtot + m0 + m) * N + n] = p[b][r];
          }
        }
      }
    } else {
      const v4i as = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, ones, v4i{0, 0, 0, 0}, 0, 0, 0);
      float asf[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) asf[r] = (float)as[r];
#pragma unroll
      for (int b = 0; b < kCB; ++b) {
        // groups past the slice (the second group of a unit past G): zero
        // scale and offset, so their products add nothing
        const uint32_t sb = gi < gn ? lds_sb[g * kC + 16 * b + fr] : 0u;
        const float s = __half2float(__ushort_as_half((unsigned short)(sb & 0xffff)));
        const float o = __half2float(__ushort_as_half((unsigned short)(sb >> 16)));
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[b][r] = fmaf(o, asf[r], fmaf(s, (float)p[b][r], facc[b][r]));
      }
    }
  };

  // 3. Units in order as they arrive; the unit D ahead reuses the registers
  //    of the one just finished.
  for (int u0 = 0; u0 < nu; u0 += D) {  // one pass when all units are in flight
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int u = u0 + s;
      if (u >= nu) break;  // wave-uniform
      {
        uint32_t d0[kCB][2], d1[kCB][2];
#pragma unroll
        for (int b = 0; b < kCB; ++b) {
          const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)wr[s][b][0], (uint32_t)wr[s][b][2], false, false);
          const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)wr[s][b][1], (uint32_t)wr[s][b][3], false, false);
          d0[b][0] = lo[0];
          d0[b][1] = hi[0];
          d1[b][0] = lo[1];
          d1[b][1] = hi[1];
        }
        if constexpr (XQ) {
          group_w4(2 * u, d0, xq_operand(2 * u));
          group_w4(2 * u + 1, d1, xq_operand(2 * u + 1));
        } else {
          group_w4(2 * u, d0, ar[s][0]);
          group_w4(2 * u + 1, d1, ar[s][1]);
        }
      }
      if (u + D < NU) issue(u + D, s);
    }
  }
  if (OUT == kOutI32) return;

  // Reduce the 8 partials of each column block (fp32): wavefront b < kCB
  // finishes column block b.
#pragma unroll
  for (int b = 0; b < kCB; ++b) {
    if (wave == b) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) lds_red[wave][b][r][lane] = facc[b][r];
  }
  __syncthreads();
  if (wave >= kCB) return;
  v4f fs = facc[0];
#pragma unroll
  for (int b = 1; b < kCB; ++b)
    if (wave == b) fs = facc[b];
  if (XQ) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sxm[r] = s_xscale[min(4 * fc + r, M - 1)];
  }
  // slices in order 0..7, the wavefront's own at its place
  v4f ft = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) ft[r] += w == wave ? fs[r] : lds_red[w][eb][r][lane];
  if (nn >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * fc + r;
    if (m >= M) continue;
    const int64_t idx = (int64_t)(m0 + m) * N + nn;
    {
      float v = fmaf(sxm[r], ft[r], bv);
      if (ep.active()) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m0 + m, nn, N);
      if (OUT == kOutF32) reinterpret_cast<float*>(y)[idx] = v;
      else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA GEMV for int8 weights (M >= 3, or K > kFusedMaxK): 16 rows x 16
// output columns per workgroup of 8 wavefronts, each owning a K slice.  An
// int8 group is 64 bytes a column, so the register layout above would read
// half lines (16 columns x 64 bytes per instruction) twice as often as for
// int4; here the weights stream through a private LDS chunk per wavefront
// with direct buffer loads of 8 rows x one full 128-byte line, in the MFMA
// fragment order, four groups a chunk (measured faster for int8 than the
// register layout: 17.1 against 19.3 us at 4 x 5120 -> 13824).
constexpr int kChunk8 = 4;        // groups per LDS chunk of one wavefront
static_assert(kXqMaxGPW % kChunk8 == 0, "XQ slices are whole chunks");

template <int OUT, bool XQ, bool AF>
__global__ __launch_bounds__(kWaves * 64) void gemv_lds8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx,
    const int8_t* __restrict__ Wq, const float* __restrict__ sw,
    const float* __restrict__ bias, void* y, int Mtot, int N, int K, Epilogue ep,
    const uint16_t* __restrict__ X, float* __restrict__ sx_out) {
  // this workgroup's 16-row block of the activations
  const int m0 = blockIdx.y * 16;
  const int M = min(16, Mtot - m0);
  if (sx != nullptr) sx += m0;
  constexpr int UB = 64;                    // bytes of one weight row per group
  constexpr int LPR = UB / 16;              // DMA lanes per (row, group)
  constexpr int GPB = 128 / UB;             // groups per 128-byte line (one DMA block)
  constexpr int WLDS = kChunk8 * 16 * UB;   // LDS bytes of one wavefront's chunk
  static_assert(kChunk8 % GPB == 0, "a chunk is whole DMA blocks");
  __shared__ __attribute__((aligned(16))) int8_t lds_w[kWaves][WLDS];
  __shared__ float lds_red[kWaves - 1][4][64];
  __shared__ float s_xamax[XQ ? kWaves : 1][kGemvXqRows];
  __shared__ float s_xscale[kGemvXqRows];

  const int G = K / 64;
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

  // Weight DMA.  The descriptor is rebased on row n0 with num_records =
  // rows*K: rows past N and groups past the matrix end read as zero.  Block
  // (r8, blk) = rows 8*r8..8*r8+7 x groups blk*GPB.. of the chunk; lane l
  // moves 16 bytes: group l/(8*LPR), row (l/LPR)%8, piece l%LPR, into LDS
  // byte 16*l of the block, which puts (row r, chunk group i) at
  // (r/8)*kChunk8*8*UB + i*8*UB + (r%8)*UB -- the fragment order.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Wq + (int64_t)n0 * K), 0, rows * K, 0x00020000);
  const int d_gg = lane / (8 * LPR), d_rr = (lane / LPR) & 7, d_pc = lane % LPR;
  const int voff = d_rr * K + d_gg * UB + d_pc * 16;
  auto issue = [&](int gs, int gc) {
#pragma unroll
    for (int blk = 0; blk < kChunk8 / GPB; ++blk) {
      if (blk * GPB < gc) {
#pragma unroll
        for (int r8 = 0; r8 < 2; ++r8) {
          lds_ptr_t dst = (lds_ptr_t)(&lds_w[wave][r8 * (kChunk8 * 8 * UB) + blk * 1024]);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, voff,
                                                   r8 * 8 * K + (gs + blk * GPB) * UB, 0, 0);
        }
      }
    }
  };
  // Activation fragments of a chunk: A row fr (< M), k chunk fc; in the
  // fragment order one contiguous 1 KB per group of the 16-row block.
  v4i fa[kChunk8];
  const int8_t* arow = AF ? A + (int64_t)blockIdx.y * G * 1024 + 16 * lane
                          : A + (int64_t)(m0 + fr) * K + fc * 16;
  auto load_a = [&](int gs, int gc) {
#pragma unroll
    for (int i = 0; i < kChunk8; ++i) {
      int4 t = make_int4(0, 0, 0, 0);
      if (i < gc && (AF || fr < M)) t = *reinterpret_cast<const int4*>(arow + (gs + i) * (AF ? 1024 : 64));
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
  issue(g0, min(gn, kChunk8));
  if (!XQ) load_a(g0, min(gn, kChunk8));
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
  const float swn = OUT != kOutI32 ? sw[nc] : 0.0f;
  float sxm[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sxm[r] = (OUT != kOutI32 && !XQ) ? sx[min(4 * fc + r, M - 1)] : 0.0f;

  if (XQ) {
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

  v4i iacc = v4i{0, 0, 0, 0};
  const int8_t* wl = &lds_w[wave][(fr >> 3) * (kChunk8 * 8 * UB) + (fr & 7) * UB + fc * (UB / 4)];
  auto group_product = [&](int i, const v4i& fa_g) {
    const int4 wv = *reinterpret_cast<const int4*>(wl + i * 8 * UB);
    iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, v4i{wv.x, wv.y, wv.z, wv.w}, iacc, 0, 0, 0);
  };
  if constexpr (XQ) {
    // Operand of slice group gi: lane fr + 16*fc (rows fr < 4) takes the
    // codes of values 16*fc..16*fc+15 from lanes 16*fr + 8*(gi%2) + 2*fc and
    // + 1 (their loads t = gi/2); rows 4-15 are zero.  Fully unrolled, so
    // the register of each load is known.
    const int src0 = 4 * (16 * (fr & 3) + 2 * fc);  // ds_bpermute byte address, gi even
#pragma unroll
    for (int c0 = 0; c0 < kXqMaxGPW; c0 += kChunk8) {
      if (c0 >= gn) break;
      const int gc = min(kChunk8, gn - c0);
      if (c0 > 0) {
        wait_vm_lgkm0<63>();  // fragment reads of the last chunk done before the DMA reuses it
        issue(g0 + c0, gc);
      }
#pragma unroll
      for (int i = 0; i < kChunk8; ++i) {
        if (i < gc) {
          const int gi = c0 + i;
          const int sa = src0 + 32 * (gi & 1);
          v4i f = v4i{__builtin_amdgcn_ds_bpermute(sa, xc[gi >> 1][0]),
                      __builtin_amdgcn_ds_bpermute(sa, xc[gi >> 1][1]),
                      __builtin_amdgcn_ds_bpermute(sa + 4, xc[gi >> 1][0]),
                      __builtin_amdgcn_ds_bpermute(sa + 4, xc[gi >> 1][1])};
          if (fr >= kGemvXqRows) f = v4i{0, 0, 0, 0};
          group_product(i, f);
        }
      }
    }
  } else {
    for (int c0 = 0; c0 < gn; c0 += kChunk8) {
      const int gc = min(kChunk8, gn - c0);
      if (c0 > 0) {
        wait_vm_lgkm0<63>();  // fragment reads of the last chunk done before the DMA reuses it
        issue(g0 + c0, gc);
        load_a(g0 + c0, gc);
      }
#pragma unroll
      for (int i = 0; i < kChunk8; ++i)
        if (i < gc) group_product(i, fa[i]);
    }
  }

  // Reduce the 8 partials (exact int32).
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) lds_red[wave - 1][r][lane] = __int_as_float(iacc[r]);
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
    for (int r = 0; r < 4; ++r) iacc[r] += __float_as_int(lds_red[w][r][lane]);
  if (nn >= N) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * fc + r;
    if (m >= M) continue;
    const int64_t idx = (int64_t)(m0 + m) * N + nn;
    if (OUT == kOutI32) {
      reinterpret_cast<int32_t*>(y)[idx] = iacc[r];
    } else {
      float v = fmaf(sxm[r] * swn, (float)iacc[r], bv);
      if (ep.active()) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m0 + m, nn, N);
      if (OUT == kOutF32) reinterpret_cast<float*>(y)[idx] = v;
      else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------
// Lane-per-column GEMV for 1 <= M <= kGemvLaneRows rows with int4 weights (K <=
// kFusedMaxK).  The weight bytes are the whole cost (each read once, 0.5625
// B per weight), so every byte a workgroup needs is in flight before it
// computes anything, and the arithmetic per byte is kept small enough to
// finish while the loads of the other wavefronts are still arriving:
//   - a workgroup of 8 wavefronts owns 32 output columns: wavefront w takes
//     columns 8*(w%4) .. +8 and K slice w/4 (one half) of each row's
//     128-byte lines (four slices, 16 wavefronts, measured slower); lane
//     (c, p) = (l/8, l%8) takes the 16-byte piece p of each of those lines
//     of column c, i.e. half p%2 of group 4i + p/2 of line i.  The 8 lanes
//     of a column read whole lines, every load instruction moves 8 columns x
//     128 bytes, and the loads go straight to registers (up to 12 lines a
//     lane), all issued at once behind the activation and scale loads, so
//     the waits for those never wait for weights;
//   - the 32 weights of a half group are 4 dwords of nibbles; nibble 2b of a
//     dword (low half of byte b) is an even k and nibble 2b+1 an odd k, so
//     the low nibbles (w & 0x0f0f0f0f) and the high ones ((w >> 4) &
//     0x0f0f0f0f) are 4 int8 values each, without reordering.  The
//     activation codes sit in LDS split the same way (the even and the odd
//     codes of each run of 8), and v_dot4_i32_i8 takes 4 products a step: 8
//     steps (two chains) give the exact int32 dot product P of the half
//     group for one row (unsigned nibbles are non-negative int8);
//   - each lane rescales its own half groups: acc += gs*P + gb*A, with A the
//     half group's code sum and gs, gb as floats, both staged in LDS by the
//     prologue (gs = gb = 0 past the last group), so no lane exchange
//     happens per group; the 8 lanes of a column add their sums (xor 1, 2,
//     4), the second K half's sums go through LDS, and lane 0 of the first
//     half applies the epilogue.
// XQ (x given): the workgroup quantizes the rows itself with the quantize
// kernel's rule and rounding (bit-pattern absmax over the whole row, the
// 1.5*2^23 shift); the token scales go to sx_out.  Codes given (XQ false):
// the quantize kernel's codes and scales.
constexpr int kLSlices = 2;               // K slices of a column set
constexpr int kLWaves = 4 * kLSlices;
constexpr int kLCols = kGemvLaneCols;  // output columns per workgroup (4 sets of 8)
static_assert(kLCols == 32 && kLWaves * 64 == kGemvLaneThreads, "lane GEMV geometry");
constexpr int kLMaxLines = (int)(kFusedMaxK / 256);
static_assert(kFusedMaxK % (256 * kLSlices) == 0, "whole lines in each K slice");

// int8 codes of the 8 bf16 values of w[0..3], as codes8_shift computes them,
// split by parity: .x = codes 0, 2, 4, 6 and .y = codes 1, 3, 5, 7.
__device__ __forceinline__ uint2 codes8_shift_eo(const uint32_t w[4], float inv) {
#pragma clang fp contract(off)  // two roundings, as the rule has them: no fma
  uint32_t t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = bf16_to_f32(w[i] & 0xFFFFu) * inv;
    const float p1 = bf16_to_f32(w[i] >> 16) * inv;
    t[2 * i] = __float_as_uint(p0 + 12582912.0f);
    t[2 * i + 1] = __float_as_uint(p1 + 12582912.0f);
  }
  // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the
  // first, 0x0c gives zero
  uint32_t d[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t lo = __builtin_amdgcn_perm(t[2 + q], t[q], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(t[6 + q], t[4 + q], 0x0c0c0400u);
    d[q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  return make_uint2(d[0], d[1]);
}

// The same split of 8 codes given in value order (c0..c3 in d0, c4..c7 in d1).
__device__ __forceinline__ uint2 codes8_eo(uint32_t d0, uint32_t d1) {
  return make_uint2(__builtin_amdgcn_perm(d1, d0, 0x06040200u), __builtin_amdgcn_perm(d1, d0, 0x07050301u));
}

// NL: lines per wavefront (each takes one K slice of a row's lines), so K
// <= 256*kLSlices*NL.  WIN: lines a lane keeps in flight.  WIN = NL issues
// every line at once (one memory latency: grids too small to fill the
// chip).  On a grid that fills it every byte in flight at once makes the
// lines land in random order, and a wavefront consumes them in issue order
// (vmcnt), so most of the arithmetic waited for the last line; with a
// window of WIN lines, line i + WIN is issued when line i is consumed and
// the arithmetic runs under the loads (5120 -> 13824, M = 1, per call:
// 10.5 -> 9.3 us at WIN = 3; 9.6 at 2, 9.7 at 4, 10.0 at 5).
template <int OUT, bool XQ, int MR, int NL, int WIN>
__global__ __launch_bounds__(kLWaves * 64) void gemv_lane_kernel(
    const uint16_t* __restrict__ X, const int8_t* __restrict__ Acodes, const float* __restrict__ sx,
    const uint8_t* __restrict__ Wq, const uint16_t* __restrict__ GS, const uint16_t* __restrict__ GB,
    const float* __restrict__ bias, void* y, int M, int N, int K, Epilogue ep,
    float* __restrict__ sx_out) {
  static_assert(kLSlices * NL <= kLMaxLines && MR >= 1 && MR <= kGemvLaneRows, "lane GEMV shape");
  static_assert(WIN >= 1 && WIN <= NL, "line window");
  constexpr int kT = kLWaves * 64;
  constexpr int kMaxK = NL * 256 * kLSlices;                // K that the slices' lines cover
  constexpr int kHPT = (MR * kMaxK / 32 + kT - 1) / kT;     // half groups per thread
  constexpr bool kScales = OUT != kOutI32;
  constexpr int kG4 = kMaxK / 64;                           // groups of kLSlices*NL lines
  constexpr int kSPT = kScales ? (kLCols * kG4 + kT - 1) / kT : 1;  // scale entries per thread
  __shared__ __attribute__((aligned(16))) uint32_t s_code[MR * kMaxK / 4];  // [row][K] split codes
  __shared__ float s_hsum[MR * kMaxK / 32];                                 // [row][half group] code sums
  __shared__ float2 s_sb[kScales ? kLCols * kG4 : 1];                       // [column][group] (gs, gb)
  __shared__ float s_amax[XQ ? kLWaves : 1][MR];
  __shared__ float s_part[kScales ? kLSlices - 1 : 1][4][MR][64];           // later K slices' sums

  const int G = K / 64, H = K / 32;
  const int nl = (G + 3) / 4;          // lines per weight row
  const int nlh = (nl + kLSlices - 1) / kLSlices;  // lines of a K slice (<= NL)
  const int G4 = 4 * nl;               // groups with padding to whole lines
  const int n0 = blockIdx.x * kLCols;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = wave & 3, kh = wave >> 2;
  const int c8 = lane >> 3, p = lane & 7;
  const int nw = n0 + 8 * cw;        // first column of this wavefront
  const int n = nw + c8;             // this lane's column (>= N: computed, not stored)
  const int l0 = kh * nlh;                  // first line of this wavefront
  const int nlw = max(0, min(nlh, nl - l0)); // its lines (later slices may have fewer)

  // 1. activations: half groups h = tid + kT*j of rows < M (clamped index;
  //    the ones past the rows are loaded and not used)
  const int HM = M * H;
  v4i xv[XQ ? kHPT : 1][4];
  uint4 cv[XQ ? 1 : kHPT][2];
#pragma unroll
  for (int j = 0; j < kHPT; ++j) {
    const int h = min(tid + kT * j, HM - 1);
    const int r = h / H, hg = h - r * H;
    if constexpr (XQ) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[j][q] = *reinterpret_cast<const v4i*>(X + (int64_t)r * K + hg * 32 + 8 * q);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        cv[j][q] = *reinterpret_cast<const uint4*>(Acodes + (int64_t)r * K + hg * 32 + 16 * q);
    }
  }
  // 2. scales and offsets: entry e = c*G4 + g for the workgroup's column c
  //    (clamped to the last column) and group g (clamped to the last group;
  //    entries g >= G are stored as zero)
  uint16_t sh[kSPT], bh[kSPT];
  if constexpr (kScales) {
#pragma unroll
    for (int j = 0; j < kSPT; ++j) {
      const int e = min(tid + kT * j, kLCols * G4 - 1);
      const int c = e / G4, g = e - c * G4;
      const int64_t src = (int64_t)min(n0 + c, N - 1) * G + min(g, G - 1);
      sh[j] = GS[src];
      bh[j] = GB[src];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 3. weights: line l0 + i of column n at byte n*(K/2) + 128*(l0 + i),
  //    piece p.  The descriptor covers this wavefront's columns < N: columns
  //    past N read as zero; lines past the wavefront's share (i >= nlw) get
  //    an offset past the descriptor, so they read zero without touching
  //    memory.  (readfirstlane: a descriptor the compiler cannot prove
  //    uniform is taken apart lane by lane in a loop around every load.)
  const int nrec = __builtin_amdgcn_readfirstlane(max(0, min(8, N - nw)) * (K / 2));
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wq + (int64_t)min(nw, N - 1) * (K / 2)), 0, nrec, 0x00020000);
  const int voff = c8 * (K / 2) + 128 * l0 + 16 * p;
  auto load_line = [&](int i) {
    return __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, i < nlw ? voff + 128 * i : 0x40000000, 0, 0));
  };
  v4i wv[NL];
#pragma unroll
  for (int i = 0; i < WIN; ++i) wv[i] = load_line(i);  // the rest as lines are consumed
  __builtin_amdgcn_sched_barrier(0);

  // 4. row scales, codes and half-group sums into LDS
  const int ones = 0x01010101;
  float sxm[MR];
  if constexpr (XQ) {
    float amj[kHPT];
#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      u16x2 mb = u16x2{0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) mb = absmax_bits2(mb, (uint32_t)xv[j][q][d]);
      amj[j] = tid + kT * j < HM ? absmax_bits_value(mb) : 0.0f;
    }
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < kHPT; ++j) a = fmaxf(a, min(tid + kT * j, HM - 1) / H == rr ? amj[j] : 0.0f);
      a = wave_max(a);
      if (lane == 0) s_amax[wave][rr] = a;
    }
    wait_vm_lgkm0<63>();  // the LDS writes (the weight loads stay in flight)
    barrier_nofence();
    float inv[MR];
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      float am = s_amax[0][rr];
#pragma unroll
      for (int w = 1; w < kLWaves; ++w) am = fmaxf(am, s_amax[w][rr]);
      inv[rr] = row_inv(am, sxm[rr]);
      if (blockIdx.x == 0 && tid == rr && rr < M && sx_out != nullptr) sx_out[rr] = sxm[rr];
    }
#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      const int h = tid + kT * j;
      if (h >= HM) continue;
      const int r = h / H, hg = h - r * H;
      float iv = inv[0];
#pragma unroll
      for (int rr = 1; rr < MR; ++rr) iv = r == rr ? inv[rr] : iv;
      uint32_t c[8];
      int s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w4[4] = {(uint32_t)xv[j][q][0], (uint32_t)xv[j][q][1], (uint32_t)xv[j][q][2],
                                (uint32_t)xv[j][q][3]};
        const uint2 eo = codes8_shift_eo(w4, iv);
        c[2 * q] = eo.x;
        c[2 * q + 1] = eo.y;
        s = __builtin_amdgcn_sdot4((int)eo.x, ones, s, false);
        s = __builtin_amdgcn_sdot4((int)eo.y, ones, s, false);
      }
      uint4* dst = reinterpret_cast<uint4*>(s_code + r * (K / 4) + hg * 8);
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
      s_hsum[r * H + hg] = (float)s;
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) sxm[rr] = kScales ? sx[min(rr, M - 1)] : 0.0f;
#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      const int h = tid + kT * j;
      if (h >= HM) continue;
      const int r = h / H, hg = h - r * H;
      uint32_t c[8];
      int s = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint2 e0 = codes8_eo(cv[j][q].x, cv[j][q].y);
        const uint2 e1 = codes8_eo(cv[j][q].z, cv[j][q].w);
        c[4 * q] = e0.x;
        c[4 * q + 1] = e0.y;
        c[4 * q + 2] = e1.x;
        c[4 * q + 3] = e1.y;
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) s = __builtin_amdgcn_sdot4((int)c[d], ones, s, false);
      uint4* dst = reinterpret_cast<uint4*>(s_code + r * (K / 4) + hg * 8);
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
      s_hsum[r * H + hg] = (float)s;
    }
  }
  if constexpr (kScales) {
#pragma unroll
    for (int j = 0; j < kSPT; ++j) {
      const int e = tid + kT * j;
      if (e >= kLCols * G4) continue;
      const bool ok = e - (e / G4) * G4 < G;
      s_sb[e] = ok ? make_float2(__half2float(__ushort_as_half(sh[j])), __half2float(__ushort_as_half(bh[j])))
                   : make_float2(0.0f, 0.0f);
    }
  }
  // The half-group sums past the rows' (the main loop reads them for the
  // padding groups past G, with a zero offset): zero, not stale LDS.
  for (int e = HM + tid; e < MR * kMaxK / 32; e += kT) s_hsum[e] = 0.0f;
  wait_vm_lgkm0<63>();
  barrier_nofence();

  // 5. the half groups, line by line as they arrive (every LDS address is a
  //    per-lane base plus a constant offset per line)
  float facc[MR];
#pragma unroll
  for (int rr = 0; rr < MR; ++rr) facc[rr] = 0.0f;
  const int hh = p & 1;
  const int g0l = 4 * l0 + (p >> 1);  // the lane's group in its first line
  const float2* sbp = s_sb + (8 * cw + c8) * G4 + g0l;
  const uint32_t* cbase = s_code + 16 * g0l + 8 * hh;
  const float* hbase = s_hsum + 2 * g0l + hh;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if (i + WIN < NL) wv[i + WIN] = load_line(i + WIN);  // keep WIN lines in flight
    if (i >= nlw) continue;  // uniform
    const int g = g0l + 4 * i;  // < G4
    float2 so = make_float2(0.0f, 0.0f);
    if constexpr (kScales) so = sbp[4 * i];
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      // codes of half group 2g + hh of row rr (inside s_code for every g <
      // G4; unused past G: the scale and offset are zero there)
      const uint4* ap = reinterpret_cast<const uint4*>(cbase + rr * (K / 4) + 64 * i);
      const uint4 a0 = ap[0], a1 = ap[1];
      const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      int acc0 = 0, acc1 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = (uint32_t)wv[i][q];
        acc0 = __builtin_amdgcn_sdot4((int)(w & 0x0F0F0F0Fu), (int)a[2 * q], acc0, false);
        acc1 = __builtin_amdgcn_sdot4((int)((w >> 4) & 0x0F0F0F0Fu), (int)a[2 * q + 1], acc1, false);
      }
      const int acc = acc0 + acc1;
      if constexpr (OUT == kOutI32) {
        // debug output: P of every group, [G, M, N]
        const int pg = acc + __builtin_amdgcn_mov_dpp(acc, 0xB1, 0xF, 0xF, false);  // + lane ^ 1
        if (hh == 0 && g < G && n < N && rr < M)
          reinterpret_cast<int32_t*>(y)[((int64_t)g * M + rr) * N + n] = pg;
      } else {
        // (past the row's H entries: the next row's sums or the zeroed
        // tail, finite either way, times a zero offset)
        const float hs = hbase[rr * H + 8 * i];
        facc[rr] = fmaf(so.y, hs, fmaf(so.x, (float)acc, facc[rr]));
      }
    }
  }
  if constexpr (OUT == kOutI32) return;

  // 6. the column's 8 lanes, the later K slices through LDS, then the
  //    epilogue in lane p = 0 of the first slice, adding the slices in order
#pragma unroll
  for (int rr = 0; rr < MR; ++rr) {
    float v = facc[rr];
    v += __shfl_xor(v, 1, kWave);
    v += __shfl_xor(v, 2, kWave);
    v += __shfl_xor(v, 4, kWave);
    facc[rr] = v;
  }
  if (kh > 0) {
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) s_part[kh - 1][cw][rr][lane] = facc[rr];
  }
  __syncthreads();
  if (kh > 0 || p != 0 || n >= N) return;
#pragma unroll
  for (int rr = 0; rr < MR; ++rr)
#pragma unroll
    for (int k = 0; k < kLSlices - 1; ++k) facc[rr] += s_part[k][cw][rr][lane];
  const float bv = bias ? bias[n] : 0.0f;
#pragma unroll
  for (int rr = 0; rr < MR; ++rr) {
    if (rr >= M) continue;
    const int64_t idx = (int64_t)rr * N + n;
    float v = fmaf(sxm[rr], facc[rr], bv);
    if (ep.active()) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, rr, n, N);
    if (OUT == kOutF32) reinterpret_cast<float*>(y)[idx] = v;
    else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
  }
}

// Lines in flight per lane on grids that fill the chip (measured best).
constexpr int kLaneWin4 = 3, kLaneWin8 = 4;

// The windowed form on a grid of at least one workgroup per CU.
inline bool lane_streams(int N) { return (N + kLCols - 1) / kLCols >= kSplitCUs; }

template <bool XQ, int MR, int NL, int WIN>
void launch_lane_win(const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                     const void* gs, const void* gb, const float* bias, void* y, int out, int M,
                     int N, int K, hipStream_t s, const Epilogue& ep, float* sx_out) {
  const dim3 grid((unsigned)((N + kLCols - 1) / kLCols)), block(kLWaves * 64);
  const uint8_t* qw = reinterpret_cast<const uint8_t*>(q);
  const uint16_t* hs = reinterpret_cast<const uint16_t*>(gs);
  const uint16_t* hb = reinterpret_cast<const uint16_t*>(gb);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemv_lane_kernel<kOutF32, XQ, MR, NL, WIN>), grid, block, 0, s, x, a, sx, qw, hs, hb, bias, y, M, N, K, ep, sx_out);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemv_lane_kernel<kOutBF16, XQ, MR, NL, WIN>), grid, block, 0, s, x, a, sx, qw, hs, hb, bias, y, M, N, K, ep, sx_out);
  else
    hipLaunchKernelGGL((gemv_lane_kernel<kOutI32, XQ, MR, NL, WIN>), grid, block, 0, s, x, a, sx, qw, hs, hb, bias, y, M, N, K, ep, sx_out);
}

template <bool XQ, int MR, int NL>
void launch_lane_out(const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                     const void* gs, const void* gb, const float* bias, void* y, int out, int M,
                     int N, int K, hipStream_t s, const Epilogue& ep, float* sx_out) {
  if constexpr (NL > kLaneWin4) {
    if (lane_streams(N)) {
      launch_lane_win<XQ, MR, NL, kLaneWin4>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
      return;
    }
  }
  launch_lane_win<XQ, MR, NL, NL>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
}

template <bool XQ, int MR>
void launch_lane_mr(int nlh, const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                    const void* gs, const void* gb, const float* bias, void* y, int out, int M,
                    int N, int K, hipStream_t s, const Epilogue& ep, float* sx_out) {
  static_assert(kLSlices * 12 == kLMaxLines, "NL = 12 covers K = kFusedMaxK");
  if (nlh <= 2)
    launch_lane_out<XQ, MR, 2>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 4)
    launch_lane_out<XQ, MR, 4>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 6)
    launch_lane_out<XQ, MR, 6>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 8)
    launch_lane_out<XQ, MR, 8>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 10)
    launch_lane_out<XQ, MR, 10>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  else
    launch_lane_out<XQ, MR, 12>(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
}

// The lane-per-column GEMV (int4 weights, M <= kGemvLaneRows, K <=
// kFusedMaxK); x != NULL: it quantizes x itself.
const char* launch_lane(const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                        const void* gs, const void* gb, const float* bias, void* y, int out,
                        int M, int N, int K, hipStream_t s, const Epilogue& ep, float* sx_out) {
  const int nlh = ((K / 64 + 3) / 4 + kLSlices - 1) / kLSlices;
  if (x != nullptr) {
    if (M == 1) launch_lane_mr<true, 1>(nlh, x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
    else launch_lane_mr<true, 2>(nlh, x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
    return "gemv_xq_w4a8_lane";
  }
  if (M == 1) launch_lane_mr<false, 1>(nlh, x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  else launch_lane_mr<false, 2>(nlh, x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out);
  return "gemv_w4a8_lane";
}

// ---------------------------------------------------------------------------
// The lane-per-column GEMV for int8 weights (M <= kGemvLaneRows, K <=
// kFusedMaxK): the same workgroup and lane geometry as the int4 kernel
// above, with 128 weights per 128-byte line.  Per line and row a lane takes
// 16 weights and the 16 matching activation codes (natural order in LDS)
// in four v_dot4_i32_i8 steps; the int32 sum runs over the whole row (the
// scale is per output channel), the 8 lanes of a column and the two K
// slices add exactly, and the epilogue is the MFMA GEMV's expression,
// fma(sx*sw, acc, bias), so the outputs equal the other routes' bit for
// bit.  Codes past K (a half line at the end) are zero in LDS.
// WIN: lines a lane keeps in flight, as in the int4 kernel (the modulation
// linear 2x3072 -> 18432: 14.2 -> 13.95 us at WIN = 4).
template <int OUT, bool XQ, int MR, int NL, int WIN>
__global__ __launch_bounds__(kLWaves * 64) void gemv_lane8_kernel(
    const uint16_t* __restrict__ X, const int8_t* __restrict__ Acodes, const float* __restrict__ sx,
    const int8_t* __restrict__ Wq, const float* __restrict__ SW, const float* __restrict__ bias,
    void* y, int M, int N, int K, Epilogue ep, float* __restrict__ sx_out) {
  static_assert(kLSlices * NL <= 2 * kLMaxLines && MR >= 1 && MR <= kGemvLaneRows, "lane GEMV shape");
  static_assert(WIN >= 1 && WIN <= NL, "line window");
  constexpr int kT = kLWaves * 64;
  constexpr int kMaxK = NL * 128 * kLSlices;                // K that the slices' lines cover
  constexpr int kHPT = (MR * kMaxK / 32 + kT - 1) / kT;     // 32-value units per thread
  __shared__ __attribute__((aligned(16))) uint32_t s_code[MR * kMaxK / 4];  // [row][kMaxK] codes
  __shared__ float s_amax[XQ ? kLWaves : 1][MR];
  __shared__ int s_part[kLSlices - 1][4][MR][64];          // later K slices' sums

  const int H = K / 32;
  const int nl = (K + 127) / 128;                  // lines per weight row
  const int nlh = (nl + kLSlices - 1) / kLSlices;  // lines of a K slice (<= NL)
  const int n0 = blockIdx.x * kLCols;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = wave & 3, kh = wave >> 2;
  const int c8 = lane >> 3, p = lane & 7;
  const int nw = n0 + 8 * cw;
  const int n = nw + c8;
  const int l0 = kh * nlh;
  const int nlw = max(0, min(nlh, nl - l0));

  // 1. activations: 32-value units h = tid + kT*j of rows < M
  const int HM = M * H;
  v4i xv[XQ ? kHPT : 1][4];
  uint4 cv[XQ ? 1 : kHPT][2];
#pragma unroll
  for (int j = 0; j < kHPT; ++j) {
    const int h = min(tid + kT * j, HM - 1);
    const int r = h / H, hg = h - r * H;
    if constexpr (XQ) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[j][q] = *reinterpret_cast<const v4i*>(X + (int64_t)r * K + hg * 32 + 8 * q);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        cv[j][q] = *reinterpret_cast<const uint4*>(Acodes + (int64_t)r * K + hg * 32 + 16 * q);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // 2. weights: line l0 + i of column n at byte n*K + 128*(l0 + i), piece p
  //    (descriptor as in the int4 kernel: columns past N and lines past the
  //    wavefront's share read zero)
  const int nrec = __builtin_amdgcn_readfirstlane(max(0, min(8, N - nw)) * K);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(Wq + (int64_t)min(nw, N - 1) * K), 0, nrec, 0x00020000);
  const int voff = c8 * K + 128 * l0 + 16 * p;
  auto load_line = [&](int i) {
    return __builtin_bit_cast(
        v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, i < nlw ? voff + 128 * i : 0x40000000, 0, 0));
  };
  v4i wv[NL];
#pragma unroll
  for (int i = 0; i < WIN; ++i) wv[i] = load_line(i);  // the rest as lines are consumed
  __builtin_amdgcn_sched_barrier(0);

  // 3. row scales and codes into LDS (rows at a kMaxK-byte stride)
  float sxm[MR];
  if constexpr (XQ) {
    float amj[kHPT];
#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      u16x2 mb = u16x2{0, 0};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) mb = absmax_bits2(mb, (uint32_t)xv[j][q][d]);
      amj[j] = tid + kT * j < HM ? absmax_bits_value(mb) : 0.0f;
    }
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < kHPT; ++j) a = fmaxf(a, min(tid + kT * j, HM - 1) / H == rr ? amj[j] : 0.0f);
      a = wave_max(a);
      if (lane == 0) s_amax[wave][rr] = a;
    }
    wait_vm_lgkm0<63>();  // the LDS writes (the weight loads stay in flight)
    barrier_nofence();
    float inv[MR];
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      float am = s_amax[0][rr];
#pragma unroll
      for (int w = 1; w < kLWaves; ++w) am = fmaxf(am, s_amax[w][rr]);
      inv[rr] = row_inv(am, sxm[rr]);
      if (blockIdx.x == 0 && tid == rr && rr < M && sx_out != nullptr) sx_out[rr] = sxm[rr];
    }
#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      const int h = tid + kT * j;
      if (h >= HM) continue;
      const int r = h / H, hg = h - r * H;
      float iv = inv[0];
#pragma unroll
      for (int rr = 1; rr < MR; ++rr) iv = r == rr ? inv[rr] : iv;
      uint32_t c[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w4[4] = {(uint32_t)xv[j][q][0], (uint32_t)xv[j][q][1], (uint32_t)xv[j][q][2],
                                (uint32_t)xv[j][q][3]};
        const uint2 cc = codes8_shift(w4, iv);
        c[2 * q] = cc.x;
        c[2 * q + 1] = cc.y;
      }
      uint4* dst = reinterpret_cast<uint4*>(s_code + r * (kMaxK / 4) + hg * 8);
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    }
  } else {
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) sxm[rr] = OUT != kOutI32 ? sx[min(rr, M - 1)] : 0.0f;
#pragma unroll
    for (int j = 0; j < kHPT; ++j) {
      const int h = tid + kT * j;
      if (h >= HM) continue;
      const int r = h / H, hg = h - r * H;
      uint4* dst = reinterpret_cast<uint4*>(s_code + r * (kMaxK / 4) + hg * 8);
      dst[0] = cv[j][0];
      dst[1] = cv[j][1];
    }
  }
  // the codes past K in each row (a half line at the end): zero
  for (int e = tid; e < MR * (kMaxK - K) / 4; e += kT) {
    const int r = e / ((kMaxK - K) / 4), d = e - r * ((kMaxK - K) / 4);
    s_code[r * (kMaxK / 4) + K / 4 + d] = 0u;
  }
  wait_vm_lgkm0<63>();
  barrier_nofence();

  // 4. the lines as they arrive: 4 dot steps per line and row
  int acc[MR];
#pragma unroll
  for (int rr = 0; rr < MR; ++rr) acc[rr] = 0;
  const uint32_t* cbase = s_code + 32 * l0 + 4 * p;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if (i + WIN < NL) wv[i + WIN] = load_line(i + WIN);  // keep WIN lines in flight
    if (i >= nlw) continue;  // uniform
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      const uint4 a = *reinterpret_cast<const uint4*>(cbase + rr * (kMaxK / 4) + 32 * i);
      acc[rr] = __builtin_amdgcn_sdot4(wv[i][0], (int)a.x, acc[rr], false);
      acc[rr] = __builtin_amdgcn_sdot4(wv[i][1], (int)a.y, acc[rr], false);
      acc[rr] = __builtin_amdgcn_sdot4(wv[i][2], (int)a.z, acc[rr], false);
      acc[rr] = __builtin_amdgcn_sdot4(wv[i][3], (int)a.w, acc[rr], false);
    }
  }

  // 5. exact int32 sums over the column's 8 lanes and the K slices, then
  //    the epilogue in lane p = 0 of the first slice
#pragma unroll
  for (int rr = 0; rr < MR; ++rr) {
    int v = acc[rr];
    v += __shfl_xor(v, 1, kWave);
    v += __shfl_xor(v, 2, kWave);
    v += __shfl_xor(v, 4, kWave);
    acc[rr] = v;
  }
  if (kh > 0) {
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) s_part[kh - 1][cw][rr][lane] = acc[rr];
  }
  __syncthreads();
  if (kh > 0 || p != 0 || n >= N) return;
#pragma unroll
  for (int rr = 0; rr < MR; ++rr)
#pragma unroll
    for (int k = 0; k < kLSlices - 1; ++k) acc[rr] += s_part[k][cw][rr][lane];
  const float swn = OUT != kOutI32 ? SW[n] : 0.0f;
  const float bv = (OUT != kOutI32 && bias) ? bias[n] : 0.0f;
#pragma unroll
  for (int rr = 0; rr < MR; ++rr) {
    if (rr >= M) continue;
    const int64_t idx = (int64_t)rr * N + n;
    if (OUT == kOutI32) {
      reinterpret_cast<int32_t*>(y)[idx] = acc[rr];
    } else {
      float v = fmaf(sxm[rr] * swn, (float)acc[rr], bv);
      if (ep.active()) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, rr, n, N);
      if (OUT == kOutF32) reinterpret_cast<float*>(y)[idx] = v;
      else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <bool XQ, int MR, int NL, int WIN>
void launch_lane8_win(const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                      const void* sw, const float* bias, void* y, int out, int M, int N, int K,
                      hipStream_t s, const Epilogue& ep, float* sx_out) {
  const dim3 grid((unsigned)((N + kLCols - 1) / kLCols)), block(kLWaves * 64);
  const int8_t* qw = reinterpret_cast<const int8_t*>(q);
  const float* swf = reinterpret_cast<const float*>(sw);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemv_lane8_kernel<kOutF32, XQ, MR, NL, WIN>), grid, block, 0, s, x, a, sx, qw, swf, bias, y, M, N, K, ep, sx_out);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemv_lane8_kernel<kOutBF16, XQ, MR, NL, WIN>), grid, block, 0, s, x, a, sx, qw, swf, bias, y, M, N, K, ep, sx_out);
  else
    hipLaunchKernelGGL((gemv_lane8_kernel<kOutI32, XQ, MR, NL, WIN>), grid, block, 0, s, x, a, sx, qw, swf, bias, y, M, N, K, ep, sx_out);
}

template <bool XQ, int MR, int NL>
void launch_lane8_out(const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                      const void* sw, const float* bias, void* y, int out, int M, int N, int K,
                      hipStream_t s, const Epilogue& ep, float* sx_out) {
  if constexpr (NL > kLaneWin8) {
    if (lane_streams(N)) {
      launch_lane8_win<XQ, MR, NL, kLaneWin8>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
      return;
    }
  }
  launch_lane8_win<XQ, MR, NL, NL>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
}

template <bool XQ, int MR>
void launch_lane8_mr(int nlh, const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                     const void* sw, const float* bias, void* y, int out, int M, int N, int K,
                     hipStream_t s, const Epilogue& ep, float* sx_out) {
  static_assert(kLSlices * 24 == 2 * kLMaxLines, "NL = 24 covers K = kFusedMaxK");
  if (nlh <= 4)
    launch_lane8_out<XQ, MR, 4>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 8)
    launch_lane8_out<XQ, MR, 8>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 12)
    launch_lane8_out<XQ, MR, 12>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 16)
    launch_lane8_out<XQ, MR, 16>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  else if (nlh <= 20)
    launch_lane8_out<XQ, MR, 20>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  else
    launch_lane8_out<XQ, MR, 24>(x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
}

// The lane-per-column GEMV for int8 weights (M <= kGemvLaneRows, K <=
// kFusedMaxK); x != NULL: it quantizes x itself.
const char* launch_lane8(const uint16_t* x, const int8_t* a, const float* sx, const void* q,
                         const void* sw, const float* bias, void* y, int out, int M, int N, int K,
                         hipStream_t s, const Epilogue& ep, float* sx_out) {
  const int nlh = ((K + 127) / 128 + kLSlices - 1) / kLSlices;
  if (x != nullptr) {
    if (M == 1) launch_lane8_mr<true, 1>(nlh, x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
    else launch_lane8_mr<true, 2>(nlh, x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
    return "gemv_xq_w8a8_lane";
  }
  if (M == 1) launch_lane8_mr<false, 1>(nlh, x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  else launch_lane8_mr<false, 2>(nlh, x, a, sx, q, sw, bias, y, out, M, N, K, s, ep, sx_out);
  return "gemv_w8a8_lane";
}

template <int OUT, bool XQ, bool AF, int NU>
void launch_w4_out(dim3 grid, size_t sb, const int8_t* a, const float* sx, const void* q,
                   const void* gs, const void* gb, const float* bias, void* y, int M, int N,
                   int K, hipStream_t s, const Epilogue& ep, const uint16_t* x, float* sx_out) {
  // Two units in flight ahead of the arithmetic (measured best of 2, 3, 4
  // and all of them: deeper pipelines cost occupancy).
  constexpr int D = NU < 2 ? NU : 2;
  hipLaunchKernelGGL((gemv_w4_kernel<OUT, XQ, AF, NU, D>), grid, dim3(kWaves * 64), sb, s, a, sx,
                     reinterpret_cast<const uint8_t*>(q), reinterpret_cast<const uint16_t*>(gs),
                     reinterpret_cast<const uint16_t*>(gb), bias, y, M, N, K, ep, x, sx_out);
}

template <bool XQ, bool AF, int NU>
void launch_w4_nu(dim3 grid, size_t sb, const int8_t* a, const float* sx, const void* q,
                  const void* gs, const void* gb, const float* bias, void* y, int out, int M,
                  int N, int K, hipStream_t s, const Epilogue& ep, const uint16_t* x,
                  float* sx_out) {
  if (out == kOutF32)
    launch_w4_out<kOutF32, XQ, AF, NU>(grid, sb, a, sx, q, gs, gb, bias, y, M, N, K, s, ep, x, sx_out);
  else if (out == kOutBF16)
    launch_w4_out<kOutBF16, XQ, AF, NU>(grid, sb, a, sx, q, gs, gb, bias, y, M, N, K, s, ep, x, sx_out);
  else
    launch_w4_out<kOutI32, XQ, AF, NU>(grid, sb, a, sx, q, gs, gb, bias, y, M, N, K, s, ep, x, sx_out);
}

template <bool XQ, bool AF>
const char* launch_w4(const int8_t* a, const float* sx, const void* q, const void* gs,
                      const void* gb, const float* bias, void* y, int out, int M, int N, int K,
                      hipStream_t s, const Epilogue& ep, const uint16_t* x, float* sx_out) {
  const dim3 grid((unsigned)((N + kGemvCols - 1) / kGemvCols), (unsigned)((M + 15) / 16));
  const size_t sb = out != kOutI32 ? (size_t)kGemvCols * (K / 64) * sizeof(uint32_t) : 0;
  const int nu = ((K / 64 + kWaves - 1) / kWaves + 1) / 2;  // load units per wavefront
#define KQ_GEMV_NU(n) \
  launch_w4_nu<XQ, AF, n>(grid, sb, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, x, sx_out)
  if constexpr (XQ) {
    // K <= kFusedMaxK: at most kXqMaxGPW groups a wavefront
    static_assert(kXqMaxGPW == 12, "XQ unit counts");
    if (nu <= 2) KQ_GEMV_NU(2);
    else if (nu <= 4) KQ_GEMV_NU(4);
    else KQ_GEMV_NU(6);
  } else {
    static_assert(kGemvMaxK / 64 / kWaves <= 32, "unit counts");
    if (nu <= 2) KQ_GEMV_NU(2);
    else if (nu <= 4) KQ_GEMV_NU(4);
    else if (nu <= 6) KQ_GEMV_NU(6);
    else if (nu <= 8) KQ_GEMV_NU(8);
    else KQ_GEMV_NU(16);
  }
#undef KQ_GEMV_NU
  return XQ ? "gemv_xq_w4a8" : "gemv_w4a8";
}

template <bool XQ, bool AF>
const char* launch_w8(const int8_t* a, const float* sx, const void* q, const void* sw,
                      const float* bias, void* y, int out, int M, int N, int K, hipStream_t s,
                      const Epilogue& ep, const uint16_t* x, float* sx_out) {
  const dim3 grid((unsigned)((N + kGemvCols8 - 1) / kGemvCols8), (unsigned)((M + 15) / 16)),
      block(kWaves * 64);
  const int8_t* qw = reinterpret_cast<const int8_t*>(q);
  const float* swf = reinterpret_cast<const float*>(sw);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemv_lds8_kernel<kOutF32, XQ, AF>), grid, block, 0, s, a, sx, qw, swf, bias, y, M, N, K, ep, x, sx_out);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemv_lds8_kernel<kOutBF16, XQ, AF>), grid, block, 0, s, a, sx, qw, swf, bias, y, M, N, K, ep, x, sx_out);
  else
    hipLaunchKernelGGL((gemv_lds8_kernel<kOutI32, XQ, AF>), grid, block, 0, s, a, sx, qw, swf, bias, y, M, N, K, ep, x, sx_out);
  return XQ ? "gemv_xq_w8a8" : "gemv_w8a8";
}

}  // namespace

const char* launch_gemv(bool w4, const int8_t* a, const float* sx, const int32_t* /*gsum*/,
                        const void* q, const void* gs, const void* gb, const float* bias,
                        void* y, int out, int M, int N, int K, hipStream_t s,
                        const Epilogue& ep, const uint16_t* x, float* sx_out, bool lane,
                        bool frag) {
  if (lane && M <= kGemvLaneRows && K <= kFusedMaxK)
    return w4 ? launch_lane(x, a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, sx_out)
              : launch_lane8(x, a, sx, q, gs, bias, y, out, M, N, K, s, ep, sx_out);
  if (x != nullptr)
    return w4 ? launch_w4<true, false>(nullptr, nullptr, q, gs, gb, bias, y, out, M, N, K, s, ep, x, sx_out)
              : launch_w8<true, false>(nullptr, nullptr, q, gs, bias, y, out, M, N, K, s, ep, x, sx_out);
  if (frag)
    return w4 ? launch_w4<false, true>(a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, nullptr, nullptr)
              : launch_w8<false, true>(a, sx, q, gs, bias, y, out, M, N, K, s, ep, nullptr, nullptr);
  return w4 ? launch_w4<false, false>(a, sx, q, gs, gb, bias, y, out, M, N, K, s, ep, nullptr, nullptr)
            : launch_w8<false, false>(a, sx, q, gs, bias, y, out, M, N, K, s, ep, nullptr, nullptr);
}

}  // namespace kq
