// Thin-N linear with the activation quantization inside the kernel: one
// launch per call for N <= 64 output columns at any M.
//
// "qlip-mlx" README, w8a8_linear bullet: the per-token activation
// quantization happens inside the kernel.  For the tiled GEMM this would
// re-read each row block once per column tile; with N <= 64 a workgroup
// covers every output column of its rows, so x is read exactly once and the
// int8 codes never leave registers.  The separate quantize pass (x in, codes
// out, codes read back) moves about 2.5x the bytes this kernel does.
//
// Same rules and math as the two-kernel route:
//   codes: amax = max |x| over the row, inv = fp32(127/amax), code =
//          clamp(rint(x*inv), -127, 127), sx = fp32(amax/127) (the quantize
//          kernel's helpers, so codes and scales are identical bit for bit);
//   int8 weights: y = (sx*sw) * acc + bias, acc the exact int32 dot product;
//   int4 weights: y = sx * sum_g (gs*P + gb*A) + bias, P the exact int32
//          dot product of one 64-wide group, A the group sum of the codes.
//
// gfx950 design (HBM-bound on x):
//   - a workgroup of 16 wavefronts owns 16 activation rows and all N
//     columns (up to 4 blocks of 16); the wavefronts split the K groups into
//     16 contiguous slices of at most 6 groups (K <= 6144);
//   - each lane loads the 32 bytes of bf16 x that form its MFMA fragment
//     (row lane%16, k = 16*(lane/16)..+15 of each group of its slice), so
//     the quantized values are already in operand order.  The two 16-byte
//     loads of a fragment touch the same lines, so the second hits the L1:
//     ordinary loads measured 13% faster than non-temporal ones here;
//   - the codes: the absmax on the bf16 bit patterns (packed 16-bit max),
//     rint through the 1.5*2^23 shift, bytes packed with v_perm_b32; about
//     5 VALU operations per element, the kernel's largest cost after the
//     loads;
//   - the row absmax: in-lane max, two cross-lane steps over the 4 lanes of
//     a row, then the 16 slice maxima through LDS;
//   - the weights (N*K bytes, shared by every workgroup and therefore served
//     by the L2) are loaded into registers in chunks; the first chunk is in
//     flight while x arrives;
//   - v_mfma_i32_16x16x64_i8 with the codes as the A operand; for int4
//     weights a second MFMA against an all-ones operand gives the group sums
//     A exactly;
//   - the 16 slice partials are reduced through LDS in slice order (exact
//     int32 for int8 weights), one output element per thread.
#include <type_traits>

#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = kFusedThreads / 64;               // K slices per workgroup
constexpr int kMaxG = (int)(kFusedMaxK / 64);            // groups per row at most
constexpr int kMaxGPW = (kMaxG + kWaves - 1) / kWaves;   // groups per slice at most
static_assert(kFusedRows == 16, "one MFMA row block per workgroup");

// W4: int4 weights (gsv/gbv fp16 [N, K/64]); else int8 (gsv fp32 [N]).
// NB: 16-column blocks (N <= 16*NB).
template <bool W4, int OUT, int NB>
__global__ __launch_bounds__(kFusedThreads) void thin_fused_kernel(
    const uint16_t* __restrict__ x, float* __restrict__ sx_out, const void* __restrict__ Wq,
    const void* __restrict__ gsv, const void* __restrict__ gbv, const float* __restrict__ bias,
    void* y, int M, int N, int K, Epilogue ep) {
  // Weight fragments per chunk: at most 24 registers, two chunks in flight
  // (VGPR budget of 128 with 16 wavefronts per workgroup; x takes 48).
  constexpr int kWRegs = W4 ? 2 : 4;  // registers per (group, column block)
  constexpr int kChCap = 24 / (kWRegs * NB);
  constexpr int kCh = kChCap < 1 ? 1 : (kChCap > kMaxGPW ? kMaxGPW : kChCap);
  constexpr bool kScales = W4 && OUT != kOutI32;
  constexpr int kSL = kScales ? (kMaxG * 16 * NB + kFusedThreads - 1) / kFusedThreads : 1;
  __shared__ float s_amax[kWaves][16];
  __shared__ float s_scale[16];
  __shared__ float s_red[kWaves][NB * 4][64];
  __shared__ uint32_t s_sb[kScales ? kMaxG * 16 * NB : 1];  // [g][n]: scale | offset << 16

  const int m0 = blockIdx.x * kFusedRows;
  const int G = K / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (readfirstlane): the slice guards are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15;  // MFMA A row / B column of this lane
  const int fc = lane >> 4;  // 16-wide k chunk of a group / output row block
  const int per = (G + kWaves - 1) / kWaves;
  const int g0 = min(wave * per, G);
  const int gn = min(per, G - g0);  // 0 for trailing slices of short K
  const int m = m0 + fr;            // this lane's activation row

  // 1. Scale/offset staging loads (int4): rows 0..N-1 of the [N, G] arrays
  //    are one contiguous run of N*G halves.
  uint32_t sreg[kSL];
  if (kScales) {
    const uint16_t* hs = reinterpret_cast<const uint16_t*>(gsv);
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(gbv);
    const int lim = N * G;
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = tid + j * kFusedThreads;
      uint32_t v = 0;
      if (e < lim) v = (uint32_t)hs[e] | ((uint32_t)hb[e] << 16);
      sreg[j] = v;
    }
  }

  // 2. x fragments: 16 bf16 of row m per group, k = 16*fc..16*fc+15.
  v4i xv[kMaxGPW][2];
  {
    const v4i* xr = reinterpret_cast<const v4i*>(x + (int64_t)min(m, M - 1) * K + 16 * fc);
#pragma unroll
    for (int i = 0; i < kMaxGPW; ++i) {
      xv[i][0] = v4i{0, 0, 0, 0};
      xv[i][1] = v4i{0, 0, 0, 0};
      if (i < gn && m < M) {
        xv[i][0] = xr[(g0 + i) * 8];
        xv[i][1] = xr[(g0 + i) * 8 + 1];
      }
    }
  }

  // 3. Weight fragments of one chunk: column n = 16*cb + fr, the 16 k of
  //    chunk fc (int8: 16 bytes; int4: 8 bytes, unpacked before use).
  typedef typename std::conditional<W4, uint2, int4>::type WFrag;
  WFrag wf[2][kCh][NB];  // chunk c0/kCh goes to wf[(c0/kCh) % 2]
  auto load_chunk = [&](int c0) {
    WFrag (&dst)[kCh][NB] = wf[(c0 / kCh) & 1];
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int n = 16 * cb + fr;
        const int g = g0 + c0 + i;
        if constexpr (W4) {
          uint2 v = make_uint2(0, 0);
          if (c0 + i < gn && n < N)
            v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(Wq) +
                                                (int64_t)n * (K / 2) + g * 32 + 8 * fc);
          dst[i][cb] = v;
        } else {
          int4 v = make_int4(0, 0, 0, 0);
          if (c0 + i < gn && n < N)
            v = *reinterpret_cast<const int4*>(reinterpret_cast<const int8_t*>(Wq) +
                                               (int64_t)n * K + g * 64 + 16 * fc);
          dst[i][cb] = v;
        }
      }
    }
  };
  load_chunk(0);

  // 4. Row absmax over the whole row: in-lane, then the 4 lanes of the row,
  //    then the 16 slices.
  //    For finite values |x| orders as its magnitude bits, so the max runs
  //    on the bf16 bit patterns, two at a time (exact, and no fp32 copy of x
  //    stays live).
  u16x2 mx = u16x2{0, 0};
#pragma unroll
  for (int i = 0; i < kMaxGPW; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, (uint32_t)xv[i][h][j] & 0x7FFF7FFFu));
  const uint32_t mbits = max((uint32_t)mx.x, (uint32_t)mx.y);
  float amax = bf16_to_f32(mbits);
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  if (fc == 0) s_amax[wave][fr] = amax;
  if (kScales) {
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = tid + j * kFusedThreads;
      if (e < N * G) {
        const int n = e / G, g = e - n * G;
        s_sb[g * (16 * NB) + n] = sreg[j];
      }
    }
  }
  wait_vm_lgkm0<63>();  // LDS writes done; weight loads may still fly
  barrier_nofence();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, s_amax[w][fr]);
  float scale;
  const float inv = row_inv(amax, scale);
  if (wave == 0 && fc == 0) {
    s_scale[fr] = scale;
    if (sx_out != nullptr && m < M) sx_out[m] = scale;
  }

  // 5. Codes in MFMA operand order.  rint(x*inv) through the 1.5*2^23
  //    shift: the product rounds once, and adding 1.5*2^23 (exact spacing 1
  //    at that magnitude) rounds it to the nearest integer, ties to even,
  //    leaving the code in the low byte of the sum's bits.  No clamp: with
  //    inv = fp32(127/amax), |x*inv| <= 127*(1 + 2^-24)^2 < 127.5.
  v4i fa[kMaxGPW];
#pragma unroll
  for (int i = 0; i < kMaxGPW; ++i) {
#pragma clang fp contract(off)  // two roundings, as the rule has them: no fma
    uint32_t t[16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)xv[i][h][j];
        const float p0 = bf16_to_f32(w & 0xFFFFu) * inv;
        const float p1 = bf16_to_f32(w >> 16) * inv;
        t[8 * h + 2 * j] = __float_as_uint(p0 + 12582912.0f);
        t[8 * h + 2 * j + 1] = __float_as_uint(p1 + 12582912.0f);
      }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // v_perm_b32 selectors: bytes 0-3 come from the second operand, 4-7
      // from the first, 0x0c gives zero
      const uint32_t lo = __builtin_amdgcn_perm(t[4 * d + 1], t[4 * d], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(t[4 * d + 3], t[4 * d + 2], 0x0c0c0400u);
      fa[i][d] = (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
  }

  // 6. Products over the slice, one weight chunk at a time.
  v4i iacc[NB];
  v4f facc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    iacc[cb] = v4i{0, 0, 0, 0};
    facc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  // the later chunks' loads stay below this point (hoisted, they would
  // hold registers next to x)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c0 = 0; c0 < kMaxGPW; c0 += kCh) {
    if (c0 + kCh < kMaxGPW) load_chunk(c0 + kCh);
    const WFrag (&cur)[kCh][NB] = wf[(c0 / kCh) & 1];
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int gi = c0 + i;
      if (gi >= kMaxGPW || gi >= gn) continue;
      const int g = g0 + gi;
      if constexpr (W4) {
        v4i as = v4i{0, 0, 0, 0};
        if (OUT != kOutI32) as = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[gi], ones, as, 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const uint2 wv = cur[i][cb];
          uint32_t u0, u1, u2, u3;
          unpack8_u4(wv.x, u0, u1);
          unpack8_u4(wv.y, u2, u3);
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              fa[gi], v4i{(int)u0, (int)u1, (int)u2, (int)u3}, v4i{0, 0, 0, 0}, 0, 0, 0);
          const int n = 16 * cb + fr;
          if (OUT == kOutI32) {
            // debug output: P of every group, [G, M, N]; p[r] = P[g, m0 + 4*fc + r, n]
            if (n < N) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int mr = m0 + 4 * fc + r;
                if (mr < M) reinterpret_cast<int32_t*>(y)[((int64_t)g * M + mr) * N + n] = p[r];
              }
            }
          } else {
            const uint32_t sb = s_sb[g * (16 * NB) + n];
            const float s = __half2float(__ushort_as_half((unsigned short)(sb & 0xffff)));
            const float b = __half2float(__ushort_as_half((unsigned short)(sb >> 16)));
#pragma unroll
            for (int r = 0; r < 4; ++r)
              facc[cb][r] = fmaf(b, (float)as[r], fmaf(s, (float)p[r], facc[cb][r]));
          }
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const int4 wv = cur[i][cb];
          iacc[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[gi], v4i{wv.x, wv.y, wv.z, wv.w},
                                                           iacc[cb], 0, 0, 0);
        }
      }
    }
  }
  if (W4 && OUT == kOutI32) return;

  // 7. Slice partials -> LDS; thread t then sums element t over the slices
  //    in order and applies the epilogue.  Element e = (cb*4 + r)*64 + l is
  //    output row m0 + 4*(l/16) + r, column 16*cb + l%16.
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      s_red[wave][cb * 4 + r][lane] = W4 ? facc[cb][r] : __int_as_float(iacc[cb][r]);
  __syncthreads();
  if (tid >= NB * 256) return;
  const int j = tid >> 6, l = tid & 63;
  const int cb = j >> 2, r = j & 3;
  const int mo = m0 + 4 * (l >> 4) + r;
  const int n = 16 * cb + (l & 15);
  if (mo >= M || n >= N) return;
  float fs = 0.0f;
  int32_t is = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (W4) fs += s_red[w][j][l];
    else is += __float_as_int(s_red[w][j][l]);
  }
  const int64_t idx = (int64_t)mo * N + n;
  if (OUT == kOutI32) {
    reinterpret_cast<int32_t*>(y)[idx] = is;
    return;
  }
  const float sm = s_scale[mo - m0];
  const float bv = bias ? bias[n] : 0.0f;
  float v;
  if (W4) {
    v = fmaf(sm, fs, bv);
  } else {
    const float swn = reinterpret_cast<const float*>(gsv)[n];
    v = fmaf(sm * swn, (float)is, bv);
  }
  if (ep.active()) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, mo, n, N);
  if (OUT == kOutF32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
}

template <bool W4, int OUT>
void launch_nb(const uint16_t* x, float* sx, const void* q, const void* gs, const void* gb,
               const float* bias, void* y, int M, int N, int K, hipStream_t s,
               const Epilogue& ep) {
  const dim3 grid((unsigned)((M + kFusedRows - 1) / kFusedRows)), block(kFusedThreads);
  switch ((N + 15) / 16) {
    case 1: hipLaunchKernelGGL((thin_fused_kernel<W4, OUT, 1>), grid, block, 0, s, x, sx, q, gs, gb, bias, y, M, N, K, ep); break;
    case 2: hipLaunchKernelGGL((thin_fused_kernel<W4, OUT, 2>), grid, block, 0, s, x, sx, q, gs, gb, bias, y, M, N, K, ep); break;
    case 3: hipLaunchKernelGGL((thin_fused_kernel<W4, OUT, 3>), grid, block, 0, s, x, sx, q, gs, gb, bias, y, M, N, K, ep); break;
    default: hipLaunchKernelGGL((thin_fused_kernel<W4, OUT, 4>), grid, block, 0, s, x, sx, q, gs, gb, bias, y, M, N, K, ep); break;
  }
}

template <bool W4>
const char* launch_fmt(const uint16_t* x, float* sx, const void* q, const void* gs, const void* gb,
                       const float* bias, void* y, int out, int M, int N, int K, hipStream_t s,
                       const Epilogue& ep) {
  if (out == kOutF32) launch_nb<W4, kOutF32>(x, sx, q, gs, gb, bias, y, M, N, K, s, ep);
  else if (out == kOutBF16) launch_nb<W4, kOutBF16>(x, sx, q, gs, gb, bias, y, M, N, K, s, ep);
  else launch_nb<W4, kOutI32>(x, sx, q, gs, gb, bias, y, M, N, K, s, ep);
  return W4 ? "thin_fused_w4a8" : "thin_fused_w8a8";
}

}  // namespace

const char* launch_thin_fused(bool w4, const uint16_t* x, float* sx, const void* q, const void* gs,
                              const void* gb, const float* bias, void* y, int out, int M, int N,
                              int K, hipStream_t s, const Epilogue& ep) {
  return w4 ? launch_fmt<true>(x, sx, q, gs, gb, bias, y, out, M, N, K, s, ep)
            : launch_fmt<false>(x, sx, q, gs, gb, bias, y, out, M, N, K, s, ep);
}

}  // namespace kq
