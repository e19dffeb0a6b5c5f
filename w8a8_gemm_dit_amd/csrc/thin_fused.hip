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
//          kernel's helpers row_inv and codes8_shift, so codes and scales
//          are identical bit for bit);
//   int8 weights: y = (sx*sw) * acc + bias, acc the exact int32 dot product;
//   int4 weights: y = sx * sum_g (gs*P + gb*A) + bias, P the exact int32
//          dot product of one 64-wide group, A the group sum of the codes.
//
// gfx950 design (HBM-bound on x):
//   - a workgroup of 16 wavefronts owns 8 activation rows and all N columns
//     (up to 4 blocks of 16); the wavefronts split the K groups into 16
//     contiguous slices, each a whole number of 128-byte weight lines (2
//     groups of int8 weights, 4 of int4), at most 8 groups (K <= 6144).
//     Eight rows per workgroup give 256 workgroups at M = 2048;
//   - x is read with whole lines: lane l loads 16 bytes (8 values) of row
//     l/8, so one load instruction covers 8 rows x 128 bytes;
//   - the row absmax: a packed 16-bit max over the bf16 bit patterns (for
//     finite values the magnitude bits order as |x|), 3 cross-lane steps
//     over the 8 lanes of a row, then the 16 slice maxima through LDS;
//   - the codes: rint(x*inv) through the 1.5*2^23 shift (codes8_shift;
//     about 5 VALU operations per element with the max), then moved into
//     MFMA operand order with 4 ds_bpermute per group (lane
//     m + 16*c takes codes 16c..16c+15 of row m % 8 from the two lanes that
//     hold them); the MFMA's rows 8-15 repeat rows 0-7 and are discarded;
//   - the weights (N*K bytes, read by every workgroup, so served by the L2)
//     stream through a wavefront-private LDS chunk with direct global->LDS
//     loads: one instruction moves 8 rows x one whole 128-byte line into
//     the MFMA fragment order.  Loading them into registers instead (16
//     rows x 64 bytes per instruction, the fragment layout) measured 1.6x
//     slower for the whole kernel.  The first chunk is issued with x;
//   - v_mfma_i32_16x16x64_i8 with the codes as the A operand; for int4
//     weights a second MFMA against an all-ones operand gives the group sums
//     A exactly;
//   - the slices are rotated by the workgroup index, so that the workgroups
//     do not all ask the same L2 channels for the same weight lines at once;
//   - the 16 slice partials go to the wavefronts' LDS chunks and are summed
//     in slice order (exact int32 for int8 weights), one output element per
//     thread.
#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

constexpr int kWaves = kFusedThreads / 64;               // K slices per workgroup
constexpr int kRows = kFusedRows;                        // activation rows per workgroup
constexpr int kMaxG = (int)(kFusedMaxK / 64);            // groups per row at most
constexpr int kMaxGPW = 8;                               // groups per slice at most
static_assert(kRows == 8, "lane l of the x loads takes row l/8");
static_assert((kWaves & (kWaves - 1)) == 0, "slice rotation by masking");
static_assert(((kMaxG + kWaves - 1) / kWaves + 3) / 4 * 4 <= kMaxGPW, "slices of whole lines");

// W4: int4 weights (gsv/gbv fp16 [N, K/64]); else int8 (gsv fp32 [N]).
// NB: 16-column blocks (N <= 16*NB).
template <bool W4, int OUT, int NB>
__global__ __launch_bounds__(kFusedThreads) void thin_fused_kernel(
    const uint16_t* __restrict__ x, float* __restrict__ sx_out, const void* __restrict__ Wq,
    const void* __restrict__ gsv, const void* __restrict__ gbv, const float* __restrict__ bias,
    void* y, int M, int N, int K, Epilogue ep) {
  constexpr int UB = W4 ? 32 : 64;     // bytes of one weight row per group
  constexpr int LPR = UB / 16;         // DMA lanes per (row, group)
  constexpr int GPB = 128 / UB;        // groups per 128-byte line = groups per chunk
  constexpr bool kScales = W4 && OUT != kOutI32;
  constexpr int kSL = kScales ? (kMaxG * 16 * NB + kFusedThreads - 1) / kFusedThreads : 1;
  __shared__ float s_amax[kWaves][kRows];
  __shared__ float s_scale[kRows];
  // per wavefront: one chunk of weight lines, [cb][r8][1 KB DMA block]; at
  // the end its partial sums
  __shared__ int4 s_w[kWaves][NB * 2 * 64];
  __shared__ uint32_t s_sb[kScales ? kMaxG * 16 * NB : 1];  // [g][n]: scale | offset << 16
  static_assert(NB * 2 * 1024 >= NB * 4 * 64 * 4, "partial sums fit the chunk");

  const int m0 = blockIdx.x * kRows;
  const int G = K / 64;
  const int RB = W4 ? K / 2 : K;    // bytes per weight row
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (readfirstlane): the slice guards are scalar branches and
  // the LDS DMA bases stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = ((G + kWaves - 1) / kWaves + GPB - 1) / GPB * GPB;
  // Slice of this wavefront, rotated by the workgroup index: every
  // workgroup reads all of the weights.
  const int slice = (wave + (int)blockIdx.x) & (kWaves - 1);
  const int g0 = min(slice * per, G);
  const int gn = min(per, G - g0);  // 0 for trailing slices of short K
  const int xr = lane >> 3;         // x loads: row m0 + xr, values 8*xc..8*xc+7 of a group
  const int xc = lane & 7;
  const int mx = m0 + xr;
  const int fr = lane & 15;         // MFMA A row (codes of row fr % 8) / B column
  const int fc = lane >> 4;         // 16-wide k chunk of a group / output row block

  // 1. Scale/offset staging loads (int4): rows 0..N-1 of the [N, G] arrays
  //    are one contiguous run of N*G halves.
  uint32_t sreg[kSL];
  if (kScales) {
    const uint16_t* hs = reinterpret_cast<const uint16_t*>(gsv);
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(gbv);
    const int lim = N * G;
    // Unconditional loads at a clamped index (lim >= 1): all of them issue
    // back to back (loads under a per-lane guard were each waited for
    // before the next one issued).
    uint16_t sl[kSL], bl[kSL];
#pragma unroll
    for (int j = 0; j < kSL; ++j) {
      const int e = min(tid + j * kFusedThreads, lim - 1);
      sl[j] = hs[e];
      bl[j] = hb[e];
    }
#pragma unroll
    for (int j = 0; j < kSL; ++j)
      sreg[j] = tid + j * kFusedThreads < lim ? (uint32_t)sl[j] | ((uint32_t)bl[j] << 16) : 0u;
  }

  // 2. x: one whole-line load per group (8 rows x 128 bytes per instruction).
  v4i xv[kMaxGPW];
  {
    const v4i* xrow = reinterpret_cast<const v4i*>(x + (int64_t)min(mx, M - 1) * K + 8 * xc);
#pragma unroll
    for (int i = 0; i < kMaxGPW; ++i) {
      xv[i] = v4i{0, 0, 0, 0};
      if (i < gn && mx < M) xv[i] = xrow[(g0 + i) * 8];
    }
  }

  // 3. Weight DMA of one chunk (the GPB groups from g0 + c): the descriptor
  //    covers rows 0..N-1, so rows past N read as zero; lane l moves the 16
  //    bytes of (group l/(8*LPR), row (l/LPR)%8, piece l%LPR) of its block
  //    to LDS byte 16*l of the block, which puts (row r, group i, chunk fc)
  //    at block (cb, r/8), byte i*8*UB + (r%8)*UB + fc*UB/4: the fragment
  //    order.  Bytes past the slice or past K (the next row's, or zeros past
  //    the last) land in groups that are never read.
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(Wq), 0, N * RB, 0x00020000);
  const int voff = ((lane / LPR) & 7) * RB + (lane / (8 * LPR)) * UB + (lane % LPR) * 16;
  auto issue = [&](int c) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r8 = 0; r8 < 2; ++r8) {
        lds_ptr_t dst = (lds_ptr_t)(&s_w[wave][(cb * 2 + r8) * 64]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, voff,
                                                 (16 * cb + 8 * r8) * RB + (g0 + c) * UB, 0, 0);
      }
  };
  if (gn > 0) issue(0);

  // 4. Row absmax over the whole row: in-lane (two values at a time, on the
  //    bit patterns), then the 8 lanes of the row, then the 16 slices.
  u16x2 mxb = u16x2{0, 0};
#pragma unroll
  for (int i = 0; i < kMaxGPW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) mxb = absmax_bits2(mxb, (uint32_t)xv[i][j]);
  float amax = absmax_bits_value(mxb);
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
  if (xc == 0) s_amax[wave][xr] = amax;
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
  wait_vm_lgkm0<63>();  // LDS writes done; the weight DMA may still fly
  barrier_nofence();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) amax = fmaxf(amax, s_amax[w][xr]);
  float scale;
  const float inv = row_inv(amax, scale);
  if (wave == 0 && xc == 0) {
    s_scale[xr] = scale;
    if (sx_out != nullptr && mx < M) sx_out[mx] = scale;
  }

  // 5. Codes (codes8_shift: the quantize kernel's rule), then operand order:
  //    lane fr + 16*fc takes its 16 codes from lanes 8*(fr%8) + 2*fc and + 1.
  const int src0 = 4 * (8 * (fr & 7) + 2 * fc);  // ds_bpermute byte address
  const int src1 = src0 + 4;
  v4i fa[kMaxGPW];
#pragma unroll
  for (int i = 0; i < kMaxGPW; ++i) {
    const uint32_t w[4] = {(uint32_t)xv[i][0], (uint32_t)xv[i][1], (uint32_t)xv[i][2],
                           (uint32_t)xv[i][3]};
    const uint2 c = codes8_shift(w, inv);
    fa[i] = v4i{__builtin_amdgcn_ds_bpermute(src0, (int)c.x), __builtin_amdgcn_ds_bpermute(src0, (int)c.y),
                __builtin_amdgcn_ds_bpermute(src1, (int)c.x), __builtin_amdgcn_ds_bpermute(src1, (int)c.y)};
  }

  // 6. Products over the slice, one chunk of weight lines at a time.
  v4i iacc[NB];
  v4f facc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    iacc[cb] = v4i{0, 0, 0, 0};
    facc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  const char* wl = reinterpret_cast<const char*>(&s_w[wave][0]) + (fr >> 3) * 1024 +
                   (fr & 7) * UB + fc * (UB / 4);
#pragma unroll
  for (int c = 0; c < kMaxGPW; c += GPB) {
    if (c >= gn) break;
    if (c > 0) {
      wait_vm_lgkm0<63>();  // fragment reads of the last chunk done before the DMA reuses it
      issue(c);
    }
    wait_vm_lgkm0<0>();     // this chunk has landed
#pragma unroll
    for (int i = 0; i < GPB; ++i) {
      const int gi = c + i;
      if (gi >= gn) continue;
      const int g = g0 + gi;
      const v4i fa_g = fa[gi];
      if constexpr (W4) {
        v4i as = v4i{0, 0, 0, 0};
        if (OUT != kOutI32) as = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, ones, as, 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const uint2 wv = *reinterpret_cast<const uint2*>(wl + cb * 2048 + i * 8 * UB);
          uint32_t u0, u1, u2, u3;
          unpack8_u4(wv.x, u0, u1);
          unpack8_u4(wv.y, u2, u3);
          const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              fa_g, v4i{(int)u0, (int)u1, (int)u2, (int)u3}, v4i{0, 0, 0, 0}, 0, 0, 0);
          const int n = 16 * cb + fr;
          if (OUT == kOutI32) {
            // debug output: P of every group, [G, M, N]; p[r] = P[g, m0 + 4*fc + r, n]
            // (lanes with fc >= 2 hold the repeated rows)
            if (n < N && fc < 2) {
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
          const int4 wv = *reinterpret_cast<const int4*>(wl + cb * 2048 + i * 8 * UB);
          iacc[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa_g, v4i{wv.x, wv.y, wv.z, wv.w},
                                                           iacc[cb], 0, 0, 0);
        }
      }
    }
  }
  if (W4 && OUT == kOutI32) return;

  // 7. Slice partials -> the wavefront's chunk buffer (its reads are done);
  //    thread t then sums element t over the slices in order and applies
  //    the epilogue.  Element e = (cb*4 + r)*64 + l is output row
  //    m0 + 4*(l/16) + r (l < 32; the rest repeat rows), column 16*cb + l%16.
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  float* part = reinterpret_cast<float*>(&s_w[wave][0]);
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      part[(cb * 4 + r) * 64 + lane] = W4 ? facc[cb][r] : __int_as_float(iacc[cb][r]);
  __syncthreads();
  if (tid >= NB * 256) return;
  const int j = tid >> 6, l = tid & 63;
  if (l >= 32) return;
  const int cb = j >> 2, r = j & 3;
  const int mo = m0 + 4 * (l >> 4) + r;
  const int n = 16 * cb + (l & 15);
  if (mo >= M || n >= N) return;
  float fs = 0.0f;
  int32_t is = 0;
#pragma unroll
  for (int sl = 0; sl < kWaves; ++sl) {  // in slice order
    const int w = (sl - (int)blockIdx.x) & (kWaves - 1);
    const float v = reinterpret_cast<const float*>(&s_w[w][0])[j * 64 + l];
    if (W4) fs += v;
    else is += __float_as_int(v);
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
