// Device-side helpers shared by the libkq kernels (gfx950 only).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;  // CDNA wavefront width

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 rounds to nearest even in one v_cvt_pk_bf16_f32 (gfx950),
// two values per instruction: the same result as adding 0x7fff plus the
// kept bit's parity to the fp32 pattern and truncating, for every finite
// input, in a fifth of the instructions.
typedef __bf16 kq_bf16x2 __attribute__((ext_vector_type(2)));
typedef float kq_f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

// Two fp32 -> packed bf16x2 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(kq_f32x2{a, b}, kq_bf16x2));
}

// Wave-wide reductions over all 64 lanes (result in every lane).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, kWave));
  return v;
}

// int8 code of one value: clamp(rint(v * inv), -127, 127).  The product is a
// single IEEE multiply (no contraction possible), rintf is round-half-even.
__device__ __forceinline__ int quant_code(float v, float inv) {
  float t = rintf(v * inv);
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return (int)t;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running max of |x| over the two bf16 values of a dword, on their bit
// patterns: for finite values the magnitude bits order as |x| (exact).
__device__ __forceinline__ u16x2 absmax_bits2(u16x2 m, uint32_t w) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}

// |x| max as a float from absmax_bits2's running value.
__device__ __forceinline__ float absmax_bits_value(u16x2 m) {
  return bf16_to_f32(max((uint32_t)m.x, (uint32_t)m.y));
}

// int8 codes of the 8 bf16 values of w[0..3] (low half first), 4 per dword
// in value order, with inv from row_inv: the same result as quant_code.
// rint(x*inv) goes through the 1.5*2^23 shift: the product rounds once, and
// adding 1.5*2^23 (exact spacing 1 at that magnitude) rounds it to the
// nearest integer, ties to even, leaving the code in the low byte of the
// sum's bits.  No clamp: inv = fp32(127/amax) gives |x*inv| <= 127*(1 +
// 2^-24)^2 < 127.5 (and inv = 0 gives 0).
__device__ __forceinline__ uint2 codes8_shift(const uint32_t w[4], float inv) {
#pragma clang fp contract(off)  // two roundings, as the rule has them: no fma
  uint32_t t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p0 = bf16_to_f32(w[i] & 0xFFFFu) * inv;
    const float p1 = bf16_to_f32(w[i] >> 16) * inv;
    t[2 * i] = __float_as_uint(p0 + 12582912.0f);
    t[2 * i + 1] = __float_as_uint(p1 + 12582912.0f);
  }
  // v_perm_b32 selectors: bytes 0-3 come from the second operand, 4-7 from
  // the first, 0x0c gives zero
  uint32_t d[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t lo = __builtin_amdgcn_perm(t[4 * q + 1], t[4 * q], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(t[4 * q + 3], t[4 * q + 2], 0x0c0c0400u);
    d[q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
  }
  return make_uint2(d[0], d[1]);
}

// Per-row scale rule of the symmetric int8 quantizer: inv = fp32(127/amax)
// and scale = fp32(amax/127); a row whose 127/amax is not a finite fp32
// (all zero, or too small) gets inv 0 (codes 0) and scale 0.
__device__ __forceinline__ float row_inv(float amax, float& scale) {
  const float inv = 127.0f / amax;
  const bool ok = inv <= 3.402823466e38f;  // false for +inf
  scale = ok ? amax / 127.0f : 0.0f;
  return ok ? inv : 0.0f;
}

// Gated residual of one output element (see kq::Epilogue): fma(g, v, r)
// with g = gate[m / gate_rows][n] (1 without a gate) and r the bf16
// residual at [m][n] (0 without one); one rounding, in fp32.
__device__ __forceinline__ float gated1(float v, const uint16_t* residual, const float* gate,
                                        int gate_rows, int64_t m, int n, int N) {
  const float g = gate ? gate[(m / gate_rows) * (int64_t)N + n] : 1.0f;
  const float r = residual ? bf16_to_f32(residual[m * (int64_t)N + n]) : 0.0f;
  return fmaf(g, v, r);
}

// Pack four int8 codes into one dword (byte i = code i).
__device__ __forceinline__ uint32_t pack4_i8(int c0, int c1, int c2, int c3) {
  return (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) |
         ((uint32_t)(c2 & 0xFF) << 16) | ((uint32_t)(c3 & 0xFF) << 24);
}

// Unpack 8 int4 codes (one dword, low nibble of byte j = code 2j, high
// nibble = code 2j+1) into 8 int8 codes in k order, as two dwords.
__device__ __forceinline__ void unpack8_u4(uint32_t d, uint32_t& lo4, uint32_t& hi4) {
  const uint32_t lo = d & 0x0F0F0F0Fu;          // codes 0,2,4,6
  const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
  // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the first.
  lo4 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // codes 0,1,2,3
  hi4 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // codes 4,5,6,7
}

// Map a linear workgroup id onto a tile id so that the workgroups one XCD
// runs (ids congruent mod 8 are dispatched to the same XCD) get a
// contiguous range of tiles, which share operand panels in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcds = 8;
  if (nblocks % kXcds != 0) return bid;
  const int per = nblocks / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

// Output tile of workgroup `bid` in a tiles_m x tiles_n grid: XCD-contiguous
// index ranges (xcd_remap), walked in groups of kGroupRows tile rows,
// column by column.  The tiles an XCD runs at the same time then form a
// compact block (4 rows x 8 columns for 32 CUs), so its L2 fetches fewer
// distinct activation and weight panels than with a row-major walk.
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n,
                                            int& tm, int& tn) {
  constexpr int kGroupRows = 4;
  const int t = xcd_remap(bid, nblocks);
  const int group = t / (kGroupRows * tiles_n);
  const int first = group * kGroupRows;
  const int rows = min(tiles_m - first, kGroupRows);  // the last group may be shorter
  const int r = t - group * kGroupRows * tiles_n;
  tm = first + r % rows;
  tn = r / rows;
}

// LDS pointer type taken by the direct global->LDS buffer loads.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// s_waitcnt with vmcnt = N (compile-time) and lgkmcnt = 0 (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt bits 6:4 left at
// "no wait", lgkmcnt bits 11:8).  N = 63 waits for LDS/scalar traffic only.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0 << 8));
}

// Workgroup barrier without a memory fence (a fence would wait for the
// loads still in flight); the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace kq
