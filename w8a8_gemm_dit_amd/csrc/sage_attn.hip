// INT8 attention, flash-attention structure ("qlip-mlx" README,
// sage_attention bullet: INT8 QK^T inside a flash-attention loop with an
// exact online softmax; "Key features": softmax and P.V in floating point,
// head dim 128, mask-free).
//
// One workgroup: 128 query rows of one (b, h), 4 wavefronts of 32 rows.
// Per step of 64 keys:
//   S^T = Kc . Qc^T on v_mfma_i32_16x16x64_i8 (key codes from LDS, query
//     codes held in registers for the whole loop).  Computing the transpose
//     leaves each lane with one query row and 16 keys, which is already the
//     operand layout the P.V product takes: no LDS round trip for P;
//   online softmax in fp32 with exp2 (the scale, the query scale and log2 e
//     folded into one factor per row, the key scale applied per column);
//     the row max is reduced across the 4 lanes that share a row;
//   O^T += V^T . P^T on v_mfma_f32_16x16x32_f16, P rounded to fp16 and V^T
//     read from LDS in the key order the S^T layout produces (the
//     preparation pass wrote V transposed in that order).
// Key codes, V^T and key scales of step j+1 move into the other half of a
// double-buffered LDS stage by direct global->LDS loads while step j
// computes; one barrier per step.
#include "kq_common.hpp"
#include "sage.hpp"

// 16-row query blocks per wavefront (a build-time choice): 2 gives 4
// wavefronts of 32 rows, 2 wavefronts per SIMD; 1 gives 8 wavefronts of 16
// rows and 4 per SIMD, but every wavefront then reads the whole key and
// value tiles for half the rows, and the LDS traffic makes it 4% slower.
#ifndef KQB
#define KQB 2
#endif

namespace kq {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kQB = KQB;      // 16-row query blocks per wavefront
constexpr int kWaves = kSageQTile / (16 * kQB);
constexpr int kKBytes = kSageKTile * kSageD;       // key codes of one step
constexpr int kVBytes = kSageD * kSageKTile * 2;   // V^T of one step
constexpr int kSBytes = kSageKTile * 4;            // key scales of one step
constexpr int kStage = kKBytes + kVBytes + kSBytes;
// The score accumulators start at the bit pattern of 1.5 * 2^23: an int32
// result then reads as the float 1.5 * 2^23 + S (exact, |S| <= 128 * 127^2
// < 2^22), and one exact subtraction replaces the int -> float conversion.
constexpr int kMagic = 0x4B400000;
constexpr float kMagicF = 12582912.0f;
static_assert(kWaves * 16 * kQB == kSageQTile && 8 % kWaves == 0, "query tile split");
constexpr int kKPerWave = 8 / kWaves;    // 1 KB key-code loads per wavefront
constexpr int kVPerWave = 16 / kWaves;   // 1 KB V^T loads per wavefront

// 16-byte chunk swizzle of 128-byte LDS rows: chunk c of row r sits at
// c ^ ((r >> 1) & 7).  16 consecutive rows read at one logical chunk then
// hit 16 distinct 16-byte bank groups (rows r and r+1 are 128 bytes apart,
// the XOR spreads the 8 even and the 8 odd rows over all 8 chunks).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// KUNI: the key scale is uniform over each 64-key step (k_block >= 64), so
// the exponent is one fma of the converted score and the step's max is an
// integer max.  It reads the key block the preparation recorded in the
// workspace (meta[0]); if that block is shorter than a step, the scales are
// not uniform and the workgroup writes NaN to its output rows instead of
// wrong values (the host cannot read the workspace without a sync).
template <bool KUNI>
__global__ __launch_bounds__(kWaves * 64) void sage_attn_kernel(
    const int8_t* __restrict__ qc, const float* __restrict__ sqs, const int8_t* __restrict__ kc,
    const float* __restrict__ sks, const uint16_t* __restrict__ vt, uint16_t* __restrict__ out,
    SageStrides so, int H, int Lq, int Lk, int Lqp, int Lkp, float c_log2,
    const int32_t* __restrict__ meta) {
  // Three stages: step j's keys are read at step j, its values at step
  // j+1 (the P.V product runs one step behind the scores), and step j+1's
  // loads land meanwhile.
  __shared__ __attribute__((aligned(16))) char lds[3][kStage];

  const int ntq = Lqp / kSageQTile;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = t / ntq, qt = t % ntq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, g = lane >> 4;
  const int q0 = qt * kSageQTile + wave * 16 * kQB;
  if (KUNI && __builtin_amdgcn_readfirstlane(meta[0]) < kSageKTile) {
    const int b = bh / H, hh = bh % H;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int q = q0 + 16 * qb + fr;
      if (q >= Lq) continue;
      uint16_t* orow = out + (int64_t)b * so.b + (int64_t)hh * so.h + (int64_t)q * so.l + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *reinterpret_cast<uint2*>(orow + 16 * db) = make_uint2(0x7E007E00u, 0x7E007E00u);
    }
    return;
  }

  // Query codes (B operand of S^T: row q = fr, 16 bytes at chunk g of each
  // 64-channel half) and the per-row exponent factor.
  v4i qf[kQB][2];
  float aq[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int8_t* qr = qc + ((int64_t)bh * Lqp + q0 + 16 * qb + fr) * kSageD + 16 * g;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) qf[qb][dh] = *reinterpret_cast<const v4i*>(qr + 64 * dh);
    aq[qb] = sqs[(int64_t)bh * Lqp + q0 + 16 * qb + fr] * c_log2;
  }

  // Direct global->LDS loads: one instruction fills 1 KB = 8 rows of 128
  // bytes; lane l writes row l/8, physical chunk l%8, which holds logical
  // chunk (l%8) ^ swz(row).  swz of row 8b+i is ((b&1)<<2) | (i>>1), so two
  // per-lane offsets (block parity) serve every block.
  const int dr = lane >> 3, dc = lane & 7;
  const uint32_t voff0 = (uint32_t)(dr * 128 + ((dc ^ (dr >> 1)) * 16));
  const uint32_t voff1 = (uint32_t)(dr * 128 + ((dc ^ (4 | (dr >> 1))) * 16));
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(kc + (int64_t)bh * Lkp * kSageD), 0, Lkp * kSageD, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vt + (int64_t)bh * Lkp * kSageD), 0, Lkp * kSageD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(sks + (int64_t)bh * Lkp), 0, Lkp * 4, 0x00020000);
  auto issue = [&](int stage, int j) {
    char* base = lds[stage];
#pragma unroll
    for (int i = 0; i < kKPerWave; ++i) {  // key codes: 8 blocks
      const int b = kKPerWave * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(base + 1024 * b), 16,
                                               (b & 1) ? voff1 : voff0,
                                               j * kKBytes + 1024 * b, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kVPerWave; ++i) {  // V^T: 16 blocks
      const int b = kVPerWave * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(base + kKBytes + 1024 * b), 16,
                                               (b & 1) ? voff1 : voff0,
                                               j * kVBytes + 1024 * b, 0, 0);
    }
    if (wave == 0 && lane < kSBytes / 16)  // key scales: 16 lanes x 16 bytes
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(base + kKBytes + kVBytes), 16,
                                               (uint32_t)(lane * 16), j * kSBytes, 0, 0);
  };

  // O^T accumulators; block 8 multiplies P by a block of ones, so it holds
  // the row sums of the rounded P (in every lane of the row), rescaled with
  // the rest.
  v4f o[9][kQB];
  float m[kQB];  // exponent reference of the row, shared by its 4 lanes
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m[qb] = -INFINITY;
#pragma unroll
    for (int db = 0; db < 9; ++db) o[db][qb] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const v8h ones = v8h{1, 1, 1, 1, 1, 1, 1, 1};

  // S^T of one step: keys 16kb + (4g + r), query fr.
  auto scores = [&](int cur, v4i (&st)[4][kQB]) {
    const char* ks = lds[cur];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int row = 16 * kb + fr;
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) st[kb][qb] = v4i{kMagic, kMagic, kMagic, kMagic};
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        const v4i kf = *reinterpret_cast<const v4i*>(ks + row * 128 + (((4 * dh + g) ^ swz(row)) * 16));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          st[kb][qb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kf, qf[qb][dh], st[kb][qb], 0, 0, 0);
      }
    }
  };

  // O^T[d][q] += V^T[d][slots] . P^T[slots][q] for the values of stage
  // `cur`; block 8: the row sums.
  auto pv = [&](int cur, const v8h (&pf)[2][kQB]) {
    const char* vs = lds[cur] + kKBytes;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int row = 16 * db + fr;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v8h vf = *reinterpret_cast<const v8h*>(vs + row * 128 + (((4 * h + g) ^ swz(row)) * 16));
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[h][qb], o[db][qb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        o[8][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[h][qb], o[8][qb], 0, 0, 0);
  };

  // Online softmax of one step's scores -> fp16 probabilities pf.  MASK:
  // the last step, keys >= kvalid take no part.  The exponent reference m
  // of a row only moves when the row's max exceeds it by more than kSlack
  // (log2 units): the probabilities then stay below 2^kSlack (exact enough
  // in fp16, far from overflow) and O, which already holds the products of
  // every earlier step, is rescaled on a handful of steps only.
  constexpr float kSlack = 8.0f;
  auto softmax = [&](int cur, const v4i (&st)[4][kQB], int kvalid, auto mask_tag,
                     v8h (&pf)[2][kQB]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const float* ss = reinterpret_cast<const float*>(lds[cur] + kKBytes + kVBytes);
    float skv[4][4];
    if (KUNI) {
      const float s0 = ss[0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) skv[kb][r] = s0;
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4 s4 = *reinterpret_cast<const float4*>(ss + 16 * kb + 4 * g);
        skv[kb][0] = s4.x; skv[kb][1] = s4.y; skv[kb][2] = s4.z; skv[kb][3] = s4.w;
      }
    }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      // exponent of key (kb, r): x * mul - m (log2 units); x is the int32
      // score converted (KUNI: mul = the step's key scale x aq) or times
      // its key scale (mul = aq); both factors are >= 0, so the max of the
      // exponents is the max of x times mul.
      float x[4][4];
      float xmax, mul;
      if (KUNI && !MASK) {
        mul = skv[0][0] * aq[qb];
        int imax = st[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            imax = max(imax, st[kb][qb][r]);
            x[kb][r] = __int_as_float(st[kb][qb][r]) - kMagicF;
          }
        xmax = __int_as_float(imax) - kMagicF;
      } else {
        mul = aq[qb];
        xmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[kb][r] = (__int_as_float(st[kb][qb][r]) - kMagicF) * skv[kb][r];
            if (!MASK || 16 * kb + 4 * g + r < kvalid) xmax = fmaxf(xmax, x[kb][r]);
          }
      }
      const float tmax = xmax * mul;
      if (__any(tmax > m[qb] + kSlack)) {  // wave-uniform: move the reference
        float rm = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        rm = fmaxf(rm, __shfl_xor(rm, 32, kWave));
        const float mnew = fmaxf(m[qb], rm);
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
        m[qb] = mnew;
#pragma unroll
        for (int db = 0; db < 9; ++db) o[db][qb] *= alpha;
      }
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(x[kb][r], mul, -m[qb]));
          p[kb][r] = (!MASK || 16 * kb + 4 * g + r < kvalid) ? e : 0.0f;
        }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pf[h][qb] = v8h{(_Float16)p[2 * h][0], (_Float16)p[2 * h][1], (_Float16)p[2 * h][2],
                        (_Float16)p[2 * h][3], (_Float16)p[2 * h + 1][0], (_Float16)p[2 * h + 1][1],
                        (_Float16)p[2 * h + 1][2], (_Float16)p[2 * h + 1][3]};
    }
  };

  using NoMask = std::integral_constant<bool, false>;
  using Mask = std::integral_constant<bool, true>;
  const int nsteps = (Lk + kSageKTile - 1) / kSageKTile;
  const bool ragged = (Lk % kSageKTile) != 0;
  const int nfull = ragged ? nsteps - 1 : nsteps;

  // Step j: the scores of step j, the P.V product of step j-1 (its MFMAs
  // do not depend on the scores, so the two run back to back), the softmax
  // of step j.  Before the first step the probabilities are zero and their
  // product (on step 0's finite values) adds nothing.  The ragged last
  // step runs outside the loop.
  v8h pf[2][kQB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) pf[h][qb] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
  int prev = 0;
  auto run = [&](int j, auto mask_tag) {
    const int cur = j % 3;
    wait_vm_lgkm0<0>();
    barrier_nofence();  // step j has landed; every wave is done with step j-1
    if (j + 1 < nsteps) issue((j + 1) % 3, j + 1);
    v4i st[4][kQB];
    // The wave issuing MFMAs gets the higher priority, so that the other
    // wave on the SIMD fills the matrix pipe's busy cycles with its softmax
    // instead of competing for issue slots.
    __builtin_amdgcn_s_setprio(1);
    scores(cur, st);
    pv(prev, pf);
    __builtin_amdgcn_s_setprio(0);
    softmax(cur, st, Lk - j * kSageKTile, mask_tag, pf);
    prev = cur;
  };
  issue(0, 0);
  for (int j = 0; j < nfull; ++j) run(j, NoMask{});
  if (ragged) run(nsteps - 1, Mask{});
  pv(prev, pf);
  wait_vm_lgkm0<0>();

  const int b = bh / H, hh = bh % H;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float inv = 1.0f / o[8][qb][0];
    const int q = q0 + 16 * qb + fr;
    if (q >= Lq) continue;
    uint16_t* orow = out + (int64_t)b * so.b + (int64_t)hh * so.h + (int64_t)q * so.l + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const v4f v = o[db][qb] * inv;
      const _Float16 h0 = (_Float16)v[0], h1 = (_Float16)v[1], h2 = (_Float16)v[2], h3 = (_Float16)v[3];
      const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * db) = make_uint2(lo, hi);
    }
  }
}

}  // namespace

const char* launch_sage_attend(const char* ws, const SageLayout& L, uint16_t* out,
                               SageStrides so, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                               float scale, bool k_uniform, hipStream_t s) {
  (void)B;
  const float c_log2 = (float)((double)scale * 1.4426950408889634);
  const int64_t tiles = L.BH * (L.Lqp / kSageQTile);
  const auto kern = k_uniform ? sage_attn_kernel<true> : sage_attn_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kWaves * 64), 0, s,
                     reinterpret_cast<const int8_t*>(ws + L.qc), reinterpret_cast<const float*>(ws + L.sq),
                     reinterpret_cast<const int8_t*>(ws + L.kc), reinterpret_cast<const float*>(ws + L.sk),
                     reinterpret_cast<const uint16_t*>(ws + L.vt), out, so, (int)H, (int)Lq, (int)Lk,
                     (int)L.Lqp, (int)L.Lkp, c_log2, reinterpret_cast<const int32_t*>(ws + L.meta));
  return k_uniform ? "sage_attn_kuni" : "sage_attn";
}

}  // namespace kq
