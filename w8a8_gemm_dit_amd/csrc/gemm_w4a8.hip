// W4A8 GEMM of libkq ("qlip-mlx" README, w4a8_linear bullet: int4 weights
// with the INT8 matmul, affine group-64 dequantization):
//   y[m,n] = sx[m] * sum_g (gs[n,g] * P[m,n,g] + gb[n,g] * A[m,g]) + bias[n]
// with P the exact int32 product of one 64-wide group of activation codes
// and unsigned 4-bit weight codes, and A the group sum of the activation
// codes.  This is the affine dequantization w = gs*q + gb (MLX pull request
// 4722, serving test: affine 4-bit g64) multiplied out: the offset
// contributes gb times the group's code sum.
//
// gfx950 design:
//   - a workgroup of 8 (or 4) wavefronts computes a BM x BN tile; each
//     wavefront owns a WTM x WTN block of fp32 accumulators;
//   - K advances one group (64 codes) per step.  Activation rows (64 bytes)
//     and packed weight rows (32 bytes) move global -> LDS with direct
//     buffer loads into a 4-slot ring, one array per slot, as in the W8A8
//     GEMM (same swizzle for the activation rows);
//   - per step and 16x16 block, v_mfma_i32_16x16x64_i8 gives P exactly
//     (activation codes are the A operand, unpacked weights the B operand,
//     so each lane holds 4 rows of one column and needs one scale), then
//     two VALU ops per element apply the group scale: acc += gs * float(P);
//   - the offset term sum_g gb*A runs on the matrix core: every 16 groups a
//     table of the group sums split exactly into fp16 parts (A = 64*hi + lo,
//     |hi| <= 128, 0 <= lo < 64) and of the fp16 offsets feeds one
//     v_mfma_f32_16x16x32_f16 per block that accumulates straight into the
//     fp32 accumulators (every product is exact in fp32);
//   - the scale/offset/group-sum tables are double-buffered in LDS: loads
//     for the next 16 groups go out at the first step of the current 16,
//     LDS writes at the ninth, so no step waits for them;
//   - the K loop is unrolled by 16 steps (4 ring turns) so every table event
//     sits at a fixed place; uniform guards on each step (steps past K skip
//     their compute) also keep the compiler from interleaving the steps'
//     fragments, which would exhaust the registers.
#include <type_traits>

#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Activation-row swizzle of the W8A8 ring: chunk index ^ ((r/2)%4 ^ 3*((r/8)%2)),
// so that the 32 lanes gfx950 serves per clock of a ds_read_b128 fragment
// read (16 rows x 2 chunks, rows r and r+8 512 bytes apart) hit distinct
// bank groups.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) & 3) ^ (((row >> 3) & 1) * 3); }

constexpr int kSG = 16;  // groups per table chunk (one f16 MFMA: 16 groups x {hi, lo})

template <int BM, int BN, int WTM, int WTN>
struct Cfg4 {
  static constexpr int kWM = BM / WTM, kWN = BN / WTN;
  static constexpr int kWaves = kWM * kWN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kTM = WTM / 16, kTN = WTN / 16;
  static constexpr int kABlk = BM / 16;   // 1 KB DMA blocks of activation rows per step
  static constexpr int kWBlk = BN / 32;   // 1 KB DMA blocks of packed weight rows per step
  static constexpr int kLPW = (kABlk + kWBlk) / kWaves;
  static constexpr int kASlots = BM * 4;  // 16-byte granules of one slot's activation part
  static constexpr int kSlots = kASlots + BN * 2;
  // table staging per thread and chunk
  static constexpr int kSBN = BN * kSG / kThreads;  // scale and offset entries
  static constexpr int kSBM = BM * kSG / kThreads;  // group-sum entries
  static_assert(kABlk % kWaves == 0 && kWBlk % kWaves == 0, "DMA blocks split evenly over the waves");
  static_assert(BN * kSG % kThreads == 0 && BM * kSG % kThreads == 0, "table staging");
};

template <int OUT>
__device__ __forceinline__ void store1(void* y, int64_t idx, float v) {
  if (OUT == kOutF32 || OUT == kOutPart) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_rne(v);
}

// GATED: the output goes through the gated residual epilogue (kq::Epilogue).
// Split K: workgroup row blockIdx.y takes groups [y*gchunk, min(G, (y+1)*
// gchunk)) (gchunk a multiple of the 16-group table chunk); with OUT ==
// kOutPart it writes its raw fp32 sums to slice y of y[splits][M][N].
// EO: every run of 8 activation codes holds its even codes, then its odd
// ones, the order in which a packed weight dword's low and high nibbles
// come out (w & 0x0f0f0f0f, (w >> 4) & 0x0f0f0f0f): the weights need no
// reordering.  Otherwise the codes are in natural order and the unpacked
// nibbles are put back into it (two v_perm_b32 a dword).  The dot product
// of a group is the same sum in another order, exact in int32.
// TV: the tables come in with 16-byte loads: thread t stages 8 consecutive
// groups of column t/2 (and of row t/2), groups 8*(t%2)..+7 of the chunk.
// It needs the table rows 16-byte aligned (K/64 a multiple of 8, aligned
// bases), so the slice's group count G is a multiple of 8 as well and an
// 8-group unit lies wholly inside or wholly past the slice.
template <int BM, int BN, int WTM, int WTN, int OUT, bool GATED, bool EO, bool TV>
// (128x128: two workgroups per CU, so at most 256 registers per lane)
__global__ __launch_bounds__((BM / WTM) * (BN / WTN) * 64, (BM == 128 && BN == 128) ? 2 : 1) void gemm_w4a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int32_t* __restrict__ gsum,
    const uint8_t* __restrict__ Q, const uint16_t* __restrict__ GS, const uint16_t* __restrict__ GB,
    const float* __restrict__ bias, void* y, int M, int N, int K, Epilogue ep, int gchunk) {
  using C = Cfg4<BM, BN, WTM, WTN>;
  constexpr bool kScaled = OUT != kOutI32;
  __shared__ int4 lds0[C::kSlots], lds1[C::kSlots], lds2[C::kSlots], lds3[C::kSlots];
  // tables, double-buffered: gs and gb as [column][16 groups] fp16, the group
  // sums as [row][32] fp16 = {64*hi of groups 0..15, lo of groups 0..15}
  // (t_gs rows padded to 18 halves: the per-step reads of 16 consecutive
  // columns then hit 16 distinct banks instead of two columns per bank)
  // (128x128: unpadded, so that two workgroups fit in a CU's 160 KB of LDS)
  constexpr int kGsPad = (BM == 128 && BN == 128) ? 0 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t t_gs[kScaled ? 2 : 1][kScaled ? BN : 1][kSG + kGsPad];
  __shared__ __attribute__((aligned(16))) uint16_t t_gb[kScaled ? 2 : 1][kScaled ? BN : 1][kSG];
  __shared__ __attribute__((aligned(16))) uint16_t t_as[kScaled ? 2 : 1][kScaled ? BM : 1][2 * kSG];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::kWN;
  const int wn = wave % C::kWN;
  const int Gall = K / 64;  // groups per row (the tables' row stride)
  const int g0 = blockIdx.y * gchunk;
  const int G = min(gchunk, Gall - g0);  // groups of this K slice
  const int KT = G;
  const int QB = K / 2;  // packed bytes per weight row
  A += (int64_t)g0 * 64;
  Q += (int64_t)g0 * 32;
  GS += g0;
  GB += g0;
  if (kScaled && gsum != nullptr) gsum += g0;
  if (OUT == kOutPart) y = reinterpret_cast<float*>(y) + (int64_t)blockIdx.y * M * N;

  // (num_records ends at the last row's end, which lies g0*64 or g0*32
  // bytes before base + rows*stride once the base moved to the slice)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(A + (int64_t)m0 * K), 0, min(BM, M - m0) * K - g0 * 64, 0x00020000);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Q + (int64_t)n0 * QB), 0, min(BN, N - n0) * QB - g0 * 32, 0x00020000);

  // DMA plan: block b = wave + kWaves*i.  Activation block b < kABlk holds
  // rows 16b..16b+15 (lane l: row 16b + l/4, physical chunk l%4 holding
  // logical chunk (l%4)^swz4(row)); weight block b' = b - kABlk holds rows
  // 32b'..32b'+31 of 32 bytes (lane l: row 32b' + l/2, physical half l%2
  // holding logical half (l%2) ^ ((row/8)%2)), stored after the activation
  // part.  The half swap makes the 8-byte fragment reads of rows r and r+8
  // land in different banks.
  const int ar = lane >> 2;
  const uint32_t voff_a = (uint32_t)(ar * K + (((lane & 3) ^ swz4(ar)) * 16));
  const uint32_t voff_q = (uint32_t)((lane >> 1) * QB + (((lane & 1) ^ ((lane >> 4) & 1)) * 16));
  auto issue = [&](int4* slot, int kt) {
    const int k = min(kt, KT - 1);  // steps past the end re-load the last slice
#pragma unroll
    for (int i = 0; i < C::kLPW; ++i) {
      const int b = wave + C::kWaves * i;
      // compile-time split (kABlk is a multiple of kWaves): no branch, so
      // the step stays one basic block
      if (i < C::kABlk / C::kWaves) {
        lds_ptr_t dst = (lds_ptr_t)(slot + 64 * b);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, voff_a, 16 * b * K + k * 64, 0, 0);
      } else {
        const int bq = b - C::kABlk;
        lds_ptr_t dst = (lds_ptr_t)(slot + C::kASlots + 64 * bq);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dst, 16, voff_q, 32 * bq * QB + k * 32, 0, 0);
      }
    }
  };

  // ---- table staging (scales, offsets, group sums of 16 groups)
  uint32_t st_s[C::kSBN], st_b[C::kSBN];
  int32_t st_a[C::kSBM];
  // Always issues the same number of loads (clamped addresses): the ring's
  // vmcnt waits count them.  The values past N, M or G are zeroed where
  // they are written, not here: a select at the load lets the compiler sink
  // the load under a branch and wait for it (and for every ring load in
  // flight) on the spot.
  static_assert(!TV || (BN * 2 == C::kThreads && BM * 2 <= C::kThreads), "vector table staging");
  v4i st_sv = v4i{0, 0, 0, 0}, st_bv = v4i{0, 0, 0, 0}, st_av[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
  const int tv_c = tid >> 1, tv_h = tid & 1;      // column (and row) and half of the chunk
  const int tv_r = min(tv_c, BM - 1);             // rows past BM repeat row BM-1's unit
  auto stage_load_v = [&](int chunk) {
    // 8-group units wholly past the slice load the slice's last unit (the
    // writes zero them); columns and rows past N / M load the last one
    const int g = min(chunk * kSG + 8 * tv_h, G - 8);
    const int64_t cn = (int64_t)min(n0 + tv_c, N - 1) * Gall + g;
    st_sv = *reinterpret_cast<const v4i*>(GS + cn);
    st_bv = *reinterpret_cast<const v4i*>(GB + cn);
    const int32_t* ga = gsum + (int64_t)min(m0 + tv_r, M - 1) * Gall + g;
    st_av[0] = *reinterpret_cast<const v4i*>(ga);
    st_av[1] = *reinterpret_cast<const v4i*>(ga + 4);
  };
  auto stage_write_v = [&](int buf, int chunk) {
    const bool inside = chunk * kSG + 8 * tv_h < G;
    const bool okn = inside && n0 + tv_c < N;
    const v4i z = v4i{0, 0, 0, 0};
    // t_gs rows may be padded to 18 halves: 4-byte aligned words
    uint32_t* ds = reinterpret_cast<uint32_t*>(&t_gs[buf][tv_c][8 * tv_h]);
    const v4i vs = okn ? st_sv : z;
#pragma unroll
    for (int i = 0; i < 4; ++i) ds[i] = (uint32_t)vs[i];
    *reinterpret_cast<v4i*>(&t_gb[buf][tv_c][8 * tv_h]) = okn ? st_bv : z;
    const bool okm = inside && m0 + tv_r < M;
    uint32_t hi2[4], lo2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hv[2], lv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int j = 2 * i + k;
        const int v = okm ? st_av[j >> 2][j & 3] : 0;
        const int hi = v >> 6;        // floor(v / 64)
        const int lo = v - hi * 64;   // 0..63
        hv[k] = __half_as_ushort(__float2half_rn((float)(hi * 64)));
        lv[k] = __half_as_ushort(__float2half_rn((float)lo));
      }
      hi2[i] = hv[0] | (hv[1] << 16);
      lo2[i] = lv[0] | (lv[1] << 16);
    }
    *reinterpret_cast<v4i*>(&t_as[buf][tv_r][8 * tv_h]) = v4i{(int)hi2[0], (int)hi2[1], (int)hi2[2], (int)hi2[3]};
    *reinterpret_cast<v4i*>(&t_as[buf][tv_r][kSG + 8 * tv_h]) = v4i{(int)lo2[0], (int)lo2[1], (int)lo2[2], (int)lo2[3]};
  };
  auto stage_load = [&](int chunk) {
    if constexpr (TV) {
      stage_load_v(chunk);
      return;
    }
    const int gbase = chunk * kSG;
#pragma unroll
    for (int u = 0; u < C::kSBN; ++u) {
      const int e = tid + u * C::kThreads;
      const int col = e / kSG, t = e % kSG;
      const int n = n0 + col, g = gbase + t;
      const int64_t idx = (int64_t)min(n, N - 1) * Gall + min(g, G - 1);
      st_s[u] = GS[idx];
      st_b[u] = GB[idx];
    }
#pragma unroll
    for (int u = 0; u < C::kSBM; ++u) {
      const int e = tid + u * C::kThreads;
      const int row = e / kSG, t = e % kSG;
      const int m = m0 + row, g = gbase + t;
      st_a[u] = gsum[(int64_t)min(m, M - 1) * Gall + min(g, G - 1)];
    }
  };
  auto stage_write = [&](int buf, int chunk) {
    if constexpr (TV) {
      stage_write_v(buf, chunk);
      return;
    }
    const int gbase = chunk * kSG;
#pragma unroll
    for (int u = 0; u < C::kSBN; ++u) {
      const int e = tid + u * C::kThreads;
      const int col = e / kSG, t = e % kSG;
      const bool ok = n0 + col < N && gbase + t < G;
      t_gs[buf][col][t] = ok ? (uint16_t)st_s[u] : (uint16_t)0;
      t_gb[buf][col][t] = ok ? (uint16_t)st_b[u] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < C::kSBM; ++u) {
      const int e = tid + u * C::kThreads;
      const int row = e / kSG, t = e % kSG;
      const int v = (m0 + row < M && gbase + t < G) ? st_a[u] : 0;
      const int hi = v >> 6;        // floor(v / 64)
      const int lo = v - hi * 64;   // 0..63
      t_as[buf][row][t] = __half_as_ushort(__float2half_rn((float)(hi * 64)));
      t_as[buf][row][kSG + t] = __half_as_ushort(__float2half_rn((float)lo));
    }
  };

  v4f acc[C::kTN][C::kTM];
#pragma unroll
  for (int i = 0; i < C::kTN; ++i)
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15;  // A row / B column within a 16-block
  const int fc = lane >> 4;  // k chunk (16 codes) / output row quad
  const int a_row0 = wm * WTM + fr;
  const int a_slot0 = a_row0 * 4 + (fc ^ swz4(a_row0));  // row block j: + 64*j (swz4 is 16-periodic)
  const int q_col0 = wn * WTN + fr;
  // column block i: + 512*i (16 rows, which keeps bit 3 of the row)
  const int q_byte0 = C::kASlots * 16 + q_col0 * 32 + ((fc * 8) ^ (((q_col0 >> 3) & 1) << 4));

  struct Frags {
    v4i a[C::kTM];
    uint2 q[C::kTN];
    uint32_t s[C::kTN];
  };
  auto read_frags = [&](Frags& f, const int4* slot, int kt) {
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
      const int4 t = slot[a_slot0 + 64 * j];
      f.a[j] = v4i{t.x, t.y, t.z, t.w};
    }
    const char* sb = reinterpret_cast<const char*>(slot);
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) f.q[i] = *reinterpret_cast<const uint2*>(sb + q_byte0 + 512 * i);
    if (kScaled) {
      const int g = min(kt, KT - 1);
      const int buf = (g / kSG) & 1, t = g % kSG;
#pragma unroll
      for (int i = 0; i < C::kTN; ++i) f.s[i] = t_gs[buf][q_col0 + 16 * i][t];
    }
  };
  auto weights = [&](const Frags& f, int i) {
    uint32_t u0, u1, u2, u3;
    if constexpr (EO) {
      u0 = f.q[i].x & 0x0F0F0F0Fu;
      u1 = (f.q[i].x >> 4) & 0x0F0F0F0Fu;
      u2 = f.q[i].y & 0x0F0F0F0Fu;
      u3 = (f.q[i].y >> 4) & 0x0F0F0F0Fu;
    } else {
      unpack8_u4(f.q[i].x, u0, u1);
      unpack8_u4(f.q[i].y, u2, u3);
    }
    return v4i{(int)u0, (int)u1, (int)u2, (int)u3};
  };
  auto compute = [&](const Frags& f, int kt) {
    // A column block's MFMAs go out together, into separate registers, and
    // the next block's go out before this block's rescale, so each rescale
    // finds its products ready instead of waiting out the latency of an
    // MFMA just issued.
    v4i pp[2][C::kTM];
    {
      const v4i fw = weights(f, 0);
#pragma unroll
      for (int j = 0; j < C::kTM; ++j)
        pp[0][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[j], fw, v4i{0, 0, 0, 0}, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      if (i + 1 < C::kTN) {
        const v4i fw = weights(f, i + 1);
#pragma unroll
        for (int j = 0; j < C::kTM; ++j)
          pp[(i + 1) & 1][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.a[j], fw, v4i{0, 0, 0, 0}, 0, 0, 0);
      }
      const float s = kScaled ? __half2float(__ushort_as_half((unsigned short)f.s[i])) : 0.f;
#pragma unroll
      for (int j = 0; j < C::kTM; ++j) {
        const v4i p = pp[i & 1][j];
        if (kScaled) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(s, (float)p[r], acc[i][j][r]);
        } else {
          // debug output: P of every group, [G, M, N]
          const int n = n0 + q_col0 + 16 * i;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * WTM + 16 * j + 4 * fc + r;
            if (m < M && n < N) reinterpret_cast<int32_t*>(y)[((int64_t)(g0 + kt) * M + m) * N + n] = p[r];
          }
        }
      }
    }
  };
  // Offset term of one table chunk: acc += sum_t (64*hi_t + lo_t) * gb_t.
  auto offset_mfmas = [&](int buf) {
    v8h fa[C::kTM], fb[C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j)
      fa[j] = *reinterpret_cast<const v8h*>(&t_as[buf][wm * WTM + 16 * j + fr][8 * fc]);
#pragma unroll
    for (int i = 0; i < C::kTN; ++i)
      fb[i] = *reinterpret_cast<const v8h*>(&t_gb[buf][q_col0 + 16 * i][8 * (fc & 1)]);
#pragma unroll
    for (int i = 0; i < C::kTN; ++i)
#pragma unroll
      for (int j = 0; j < C::kTM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[j], fb[i], acc[i][j], 0, 0, 0);
  };

  // One step of the ring (see the W8A8 GEMM): wait until step kt+1 landed,
  // barrier, read step kt+1's fragments, refill step kt's slot with kt+4,
  // compute step kt.  EXTRA = VMEM ops issued after step kt+1's loads
  // besides the ring's own (the table loads, at two places per chunk).
  auto step = [&](Frags& cur, Frags& nxt, int4* cur_slot, const int4* nxt_slot, int kt,
                  auto extra_tag, auto s_tag) {
    constexpr int EXTRA = decltype(extra_tag)::value;
    constexpr int S = decltype(s_tag)::value;  // position in the 16-step chunk
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<2 * C::kLPW + EXTRA>();
    barrier_nofence();
    read_frags(nxt, nxt_slot, kt + 1);
    if (kScaled && S == 0) stage_load(kt / kSG + 1);
    issue(cur_slot, kt + 4);
    if (kt < KT) compute(cur, kt);
    if (kScaled && S == 8) {
      const int c = kt / kSG + 1;
      if (c * kSG < G) stage_write(c & 1, c);
    }
    if (kScaled && S == kSG - 1) {
      if (kt < KT) offset_mfmas((kt / kSG) & 1);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  constexpr int kStageOps = !kScaled ? 0 : TV ? 4 : 2 * C::kSBN + C::kSBM;
  using IX = std::integral_constant<int, kStageOps>;

  // prologue: table chunk 0, ring steps 0..3
  if (kScaled) {
    stage_load(0);
    stage_write(0, 0);
  }
  issue(lds0, 0);
  issue(lds1, 1);
  issue(lds2, 2);
  issue(lds3, 3);
  wait_vm_lgkm0<3 * C::kLPW>();
  barrier_nofence();
  Frags f0, f1;
  read_frags(f0, lds0, 0);

  // With the table loads issued at position 0 before that step's ring
  // loads, the waits at positions 1 and 2 allow them to stay in flight.
  for (int kt = 0; kt < KT; kt += kSG) {
#define KQ_STEP4(base, X1, X2)                                                   \
    step(f0, f1, lds0, lds1, kt + base + 0, I0{}, std::integral_constant<int, base + 0>{}); \
    step(f1, f0, lds1, lds2, kt + base + 1, X1{}, std::integral_constant<int, base + 1>{}); \
    step(f0, f1, lds2, lds3, kt + base + 2, X2{}, std::integral_constant<int, base + 2>{}); \
    step(f1, f0, lds3, lds0, kt + base + 3, I0{}, std::integral_constant<int, base + 3>{});
    KQ_STEP4(0, IX, IX)
    if (kt + 4 < KT) { KQ_STEP4(4, I0, I0) }
    if (kt + 8 < KT) { KQ_STEP4(8, I0, I0) }
    if (kt + 12 < KT) { KQ_STEP4(12, I0, I0) }
#undef KQ_STEP4
    if (kt + kSG > KT) {
      // partial last chunk: its offset term was not applied at position 15
      if (kScaled) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<63>();
        barrier_nofence();
        offset_mfmas((kt / kSG) & 1);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<0>();  // drain the dead loads before the workgroup exits

  if (!kScaled) return;
  // Epilogue: lane holds D[m = 4*fc + r][n = fr] of each 16x16 block.
  // bf16 output of a full tile goes through LDS: each wavefront writes its
  // block row-major into a free ring slot (16-byte chunk index XORed with
  // row % 8) and stores whole 16-byte row chunks, instead of scattered
  // 2-byte values.
  constexpr int kStage = WTM * WTN * 2;                  // bytes of one wave's bf16 block
  constexpr int kPerSlot = (C::kSlots * 16) / kStage;    // blocks per ring slot
  constexpr int kRowChunks = WTN / 8;                    // 16-byte chunks per block row
  if (OUT == kOutBF16 && kPerSlot * 4 >= C::kWaves && kRowChunks >= 8 && (N % 8) == 0 &&
      m0 + BM <= M && n0 + BN <= N) {
    __builtin_amdgcn_sched_barrier(0);
    barrier_nofence();  // every wave is done with the ring (its loads drained above)
    const int sidx = wave / kPerSlot;
    char* stage = reinterpret_cast<char*>(sidx == 0 ? lds0 : sidx == 1 ? lds1 : sidx == 2 ? lds2 : lds3) +
                  (wave % kPerSlot) * kStage;
    // The lane's token scales and biases, loaded together up front (loaded
    // at their uses, each waited for before the next one issued).
    float s_m[C::kTM][4], b_n[C::kTN];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_m[j][r] = sx[m0 + wm * WTM + 16 * j + 4 * fc + r];
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) b_n[i] = bias != nullptr ? bias[n0 + q_col0 + 16 * i] : 0.0f;
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int cl = 16 * i + fr;  // column within the block
      const float bv = b_n[i];
#pragma unroll
      for (int j = 0; j < C::kTM; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = 16 * j + 4 * fc + r;  // row within the block
          float v = fmaf(s_m[j][r], acc[i][j][r], bv);
          if (GATED)
            v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m0 + wm * WTM + rl, n0 + q_col0 + 16 * i, N);
          *reinterpret_cast<uint16_t*>(stage + rl * (WTN * 2) + (((cl >> 3) ^ (rl & 7)) * 16) +
                                       (cl & 7) * 2) = (uint16_t)f32_to_bf16_rne(v);
        }
      }
    }
    uint16_t* yb = reinterpret_cast<uint16_t*>(y) + (int64_t)(m0 + wm * WTM) * N + n0 + wn * WTN;
#pragma unroll
    for (int u = 0; u < WTM * kRowChunks / 64; ++u) {
      const int e = lane + 64 * u;
      const int rl = e / kRowChunks, c = e % kRowChunks;
      const v4i v = *reinterpret_cast<const v4i*>(stage + rl * (WTN * 2) + ((c ^ (rl & 7)) * 16));
      __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(yb + (int64_t)rl * N + 8 * c));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::kTN; ++i) {
    const int n = n0 + q_col0 + 16 * i;
    const float bv = (bias != nullptr && n < N) ? bias[n] : 0.0f;
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * WTM + 16 * j + 4 * fc + r;
        if (m < M && n < N) {
          if (OUT == kOutPart) {
            store1<OUT>(y, (int64_t)m * N + n, acc[i][j][r]);
          } else {
            float v = fmaf(sx[m], acc[i][j][r], bv);
            if (GATED) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m, n, N);
            store1<OUT>(y, (int64_t)m * N + n, v);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WTM, int WTN, bool EO, bool TV>
const char* launch_tile4_tv(const int8_t* a, const float* sx, const int32_t* gsum, const uint8_t* q4,
                         const uint16_t* gs, const uint16_t* gb, const float* bias, void* y,
                         int out, int M, int N, int K, hipStream_t s, const Epilogue& ep,
                         const char* name, int splits, int gchunk) {
  using C = Cfg4<BM, BN, WTM, WTN>;
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles, (unsigned)splits), block(C::kThreads);
  if (out == kOutPart) {
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, WTM, WTN, kOutPart, false, EO, TV>), grid, block, 0, s, a, sx, gsum, q4, gs, gb, bias, y, M, N, K, ep, gchunk);
    return name;
  }
  if (ep.active() && out == kOutF32)
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, WTM, WTN, kOutF32, true, EO, TV>), grid, block, 0, s, a, sx, gsum, q4, gs, gb, bias, y, M, N, K, ep, gchunk);
  else if (ep.active() && out == kOutBF16)
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, WTM, WTN, kOutBF16, true, EO, TV>), grid, block, 0, s, a, sx, gsum, q4, gs, gb, bias, y, M, N, K, ep, gchunk);
  else if (out == kOutF32)
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, WTM, WTN, kOutF32, false, EO, TV>), grid, block, 0, s, a, sx, gsum, q4, gs, gb, bias, y, M, N, K, ep, gchunk);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, WTM, WTN, kOutBF16, false, EO, TV>), grid, block, 0, s, a, sx, gsum, q4, gs, gb, bias, y, M, N, K, ep, gchunk);
  else
    hipLaunchKernelGGL((gemm_w4a8_kernel<BM, BN, WTM, WTN, kOutI32, false, EO, false>), grid, block, 0, s, a, sx, gsum, q4, gs, gb, bias, y, M, N, K, ep, gchunk);
  return name;
}

// 16-byte table loads where the split-order (linear) kernels can take them:
// table rows of a multiple of 8 groups on 16-byte aligned bases.
template <int BM, int BN, int WTM, int WTN, bool EO>
const char* launch_tile4(const int8_t* a, const float* sx, const int32_t* gsum, const uint8_t* q4,
                         const uint16_t* gs, const uint16_t* gb, const float* bias, void* y,
                         int out, int M, int N, int K, hipStream_t s, const Epilogue& ep,
                         const char* name, int splits, int gchunk) {
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if constexpr (EO) {
    if ((K / 64) % 8 == 0 && a16(gs) && a16(gb) && a16(gsum) && out != kOutI32)
      return launch_tile4_tv<BM, BN, WTM, WTN, EO, true>(a, sx, gsum, q4, gs, gb, bias, y, out, M, N,
                                                         K, s, ep, name, splits, gchunk);
  }
  return launch_tile4_tv<BM, BN, WTM, WTN, EO, false>(a, sx, gsum, q4, gs, gb, bias, y, out, M, N, K,
                                                      s, ep, name, splits, gchunk);
}

// Fold of a split int4 GEMM: the fp32 slice sums added in slice order,
// then the unsplit epilogue expression (token scale, bias, gated residual),
// rounded once to the output type.
template <int OUT, bool GATED>
__global__ __launch_bounds__(256) void splitk_fold4(const float* __restrict__ P, int S,
                                                    const float* __restrict__ sx,
                                                    const float* __restrict__ bias, void* y,
                                                    int M, int N, Epilogue ep) {
  const int64_t MN = (int64_t)M * N;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= MN) return;
  // Four slices' loads at a time, all issued before they are added, in
  // slice order (a load-add loop waited for each load before issuing the
  // next); indices past the last slice are clamped and not added.
  float acc = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 4) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = P[(int64_t)min(s0 + j, S - 1) * MN + e];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s0 + j < S) acc = (s0 + j == 0) ? v[j] : acc + v[j];
  }
  const int m = (int)(e / N), n = (int)(e % N);
  float v = fmaf(sx[m], acc, bias != nullptr ? bias[n] : 0.0f);
  if (GATED) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m, n, N);
  if (OUT == kOutF32) reinterpret_cast<float*>(y)[e] = v;
  else reinterpret_cast<uint16_t*>(y)[e] = (uint16_t)f32_to_bf16_rne(v);
}

void launch_fold4(const float* P, int S, const float* sx, const float* bias, void* y, int out,
                  int M, int N, hipStream_t s, const Epilogue& ep) {
  const dim3 grid((unsigned)(((int64_t)M * N + 255) / 256)), block(256);
  const bool g = ep.active();
  if (out == kOutF32 && g)
    hipLaunchKernelGGL((splitk_fold4<kOutF32, true>), grid, block, 0, s, P, S, sx, bias, y, M, N, ep);
  else if (out == kOutF32)
    hipLaunchKernelGGL((splitk_fold4<kOutF32, false>), grid, block, 0, s, P, S, sx, bias, y, M, N, ep);
  else if (g)
    hipLaunchKernelGGL((splitk_fold4<kOutBF16, true>), grid, block, 0, s, P, S, sx, bias, y, M, N, ep);
  else
    hipLaunchKernelGGL((splitk_fold4<kOutBF16, false>), grid, block, 0, s, P, S, sx, bias, y, M, N, ep);
}

}  // namespace

const char* launch_gemm_w4a8(int tile, const int8_t* a, const float* sx, const int32_t* gsum,
                             const uint8_t* q4, const void* gs, const void* gb,
                             const float* bias, void* y, int out, int M, int N, int K,
                             hipStream_t s, const Epilogue& ep, int splits, float* partials,
                             bool eo) {
  const uint16_t* hs = reinterpret_cast<const uint16_t*>(gs);
  const uint16_t* hb = reinterpret_cast<const uint16_t*>(gb);
  int sp = 1, gchunk = K / 64;
  if (splits > 1) {
    int64_t chunk = K;
    sp = split_chunk(K, splits, chunk, kSplitUnitW4);
    gchunk = (int)(chunk / 64);
  }
  // the slices' output: the caller's y for one slice or for the int32
  // per-group products (each slice writes its own groups), else partials
  const bool fold = sp > 1 && out != kOutI32;
  void* dst = fold ? static_cast<void*>(partials) : y;
  const int dout = fold ? kOutPart : out;
  const Epilogue dep = fold ? Epilogue() : ep;
  auto run = [&](auto eo_tag) {
    constexpr bool E = decltype(eo_tag)::value;
    return tile == kTile128x256
               ? launch_tile4<128, 256, 64, 64, E>(a, sx, gsum, q4, hs, hb, bias, dst, dout, M, N,
                                                   K, s, dep, "gemm_w4a8_128x256", sp, gchunk)
           : tile == kTile128x128
               ? launch_tile4<128, 128, 64, 64, E>(a, sx, gsum, q4, hs, hb, bias, dst, dout, M, N,
                                                   K, s, dep, "gemm_w4a8_128x128", sp, gchunk)
               : launch_tile4<64, 128, 32, 64, E>(a, sx, gsum, q4, hs, hb, bias, dst, dout, M, N,
                                                  K, s, dep, "gemm_w4a8_64x128", sp, gchunk);
  };
  const char* name = eo ? run(std::true_type{}) : run(std::false_type{});
  if (fold) launch_fold4(partials, sp, sx, bias, y, out, M, N, s, ep);
  return name;
}

}  // namespace kq
