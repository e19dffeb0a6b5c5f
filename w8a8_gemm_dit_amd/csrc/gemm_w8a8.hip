// W8A8 GEMM of libkq: y[m,n] = sx[m]*sw[n]*sum_k a[m,k]*q[n,k] + bias[n].
//
// "qlip-mlx" README, w8a8_linear bullet: INT8xINT8->INT32 matmul with
// dequant+bias fused into one node.  Both operands are K-contiguous ([M,K]
// codes and [N,K] weights, MLX pull request 4722 "Selector rules": 2-D
// transposed weights).
//
// gfx950 design:
//   - a workgroup of 4 (2x2) or 8 (4x2) wavefronts computes a BM x BN output
//     tile; each wavefront owns its block of int32 accumulators built from
//     v_mfma_i32_16x16x64_i8 (16x16 outputs, K = 64 per instruction).  With
//     8 wavefronts (the 256x192 tile) each SIMD runs two, so the MFMA pipe
//     keeps issuing while one of them waits on a full load queue;
//   - K advances 64 bytes per step.  Operand tiles move global -> LDS with
//     buffer_load_dwordx4 ... lds (no staging registers): 64 lanes write
//     1 KB of LDS per instruction, each lane fetching the global 16-byte
//     chunk that belongs at its LDS slot.  One instruction covers 8 rows x
//     128 bytes, i.e. two K steps of 8 whole cache lines: a CU's load path
//     moves about 1.7x more bytes per clock that way than with 16 rows of
//     64 bytes (half lines).  In LDS the rows are 64 bytes with the 16-byte
//     chunk index XOR-swizzled per row, so every 16-lane phase of the
//     fragment ds_read_b128 hits 16 distinct banks;
//   - two pair buffers (4 K steps) form the ring, and fragments are
//     software-pipelined: step k reads step k+1's fragments while its MFMAs
//     run on step k's; each odd step refills the pair it has finished with
//     the pair two ahead.  Each step costs one s_waitcnt of known depth and
//     one barrier without a memory fence.  Each pair buffer is its own LDS
//     array (the compiler tracks the asynchronous LDS writes per array, so
//     reads of one buffer never wait for loads landing in the other), the K
//     loop is unrolled by 4, and scheduling barriers between steps keep the
//     accumulators in place;
//   - no data-dependent branches: buffer descriptors are rebased per
//     workgroup so rows past M or N read as zero, and loads past the last
//     K step re-load the final pair into a buffer that is never read;
//   - the weights are the MFMA A operand and the activations the B operand,
//     so each lane ends with 4 consecutive output columns of one row;
//   - workgroup ids are remapped so each XCD (ids congruent mod 8) works on
//     a compact 2-D block of tiles (groups of 4 tile rows walked column by
//     column) whose operand panels its L2 shares;
//   - epilogue: fp32 acc * (sx[m]*sw[n]) + bias[n] with one fma, rounded
//     once to fp32 or bf16 (round-to-nearest-even).
#include <climits>
#include <cstdlib>
#include <type_traits>

#include "kq_common.hpp"
#include "kq_launch.hpp"
#include "kq_route.hpp"

namespace kq {

namespace {

template <int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int kWaves = WM * WN;     // wavefront grid WM (rows) x WN (columns)
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWTM = BM / WM;       // wave tile rows (m)
  static constexpr int kWTN = BN / WN;       // wave tile columns (n)
  static constexpr int kTM = kWTM / 16;
  static constexpr int kTN = kWTN / 16;
  static constexpr int kRows = BM + BN;      // LDS rows (A rows, then W rows)
  static constexpr int kBlocks = kRows / 8;  // 1 KB DMA blocks per pair of K steps
  static constexpr int kPairSlots = kBlocks * 64;  // 16-byte slots of one pair buffer
  // The first kDmaWaves waves move kLPW consecutive blocks each (the
  // smallest divisor of kBlocks that covers them all), the rest none (their
  // vmcnt waits are then no-ops; the barrier covers them).
  static constexpr int lpw() {
    int d = (kBlocks + kWaves - 1) / kWaves;
    while (kBlocks % d != 0) ++d;
    return d;
  }
  static constexpr int kLPW = lpw();
  static constexpr int kDmaWaves = kBlocks / kLPW;
  static_assert(kBlocks % kLPW == 0 && kLPW < 64, "DMA blocks split into whole per-wave runs");
  static_assert(BM % 64 == 0 && BN % 32 == 0 && kTM >= 1 && kTN >= 1, "tile shape");
};

// LDS row swizzle: the 16-byte chunk index of row r is XORed with
// ((r/2)%4) ^ 3*((r/8)%2).  gfx950 serves 32 lanes of a ds_read_b128 per
// clock from a 512-byte bank period; a fragment read (16 consecutive rows,
// chunk c for lanes 0-15 and c^1 for lanes 16-31) then needs rows r and
// r+8, which sit a multiple of 512 bytes apart, to differ in bit 1 of the XOR (with
// ^1 instead of ^3 they collide pairwise: 2-way conflicts, measured).
// Every 8, 16 and 32 consecutive lanes hit distinct 16-byte bank groups.
// The value depends on r % 16 only.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) ^ (((row >> 3) & 1) * 3); }

// A pair buffer holds two consecutive K steps (64 bytes of every row each)
// as 1 KB blocks of 8 rows: [step 2p: 8 rows x 64 B][step 2p+1: 8 rows x
// 64 B].  One DMA instruction fills one block, so each of its 8 rows is
// read as one whole 128-byte line (16 rows of 64 bytes would touch twice as
// many lines per instruction for the same bytes, which cuts the load
// throughput of a CU by about 40%).  16-byte slot of (row, logical chunk) in half h:
__device__ __forceinline__ int pair_slot(int row, int chunk, int h) {
  return (row >> 3) * 64 + h * 32 + (row & 7) * 4 + (chunk ^ swz(row));
}

// Instruction interleave of one K step.  Steps that refill a pair buffer:
// NV groups of [MFMA x a, DS read x b, MFMA x a, VMEM x 1], then the
// leftovers; the other steps: ND groups of [MFMA x a, DS read x 1].  The
// MFMA pipe stays busy while the fragment reads and the LDS DMA loads issue
// (sched_group_barrier mask bits: 0x008 MFMA, 0x100 DS read, 0x020 VMEM).
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave_step() {
  if constexpr (ND == 0 && NV == 0) {
    // MFMAs only: nothing to interleave
  } else if constexpr (NV == 0) {
    constexpr int a = NM / ND;
#pragma unroll
    for (int g = 0; g < ND; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, a, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - a * ND, 0);
  } else {
    constexpr int a = NM / (2 * NV) > 0 ? NM / (2 * NV) : 1;
    constexpr int b = ND / NV;
#pragma unroll
    for (int g = 0; g < NV; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, a, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, b, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, a, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, ND - b * NV, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM - 2 * a * NV > 0 ? NM - 2 * a * NV : 0, 0);
  }
}

template <int OUT>
__device__ __forceinline__ void store4(void* y, int64_t idx, const float v[4], const int32_t iv[4],
                                       int valid, bool vec_ok) {
  if (OUT == kOutI32) {
    int32_t* p = reinterpret_cast<int32_t*>(y) + idx;
    if (vec_ok && valid == 4) *reinterpret_cast<int4*>(p) = make_int4(iv[0], iv[1], iv[2], iv[3]);
    else for (int i = 0; i < valid; ++i) p[i] = iv[i];
  } else if (OUT == kOutF32) {
    float* p = reinterpret_cast<float*>(y) + idx;
    if (vec_ok && valid == 4) *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else for (int i = 0; i < valid; ++i) p[i] = v[i];
  } else {
    uint16_t* p = reinterpret_cast<uint16_t*>(y) + idx;
    if (vec_ok && valid == 4)
      *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    else for (int i = 0; i < valid; ++i) p[i] = (uint16_t)f32_to_bf16_rne(v[i]);
  }
}

// The K loop is unrolled by 4 steps (two pair buffers); where K/64 is a
// multiple of 4 the last group issues no refills (its pairs are all
// loaded), so nothing is in flight when the epilogue starts.  REM: K/64 is
// not a multiple of 4, so guarded tail steps follow the loop; the
// conditional tail makes the register allocator copy accumulators at the
// loop back-edge, so it is compiled only into the variant that needs it.
// GATED: the output goes through the gated residual epilogue (kq::Epilogue).
// Split K: workgroup row blockIdx.y takes codes [y*kchunk, min(K, (y+1)*
// kchunk)) of every row (K stays the row stride) and, with OUT == I32,
// writes its int32 sums to slice y of y[splits][M][N]; kchunk = K and one
// grid row otherwise.
// NB: pair buffers in the ring (2, or 4 where a small tile runs one
// workgroup per CU on a grid that does not fill the chip twice: the
// kernel is then bound by the bytes it keeps in flight, and 4 buffers hold
// three pairs in flight instead of one).  NB = 4 needs K/64 a multiple of
// 8 in every slice and no REM.
template <int BM, int BN, int WM, int WN, int OUT, bool REM, bool GATED, int NB = 2>
__global__ __launch_bounds__(64 * WM * WN) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const float* __restrict__ bias, void* y, int M,
    int N, int K, Epilogue ep, int kchunk) {
  using C = Cfg<BM, BN, WM, WN>;
  static_assert(NB == 2 || (NB == 4 && !REM), "ring depth");
  // NB pair buffers (pair p, steps 2p and 2p+1, in buffer p % NB): each its
  // own array, so the compiler's tracking of the asynchronous LDS writes
  // never couples reads of one buffer to loads landing in another.
  __shared__ int4 lds0[C::kPairSlots], lds1[C::kPairSlots];
  __shared__ int4 lds2[NB > 2 ? C::kPairSlots : 1], lds3[NB > 2 ? C::kPairSlots : 1];
  // bf16 output: the staged epilogue's operands (token scales of the BM
  // rows, then channel scales and biases of the BN columns), moved into
  // LDS by DMA ahead of the first pair, so the epilogue waits for no load.
  constexpr bool kEops = OUT == kOutBF16;
  constexpr int kEU = (BM + 2 * BN) / 64;           // 64-float DMA units
  constexpr int kEH = (kEU + C::kWaves - 1) / C::kWaves;  // units per wave
  static_assert(!kEops || (BM + 2 * BN) % 64 == 0, "whole epilogue operand units");
  __shared__ __attribute__((aligned(16))) float eops[kEops ? BM + 2 * BN : 1];

  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA bases stay scalar
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int k0 = blockIdx.y * kchunk;
  A += k0;
  W += k0;
  if (OUT == kOutI32) y = reinterpret_cast<int32_t*>(y) + (int64_t)blockIdx.y * M * N;

  // Buffer descriptors rebased on this tile's first row (and the slice's
  // first code): rows past the matrix edge fall outside num_records and
  // read as zero.  num_records ends at the last row's end, K - k0 bytes
  // into it, so the dead second half of an odd slice's last pair (bytes
  // past the row end) reads zeros there instead of memory past the buffer.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(A + (int64_t)m0 * K), 0, min(BM, M - m0) * K - k0, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(W + (int64_t)n0 * K), 0, min(BN, N - n0) * K - k0, 0x00020000);

  // DMA plan: wave w < kDmaWaves moves blocks b = w*kLPW + i (rows 8b..8b+7
  // of the pair); lane l fills slot 64*b + l: half h = l/32 (the pair's
  // step), row r = 8*b + (l%32)/4, physical chunk l%4 holding logical chunk
  // (l%4) ^ swz(r).  swz(r) depends on (l%32)/4 and the parity of b only,
  // so two per-lane offsets serve every block; the block's first row and
  // the pair's K offset go into the scalar offset, which the buffer
  // addressing needs non-negative.  Blocks b < BM/8 are activation rows,
  // the rest weight rows.
  const int rr = (lane & 31) >> 2;
  const uint32_t vbase = (uint32_t)(rr * K + (lane >> 5) * 64);
  const uint32_t voff0 = vbase + (uint32_t)(((lane & 3) ^ ((rr >> 1) & 3)) * 16);
  const uint32_t voff1 = vbase + (uint32_t)(((lane & 3) ^ ((rr >> 1) & 3) ^ 3) * 16);
  const int KT = min(kchunk, K - k0) / 64;
  // Fill a pair buffer with K steps 2*pi and 2*pi+1.  Pairs past the end
  // re-load the last one into a buffer that is never read again; with an
  // odd step count the last pair's second half holds bytes past the row
  // (the next row's, or zeros past the descriptor), which no step reads.
  auto issue = [&](int4* buf, int pi) {
    // (a branch here would split the step's basic block and keep the
    // scheduler from interleaving the loads with the MFMAs)
    if (C::kDmaWaves < C::kWaves && wave >= C::kDmaWaves) return;
    const int ks = min(pi, (KT - 1) >> 1) * 128;
#pragma unroll
    for (int i = 0; i < C::kLPW; ++i) {
      const int b = wave * C::kLPW + i;
      lds_ptr_t dst = (lds_ptr_t)(buf + 64 * b);
      const uint32_t vo = (b & 1) ? voff1 : voff0;
      if (b < BM / 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, vo, ks + 8 * b * K, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, vo, ks + (8 * b - BM) * K, 0, 0);
    }
  };

  // bf16 output of a full tile leaves through an LDS stage (epilogue below).
  constexpr int kStage = C::kWTM * C::kWTN * 2;          // bytes of one wave's bf16 block
  constexpr int kPerSlot = (C::kPairSlots * 16) / kStage;  // blocks per pair buffer
  constexpr int kRowChunks = C::kWTN / 8;                // 16-byte chunks per block row
  constexpr int kResLoads = C::kWTM * kRowChunks / 64;   // 16-byte residual loads per lane
  const bool staged = OUT == kOutBF16 && kPerSlot * 2 >= C::kWaves && (N % 8) == 0 &&
                      m0 + BM <= M && n0 + BN <= N;
  // Gated, staged: the wave's residual block, read with whole 16-byte row
  // chunks.  Where registers allow, the loads go out before the K loop and
  // land while it runs (the vmcnt waits of the loop's first step then
  // include them); otherwise they go out in the epilogue.
  constexpr bool kResEarly = GATED && kResLoads <= 16;
  const int64_t mrow0 = m0 + wm * C::kWTM;
  v4i res[GATED ? kResLoads : 1];
  auto load_residual = [&]() {
    const uint16_t* rb = ep.residual + mrow0 * N + n0 + wn * C::kWTN;
#pragma unroll
    for (int u = 0; u < kResLoads; ++u) {
      const int e = lane + 64 * u;
      res[u] = *reinterpret_cast<const v4i*>(rb + (int64_t)(e / kRowChunks) * N + 8 * (e % kRowChunks));
    }
  };
  if (kResEarly && staged && ep.residual != nullptr) load_residual();

  v4i acc[C::kTN][C::kTM];
#pragma unroll
  for (int i = 0; i < C::kTN; ++i)
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int fr = lane & 15;  // fragment row within a 16-row tile
  const int fc = lane >> 4;  // fragment 16-byte chunk
  // Fragment slots in the first half of a pair buffer: 16-row tile j sits
  // 128 slots (two blocks) after tile j-1; the second half is 32 slots on.
  const int a_slot0 = pair_slot(wm * C::kWTM + fr, fc, 0);
  const int w_slot0 = pair_slot(BM + wn * C::kWTN + fr, fc, 0);

  struct Frags {
    v4i a[C::kTM], w[C::kTN];
  };
  auto read_frags = [&](Frags& f, const int4* slot) {
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
      const int4 t = slot[a_slot0 + 128 * j];
      f.a[j] = v4i{t.x, t.y, t.z, t.w};
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int4 t = slot[w_slot0 + 128 * i];
      f.w[i] = v4i{t.x, t.y, t.z, t.w};
    }
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < C::kTN; ++i)
#pragma unroll
      for (int j = 0; j < C::kTM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[i], f.a[j], acc[i][j], 0, 0, 0);
  };
  // One step kt: (1) wait until step kt+1 has landed and this wave's reads
  // of step kt's fragments are done, then barrier; (2) issue the reads of
  // step kt+1's fragments and, at odd kt, refill step kt's pair buffer
  // (both of its steps are read by now) with the pair NB ahead, interleaved
  // with (3) the MFMAs on step kt's fragments.  VM: the loads that may
  // still be in flight at the wait (vmcnt retires in issue order): at an
  // even step the next step is in the pair waited for at the odd step
  // before, so the NB - 1 youngest refills may fly; at an odd step the next
  // step's pair was issued NB - 1 refills ago, so NB - 2 may (fewer in the
  // last group, which issues no refills).
  // LAST: a step of the last group (no refill; at the last step no reads).
  auto step = [&](Frags& cur, Frags& nxt, int4* cur_buf, const int4* nxt_slot, int kt,
                  auto odd_tag, auto last_tag, auto final_tag, auto vm_tag) {
    constexpr bool kOdd = decltype(odd_tag)::value;
    constexpr bool kRefill = kOdd && !decltype(last_tag)::value;
    constexpr bool kReads = !decltype(final_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<decltype(vm_tag)::value>();
    barrier_nofence();
    if (kReads) read_frags(nxt, nxt_slot);
    if (kRefill) issue(cur_buf, ((kt - 1) >> 1) + NB);
    mfmas(cur);
    interleave_step<C::kTM * C::kTN, kReads ? C::kTM + C::kTN : 0, kRefill ? C::kLPW : 0>();
  };
  using Even = std::integral_constant<bool, false>;
  using Odd = std::integral_constant<bool, true>;
  // pair buffer b of the ring
  auto bufp = [&](auto b_tag) -> int4* {
    constexpr int b = decltype(b_tag)::value;
    if constexpr (b == 0) return lds0;
    else if constexpr (b == 1) return lds1;
    else if constexpr (b == 2) return lds2;
    else return lds3;
  };
#define KQ_BUF(b) bufp(std::integral_constant<int, (b)>{})
  // loads that may fly at step j of a group of 2*NB (steady state; in the
  // last group an odd step j has (NB - 2 - (j - 1)/2) younger pairs at most)
#define KQ_VM(j, LAST)                                                                   \
  std::integral_constant<int, (j) % 2 == 0 ? (NB - 1) * C::kLPW                          \
                              : (LAST ? (NB - 2 - ((j) - 1) / 2 > 0 ? NB - 2 - ((j) - 1) / 2 : 0) \
                                      : NB - 2) * C::kLPW>{}
  // step j of an unrolled group of 2*NB: pair buffer j/2, next step's slot
  // (the pair's second half, or the next buffer's first), parity
#define KQ_STEPX(j, LAST)                                                                \
  step((j) % 2 ? f1 : f0, (j) % 2 ? f0 : f1, KQ_BUF((j) / 2),                           \
       (j) % 2 == 0 ? KQ_BUF((j) / 2) + 32 : KQ_BUF(((j) / 2 + 1) % NB), kt + (j),       \
       std::conditional_t<(j) % 2 == 1, Odd, Even>{}, std::integral_constant<bool, LAST>{}, \
       std::integral_constant<bool, LAST && (j) == 2 * NB - 1>{}, KQ_VM(j, LAST))
#define KQ_STEP(j) KQ_STEPX(j, false)
#define KQ_LAST(j) KQ_STEPX(j, true)

  Frags f0, f1;
  if (kEops && staged) {
    // every wave moves units wave + h*kWaves (a unit past kEU repeats the
    // last one, writing the same values again); a missing bias reads as
    // zero.  Issued first, so the waits for the first pairs cover them.
#pragma unroll
    for (int h = 0; h < kEH; ++h) {
      const int u = min(wave + h * C::kWaves, kEU - 1);
      const bool is_sx = u < BM / 64, is_sw = !is_sx && u < (BM + BN) / 64;
      const float* base = is_sx ? sx + m0 : is_sw ? sw + n0 : (bias ? bias + n0 : sw);
      const int valid = is_sx ? BM : bias || is_sw ? BN : 0;
      const int first = 64 * (is_sx ? u : is_sw ? u - BM / 64 : u - (BM + BN) / 64);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(base), 0, valid * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)&eops[64 * u], 4, lane * 4,
                                               first * 4, 0, 0);
    }
  }
  issue(lds0, 0);
  issue(lds1, 1);
  if constexpr (NB > 2) {
    issue(lds2, 2);
    issue(lds3, 3);
  }
  wait_vm_lgkm0<(NB - 1) * C::kLPW>();  // pair 0
  barrier_nofence();
  read_frags(f0, lds0);
  int kt = 0;
  if constexpr (!REM && NB == 4) {
    for (; kt + 8 < KT; kt += 8) {
      KQ_STEP(0); KQ_STEP(1); KQ_STEP(2); KQ_STEP(3);
      KQ_STEP(4); KQ_STEP(5); KQ_STEP(6); KQ_STEP(7);
    }
    // the last group: its pairs are in the buffers, so no refills (and no
    // reads for a step past the end)
    KQ_LAST(0); KQ_LAST(1); KQ_LAST(2); KQ_LAST(3);
    KQ_LAST(4); KQ_LAST(5); KQ_LAST(6); KQ_LAST(7);
  } else if constexpr (!REM) {
    for (; kt + 4 < KT; kt += 4) {
      KQ_STEP(0); KQ_STEP(1); KQ_STEP(2); KQ_STEP(3);
    }
    // the last group: its pairs are in the buffers, so no refills (and no
    // reads for a step past the end)
    KQ_LAST(0); KQ_LAST(1); KQ_LAST(2); KQ_LAST(3);
  } else {
    for (; kt + 4 <= KT; kt += 4) {
      KQ_STEP(0); KQ_STEP(1); KQ_STEP(2); KQ_STEP(3);
    }
    // the K steps beyond a multiple of 4
    if (kt < KT) KQ_STEP(0);
    if (kt + 1 < KT) KQ_STEP(1);
    if (kt + 2 < KT) KQ_STEP(2);
  }
#undef KQ_STEP
#undef KQ_LAST
#undef KQ_STEPX
#undef KQ_VM
#undef KQ_BUF
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<0>();  // drain the dead loads of a tail before the workgroup exits

  // Epilogue: lane holds D[n = nb + 4*(lane/16) + r][m = mb + lane%16].
  // bf16 output of a full tile goes through LDS: each wavefront writes its
  // block, row-major, into a free ring slot and then stores whole 16-byte
  // row chunks (non-temporal), instead of 8-byte pieces of 16 rows.
  if (staged) {
    __builtin_amdgcn_sched_barrier(0);
    barrier_nofence();  // every wave is done with the ring (its loads drained above)
    const int sidx = wave / kPerSlot;
    char* stage = reinterpret_cast<char*>(sidx == 0 ? lds0 : lds1) +
                  (wave % kPerSlot) * kStage;
    // token scales, channel scales and biases: in LDS since the first pair
    float s_m[C::kTM];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) s_m[j] = eops[wm * C::kWTM + j * 16 + fr];
    // (channel scales and biases are read per column group below)
    // Gated: the residual block goes into the stage at the places its
    // outputs take (each lane then reads its 4 values where it writes the
    // result); a tile whose rows share one gate row reads that row once per
    // column group.
    const bool one_gate = GATED && ep.gate != nullptr &&
                          m0 / ep.gate_rows == (m0 + BM - 1) / ep.gate_rows;
    if (GATED && ep.residual != nullptr) {
      if (!kResEarly) load_residual();
#pragma unroll
      for (int u = 0; u < kResLoads; ++u) {
        const int e = lane + 64 * u;
        const int r = e / kRowChunks, c = e % kRowChunks;
        *reinterpret_cast<v4i*>(stage + r * (C::kWTN * 2) + ((c ^ (r & 3)) * 16)) = res[u];
      }
      // lanes read what other lanes of the wave wrote: keep the order
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int n = n0 + wn * C::kWTN + i * 16 + fc * 4;
      float g4[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if (one_gate) {
        const float* gr = ep.gate + (int64_t)(m0 / ep.gate_rows) * N + n;
        g4[0] = gr[0]; g4[1] = gr[1]; g4[2] = gr[2]; g4[3] = gr[3];
      }
      const int ce = wn * C::kWTN + i * 16 + fc * 4;
      const float4 swv = *reinterpret_cast<const float4*>(eops + BM + ce);
      const float4 bv = *reinterpret_cast<const float4*>(eops + BM + BN + ce);
      const int c = 2 * i + (fc >> 1);  // 16-byte chunk of the block row
#pragma unroll
      for (int j = 0; j < C::kTM; ++j) {
        const int r = 16 * j + fr;
        const float sm = s_m[j];
        float v[4] = {fmaf(sm * swv.x, (float)acc[i][j][0], bv.x),
                      fmaf(sm * swv.y, (float)acc[i][j][1], bv.y),
                      fmaf(sm * swv.z, (float)acc[i][j][2], bv.z),
                      fmaf(sm * swv.w, (float)acc[i][j][3], bv.w)};
        uint2* slot = reinterpret_cast<uint2*>(stage + r * (C::kWTN * 2) + ((c ^ (r & 3)) * 16) +
                                               (fc & 1) * 8);
        if (GATED) {
          float g[4] = {g4[0], g4[1], g4[2], g4[3]};
          if (ep.gate != nullptr && !one_gate) {
            const float* gr = ep.gate + ((mrow0 + r) / ep.gate_rows) * N + n;
            g[0] = gr[0]; g[1] = gr[1]; g[2] = gr[2]; g[3] = gr[3];
          }
          float rv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (ep.residual != nullptr) {
            const uint2 u = *slot;
            rv[0] = bf16_to_f32(u.x & 0xFFFFu); rv[1] = bf16_to_f32(u.x >> 16);
            rv[2] = bf16_to_f32(u.y & 0xFFFFu); rv[3] = bf16_to_f32(u.y >> 16);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fmaf(g[q], v[q], rv[q]);
        }
        *slot = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    uint16_t* yb = reinterpret_cast<uint16_t*>(y) + (int64_t)(m0 + wm * C::kWTM) * N + n0 +
                   wn * C::kWTN;
#pragma unroll
    for (int u = 0; u < C::kWTM * kRowChunks / 64; ++u) {
      const int e = lane + 64 * u;
      const int r = e / kRowChunks, c = e % kRowChunks;
      const v4i v = *reinterpret_cast<const v4i*>(stage + r * (C::kWTN * 2) + ((c ^ (r & 3)) * 16));
      __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(yb + (int64_t)r * N + 8 * c));
    }
    return;
  }
  const bool vec_ok = (N % 4) == 0;
  float s_m[C::kTM];
#pragma unroll
  for (int j = 0; j < C::kTM; ++j) {
    const int m = min(m0 + wm * C::kWTM + j * 16 + fr, M - 1);
    s_m[j] = (OUT == kOutI32) ? 0.0f : sx[m];
  }
#pragma unroll
  for (int i = 0; i < C::kTN; ++i) {
    const int n = n0 + wn * C::kWTN + i * 16 + fc * 4;
    float swv[4], bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int nn = min(n + r, N - 1);
      swv[r] = (OUT == kOutI32) ? 0.f : sw[nn];
      bv[r] = (OUT == kOutI32 || bias == nullptr) ? 0.f : bias[nn];
    }
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
      const int m = m0 + wm * C::kWTM + j * 16 + fr;
      if (m >= M) continue;
      float v[4];
      int32_t iv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        iv[r] = acc[i][j][r];
        v[r] = fmaf(s_m[j] * swv[r], (float)iv[r], bv[r]);
      }
      if (GATED) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) v[r] = gated1(v[r], ep.residual, ep.gate, ep.gate_rows, m, n + r, N);
      }
      store4<OUT>(y, (int64_t)m * N + n, v, iv, min(4, N - n), vec_ok);
    }
  }
}

// Persistent form, for unsplit products whose K steps are a multiple of 4
// (K % 256 == 0) and that have more tiles than the GPU has CUs: a grid of
// one workgroup per CU (a multiple of 8), each looping over tiles t =
// blockIdx.x, blockIdx.x + gridDim.x, ... in the one-tile kernel's
// XCD-aware order (t keeps running on XCD t % 8).  Per tile, the same K
// loop as the one-tile kernel, except that the last two refills, which the
// one-tile kernel spends on dead re-loads of the final pair, fetch the next
// tile's first two pairs, and the last step reads the next tile's first
// fragments: the next tile's MFMAs start without a load round trip.  The
// epilogue stores straight from the accumulators (the LDS ring already
// holds the next tile's operands); its token scales, channel scales and
// biases were moved into LDS by DMA during the tile's first steps (double
// buffered by tile parity), so no epilogue load waits behind the next
// tile's operand loads.  The arithmetic and the output expression are the
// one-tile kernel's, so the results are identical bit for bit.
//
// Whole tiles only (M % BM == 0, N % BN == 0) and no gated epilogue: the
// epilogue is straight-line code.  Wait accounting at a tile's first steps
// (vmcnt retires in issue order): the epilogue issues exactly kStores
// vector stores after the next tile's pair-1 loads, so "at most kStores
// outstanding" at step 1 means pair 1 has landed, and steps 0 and 2 need
// nothing new; the first tile's prologue waits for both pairs.
template <int BM, int BN, int WM, int WN, int OUT>
__global__ __launch_bounds__(64 * WM * WN) void gemm_w8a8_persist(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const float* __restrict__ bias, void* y, int M, int N, int K) {
  using C = Cfg<BM, BN, WM, WN>;
  __shared__ int4 lds0[C::kPairSlots], lds1[C::kPairSlots];
  // Epilogue operands per tile parity: token scales of the BM rows, then
  // channel scales and biases of the BN columns (64-float DMA units).
  constexpr int kEU = (BM + 2 * BN) / 64;
  static_assert((BM + 2 * BN) % 64 == 0 && BM % 64 == 0 && BN % 64 == 0 && kEU <= 2 * C::kWaves,
                "epilogue operand units: two per wave at most");
  __shared__ __attribute__((aligned(16))) float eops[2][BM + 2 * BN];
  constexpr int kStores = C::kTN * C::kTM;  // vector stores of a full tile's epilogue
  constexpr int kExtra = 2;                 // epilogue-operand DMAs per wave and tile
  static_assert(C::kLPW + kStores + kExtra < 64, "vmcnt range");
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int KT = K / 64;  // a multiple of 4
  const int NP = KT / 2;  // K-step pairs per tile

  const int rr = (lane & 31) >> 2;
  const uint32_t vbase = (uint32_t)(rr * K + (lane >> 5) * 64);
  const uint32_t voff0 = vbase + (uint32_t)(((lane & 3) ^ ((rr >> 1) & 3)) * 16);
  const uint32_t voff1 = vbase + (uint32_t)(((lane & 3) ^ ((rr >> 1) & 3) ^ 3) * 16);

  // This tile (m0, n0) and the next one (m1, n1); has_next false at the last.
  int t = blockIdx.x;
  int m0, n0, m1, n1;
  {
    int tm, tn;
    tile_coords(t, ntiles, tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  }
  bool has_next = t + (int)gridDim.x < ntiles;
  auto next_coords = [&]() {
    int tm, tn;
    tile_coords(has_next ? t + (int)gridDim.x : t, ntiles, tiles_m, tiles_n, tm, tn);
    m1 = tm * BM;
    n1 = tn * BN;
  };
  next_coords();

  // Fill a pair buffer with pair pi of this tile; pi >= NP: pair pi - NP
  // of the next tile (or, at the last tile, a dead re-load of this tile's
  // final pair).  Uniform selects, no branch: the step stays one block.
  auto issue = [&](int4* buf, int pi) {
    if (C::kDmaWaves < C::kWaves && wave >= C::kDmaWaves) return;
    const bool nx = pi >= NP && has_next;
    const int mb = nx ? m1 : m0, nb = nx ? n1 : n0;
    const int ks = (pi < NP ? pi : has_next ? pi - NP : NP - 1) * 128;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(A + (int64_t)mb * K), 0, min(BM, M - mb) * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(W + (int64_t)nb * K), 0, min(BN, N - nb) * K, 0x00020000);
#pragma unroll
    for (int i = 0; i < C::kLPW; ++i) {
      const int b = wave * C::kLPW + i;
      lds_ptr_t dst = (lds_ptr_t)(buf + 64 * b);
      const uint32_t vo = (b & 1) ? voff1 : voff0;
      if (b < BM / 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, vo, ks + 8 * b * K, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, vo, ks + (8 * b - BM) * K, 0, 0);
    }
  };
  // The epilogue operands of the tile at (mb, nb) into eops[buf]: every
  // wave moves units wave and wave + kWaves (a unit past kEU repeats the
  // last one, writing the same values again); rows or columns past the
  // matrix edge, and a missing bias, read as zero.
  auto issue_eops = [&](int buf, int mb, int nb) {
    if (OUT == kOutI32) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = min(wave + h * C::kWaves, kEU - 1);
      const bool is_sx = u < BM / 64, is_sw = !is_sx && u < (BM + BN) / 64;
      const float* base = is_sx ? sx + mb : is_sw ? sw + nb : (bias ? bias + nb : sw);
      const int valid = is_sx ? M - mb : bias || is_sw ? N - nb : 0;
      const int first = 64 * (is_sx ? u : is_sw ? u - BM / 64 : u - (BM + BN) / 64);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(base), 0, valid * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)&eops[buf][64 * u], 4, lane * 4,
                                               first * 4, 0, 0);
    }
  };

  v4i acc[C::kTN][C::kTM];
  const int fr = lane & 15;
  const int fc = lane >> 4;
  const int a_slot0 = pair_slot(wm * C::kWTM + fr, fc, 0);
  const int w_slot0 = pair_slot(BM + wn * C::kWTN + fr, fc, 0);
  struct Frags {
    v4i a[C::kTM], w[C::kTN];
  };
  auto read_frags = [&](Frags& f, const int4* slot) {
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) {
      const int4 v = slot[a_slot0 + 128 * j];
      f.a[j] = v4i{v.x, v.y, v.z, v.w};
    }
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int4 v = slot[w_slot0 + 128 * i];
      f.w[i] = v4i{v.x, v.y, v.z, v.w};
    }
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < C::kTN; ++i)
#pragma unroll
      for (int j = 0; j < C::kTM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.w[i], f.a[j], acc[i][j], 0, 0, 0);
  };
  int par = 0;  // tile parity: eops[par] holds this tile's epilogue operands
  // One step (the one-tile kernel's): VM is the vmcnt this wave waits for
  // before the barrier; EO: also move the next tile's epilogue operands
  // (after the barrier, so every wave is past the previous epilogue).
  auto step = [&](Frags& cur, Frags& nxt, int4* cur_buf, const int4* nxt_slot, int kt,
                  auto odd_tag, auto vm_tag, auto eo_tag) {
    constexpr bool kOdd = decltype(odd_tag)::value;
    constexpr int VM = decltype(vm_tag)::value;
    constexpr bool EO = decltype(eo_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<VM>();
    barrier_nofence();
    read_frags(nxt, nxt_slot);
    if (kOdd) issue(cur_buf, (kt + 3) >> 1);
    if (EO) issue_eops(par ^ 1, m1, n1);
    mfmas(cur);
    interleave_step<C::kTM * C::kTN, C::kTM + C::kTN, kOdd ? C::kLPW : 0>();
  };
  using Even = std::integral_constant<bool, false>;
  using Odd = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  using Yes = std::integral_constant<bool, true>;
  using VmEven = std::integral_constant<int, C::kLPW>;
  using VmOdd = std::integral_constant<int, 0>;
  using VmFirst = std::integral_constant<int, C::kLPW + kStores + kExtra>;  // steps 0 and 2
  using VmSecond = std::integral_constant<int, kStores>;                   // step 1
#define KQ_PSTEP(j, VMT, EOT)                                                            \
  step((j) % 2 ? f1 : f0, (j) % 2 ? f0 : f1, (j) < 2 ? lds0 : lds1,                     \
       (j) == 0 ? lds0 + 32 : (j) == 1 ? lds1 : (j) == 2 ? lds1 + 32 : lds0, kt + (j),    \
       std::conditional_t<(j) % 2 == 1, Odd, Even>{}, VMT{}, EOT{})

  Frags f0, f1;
  issue_eops(0, m0, n0);
  issue(lds0, 0);
  issue(lds1, 1);
  wait_vm_lgkm0<0>();  // both pairs: a tile's relaxed first waits then hold for the first tile
  barrier_nofence();
  read_frags(f0, lds0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < C::kTN; ++i)
#pragma unroll
      for (int j = 0; j < C::kTM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    int kt = 0;
    KQ_PSTEP(0, VmFirst, No); KQ_PSTEP(1, VmSecond, Yes);
    KQ_PSTEP(2, VmFirst, No); KQ_PSTEP(3, VmOdd, No);
    for (kt = 4; kt + 4 <= KT; kt += 4) {
      KQ_PSTEP(0, VmEven, No); KQ_PSTEP(1, VmOdd, No);
      KQ_PSTEP(2, VmEven, No); KQ_PSTEP(3, VmOdd, No);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue: lane holds D[n = nb + 4*(lane/16) + r][m = mb + lane%16];
    // whole tiles only (checked at launch): exactly kStores vector stores,
    // straight-line code.
    const float* ebuf = eops[par];
    float s_m[C::kTM];
#pragma unroll
    for (int j = 0; j < C::kTM; ++j) s_m[j] = ebuf[wm * C::kWTM + j * 16 + fr];
#pragma unroll
    for (int i = 0; i < C::kTN; ++i) {
      const int c = wn * C::kWTN + i * 16 + fc * 4;
      const int n = n0 + c;
      const float4 swv = *reinterpret_cast<const float4*>(ebuf + BM + c);
      const float4 bv = *reinterpret_cast<const float4*>(ebuf + BM + BN + c);
#pragma unroll
      for (int j = 0; j < C::kTM; ++j) {
        const int64_t idx = (int64_t)(m0 + wm * C::kWTM + j * 16 + fr) * N + n;
        const float sm = s_m[j];
        if (OUT == kOutI32) {
          *reinterpret_cast<int4*>(reinterpret_cast<int32_t*>(y) + idx) =
              make_int4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          const float v0 = fmaf(sm * swv.x, (float)acc[i][j][0], bv.x);
          const float v1 = fmaf(sm * swv.y, (float)acc[i][j][1], bv.y);
          const float v2 = fmaf(sm * swv.z, (float)acc[i][j][2], bv.z);
          const float v3 = fmaf(sm * swv.w, (float)acc[i][j][3], bv.w);
          if (OUT == kOutF32)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + idx) = make_float4(v0, v1, v2, v3);
          else
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) =
                make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        }
      }
    }
    if (!has_next) break;
    t += gridDim.x;
    m0 = m1;
    n0 = n1;
    par ^= 1;
    has_next = t + (int)gridDim.x < ntiles;
    next_coords();
  }
#undef KQ_PSTEP
  __builtin_amdgcn_sched_barrier(0);
  wait_vm_lgkm0<0>();  // drain the dead loads before the workgroup exits
}

// CUs of the current device (cached per device), for the persistent grid.
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// KQ_DEEP_RING=0 keeps the 2-buffer ring everywhere (A/B runs).
bool deep_ring_enabled() {
  const char* v = getenv("KQ_DEEP_RING");
  return !(v && v[0] == '0');
}

// KQ_PERSIST=1 takes the persistent form where it applies (off by
// default: measured slower at the 4K shape, the next tile's refills wait
// behind the previous tile's output stores).
bool persist_enabled() {
  const char* v = getenv("KQ_PERSIST");
  return v && v[0] == '1';
}

template <int BM, int BN, int WM, int WN>
bool launch_persist(const int8_t* a, const float* sx, const int8_t* q, const float* sw,
                    const float* bias, void* y, int out, int M, int N, int K, hipStream_t s,
                    const Epilogue& ep) {
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int cus = device_cus() / 8 * 8;
  if (!persist_enabled() || ep.active() || (K / 64) % 4 != 0 || M % BM != 0 || N % BN != 0 ||
      cus < 8 || tiles <= cus || tiles > INT32_MAX)
    return false;
  const dim3 grid((unsigned)cus), block(64 * WM * WN);
  if (out == kOutF32)
    hipLaunchKernelGGL((gemm_w8a8_persist<BM, BN, WM, WN, kOutF32>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemm_w8a8_persist<BM, BN, WM, WN, kOutBF16>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K);
  else
    hipLaunchKernelGGL((gemm_w8a8_persist<BM, BN, WM, WN, kOutI32>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K);
  return true;
}

template <int BM, int BN, int WM, int WN, bool REM, int NB = 2>
void launch_rem(const int8_t* a, const float* sx, const int8_t* q, const float* sw,
                const float* bias, void* y, int out, int M, int N, int K, hipStream_t s,
                const Epilogue& ep, int splits, int kchunk) {
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles, (unsigned)splits), block(64 * WM * WN);
  const bool g = ep.active();
  if (out == kOutF32 && g)
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WM, WN, kOutF32, REM, true, NB>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K, ep, kchunk);
  else if (out == kOutF32)
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WM, WN, kOutF32, REM, false, NB>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K, ep, kchunk);
  else if (out == kOutBF16 && g)
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WM, WN, kOutBF16, REM, true, NB>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K, ep, kchunk);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WM, WN, kOutBF16, REM, false, NB>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K, ep, kchunk);
  else
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WM, WN, kOutI32, REM, false, NB>), grid, block, 0, s, a, sx, q, sw, bias, y, M, N, K, ep, kchunk);
}

template <int BM, int BN, int WM = 2, int WN = 2>
const char* launch_tile(const int8_t* a, const float* sx, const int8_t* q, const float* sw,
                        const float* bias, void* y, int out, int M, int N, int K,
                        hipStream_t s, const Epilogue& ep, const char* name, int splits,
                        int kchunk) {
  const int klast = K - (splits - 1) * kchunk;  // the last slice's codes
  if constexpr (WM * WN == 8 && BN == 192) {  // (the 8-wave 256x256 tile would spill)
    if (splits == 1 && launch_persist<BM, BN, WM, WN>(a, sx, q, sw, bias, y, out, M, N, K, s, ep))
      return name;
  }
  // the 4-buffer ring: tiles of at most 128x128 (4 pairs fit the LDS),
  // K steps a multiple of 8 in every slice, a grid of at most one
  // workgroup per CU (the ring's LDS then costs no occupancy)
  if constexpr (BM + BN <= 256) {
    const int64_t wgs = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN) * splits;
    if ((kchunk / 64) % 8 == 0 && (klast / 64) % 8 == 0 && wgs <= device_cus() &&
        deep_ring_enabled()) {
      launch_rem<BM, BN, WM, WN, false, 4>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, splits,
                                           kchunk);
      return name;
    }
  }
  if ((kchunk / 64) % 4 == 0 && (klast / 64) % 4 == 0)
    launch_rem<BM, BN, WM, WN, false>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, splits, kchunk);
  else
    launch_rem<BM, BN, WM, WN, true>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, splits, kchunk);
  return name;
}

// Fold of a split GEMM: the exact int32 sum of the slices, then the same
// epilogue expression as the unsplit kernel (one rounding), so the output
// matches it bit for bit.  One thread per output element.
template <int OUT, bool GATED>
__global__ __launch_bounds__(256) void splitk_fold(const int32_t* __restrict__ P, int S,
                                                   const float* __restrict__ sx,
                                                   const float* __restrict__ sw,
                                                   const float* __restrict__ bias, void* y,
                                                   int M, int N, Epilogue ep) {
  const int64_t MN = (int64_t)M * N;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= MN) return;
  // Four slices' loads at a time, all issued before they are added (a
  // load-add loop waited for each load before issuing the next); indices
  // past the last slice are clamped and their values not added.
  int32_t acc = 0;
  for (int s0 = 0; s0 < S; s0 += 4) {
    int32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = P[(int64_t)min(s0 + j, S - 1) * MN + e];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s0 + j < S) acc += v[j];
  }
  if (OUT == kOutI32) {
    reinterpret_cast<int32_t*>(y)[e] = acc;
    return;
  }
  const int m = (int)(e / N), n = (int)(e % N);
  float v = fmaf(sx[m] * sw[n], (float)acc, bias != nullptr ? bias[n] : 0.0f);
  if (GATED) v = gated1(v, ep.residual, ep.gate, ep.gate_rows, m, n, N);
  if (OUT == kOutF32) reinterpret_cast<float*>(y)[e] = v;
  else reinterpret_cast<uint16_t*>(y)[e] = (uint16_t)f32_to_bf16_rne(v);
}

void launch_fold(const int32_t* P, int S, const float* sx, const float* sw, const float* bias,
                 void* y, int out, int M, int N, hipStream_t s, const Epilogue& ep) {
  const dim3 grid((unsigned)(((int64_t)M * N + 255) / 256)), block(256);
  const bool g = ep.active();
  if (out == kOutF32 && g)
    hipLaunchKernelGGL((splitk_fold<kOutF32, true>), grid, block, 0, s, P, S, sx, sw, bias, y, M, N, ep);
  else if (out == kOutF32)
    hipLaunchKernelGGL((splitk_fold<kOutF32, false>), grid, block, 0, s, P, S, sx, sw, bias, y, M, N, ep);
  else if (out == kOutBF16 && g)
    hipLaunchKernelGGL((splitk_fold<kOutBF16, true>), grid, block, 0, s, P, S, sx, sw, bias, y, M, N, ep);
  else if (out == kOutBF16)
    hipLaunchKernelGGL((splitk_fold<kOutBF16, false>), grid, block, 0, s, P, S, sx, sw, bias, y, M, N, ep);
  else
    hipLaunchKernelGGL((splitk_fold<kOutI32, false>), grid, block, 0, s, P, S, sx, sw, bias, y, M, N, ep);
}

}  // namespace

// One launch of the tile kernel over `splits` K slices of kchunk codes.
const char* launch_gemm_slices(int tile, const int8_t* a, const float* sx, const int8_t* q,
                               const float* sw, const float* bias, void* y, int out, int M,
                               int N, int K, hipStream_t s, const Epilogue& ep, int splits,
                               int kchunk);

const char* launch_gemm_w8a8(int tile, const int8_t* a, const float* sx, const int8_t* q,
                             const float* sw, const float* bias, void* y, int out, int M,
                             int N, int K, hipStream_t s, const Epilogue& ep, int splits,
                             int32_t* partials) {
  if (splits > 1) {
    int64_t chunk = K;
    const int sp = split_chunk(K, splits, chunk);
    const char* name = launch_gemm_slices(tile, a, sx, q, sw, bias, partials, kOutI32, M, N, K,
                                          s, Epilogue(), sp, (int)chunk);
    launch_fold(partials, sp, sx, sw, bias, y, out, M, N, s, ep);
    return name;
  }
  return launch_gemm_slices(tile, a, sx, q, sw, bias, y, out, M, N, K, s, ep, 1, K);
}

const char* launch_gemm_slices(int tile, const int8_t* a, const float* sx, const int8_t* q,
                               const float* sw, const float* bias, void* y, int out, int M,
                               int N, int K, hipStream_t s, const Epilogue& ep, int splits,
                               int kchunk) {
  switch (tile) {
    case kTile256x256:
      return launch_tile<256, 256>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_256x256", splits, kchunk);
    case kTile256x256w8:
      // its gated bf16 instance spills (128 accumulators plus the
      // residual block in the epilogue): gated calls take 256x192
      if (ep.active())
        return launch_tile<256, 192, 4, 2>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_256x192", splits, kchunk);
      return launch_tile<256, 256, 4, 2>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_256x256w8", splits, kchunk);
    case kTile256x192:
      return launch_tile<256, 192, 4, 2>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_256x192", splits, kchunk);
    case kTile256x128:
      return launch_tile<256, 128>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_256x128", splits, kchunk);
    case kTile128x128:
      return launch_tile<128, 128>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_128x128", splits, kchunk);
    default:
      return launch_tile<64, 64>(a, sx, q, sw, bias, y, out, M, N, K, s, ep, "gemm_w8a8_64x64", splits, kchunk);
  }
}

}  // namespace kq
