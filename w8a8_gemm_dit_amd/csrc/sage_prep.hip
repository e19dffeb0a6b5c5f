// Preparation kernels of the INT8 attention: the key means, the smoothed
// and quantized keys, the quantized queries and the transposed values
// ("qlip-mlx" README, sage_attention bullet and "Key features": INT8 QK^T
// with per-token / per-block scales, softmax and P.V in floating point; the
// smoothing of K is the SageAttention method's).  All bandwidth-bound:
// coalesced 16-byte loads, one pass per tensor (two for K).
#include "kq_common.hpp"
#include "sage.hpp"

namespace kq {
namespace {

// Per (b*h, chunk of 256 tokens): the column sums of the keys as int64
// counts of 2^-24 (every fp16 value is a whole number of them, so the sums
// are exact).
// Thread t reads channels 8*(t%16)..+7 of rows t/16, t/16 + 16, ... with
// 16-byte loads; the 16 row lanes of a channel group then add up in LDS.
__global__ __launch_bounds__(256) void sage_k_colsum(const uint16_t* __restrict__ k,
                                                     SageStrides st, int H, int Lk,
                                                     int nchunk, int64_t* __restrict__ colsum) {
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int cg = tid & 15, rl = tid >> 4;
  const uint16_t* kb = k + (int64_t)(bh / H) * st.b + (int64_t)(bh % H) * st.h + 8 * cg;
  const int t0 = blockIdx.x * kSageChunk;
  const int t1 = min(Lk, t0 + kSageChunk);
  // The lane's 16 rows are summed in fp64, exactly: every fp16 value is a
  // multiple of 2^-24 below 2^16, so the partial sums need at most 45 of
  // fp64's 53 significant bits.  One conversion to units per channel
  // follows (3 VALU operations per value instead of the ~12 of an integer
  // conversion each).
  // Rows go in batches of 8 loads (clamped to the last token, masked
  // after), all issued before any is added: a load-add loop waited for each
  // load before issuing the next.
  double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  constexpr int kBatch = 8;
#pragma unroll
  for (int b = 0; b < kSageChunk / 16; b += kBatch) {
    uint4 u[kBatch];
#pragma unroll
    for (int it = 0; it < kBatch; ++it)
      u[it] = *reinterpret_cast<const uint4*>(kb + (int64_t)min(t0 + rl + 16 * (b + it), Lk - 1) * st.l);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int it = 0; it < kBatch; ++it) {
      if (t0 + rl + 16 * (b + it) >= t1) continue;
      const uint32_t w[4] = {u[it].x, u[it].y, u[it].z, u[it].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[2 * j] += (double)__half2float(__ushort_as_half((uint16_t)(w[j] & 0xFFFFu)));
        s[2 * j + 1] += (double)__half2float(__ushort_as_half((uint16_t)(w[j] >> 16)));
      }
    }
  }
  __shared__ int64_t red[16][kSageD];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[rl][8 * cg + i] = (int64_t)(s[i] * 16777216.0);  // exact
  __syncthreads();
  if (tid < kSageD) {
    int64_t tot = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) tot += red[r][tid];
    colsum[((int64_t)bh * nchunk + blockIdx.x) * kSageD + tid] = tot;
  }
}

// Per b*h: the key means from the column sums (int64 total -> fp64 ->
// x 2^-24 -> / L in fp64 -> fp32, each step rounded to nearest even).
// Workgroup 0 also records the block sizes in the workspace's meta region.
__global__ __launch_bounds__(kSageD) void sage_k_mean(const int64_t* __restrict__ colsum,
                                                      int nchunk, int Lk,
                                                      float* __restrict__ kmean, int k_block,
                                                      int q_block, int32_t* __restrict__ meta) {
  const int bh = blockIdx.x, d = threadIdx.x;
  if (bh == 0 && d < 4) meta[d] = d == 0 ? k_block : d == 1 ? q_block : 0;
  const int64_t* cs = colsum + (int64_t)bh * nchunk * kSageD + d;
  int64_t tot = 0;
  for (int c = 0; c < nchunk; ++c) tot += cs[(int64_t)c * kSageD];
  kmean[(int64_t)bh * kSageD + d] = (float)(((double)tot / 16777216.0) / (double)Lk);
}

// Quantizes 128 tokens of one (b, h): one absmax scale per `block` tokens
// (a power of two <= 128, so blocks never straddle workgroups).  SMOOTH:
// the keys, less their mean (kmean).  Thread t holds token t/2, channels
// 64*(t%2)..+63.
template <bool SMOOTH>
__global__ __launch_bounds__(256) void sage_quant(const uint16_t* __restrict__ x, SageStrides st,
                                                  int H, int L, int Lp, int block,
                                                  const float* __restrict__ kmean,
                                                  int8_t* __restrict__ codes,
                                                  float* __restrict__ scales) {
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tk = blockIdx.x * kSageRowTile + (tid >> 1);
  const int c0 = (tid & 1) * 64;
  __shared__ float s_mean[kSageD];
  __shared__ float s_wmax[4];
  if (SMOOTH) {
    if (tid < kSageD) s_mean[tid] = kmean[(int64_t)bh * kSageD + tid];
    __syncthreads();
  }
  float v[64];
  if (tk < L) {
    const uint4* src = reinterpret_cast<const uint4*>(
        x + (int64_t)(bh / H) * st.b + (int64_t)(bh % H) * st.h + (int64_t)tk * st.l + c0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 u = src[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __half2float(__ushort_as_half((uint16_t)(w[j] & 0xFFFFu)));
        v[8 * i + 2 * j + 1] = __half2float(__ushort_as_half((uint16_t)(w[j] >> 16)));
      }
    }
    if (SMOOTH) {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = __fsub_rn(v[i], s_mean[c0 + i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // the block's 2*block threads are consecutive and aligned
  const int span = 2 * block;
  for (int off = 1; off < span && off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  if (span > 64) {
    if (lane == 0) s_wmax[wave] = amax;
    __syncthreads();
    const int per = span / 64, w0 = wave / per * per;
    amax = s_wmax[w0];
    for (int w = 1; w < per; ++w) amax = fmaxf(amax, s_wmax[w0 + w]);
  }
  float scale;
  const float inv = row_inv(amax, scale);
  uint32_t pk[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    pk[i] = pack4_i8(quant_code(v[4 * i], inv), quant_code(v[4 * i + 1], inv),
                     quant_code(v[4 * i + 2], inv), quant_code(v[4 * i + 3], inv));
  uint4* dst = reinterpret_cast<uint4*>(codes + ((int64_t)bh * Lp + tk) * kSageD + c0);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]);
  if ((tid & 1) == 0) scales[(int64_t)bh * Lp + tk] = tk < L ? scale : 0.0f;
}

// V [64 keys][128] -> vt [128][64 slots] for one 64-key block, keys
// permuted within each 32-key half (slot 8g+i <- key 4g+i, i < 4; key
// 16+4g+(i-4), i >= 4); keys past Lk are zero.
__global__ __launch_bounds__(256) void sage_v_transpose(const uint16_t* __restrict__ v,
                                                        SageStrides st, int H, int Lk, int nblk,
                                                        uint16_t* __restrict__ vt) {
  const int bh = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  __shared__ uint16_t sv[kSageKTile][kSageD + 8];
  const uint16_t* vb = v + (int64_t)(bh / H) * st.b + (int64_t)(bh % H) * st.h;
  // loads at clamped rows, all issued before any is used (guarded loads
  // were each waited for before the next one issued); keys past Lk -> 0
  uint4 u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    const int t = blk * kSageKTile + (e >> 4);
    u[i] = *reinterpret_cast<const uint4*>(vb + (int64_t)min(t, Lk - 1) * st.l + 8 * (e & 15));
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    const int key = e >> 4, c = e & 15;
    const int t = blk * kSageKTile + key;
    *reinterpret_cast<uint4*>(&sv[key][8 * c]) = t < Lk ? u[i] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  uint16_t* out = vt + ((int64_t)bh * nblk + blk) * kSageD * kSageKTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    const int d = e >> 3, c = e & 7;
    const int half = c >> 2, g = c & 3;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s0 = 2 * j, s1 = 2 * j + 1;  // slots within the 8
      const int k0 = 32 * half + (s0 < 4 ? 4 * g + s0 : 16 + 4 * g + s0 - 4);
      const int k1 = 32 * half + (s1 < 4 ? 4 * g + s1 : 16 + 4 * g + s1 - 4);
      w[j] = (uint32_t)sv[k0][d] | ((uint32_t)sv[k1][d] << 16);
    }
    *reinterpret_cast<uint4*>(out + (int64_t)d * kSageKTile + 8 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

const char* launch_sage_prepare(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                SageStrides sq, SageStrides sk, SageStrides sv, int64_t B,
                                int64_t H, int64_t Lq, int64_t Lk, int q_block, int k_block,
                                char* ws, const SageLayout& L, hipStream_t s) {
  (void)B;
  int64_t* colsum = reinterpret_cast<int64_t*>(ws + L.colsum);
  const dim3 blk(256);
  hipLaunchKernelGGL(sage_k_colsum, dim3((unsigned)L.nchunk, (unsigned)L.BH), blk, 0, s, k, sk,
                     (int)H, (int)Lk, (int)L.nchunk, colsum);
  float* kmean = reinterpret_cast<float*>(ws + L.kmean);
  hipLaunchKernelGGL(sage_k_mean, dim3((unsigned)L.BH), dim3(kSageD), 0, s, colsum, (int)L.nchunk,
                     (int)Lk, kmean, k_block, q_block, reinterpret_cast<int32_t*>(ws + L.meta));
  hipLaunchKernelGGL(sage_quant<true>, dim3((unsigned)(L.Lkp / kSageRowTile), (unsigned)L.BH), blk,
                     0, s, k, sk, (int)H, (int)Lk, (int)L.Lkp, k_block, kmean,
                     reinterpret_cast<int8_t*>(ws + L.kc), reinterpret_cast<float*>(ws + L.sk));
  hipLaunchKernelGGL(sage_quant<false>, dim3((unsigned)(L.Lqp / kSageRowTile), (unsigned)L.BH), blk,
                     0, s, q, sq, (int)H, (int)Lq, (int)L.Lqp, q_block, nullptr,
                     reinterpret_cast<int8_t*>(ws + L.qc), reinterpret_cast<float*>(ws + L.sq));
  const int nblk = (int)(L.Lkp / kSageKTile);
  hipLaunchKernelGGL(sage_v_transpose, dim3((unsigned)nblk, (unsigned)L.BH), blk, 0, s, v, sv,
                     (int)H, (int)Lk, nblk, reinterpret_cast<uint16_t*>(ws + L.vt));
  return "sage_v_transpose";
}

}  // namespace kq
