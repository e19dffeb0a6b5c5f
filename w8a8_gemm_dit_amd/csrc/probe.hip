// Measurement probes of libkq: the machine's own floors beside its
// published peaks, for the roofline figures of the benchmark
// (mlx-kquant pull request 89 commit list: a DiT-shape harness with a
// three-floor roofline, compute, bytes and the measured machine).
//
//   - probe_read: a streaming read of a buffer, split into equal contiguous
//     ranges over a given grid (the GEMV's grid reads the same bytes the
//     same way), 16-byte non-temporal loads, four in flight per thread.
//     It writes nothing (the sink store is conditional on a value the XOR
//     of the data practically never takes), so the bytes moved are the
//     buffer's.
//   - probe_mfma_i8: v_mfma_i32_16x16x64_i8 back to back on register
//     operands, eight independent accumulators per wavefront, eight
//     wavefronts per workgroup (two per SIMD): the INT8 matrix rate the
//     chip sustains at its running clock, with no memory traffic.
#include "kq_common.hpp"
#include "kq_launch.hpp"

namespace kq {

namespace {

__global__ __launch_bounds__(1024) void probe_read_kernel(const v4i* __restrict__ src, int64_t n16,
                                                          int64_t per_wg, uint32_t* sink) {
  const int64_t b = (int64_t)blockIdx.x * per_wg;
  const int64_t e = min(n16, b + per_wg);
  const int64_t T = blockDim.x;
  uint32_t acc = 0;
  int64_t i = b + threadIdx.x;
  for (; i + 3 * T < e; i += 4 * T) {
    const v4i v0 = __builtin_nontemporal_load(src + i);
    const v4i v1 = __builtin_nontemporal_load(src + i + T);
    const v4i v2 = __builtin_nontemporal_load(src + i + 2 * T);
    const v4i v3 = __builtin_nontemporal_load(src + i + 3 * T);
    const v4i x = v0 ^ v1 ^ v2 ^ v3;
    acc ^= (uint32_t)(x[0] ^ x[1] ^ x[2] ^ x[3]);
  }
  for (; i < e; i += T) {
    const v4i v = __builtin_nontemporal_load(src + i);
    acc ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(512) void probe_mfma_kernel(int iters, int32_t* sink) {
  const int t = threadIdx.x;
  const v4i a = v4i{t, t * 3, t * 5, t * 7};
  const v4i b = v4i{t ^ 0x55, t ^ 0x33, t ^ 0x0F, t ^ 0x71};
  v4i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4i{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == 0x12345678) sink[blockIdx.x] = s;
}

}  // namespace

const char* launch_probe_read(const void* src, int64_t bytes, int64_t grid, int threads,
                              uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)grid), dim3((unsigned)threads), 0, s,
                     reinterpret_cast<const v4i*>(src), n16, per, sink);
  return "probe_read";
}

const char* launch_probe_mfma(int iters, int64_t grid, int32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)grid), dim3(512), 0, s, iters, sink);
  return "probe_mfma_i8";
}

}  // namespace kq
