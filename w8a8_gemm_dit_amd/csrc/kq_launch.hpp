// Host-side launchers of the libkq kernels (internal interface between the
// C ABI in kq_api.cpp and the kernel translation units).  Each launcher
// enqueues on `s` without synchronizing and returns the kernel's name (for
// the KQ_LOG route log); launch errors are read by the caller with
// hipGetLastError.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq.h"

namespace kq {

// kOutPart (internal): the raw fp32 sums of one K slice of a split int4
// GEMM, before the token scale and the bias.
enum OutKind : int { kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2, kOutPart = 3 };

// Optional gated residual epilogue of the linears: out = residual +
// gate[m / gate_rows] * y, one fma per element before the output rounding.
// A null residual reads as 0 and a null gate as 1; plain launches pass {}.
struct Epilogue {
  const uint16_t* residual = nullptr;  // bf16 [M,N], may be the output itself
  const float* gate = nullptr;         // fp32 [ceil(M/gate_rows), N]
  int gate_rows = 1;                   // token rows per gate row (>= 1)
  __host__ __device__ bool active() const { return residual != nullptr || gate != nullptr; }
};

// frag: where the codes go: 0 row-major [M][K]; 1 / 2 the MFMA GEMV's
// fragment order for int8 / int4 weights (kq::gemv_frag_offset, rows
// rounded up to 16; the padding rows are not written); 3 row-major with
// each run of 8 codes as its even codes, then its odd ones (the int4
// GEMM's unpack order, launch_gemm_w4a8's eo).
const char* launch_quant_act(const uint16_t* x, int64_t M, int K, int8_t* a, float* sx,
                             int32_t* gsum, hipStream_t s, int frag = 0);
const char* launch_quant_w8(const float* w, int64_t N, int K, int8_t* q, float* sw,
                            hipStream_t s);
const char* launch_quant_w4(const float* w, int64_t N, int K, uint8_t* q4, void* gs, void* gb,
                            hipStream_t s);

// W8A8 GEMM on quantized activations: y = sx*sw*(a . q^T) + bias.
// splits > 1: K in that many slices (kq::split_chunk), int32 partial sums
// into `partials` [splits][M][N], then a fold kernel writes y.
const char* launch_gemm_w8a8(int tile, const int8_t* a, const float* sx, const int8_t* q,
                             const float* sw, const float* bias, void* y, int out, int M,
                             int N, int K, hipStream_t s, const Epilogue& ep = Epilogue(),
                             int splits = 1, int32_t* partials = nullptr);

// W4A8 GEMM: y = sx * sum_g (gs*P + gb*A) + bias (or P per group for I32).
// splits > 1: K in that many slices of whole 16-group chunks; fp32 slice
// sums into `partials` [splits][M][N], then a fold kernel applies the token
// scale and the bias (I32 output: each slice writes its own groups).
// eo: the codes a are in launch_quant_act's frag-3 order, else natural.
const char* launch_gemm_w4a8(int tile, const int8_t* a, const float* sx, const int32_t* gsum,
                             const uint8_t* q4, const void* gs, const void* gb,
                             const float* bias, void* y, int out, int M, int N, int K,
                             hipStream_t s, const Epilogue& ep = Epilogue(),
                             int splits = 1, float* partials = nullptr, bool eo = false);

// GEMV for 1 <= M <= 16 (w4: q is packed int4 with gs/gb; w8: q int8, gs = fp32 [N]).
// x != NULL: the kernel quantizes the bf16 rows x itself (a, sx unused;
// M <= kGemvXqRows, K <= kFusedMaxK) and writes the token scales to sx_out.
// lane: M <= kGemvLaneRows and K <= kFusedMaxK take the lane-per-column
// kernels (the route's lane flag).  frag: the codes a are in the MFMA
// GEMV's fragment order (launch_quant_act's frag 1 / 2), else row-major.
const char* launch_gemv(bool w4, const int8_t* a, const float* sx, const int32_t* gsum,
                        const void* q, const void* gs, const void* gb, const float* bias,
                        void* y, int out, int M, int N, int K, hipStream_t s,
                        const Epilogue& ep = Epilogue(), const uint16_t* x = nullptr,
                        float* sx_out = nullptr, bool lane = true, bool frag = false);

// Thin-N linear with the activation quantization inside (N <= 64, K <=
// kFusedMaxK): reads bf16 x, writes the token scales to sx (if not NULL)
// and y; same weight arguments as launch_gemv.
const char* launch_thin_fused(bool w4, const uint16_t* x, float* sx, const void* q, const void* gs,
                              const void* gb, const float* bias, void* y, int out, int M, int N,
                              int K, hipStream_t s, const Epilogue& ep = Epilogue());

// The library's device scratch (noalloc.hip): kScratchBytes per GPU, for
// the entry point that allocates nothing.  scratch_address returns its
// device address on the current device (fetched once per device), or NULL
// with *err set.
constexpr size_t kScratchBytes = (size_t)KQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
void* scratch_address(hipError_t* err);

// Measurement probes (probe.hip): a streaming read of `bytes` (a multiple
// of 16) in equal contiguous ranges over `grid` workgroups of `threads`,
// and `iters` x 8 int8 MFMAs per wavefront over `grid` workgroups of 8
// wavefronts.  sink: device, at least grid entries, written only if a
// data-dependent test that practically never holds succeeds.
const char* launch_probe_read(const void* src, int64_t bytes, int64_t grid, int threads,
                              uint32_t* sink, hipStream_t s);
const char* launch_probe_mfma(int iters, int64_t grid, int32_t* sink, hipStream_t s);

}  // namespace kq
