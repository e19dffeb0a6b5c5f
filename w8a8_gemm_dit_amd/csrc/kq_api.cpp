// C ABI of libkq: argument checks, routing and kernel launches.
//
// Every entry point validates its arguments on the host before touching the
// device, records a "[op] message" on failure (the MLX "[op] ... not
// supported" invalid_argument convention, MLX pull request 3026's fast.cpp
// checks) and returns a status; no exception crosses the ABI.  A declined
// route is not an error (mlx-kquant pull request 89 commit list: raise on
// errors other than a declined route).  Launches are asynchronous on the
// caller's stream; nothing here allocates device memory or synchronizes.
//
// Environment levers, read on every call:
//   KQ_LOG=1            one stderr line per call: op, route, kernels, grid
//   KQ_FORCE_ROUTE=gemm|gemv   override the M <= 16 GEMV routing
//   KQ_TILE=256x256|256x192|256x128|128x128|64x64   pin the GEMM tile (A/B runs)
//   KQ_SPLIT=n          K slices of a GEMM (1: never split)
//   KQ_FUSE=0           no fused thin-N route (quantize kernel + GEMV instead)
//   KQ_GEMV_LANE=0      GEMVs at M <= 2 on the MFMA GEMV kernel instead of
//                       the lane-per-column ones
//   KQ_DEEP_RING=0      the W8A8 GEMM keeps its 2-buffer pair ring on every
//                       grid (A/B runs of the 4-buffer ring)
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "kq.h"
#include "kq_launch.hpp"
#include "kq_route.hpp"
#include "sage.hpp"

namespace {

thread_local std::string g_last_error;

kq_status fail(kq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

int env_force_route() {
  const char* v = getenv("KQ_FORCE_ROUTE");
  if (!v) return 0;
  if (!strcmp(v, "gemm")) return 1;
  if (!strcmp(v, "gemv")) return 2;
  return 0;
}

int env_tile() { return kq::tile_from_name(getenv("KQ_TILE")); }

// KQ_SPLIT=n: n K slices for int8-weight GEMMs (1: never); unset: automatic.
int env_split() {
  const char* v = getenv("KQ_SPLIT");
  if (!v || !v[0]) return -1;
  const int n = atoi(v);
  return n >= 1 ? n : -1;
}

// KQ_FUSE=0 turns the fused thin-N route off.
bool env_fuse() {
  const char* v = getenv("KQ_FUSE");
  return !(v && !strcmp(v, "0"));
}

// KQ_GEMV_LANE=0 turns the lane-per-column GEMVs off.
bool env_gemv_lane() {
  const char* v = getenv("KQ_GEMV_LANE");
  return !(v && !strcmp(v, "0"));
}

bool env_log() {
  const char* v = getenv("KQ_LOG");
  return v && v[0] && strcmp(v, "0");
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Checks that the current device is gfx950 (cached per device).
kq_status check_device(const char* op) {
  static int cache[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(KQ_ERR_NO_DEVICE, "[%s] no HIP device", op);
  if (dev < 64 && cache[dev] == 1) return KQ_SUCCESS;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(KQ_ERR_NO_DEVICE, "[%s] cannot query device %d", op, dev);
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev] = ok ? 1 : 2;
  if (!ok) return fail(KQ_ERR_NO_DEVICE, "[%s] device %d is %s, not gfx950", op, dev, prop.gcnArchName);
  return KQ_SUCCESS;
}

kq_status check_launch(const char* op) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KQ_ERR_LAUNCH, "[%s] launch failed: %s", op, hipGetErrorString(e));
  return KQ_SUCCESS;
}

int out_kind(kq_dtype d) {
  return d == KQ_DTYPE_F32 ? kq::kOutF32 : d == KQ_DTYPE_BF16 ? kq::kOutBF16 : kq::kOutI32;
}

const char* dtype_name(kq_dtype d) {
  return d == KQ_DTYPE_F32 ? "f32" : d == KQ_DTYPE_BF16 ? "bf16" : "i32";
}

// Launches the GEMM/GEMV stage of a validated linear on quantized
// activations (codes, scales and, for int4 weights, group sums).
// partials: int32 workspace of a split GEMM, or NULL (then K is never split).
// frag: the codes are in the MFMA GEMV's fragment order (the linears'
// quantize kernel writes them so when the route takes that kernel).
// eo: int4 weights on the tiled GEMM, codes in the quantize kernel's
// frag-3 order (each run of 8 as its even codes, then its odd ones).
kq_status launch_main(const char* op, int force, kq_wformat fmt, const int8_t* codes,
                      const float* sx, const int32_t* gsum, int64_t M, int64_t K, int64_t N,
                      const void* wq, const void* scale, const void* gbias, const float* bias,
                      void* y, kq_dtype y_dtype, hipStream_t s, const char* kq_name,
                      const kq::Epilogue& ep = kq::Epilogue(), int32_t* partials = nullptr,
                      bool frag = false, bool eo = false) {
  const kq_route_info r =
      kq::choose_route(M, N, K, fmt, force, env_tile(), partials ? env_split() : 0, false,
                       env_gemv_lane());
  const int out = out_kind(y_dtype);
  const char* k2;
  if (eo && (r.kind == KQ_ROUTE_GEMV || fmt != KQ_W4_AFFINE_G64))
    return fail(KQ_ERR_UNSUPPORTED, "[%s] internal: split-order codes on a route that reads them in natural order", op);
  if (r.kind == KQ_ROUTE_GEMV) {
    k2 = kq::launch_gemv(fmt == KQ_W4_AFFINE_G64, codes, sx, gsum, wq, scale, gbias, bias, y, out,
                         (int)M, (int)N, (int)K, s, ep, nullptr, nullptr, env_gemv_lane(),
                         frag && kq::gemv_frag_codes(r));
  } else {
    int tile = 0;
    for (int t = 0; t < kq::kNumTiles; ++t)
      if (kq::tile_shape(t).bm == r.tile_m && kq::tile_shape(t).bn == r.tile_n &&
          kq::tile_shape(t).threads == r.threads)
        tile = t;
    if (fmt == KQ_W8_PER_CHANNEL)
      k2 = kq::launch_gemm_w8a8(tile, codes, sx, reinterpret_cast<const int8_t*>(wq),
                                reinterpret_cast<const float*>(scale), bias, y, out, (int)M,
                                (int)N, (int)K, s, ep, r.splits, partials);
    else
      k2 = kq::launch_gemm_w4a8(tile, codes, sx, gsum, reinterpret_cast<const uint8_t*>(wq),
                                scale, gbias, bias, y, out, (int)M, (int)N, (int)K, s, ep,
                                r.splits, reinterpret_cast<float*>(partials), eo);
  }
  const kq_status st = check_launch(op);
  if (st != KQ_SUCCESS) return st;
  if (env_log())
    fprintf(stderr, "[kq] %s M=%lld N=%lld K=%lld out=%s%s route=%s kernels=%s%s%s%s tile=%dx%d splits=%d grid=%lld\n",
            op, (long long)M, (long long)N, (long long)K, dtype_name(y_dtype),
            ep.active() ? " gated" : "",
            r.kind == KQ_ROUTE_GEMV ? "gemv" : "gemm", kq_name ? kq_name : "",
            kq_name ? "," : "", k2, r.splits > 1 ? ",splitk_fold" : "", r.tile_m, r.tile_n,
            r.splits, (long long)r.grid);
  return KQ_SUCCESS;
}

// Checks shared by every linear entry point (scalars, pointers, alignment).
kq_status check_linear_args(const char* op, int force, kq_wformat fmt, int64_t M, int64_t K,
                            int64_t N, kq_dtype y_dtype, const void* x, const void* wq,
                            const void* scale, const void* gbias, const void* y) {
  std::string err;
  kq_status st = kq::validate_linear(op, M, K, N, fmt, y_dtype, err);
  if (st != KQ_SUCCESS) return fail(st, "%s", err.c_str());
  if (M == 0 || N == 0) return KQ_SUCCESS;
  if (!x || !wq || !scale || !y) return fail(KQ_ERR_INVALID_VALUE, "[%s] null tensor pointer", op);
  if (fmt == KQ_W4_AFFINE_G64 && !gbias)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] int4 weights need the group offsets", op);
  if (!aligned16(x) || !aligned16(wq) || !aligned16(y))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] x, weights, y and workspace must be 16-byte aligned", op);
  if (force >= 2 && M > KQ_GEMV_MAX_M)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] M=%lld exceeds the GEMV limit %d", op, (long long)M,
                KQ_GEMV_MAX_M);
  if (force >= 2 && K > kq::kGemvMaxK)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] K=%lld exceeds the GEMV limit %lld", op, (long long)K,
                (long long)kq::kGemvMaxK);
  return KQ_SUCCESS;
}

// Shared body of the three linear entry points that quantize x themselves.
kq_status run_linear(const char* op, int force, kq_wformat fmt, const void* x, int64_t M,
                     int64_t K, int64_t N, const void* wq, const void* scale, const void* gbias,
                     const float* bias, void* y, kq_dtype y_dtype, void* ws, size_t ws_bytes,
                     void* stream, const kq::Epilogue& ep = kq::Epilogue()) {
  kq_status st = check_linear_args(op, force, fmt, M, K, N, y_dtype, x, wq, scale, gbias, y);
  if (st != KQ_SUCCESS || M == 0 || N == 0) return st;
  if (!aligned16(ws))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] x, weights, y and workspace must be 16-byte aligned", op);
  const kq_route_info r = kq::choose_route(M, N, K, fmt, force, env_tile(), env_split(), env_fuse(),
                                           env_gemv_lane());
  const int splits = r.splits;
  const bool fused = r.kind == KQ_ROUTE_FUSED;
  const kq::WorkspaceLayout wl = kq::workspace_layout(M, N, K, fmt, splits, fused);
  if (!ws || ws_bytes < wl.total)
    return fail(KQ_ERR_WORKSPACE, "[%s] workspace of %zu bytes is smaller than the %zu required", op,
                ws_bytes, wl.total);
  st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsb = reinterpret_cast<char*>(ws);
  if (fused) {
    const bool w4 = fmt == KQ_W4_AFFINE_G64;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    float* sxo = reinterpret_cast<float*>(wsb + wl.scale_off);
    const char* k =
        M <= kq::kGemvXqRows
            ? kq::launch_gemv(w4, nullptr, nullptr, nullptr, wq, scale, gbias, bias, y,
                              out_kind(y_dtype), (int)M, (int)N, (int)K, s, ep, xb, sxo,
                              env_gemv_lane())
            : kq::launch_thin_fused(w4, xb, sxo, wq, scale, gbias, bias, y, out_kind(y_dtype),
                                    (int)M, (int)N, (int)K, s, ep);
    st = check_launch(op);
    if (st != KQ_SUCCESS) return st;
    if (env_log())
      fprintf(stderr, "[kq] %s M=%lld N=%lld K=%lld out=%s%s route=fused kernels=%s grid=%lld\n", op,
              (long long)M, (long long)N, (long long)K, dtype_name(y_dtype),
              ep.active() ? " gated" : "", k, (long long)r.grid);
    return KQ_SUCCESS;
  }
  int8_t* codes = reinterpret_cast<int8_t*>(wsb + wl.codes_off);
  float* sx = reinterpret_cast<float*>(wsb + wl.scale_off);
  int32_t* gsum = fmt == KQ_W4_AFFINE_G64 ? reinterpret_cast<int32_t*>(wsb + wl.gsum_off) : nullptr;
  // the MFMA GEMV reads the codes in its fragment order (whole 1 KB
  // operands per load), the int4 GEMM row-major with each run of 8 split
  // into its even and odd codes (its weights' unpack order), every other
  // route row-major
  const bool frag = kq::gemv_frag_codes(r);
  const bool eo = !frag && fmt == KQ_W4_AFFINE_G64 && r.kind != KQ_ROUTE_GEMV;
  const char* kq_name = kq::launch_quant_act(reinterpret_cast<const uint16_t*>(x), M, (int)K, codes,
                                             sx, gsum, s,
                                             frag ? (fmt == KQ_W4_AFFINE_G64 ? 2 : 1) : eo ? 3 : 0);
  st = check_launch(op);
  if (st != KQ_SUCCESS) return st;
  int32_t* partials = splits > 1 ? reinterpret_cast<int32_t*>(wsb + wl.part_off) : nullptr;
  return launch_main(op, force, fmt, codes, sx, gsum, M, K, N, wq, scale, gbias, bias, y, y_dtype,
                     s, kq_name, ep, partials, frag, eo);
}

// Shared body of the activation-quantization entry points.
kq_status quantize_act(const char* op, const void* x, int64_t M, int64_t K, int8_t* a, float* sx,
                       int32_t* gsum, kq_code_order order, void* stream) {
  if (order != KQ_CODES_NATURAL && order != KQ_CODES_SPLIT8)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] unknown code order %d", op, (int)order);
  if (M < 0 || K < 0) return fail(KQ_ERR_INVALID_VALUE, "[%s] negative size", op);
  if (K == 0) return fail(KQ_ERR_UNSUPPORTED, "[%s] K must be positive", op);
  if (K > INT32_MAX / 2) return fail(KQ_ERR_UNSUPPORTED, "[%s] K=%lld too large", op, (long long)K);
  if (order == KQ_CODES_SPLIT8 && K % 8)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] split code order needs K %% 8 == 0 (K=%lld)", op, (long long)K);
  if (gsum && K % 64)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] group sums need K %% 64 == 0 (K=%lld)", op, (long long)K);
  if (M == 0) return KQ_SUCCESS;
  if (!x || !a || !sx) return fail(KQ_ERR_INVALID_VALUE, "[%s] null tensor pointer", op);
  if (K % 8 == 0 && (!aligned16(x) || ((uintptr_t)a & 7)))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] x must be 16-byte and a 8-byte aligned", op);
  kq_status st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  const char* name = kq::launch_quant_act(reinterpret_cast<const uint16_t*>(x), M, (int)K, a, sx,
                                          gsum, reinterpret_cast<hipStream_t>(stream),
                                          order == KQ_CODES_SPLIT8 ? 3 : 0);
  st = check_launch(op);
  if (st == KQ_SUCCESS && env_log())
    fprintf(stderr, "[kq] %s M=%lld K=%lld kernel=%s\n", op, (long long)M, (long long)K, name);
  return st;
}

// Shared body of the entry points on pre-quantized activations.
kq_status run_gemm(const char* op, kq_wformat fmt, const int8_t* a, const float* sx,
                   const int32_t* gsum, int64_t M, int64_t K, int64_t N, const void* wq,
                   const void* scale, const void* gbias, const float* bias, void* y,
                   kq_dtype y_dtype, void* stream, kq_code_order order = KQ_CODES_NATURAL) {
  if (order != KQ_CODES_NATURAL && order != KQ_CODES_SPLIT8)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] unknown code order %d", op, (int)order);
  const bool eo = order == KQ_CODES_SPLIT8;
  int force = env_force_route();
  if (eo && force == 2)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] the GEMV reads natural-order codes (KQ_FORCE_ROUTE=gemv)", op);
  if (eo) force = 1;  // the tiled int4 GEMM reads split-order codes
  kq_status st = check_linear_args(op, force, fmt, M, K, N, y_dtype, a, wq, scale, gbias, y);
  if (st != KQ_SUCCESS || M == 0 || N == 0) return st;
  if (!sx || (fmt == KQ_W4_AFFINE_G64 && !gsum))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] null scale or group-sum pointer", op);
  st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  return launch_main(op, force, fmt, a, sx, gsum, M, K, N, wq, scale, gbias, bias, y, y_dtype,
                     reinterpret_cast<hipStream_t>(stream), nullptr, kq::Epilogue(), nullptr,
                     false, eo);
}

// ------------------------------------------------------------ attention
kq::SageStrides sage_strides(kq_layout layout, int64_t H, int64_t L) {
  if (layout == KQ_LAYOUT_BLHD) return kq::SageStrides{L * H * kq::kSageD, kq::kSageD, H * kq::kSageD};
  return kq::SageStrides{H * L * kq::kSageD, L * kq::kSageD, kq::kSageD};
}

bool pow2_block(int64_t b) { return b >= 1 && b <= 128 && (b & (b - 1)) == 0; }

// Shape checks shared by the attention entry points; *empty is set when
// there is nothing to do.
kq_status check_sage_shape(const char* op, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                           int64_t D, kq_layout layout, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return fail(KQ_ERR_INVALID_VALUE, "[%s] negative size", op);
  if (layout != KQ_LAYOUT_BHLD && layout != KQ_LAYOUT_BLHD)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] unknown layout %d", op, (int)layout);
  if (D != kq::kSageD)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] head dim %lld: only 128 is supported", op, (long long)D);
  if (B * H > 65535)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] B*H=%lld exceeds 65535", op, (long long)(B * H));
  if (Lq > (1 << 22) || Lk > (1 << 22))
    return fail(KQ_ERR_UNSUPPORTED, "[%s] sequence lengths are limited to 2^22", op);
  if (B == 0 || H == 0 || Lq == 0) {
    *empty = true;
    return KQ_SUCCESS;
  }
  if (Lk == 0) return fail(KQ_ERR_INVALID_VALUE, "[%s] no keys (Lk = 0) for %lld queries", op, (long long)Lq);
  return KQ_SUCCESS;
}

kq_status check_sage_ws(const char* op, const void* ws, size_t ws_bytes, const kq::SageLayout& L) {
  if (!ws || ws_bytes < L.total)
    return fail(KQ_ERR_WORKSPACE, "[%s] workspace of %zu bytes is smaller than the %zu required", op,
                ws_bytes, L.total);
  if (!aligned16(ws)) return fail(KQ_ERR_INVALID_VALUE, "[%s] workspace must be 16-byte aligned", op);
  return KQ_SUCCESS;
}

// The last preparation this process issued on each workspace address: its
// shape and key block.  The attention checks a call against it on the host,
// so a workspace prepared with per-token (or sub-step) key scales is refused
// before anything is enqueued when the call asserts uniform 64-key steps.  A
// workspace the process never prepared (filled by another process, or
// copied) is not in the table; the kernel's own check of the key block the
// preparation wrote into the workspace covers it.
struct SagePrepRecord {
  int64_t B, H, Lq, Lk, k_block;
};
std::mutex g_sage_mu;
std::unordered_map<const void*, SagePrepRecord> g_sage_prep;

void sage_record(const void* ws, const SagePrepRecord& r) {
  std::lock_guard<std::mutex> lk(g_sage_mu);
  g_sage_prep[ws] = r;
}

bool sage_lookup(const void* ws, SagePrepRecord* r) {
  std::lock_guard<std::mutex> lk(g_sage_mu);
  auto it = g_sage_prep.find(ws);
  if (it == g_sage_prep.end()) return false;
  *r = it->second;
  return true;
}

kq_status sage_prepare_impl(const char* op, const void* q, const void* k, const void* v, int64_t B,
                            int64_t H, int64_t Lq, int64_t Lk, int64_t D, kq_layout layout,
                            int64_t q_block, int64_t k_block, void* ws, size_t ws_bytes,
                            void* stream, bool* empty) {
  kq_status st = check_sage_shape(op, B, H, Lq, Lk, D, layout, empty);
  if (st != KQ_SUCCESS || *empty) return st;
  if (!pow2_block(q_block) || !pow2_block(k_block))
    return fail(KQ_ERR_UNSUPPORTED, "[%s] q_block=%lld, k_block=%lld: blocks are powers of two in [1, 128]",
                op, (long long)q_block, (long long)k_block);
  if (!q || !k || !v) return fail(KQ_ERR_INVALID_VALUE, "[%s] null tensor pointer", op);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] q, k and v must be 16-byte aligned", op);
  const kq::SageLayout L = kq::sage_layout(B, H, Lq, Lk);
  st = check_sage_ws(op, ws, ws_bytes, L);
  if (st != KQ_SUCCESS) return st;
  st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  const char* name = kq::launch_sage_prepare(
      reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
      reinterpret_cast<const uint16_t*>(v), sage_strides(layout, H, Lq), sage_strides(layout, H, Lk),
      sage_strides(layout, H, Lk), B, H, Lq, Lk, (int)q_block, (int)k_block,
      reinterpret_cast<char*>(ws), L, reinterpret_cast<hipStream_t>(stream));
  st = check_launch(op);
  if (st == KQ_SUCCESS) sage_record(ws, SagePrepRecord{B, H, Lq, Lk, k_block});
  if (st == KQ_SUCCESS && env_log())
    fprintf(stderr, "[kq] %s B=%lld H=%lld Lq=%lld Lk=%lld q_block=%lld k_block=%lld kernels=%s\n", op,
            (long long)B, (long long)H, (long long)Lq, (long long)Lk, (long long)q_block,
            (long long)k_block, name);
  return st;
}

kq_status sage_attend_impl(const char* op, const void* ws, size_t ws_bytes, void* out, int64_t B,
                           int64_t H, int64_t Lq, int64_t Lk, int64_t D, kq_layout layout,
                           float scale, int64_t k_block, void* stream) {
  bool empty = false;
  kq_status st = check_sage_shape(op, B, H, Lq, Lk, D, layout, &empty);
  if (st != KQ_SUCCESS || empty) return st;
  if (!(scale > 0.0f) || !(scale <= 3.402823466e38f))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] scale must be positive and finite", op);
  if (!pow2_block(k_block))
    return fail(KQ_ERR_UNSUPPORTED, "[%s] k_block=%lld: blocks are powers of two in [1, 128]", op,
                (long long)k_block);
  if (!out) return fail(KQ_ERR_INVALID_VALUE, "[%s] null output pointer", op);
  if (!aligned16(out)) return fail(KQ_ERR_INVALID_VALUE, "[%s] out must be 16-byte aligned", op);
  const kq::SageLayout L = kq::sage_layout(B, H, Lq, Lk);
  const bool k_uniform = k_block >= kq::kSageKTile;
  st = check_sage_ws(op, ws, ws_bytes, L);
  if (st != KQ_SUCCESS) return st;
  SagePrepRecord rec;
  if (sage_lookup(ws, &rec)) {
    if (rec.B != B || rec.H != H || rec.Lq != Lq || rec.Lk != Lk)
      return fail(KQ_ERR_INVALID_VALUE,
                  "[%s] workspace was prepared for B=%lld H=%lld Lq=%lld Lk=%lld, not B=%lld H=%lld "
                  "Lq=%lld Lk=%lld",
                  op, (long long)rec.B, (long long)rec.H, (long long)rec.Lq, (long long)rec.Lk,
                  (long long)B, (long long)H, (long long)Lq, (long long)Lk);
    if (k_uniform && rec.k_block < kq::kSageKTile)
      return fail(KQ_ERR_INVALID_VALUE,
                  "[%s] k_block=%lld asserts one key scale per %d-key step, but the workspace was "
                  "prepared with k_block=%lld",
                  op, (long long)k_block, kq::kSageKTile, (long long)rec.k_block);
  }
  st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  const char* name = kq::launch_sage_attend(reinterpret_cast<const char*>(ws), L,
                                            reinterpret_cast<uint16_t*>(out),
                                            sage_strides(layout, H, Lq), B, H, Lq, Lk, scale,
                                            k_uniform, reinterpret_cast<hipStream_t>(stream));
  st = check_launch(op);
  if (st == KQ_SUCCESS && env_log())
    fprintf(stderr, "[kq] %s B=%lld H=%lld Lq=%lld Lk=%lld kernel=%s grid=%lld\n", op, (long long)B,
            (long long)H, (long long)Lq, (long long)Lk, name,
            (long long)(L.BH * (L.Lqp / kq::kSageQTile)));
  return st;
}

}  // namespace

extern "C" {

int kq_is_available(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 0;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
  return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

const char* kq_last_error(void) { return g_last_error.c_str(); }

size_t kq_workspace_bytes(int64_t M, int64_t N, int64_t K, kq_wformat fmt) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  // Sized for the two-kernel layout even where the route is fused (which
  // needs only the scales): the same workspace then serves every entry
  // point and lever for this shape (KQ_FUSE=0, kq_gemv_small_m), whose
  // routes never split K where the fused ones apply (K <= 6144).
  const kq_route_info r =
      kq::choose_route(M, N, K, fmt, env_force_route(), env_tile(), env_split(), env_fuse(),
                       env_gemv_lane());
  return kq::workspace_layout(M, N, K, fmt, r.splits, false).total;
}

kq_status kq_route(int64_t M, int64_t N, int64_t K, kq_wformat fmt, kq_dtype y_dtype,
                   kq_route_info* out) {
  std::string err;
  kq_status st = kq::validate_linear("kq_route", M, K, N, fmt, y_dtype, err);
  if (st != KQ_SUCCESS) return fail(st, "%s", err.c_str());
  if (!out) return fail(KQ_ERR_INVALID_VALUE, "[kq_route] null output");
  const int force = env_force_route();
  if (force == 2 && M > KQ_GEMV_MAX_M)
    return fail(KQ_ERR_UNSUPPORTED, "[kq_route] M=%lld exceeds the GEMV limit %d", (long long)M,
                KQ_GEMV_MAX_M);
  if (force == 2 && K > kq::kGemvMaxK)
    return fail(KQ_ERR_UNSUPPORTED, "[kq_route] K=%lld exceeds the GEMV limit %lld", (long long)K,
                (long long)kq::kGemvMaxK);
  *out = kq::choose_route(M, N, K, fmt, force, env_tile(), env_split(), env_fuse(),
                                           env_gemv_lane());
  return KQ_SUCCESS;
}

kq_status kq_quantize_weights(const float* w, int64_t N, int64_t K, kq_wformat fmt, void* wq,
                              void* scale, void* gbias, void* stream) {
  const char* op = "kq_quantize_weights";
  if (N < 0 || K < 0) return fail(KQ_ERR_INVALID_VALUE, "[%s] negative size", op);
  if (fmt != KQ_W8_PER_CHANNEL && fmt != KQ_W4_AFFINE_G64)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] unknown weight format %d", op, (int)fmt);
  if (K == 0) return fail(KQ_ERR_UNSUPPORTED, "[%s] K must be positive", op);
  if (K > INT32_MAX / 2) return fail(KQ_ERR_UNSUPPORTED, "[%s] K=%lld too large", op, (long long)K);
  if (fmt == KQ_W4_AFFINE_G64 && K % 64)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] K=%lld must be a multiple of 64 for int4 weights", op,
                (long long)K);
  if (fmt == KQ_W8_PER_CHANNEL && gbias)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] int8 weights take no group offsets (gbias must be NULL)", op);
  if (N == 0) return KQ_SUCCESS;
  if (!w || !wq || !scale || (fmt == KQ_W4_AFFINE_G64 && !gbias))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] null tensor pointer", op);
  if (!aligned16(w) || !aligned16(wq))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] w and wq must be 16-byte aligned", op);
  kq_status st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* name;
  if (fmt == KQ_W8_PER_CHANNEL)
    name = kq::launch_quant_w8(w, N, (int)K, reinterpret_cast<int8_t*>(wq),
                               reinterpret_cast<float*>(scale), s);
  else
    name = kq::launch_quant_w4(w, N, (int)K, reinterpret_cast<uint8_t*>(wq), scale, gbias, s);
  st = check_launch(op);
  if (st == KQ_SUCCESS && env_log())
    fprintf(stderr, "[kq] %s N=%lld K=%lld kernel=%s\n", op, (long long)N, (long long)K, name);
  return st;
}

kq_status kq_quantize_act(const void* x, int64_t M, int64_t K, int8_t* a, float* sx,
                          int32_t* gsum, void* stream) {
  return quantize_act("kq_quantize_act", x, M, K, a, sx, gsum, KQ_CODES_NATURAL, stream);
}

kq_status kq_quantize_act_ordered(const void* x, int64_t M, int64_t K, int8_t* a, float* sx,
                                  int32_t* gsum, kq_code_order order, void* stream) {
  return quantize_act("kq_quantize_act_ordered", x, M, K, a, sx, gsum, order, stream);
}

kq_status kq_w8a8_linear(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq,
                         const float* sw, const float* bias, void* y, kq_dtype y_dtype, void* ws,
                         size_t ws_bytes, void* stream) {
  return run_linear("kq_w8a8_linear", env_force_route(), KQ_W8_PER_CHANNEL, x, M, K, N, wq, sw,
                    nullptr, bias, y, y_dtype, ws, ws_bytes, stream);
}

kq_status kq_w4a8_linear(const void* x, int64_t M, int64_t K, int64_t N, const uint8_t* wq4,
                         const void* gscale, const void* gbias, const float* bias, void* y,
                         kq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  return run_linear("kq_w4a8_linear", env_force_route(), KQ_W4_AFFINE_G64, x, M, K, N, wq4, gscale,
                    gbias, bias, y, y_dtype, ws, ws_bytes, stream);
}

kq_status kq_w8a8_gemm(const int8_t* a, const float* sx, int64_t M, int64_t K, int64_t N,
                       const int8_t* wq, const float* sw, const float* bias, void* y,
                       kq_dtype y_dtype, void* stream) {
  return run_gemm("kq_w8a8_gemm", KQ_W8_PER_CHANNEL, a, sx, nullptr, M, K, N, wq, sw, nullptr, bias,
                  y, y_dtype, stream);
}

kq_status kq_w4a8_gemm(const int8_t* a, const float* sx, const int32_t* gsum, int64_t M, int64_t K,
                       int64_t N, const uint8_t* wq4, const void* gscale, const void* gbias,
                       const float* bias, void* y, kq_dtype y_dtype, void* stream) {
  return run_gemm("kq_w4a8_gemm", KQ_W4_AFFINE_G64, a, sx, gsum, M, K, N, wq4, gscale, gbias, bias,
                  y, y_dtype, stream);
}

kq_status kq_w4a8_gemm_ordered(const int8_t* a, const float* sx, const int32_t* gsum, int64_t M,
                               int64_t K, int64_t N, const uint8_t* wq4, const void* gscale,
                               const void* gbias, const float* bias, void* y, kq_dtype y_dtype,
                               kq_code_order order, void* stream) {
  return run_gemm("kq_w4a8_gemm_ordered", KQ_W4_AFFINE_G64, a, sx, gsum, M, K, N, wq4, gscale,
                  gbias, bias, y, y_dtype, stream, order);
}

kq_status kq_gemv_small_m(kq_wformat fmt, const void* x, int64_t M, int64_t K, int64_t N,
                          const void* wq, const void* scale, const void* gbias, const float* bias,
                          void* y, kq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  const char* op = "kq_gemv_small_m";
  if (M > KQ_GEMV_MAX_M)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] M=%lld exceeds the GEMV limit %d", op, (long long)M,
                KQ_GEMV_MAX_M);
  if (fmt == KQ_W8_PER_CHANNEL && gbias)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] int8 weights take no group offsets (gbias must be NULL)", op);
  // the GEMV kernel, quantizing x in its prologue where it can (force 3),
  // unless KQ_FORCE_ROUTE=gemv asks for the plain two-kernel GEMV (force 2)
  return run_linear(op, env_force_route() == 2 ? 2 : 3, fmt, x, M, K, N, wq, scale, gbias, bias, y, y_dtype, ws, ws_bytes,
                    stream);
}

kq_status kq_linear_gated(kq_wformat fmt, const void* x, int64_t M, int64_t K, int64_t N,
                          const void* wq, const void* scale, const void* gbias, const float* bias,
                          const void* residual, const float* gate, int64_t gate_rows, void* y,
                          kq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  const char* op = "kq_linear_gated";
  if (fmt != KQ_W8_PER_CHANNEL && fmt != KQ_W4_AFFINE_G64)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] unknown weight format %d", op, (int)fmt);
  if (fmt == KQ_W8_PER_CHANNEL && gbias)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] int8 weights take no group offsets (gbias must be NULL)", op);
  if (y_dtype != KQ_DTYPE_F32 && y_dtype != KQ_DTYPE_BF16)
    return fail(KQ_ERR_UNSUPPORTED, "[%s] the gated epilogue writes f32 or bf16, not %s", op,
                dtype_name(y_dtype));
  if (gate_rows < 1 || gate_rows > INT32_MAX)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] gate_rows=%lld must be in [1, 2^31)", op,
                (long long)gate_rows);
  if (residual && !aligned16(residual))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] residual must be 16-byte aligned", op);
  if (gate && ((uintptr_t)gate & 3))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] gate must be 4-byte aligned", op);
  if (residual && y && residual != y && M > 0 && N > 0) {
    // Only an exact alias is race-free: each output element reads its own
    // residual element before writing it, but overlapping shifted ranges
    // would read elements another workgroup has already written.
    const uintptr_t r0 = (uintptr_t)residual, r1 = r0 + (uintptr_t)(M * N * 2);
    const uintptr_t y0 = (uintptr_t)y, y1 = y0 + (uintptr_t)(M * N * (y_dtype == KQ_DTYPE_F32 ? 4 : 2));
    if (r0 < y1 && y0 < r1)
      return fail(KQ_ERR_INVALID_VALUE, "[%s] residual overlaps y without being y itself", op);
  }
  if (residual && residual == y && y_dtype != KQ_DTYPE_BF16)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] an in-place residual needs a bf16 output", op);
  kq::Epilogue ep;
  ep.residual = reinterpret_cast<const uint16_t*>(residual);
  ep.gate = gate;
  ep.gate_rows = (int)gate_rows;
  return run_linear(op, env_force_route(), fmt, x, M, K, N, wq, scale, gbias, bias, y, y_dtype,
                    ws, ws_bytes, stream, ep);
}

kq_status kq_sage_workspace_layout(int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                                   kq_sage_workspace* out) {
  const char* op = "kq_sage_workspace_layout";
  if (!out) return fail(KQ_ERR_INVALID_VALUE, "[%s] null output", op);
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return fail(KQ_ERR_INVALID_VALUE, "[%s] negative size", op);
  if (B * H > 65535 || Lq > (1 << 22) || Lk > (1 << 22))
    return fail(KQ_ERR_UNSUPPORTED, "[%s] shape outside the supported envelope", op);
  const kq::SageLayout L = kq::sage_layout(B, H, Lq, Lk);
  out->lq_pad = L.Lqp;
  out->lk_pad = L.Lkp;
  out->chunks = L.nchunk;
  out->qc = L.qc;
  out->sq = L.sq;
  out->kc = L.kc;
  out->sk = L.sk;
  out->vt = L.vt;
  out->kmean = L.kmean;
  out->colsum = L.colsum;
  out->meta = L.meta;
  out->total = L.total;
  return KQ_SUCCESS;
}

kq_status kq_sage_prepare(const void* q, const void* k, const void* v, int64_t B, int64_t H,
                          int64_t Lq, int64_t Lk, int64_t D, kq_layout layout, int64_t q_block,
                          int64_t k_block, void* ws, size_t ws_bytes, void* stream) {
  bool empty = false;
  return sage_prepare_impl("kq_sage_prepare", q, k, v, B, H, Lq, Lk, D, layout, q_block, k_block,
                           ws, ws_bytes, stream, &empty);
}

kq_status kq_sage_attend(const void* ws, size_t ws_bytes, void* out, int64_t B, int64_t H,
                         int64_t Lq, int64_t Lk, int64_t D, kq_layout layout, float scale,
                         int64_t k_block, void* stream) {
  return sage_attend_impl("kq_sage_attend", ws, ws_bytes, out, B, H, Lq, Lk, D, layout, scale,
                          k_block, stream);
}

kq_status kq_sage_attention(const void* q, const void* k, const void* v, void* out, int64_t B,
                            int64_t H, int64_t Lq, int64_t Lk, int64_t D, kq_layout layout,
                            float scale, int64_t q_block, int64_t k_block, void* ws,
                            size_t ws_bytes, void* stream) {
  const char* op = "kq_sage_attention";
  // validate everything before enqueueing anything
  bool empty = false;
  kq_status st = check_sage_shape(op, B, H, Lq, Lk, D, layout, &empty);
  if (st != KQ_SUCCESS || empty) return st;
  if (!(scale > 0.0f) || !(scale <= 3.402823466e38f))
    return fail(KQ_ERR_INVALID_VALUE, "[%s] scale must be positive and finite", op);
  if (!out) return fail(KQ_ERR_INVALID_VALUE, "[%s] null output pointer", op);
  if (!aligned16(out)) return fail(KQ_ERR_INVALID_VALUE, "[%s] out must be 16-byte aligned", op);
  st = sage_prepare_impl(op, q, k, v, B, H, Lq, Lk, D, layout, q_block, k_block, ws, ws_bytes,
                         stream, &empty);
  if (st != KQ_SUCCESS) return st;
  return sage_attend_impl(op, ws, ws_bytes, out, B, H, Lq, Lk, D, layout, scale, k_block, stream);
}

kq_status kq_w8a8_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t N,
                                 const int8_t* wq, const float* sw, const float* bias, void* y,
                                 kq_dtype y_dtype, void* stream) {
  const char* op = "kq_w8a8_linear_noalloc";
  const int force = env_force_route();
  kq_status st = check_linear_args(op, force, KQ_W8_PER_CHANNEL, M, K, N, y_dtype, x, wq, sw,
                                   nullptr, y);
  if (st != KQ_SUCCESS || M == 0 || N == 0) return st;
  const size_t need = kq_workspace_bytes(M, N, K, KQ_W8_PER_CHANNEL);
  if (need > kq::kScratchBytes)
    return fail(KQ_ERR_UNSUPPORTED,
                "[%s] M=%lld, N=%lld, K=%lld needs %zu bytes of scratch; the library holds %zu",
                op, (long long)M, (long long)N, (long long)K, need, kq::kScratchBytes);
  st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  hipError_t e = hipSuccess;
  void* ws = kq::scratch_address(&e);
  if (ws == nullptr)
    return fail(KQ_ERR_NO_DEVICE, "[%s] no device address for the scratch: %s", op,
                hipGetErrorString(e));
  return run_linear(op, force, KQ_W8_PER_CHANNEL, x, M, K, N, wq, sw, nullptr, bias, y, y_dtype,
                    ws, kq::kScratchBytes, stream);
}

// ------------------------------------------------------------ probes
kq_status kq_probe_read(const void* src, int64_t bytes, int64_t grid, int32_t threads,
                        uint32_t* sink, void* stream) {
  const char* op = "kq_probe_read";
  if (bytes < 0 || bytes % 16 != 0)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] bytes=%lld must be a non-negative multiple of 16", op,
                (long long)bytes);
  if (grid < 1 || grid > INT32_MAX || threads < 64 || threads > 1024 || threads % 64 != 0)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] grid=%lld, threads=%d out of range", op,
                (long long)grid, (int)threads);
  if (bytes == 0) return KQ_SUCCESS;
  if (!src || !sink) return fail(KQ_ERR_INVALID_VALUE, "[%s] null pointer", op);
  if (!aligned16(src)) return fail(KQ_ERR_INVALID_VALUE, "[%s] src must be 16-byte aligned", op);
  kq_status st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  kq::launch_probe_read(src, bytes, grid, threads, sink, reinterpret_cast<hipStream_t>(stream));
  return check_launch(op);
}

kq_status kq_probe_mfma_i8(int64_t iters, int64_t grid, int32_t* sink, void* stream) {
  const char* op = "kq_probe_mfma_i8";
  if (iters < 1 || iters > INT32_MAX || grid < 1 || grid > INT32_MAX)
    return fail(KQ_ERR_INVALID_VALUE, "[%s] iters=%lld, grid=%lld out of range", op,
                (long long)iters, (long long)grid);
  if (!sink) return fail(KQ_ERR_INVALID_VALUE, "[%s] null sink", op);
  kq_status st = check_device(op);
  if (st != KQ_SUCCESS) return st;
  kq::launch_probe_mfma((int)iters, grid, sink, reinterpret_cast<hipStream_t>(stream));
  return check_launch(op);
}

}  // extern "C"
