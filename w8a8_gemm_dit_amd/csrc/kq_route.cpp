// Argument validation and route selection (pure host code, no HIP).
//
// The envelope follows MLX pull request 4722, "Selector rules" (2-D [N,K]
// weights, K % 64 == 0, K/64 <= 1024, non-batched), without its M >= 64
// gate, which the pull request calls a coverage choice; M <= 16 takes the
// GEMV ("qlip-mlx" README, w4a8_linear bullet).  The decision is one tested
// function (mlx-kquant pull request 89 commit list).
#include "kq_route.hpp"

#include <cstdio>
#include <cstdlib>

namespace kq {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

TileShape tile_shape(int32_t tile) {
  switch (tile) {
    case kTile256x256: return {256, 256, 256};
    case kTile256x192: return {256, 192, 512};
    case kTile256x128: return {256, 128, 256};
    case kTile128x128: return {128, 128, 256};
    case kTile128x256: return {128, 256, 512};
    case kTile64x128: return {64, 128, 256};
    default: return {64, 64, 256};
  }
}

static const char* const kTileNames[kNumTiles] = {"256x256", "256x192", "256x128", "128x128",
                                                  "64x64",   "128x256", "64x128"};

const char* tile_name(int32_t tile) {
  return (tile >= 0 && tile < kNumTiles) ? kTileNames[tile] : "?";
}

int32_t tile_from_name(const char* name) {
  if (!name) return -1;
  for (int32_t t = 0; t < kNumTiles; ++t)
    if (std::string(name) == kTileNames[t]) return t;
  return -1;
}

kq_status validate_linear(const char* op, int64_t M, int64_t K, int64_t N,
                          kq_wformat fmt, kq_dtype y_dtype, std::string& err) {
  char buf[256];
  if (M < 0 || N < 0 || K < 0) {
    snprintf(buf, sizeof buf, "[%s] negative size (M=%lld, N=%lld, K=%lld)", op,
             (long long)M, (long long)N, (long long)K);
    err = buf;
    return KQ_ERR_INVALID_VALUE;
  }
  if (fmt != KQ_W8_PER_CHANNEL && fmt != KQ_W4_AFFINE_G64) {
    snprintf(buf, sizeof buf, "[%s] unknown weight format %d", op, (int)fmt);
    err = buf;
    return KQ_ERR_INVALID_VALUE;
  }
  if (y_dtype != KQ_DTYPE_F32 && y_dtype != KQ_DTYPE_BF16 && y_dtype != KQ_DTYPE_I32) {
    snprintf(buf, sizeof buf, "[%s] unknown output dtype %d", op, (int)y_dtype);
    err = buf;
    return KQ_ERR_INVALID_VALUE;
  }
  if (K % 64 != 0 || K == 0) {
    snprintf(buf, sizeof buf, "[%s] K=%lld must be a positive multiple of 64", op,
             (long long)K);
    err = buf;
    return KQ_ERR_UNSUPPORTED;
  }
  if (K > KQ_MAX_K) {
    snprintf(buf, sizeof buf, "[%s] K=%lld exceeds %d (int32 accumulator bound)", op,
             (long long)K, KQ_MAX_K);
    err = buf;
    return KQ_ERR_UNSUPPORTED;
  }
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 30 || M * K > ((int64_t)1 << 40)) {
    snprintf(buf, sizeof buf, "[%s] shape too large (M=%lld, N=%lld)", op,
             (long long)M, (long long)N);
    err = buf;
    return KQ_ERR_UNSUPPORTED;
  }
  return KQ_SUCCESS;
}

kq_route_info choose_route(int64_t M, int64_t N, int64_t K, kq_wformat fmt,
                           int force, int tile_override) {
  kq_route_info r{};
  const bool fits = M <= KQ_GEMV_MAX_M && K <= kGemvMaxK;
  // Thin N: the GEMM's tiles would leave most CUs idle, while the GEMV
  // kernel's 16x16 blocks over all of K give ceil(N/16)*ceil(M/16)
  // workgroups.
  // (the row blocks are the grid's y dimension, at most 65535)
  const bool thin = N <= kGemvThinN && K <= kGemvMaxK && (M + kGemvRows - 1) / kGemvRows <= 65535;
  const bool gemv = (force == 2) ? fits : (force == 1) ? false : (M >= 1 && (fits || thin));
  if (gemv) {
    r.kind = KQ_ROUTE_GEMV;
    r.tile_m = kGemvRows;
    r.tile_n = kGemvCols;
    r.threads = kGemvThreads;
    r.grid = ((N + kGemvCols - 1) / kGemvCols) * ((M + kGemvRows - 1) / kGemvRows);
    return r;
  }
  // Tiles each kernel offers.  The int4 GEMM keeps fp32 accumulators that
  // its VALU rescale updates every group, so it uses 64x64 (or 32x64)
  // blocks per wavefront.
  static const int32_t kW8Tiles[] = {kTile256x256, kTile256x192, kTile256x128, kTile128x128,
                                     kTile64x64};
  static const int32_t kW4Tiles[] = {kTile128x256, kTile64x128};
  const bool w8 = fmt == KQ_W8_PER_CHANNEL;
  const int32_t* cand = w8 ? kW8Tiles : kW4Tiles;
  const int ncand = w8 ? 5 : 2;
  int32_t tile = -1;
  if (tile_override >= 0 && tile_override < kNumTiles) {
    // a tile this kernel lacks: the one nearest in area (larger on a tie)
    const TileShape want = tile_shape(tile_override);
    int64_t best_d = -1;
    for (int i = 0; i < ncand; ++i) {
      const TileShape s = tile_shape(cand[i]);
      const int64_t d = std::llabs((int64_t)s.bm * s.bn - (int64_t)want.bm * want.bn);
      if (best_d < 0 || d < best_d) {
        best_d = d;
        tile = cand[i];
      }
    }
  } else {
    // Minimize (waves of 256 workgroups) x (tile area / relative tile
    // efficiency): larger tiles reuse operands better, but a partial last
    // wave leaves CUs idle.
    double best = 0;
    for (int i = 0; i < ncand; ++i) {
      const TileShape s = tile_shape(cand[i]);
      const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
      const int64_t waves = (tiles + 255) / 256;
      static const double kEff[kNumTiles] = {0.95, 1.0, 0.9, 0.75, 0.45, 1.0, 0.7};
      const double cost = (double)waves * s.bm * s.bn / kEff[cand[i]];
      if (tile < 0 || cost < best) {
        best = cost;
        tile = cand[i];
      }
    }
  }
  TileShape s = tile_shape(tile);
  r.kind = KQ_ROUTE_GEMM;
  r.tile_m = s.bm;
  r.tile_n = s.bn;
  r.threads = s.threads;
  r.grid = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
  return r;
}

WorkspaceLayout workspace_layout(int64_t M, int64_t K, kq_wformat fmt) {
  WorkspaceLayout w{};
  if (M <= 0 || K <= 0) return w;
  size_t off = 0;
  w.codes_off = off;
  w.codes_bytes = (size_t)M * (size_t)K;
  off = align256(off + w.codes_bytes);
  w.scale_off = off;
  w.scale_bytes = 4 * (size_t)M;
  off = align256(off + w.scale_bytes);
  if (fmt == KQ_W4_AFFINE_G64) {
    w.gsum_off = off;
    w.gsum_bytes = 4 * (size_t)M * (size_t)(K / 64);
    off = align256(off + w.gsum_bytes);
  }
  w.total = off;
  return w;
}

}  // namespace kq
