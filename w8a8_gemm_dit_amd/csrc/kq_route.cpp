// Argument validation and route selection (pure host code, no HIP).
//
// The envelope follows MLX pull request 4722, "Selector rules" (2-D [N,K]
// weights, K % 64 == 0, K/64 <= 1024, non-batched), without its M >= 64
// gate, which the pull request calls a coverage choice; M <= 16 takes the
// GEMV ("qlip-mlx" README, w4a8_linear bullet).  The decision is one tested
// function (mlx-kquant pull request 89 commit list).
#include "kq_route.hpp"

#include <cstdio>
#include <algorithm>
#include <cstdint>
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
    case kTile256x256w8: return {256, 256, 512};
    default: return {64, 64, 256};
  }
}

static const char* const kTileNames[kNumTiles] = {"256x256", "256x192", "256x128", "128x128",
                                                  "64x64",   "128x256", "64x128",  "256x256w8"};

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

int split_chunk(int64_t K, int want, int64_t& chunk, int64_t unit) {
  const int64_t units = (K + unit - 1) / unit;
  if (want < 2 || units < 2) {
    chunk = K;
    return 1;
  }
  const int64_t per = (units + want - 1) / want;  // units per slice
  chunk = per * unit;
  return (int)((K + chunk - 1) / chunk);
}

kq_route_info choose_route(int64_t M, int64_t N, int64_t K, kq_wformat fmt,
                           int force, int tile_override, int split_override, bool fuse,
                           bool lane) {
  kq_route_info r{};
  r.splits = 1;
  const bool lane_gemv = lane && M >= 1 && M <= kGemvLaneRows && K <= kFusedMaxK;
  auto lane_geometry = [&]() {
    r.tile_m = kGemvLaneRows;
    r.tile_n = kGemvLaneCols;
    r.threads = kGemvLaneThreads;
    r.grid = (N + kGemvLaneCols - 1) / kGemvLaneCols;
  };
  // Up to 4 rows the GEMV quantizes x in its prologue (the separate
  // quantize kernel would cost a launch and a round trip for a few rows).
  if (fuse && (force == 0 || force == 3) && M >= 1 && M <= kGemvXqRows && K <= kFusedMaxK) {
    const int cols = fmt == KQ_W4_AFFINE_G64 ? kGemvCols : kGemvCols8;
    r.kind = KQ_ROUTE_FUSED;
    r.tile_m = kGemvXqRows;
    r.tile_n = cols;
    r.threads = kGemvThreads;
    r.grid = (N + cols - 1) / cols;
    if (lane_gemv) lane_geometry();
    return r;
  }
  // Thin N with more than one 16-row block: one kernel quantizes its rows
  // and covers every column, so x is read once and no codes are stored.
  if (fuse && force == 0 && N <= kGemvThinN && M > KQ_GEMV_MAX_M && K <= kFusedMaxK &&
      (N <= kFusedAnyM_N || M * N <= kFusedMaxMN) &&
      (M + kFusedRows - 1) / kFusedRows <= INT32_MAX) {
    r.kind = KQ_ROUTE_FUSED;
    r.tile_m = kFusedRows;
    r.tile_n = (int32_t)((N + 15) / 16 * 16);
    r.threads = kFusedThreads;
    r.grid = (M + kFusedRows - 1) / kFusedRows;
    return r;
  }
  const bool fits = M <= KQ_GEMV_MAX_M && K <= kGemvMaxK;
  // Up to kGemvAutoRows rows the GEMV kernel (one weight pass per 16-row
  // block, the later ones mostly from the caches) still beats the GEMM.
  const bool small = M <= kGemvAutoRows && K <= kGemvMaxK;
  // Thin N: the GEMM's tiles would leave most CUs idle, while the GEMV
  // kernel's 16x16 blocks over all of K give ceil(N/16)*ceil(M/16)
  // workgroups.
  // (the row blocks are the grid's y dimension, at most 65535)
  const bool thin = N <= kGemvThinN && K <= kGemvMaxK && (M + kGemvRows - 1) / kGemvRows <= 65535;
  const bool gemv = (force >= 2) ? fits : (force == 1) ? false : (M >= 1 && (small || thin));
  if (gemv) {
    const int cols = fmt == KQ_W4_AFFINE_G64 ? kGemvCols : kGemvCols8;
    r.kind = KQ_ROUTE_GEMV;
    r.tile_m = kGemvRows;
    r.tile_n = cols;
    r.threads = kGemvThreads;
    r.grid = ((N + cols - 1) / cols) * ((M + kGemvRows - 1) / kGemvRows);
    if (lane_gemv) lane_geometry();
    return r;
  }
  // Tiles each kernel offers.  The int4 GEMM keeps fp32 accumulators that
  // its VALU rescale updates every group, so it uses 64x64 (or 32x64)
  // blocks per wavefront.
  static const int32_t kW8Tiles[] = {kTile256x256, kTile256x192, kTile256x128, kTile128x128,
                                     kTile64x64, kTile256x256w8};
  static const int32_t kW4Tiles[] = {kTile128x256, kTile128x128, kTile64x128};
  const bool w8 = fmt == KQ_W8_PER_CHANNEL;
  const int32_t* cand = w8 ? kW8Tiles : kW4Tiles;
  const int ncand = w8 ? 6 : 3;
  int32_t tile = -1;
  for (int i = 0; i < ncand && tile_override >= 0; ++i)
    if (cand[i] == tile_override) tile = tile_override;
  if (tile < 0 && tile_override >= 0 && tile_override < kNumTiles) {
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
  }
  // Modelled time of a tile grid with `sp` K slices (seconds): waves of 256
  // workgroups, each tile at about 45% of a CU's share of the INT8 peak
  // times the tile's relative efficiency; a split adds its int32 partials'
  // HBM round trip (written, then read by the fold, at ~4 TB/s) and the
  // fold's launch.
  // (256x256w8: measured 5% faster than 256x192 at 16384 x 3072 -> 12288,
  // 12 rounds of tiles against 16; slower on single-round grids, which the
  // model leaves to 256x192 since its tiles there cost more)
  static const double kEff[kNumTiles] = {0.95, 1.0, 0.9, 0.75, 0.45, 1.0, 0.7, 1.04};
  // the int4 GEMM's 128x128 tile runs two workgroups per CU: measured 7%
  // faster than 128x256 on 2048 x 4096 -> 12288 and equal on 12288 -> 4096
  constexpr double kEffW4_128x128 = 1.05;
  // int4 tiles run at about 18% of the INT8 peak (their rescale is
  // VALU-bound), the int8 ones at about 45%
  const double cu_rate = (w8 ? 0.45 : 0.18) * 5.0e15 / kSplitCUs;
  const int64_t unit = w8 ? kSplitUnitW8 : kSplitUnitW4;
  auto model = [&](int32_t t, int sp, int64_t chunk) {
    const TileShape sh = tile_shape(t);
    const int64_t tiles = ((M + sh.bm - 1) / sh.bm) * ((N + sh.bn - 1) / sh.bn);
    const int64_t waves = (tiles * sp + kSplitCUs - 1) / kSplitCUs;
    const double eff = (!w8 && t == kTile128x128) ? kEffW4_128x128 : kEff[t];
    const double tile_s = 2.0 * sh.bm * sh.bn * (double)chunk / (cu_rate * eff);
    double cost = (double)waves * tile_s;
    if (sp > 1) cost += 8.0 * sp * (double)M * (double)N / 4.0e12 + 3e-6;
    return cost;
  };
  // Slices for a tile: the best modelled count up to kSplitMax with
  // slices of at least kSplitMinK codes, or the forced count.  int8
  // weights fold exact int32 partials; int4 weights fp32 ones.
  auto best_split = [&](int32_t t, int64_t& chunk) -> int {
    chunk = K;
    if (split_override == 0 || split_override == 1) return 1;
    if (split_override > 1)
      return split_chunk(K, std::min(split_override, kSplitMax), chunk, unit);
    int best_sp = 1;
    double best_cost = model(t, 1, K);
    for (int want = 2; want <= kSplitMax && K / want >= kSplitMinK; ++want) {
      int64_t c;
      const int sp = split_chunk(K, want, c, unit);
      const double cost = model(t, sp, c);
      if (cost < best_cost) {
        best_cost = cost;
        best_sp = sp;
        chunk = c;
      }
    }
    return best_sp;
  };
  if (tile < 0) {
    double best = 0;
    for (int i = 0; i < ncand; ++i) {
      int64_t chunk;
      const int sp = best_split(cand[i], chunk);
      const double cost = model(cand[i], sp, chunk);
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
  const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
  int64_t chunk;
  r.splits = best_split(tile, chunk);
  r.grid = tiles * r.splits;
  return r;
}

WorkspaceLayout workspace_layout(int64_t M, int64_t N, int64_t K, kq_wformat fmt, int splits,
                                 bool fused) {
  WorkspaceLayout w{};
  if (M <= 0 || K <= 0 || N <= 0) return w;
  size_t off = 0;
  if (fused) {
    w.scale_bytes = 4 * (size_t)M;
    w.total = align256(w.scale_bytes);
    return w;
  }
  w.codes_off = off;
  // rows rounded up to the GEMV's 16-row blocks (its fragment order covers
  // whole blocks; the padding rows are never written and only reach output
  // rows past M, which are not stored)
  w.codes_bytes = (size_t)((M + 15) / 16 * 16) * (size_t)K;
  off = align256(off + w.codes_bytes);
  w.scale_off = off;
  w.scale_bytes = 4 * (size_t)M;
  off = align256(off + w.scale_bytes);
  if (fmt == KQ_W4_AFFINE_G64) {
    w.gsum_off = off;
    w.gsum_bytes = 4 * (size_t)M * (size_t)(K / 64);
    off = align256(off + w.gsum_bytes);
  }
  if (splits > 1) {
    w.part_off = off;
    w.part_bytes = 4 * (size_t)splits * (size_t)M * (size_t)N;
    off = align256(off + w.part_bytes);
  }
  w.total = off;
  return w;
}

bool gemv_frag_codes(const kq_route_info& r) {
  return r.kind == KQ_ROUTE_GEMV && r.tile_m == kGemvRows;  // not the lane kernels
}

}  // namespace kq
