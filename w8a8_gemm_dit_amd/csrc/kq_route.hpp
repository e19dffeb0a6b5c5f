// Argument validation and route selection for the libkq linears.
// Pure host code with no HIP dependency, so it is testable without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "kq.h"

namespace kq {

// Tile configurations of the W8A8 (ids 0-4) and W4A8 (ids 5-6) GEMM kernels.
enum GemmTile : int32_t {
  kTile256x256 = 0,  // 256 rows x 256 columns, 4 waves of 128x128
  kTile256x192 = 1,  // 256 x 192, 8 waves of 64x96 (4x2)
  kTile256x128 = 2,  // 256 x 128, 4 waves of 128x64 (2x2)
  kTile128x128 = 3,  // 128 x 128, 4 waves of 64x64
  kTile64x64 = 4,    // 64 x 64, 4 waves of 32x32 (thin shapes)
  kTile128x256 = 5,  // int4 GEMM: 128 x 256, 8 waves of 64x64 (2x4)
  kTile64x128 = 6,   // int4 GEMM: 64 x 128, 4 waves of 32x64 (2x2)
  kTile256x256w8 = 7,  // 256 x 256, 8 waves of 64x128 (4x2)
  kNumTiles = 8,
};

const char* tile_name(int32_t tile);
int32_t tile_from_name(const char* name);  // -1 if unknown

struct TileShape {
  int32_t bm, bn, threads;
};

TileShape tile_shape(int32_t tile);

// Validates a linear call's scalar arguments; on failure writes the message
// (with the "[op] " prefix) to err and returns the status.
kq_status validate_linear(const char* op, int64_t M, int64_t K, int64_t N,
                          kq_wformat fmt, kq_dtype y_dtype, std::string& err);

// Route of a validated linear call.  force: 0 = automatic, 1 = GEMM, 2 = GEMV
// after the quantize kernel, 3 = GEMV, quantizing x in its prologue where it
// can (M <= kGemvXqRows, K <= kFusedMaxK, fuse).
// tile_override: -1 = automatic, else a GemmTile.  split_override: -1 =
// automatic, 0 or 1 = never split K, n > 1 = n slices (fewer if K is short).
// fuse: the call quantizes x itself and may take the fused thin-N kernel.
// lane: M <= kGemvLaneRows and K <= kFusedMaxK take the lane-per-column
// GEMV kernels (int4 and int8 weights, on both GEMV routes).
kq_route_info choose_route(int64_t M, int64_t N, int64_t K, kq_wformat fmt,
                           int force, int tile_override, int split_override = 0,
                           bool fuse = false, bool lane = true);

// K slicing of a split GEMM: slices of `chunk` codes, a multiple of `unit`
// (int8 weights: 256, so that only the last slice can end between the
// kernel's 4-step unrolls; int4 weights: 1024, whole 16-group table
// chunks); returns the number of slices, at most `want`.
constexpr int64_t kSplitUnitW8 = 256;
constexpr int64_t kSplitUnitW4 = 1024;
int split_chunk(int64_t K, int want, int64_t& chunk, int64_t unit = kSplitUnitW8);

// Workspace layout of one linear call (the fused route keeps only the
// token scales).
struct WorkspaceLayout {
  size_t codes_off, codes_bytes;   // int8 [M rounded up to 16, K]
  size_t scale_off, scale_bytes;   // fp32 [M]
  size_t gsum_off, gsum_bytes;     // int32 [M,K/64] (int4 format only)
  size_t part_off, part_bytes;     // int32 [splits,M,N] (split GEMM only)
  size_t total;
};
WorkspaceLayout workspace_layout(int64_t M, int64_t N, int64_t K, kq_wformat fmt,
                                 int splits = 1, bool fused = false);

// The MFMA GEMV of a linear reads the activation codes in its fragment
// order (gemv_frag_offset: per 16-row block and group of 64, four k chunks
// x 16 rows x 16 bytes), which the quantize kernel writes for it; the
// other routes read them row-major.
bool gemv_frag_codes(const kq_route_info& r);
// Byte offset of code (row, k) in the fragment order for int8 (w4 false)
// or int4 weights: k chunk h = (k%64)/16 of a group sits at slot h for
// int8 and at the bit-swapped slot ((h&1)<<1 | h>>1) for int4, whose
// operand pairs its k chunks that way.
constexpr int64_t gemv_frag_offset(int64_t row, int64_t k, int64_t K, bool w4) {
  const int64_t G = K / 64, g = k / 64, h = (k % 64) / 16;
  const int64_t q = w4 ? (((h & 1) << 1) | (h >> 1)) : h;
  return (((row / 16) * G + g) * 4 + q) * 256 + (row % 16) * 16 + k % 16;
}

// Split-K policy: the slice count (at most kSplitMax, slices of at least
// kSplitMinK codes) that minimizes a simple time model of the grid (waves
// of kSplitCUs workgroups) plus the partial sums' round trip.
constexpr int kSplitCUs = 256;
constexpr int kSplitMax = 16;
constexpr int64_t kSplitMinK = 512;

// GEMV route geometry: 32 output columns (two MFMA column blocks) per
// workgroup of 8 wavefronts for int4 weights, 16 for int8; the wavefronts
// split K into slices of up to 32 groups of 64, so the GEMV takes K <=
// 16384.
constexpr int kGemvCols = 32;
constexpr int kGemvCols8 = 16;
constexpr int kGemvRows = 16;   // activation rows per GEMV workgroup
constexpr int kGemvThinN = 64;  // N up to this takes the GEMV at any M
constexpr int kGemvAutoRows = 32;  // the automatic route's GEMV takes M up to this
constexpr int kGemvThreads = 512;
constexpr int kGemvXqRows = 4;  // the GEMV quantizes x itself up to this many rows
// Lane-per-column GEMVs (M <= kGemvLaneRows, K <= kFusedMaxK, either weight
// format): 32 output columns per workgroup of 8 wavefronts, 8 lanes per
// column.
constexpr int kGemvLaneRows = 2;
constexpr int kGemvLaneCols = 32;
constexpr int kGemvLaneThreads = 512;
constexpr int64_t kGemvMaxK = KQ_GEMV_MAX_K;

// Fused thin-N route (N <= kGemvThinN, M > 16): 8 rows and all columns
// per workgroup of 16 wavefronts, each holding its K slice of bf16 x in
// registers, at most 8 groups of 64, so K <= 6144.  Every workgroup reads
// all N*K weight bytes, N/16 times the bytes of its x: past M*N = 2^19 the
// two-kernel route (quantize + GEMV) measured as fast or faster, unless N
// <= 32.
constexpr int kFusedRows = 8;
constexpr int kFusedThreads = 1024;
constexpr int64_t kFusedMaxK = 6144;
constexpr int64_t kFusedMaxMN = (int64_t)1 << 19;
constexpr int kFusedAnyM_N = 32;

}  // namespace kq
