// tile_order.hpp -- which output tile a persistent GEMM workgroup computes.
//
// Host- and device-callable, so the CPU tests check the exact mapping the
// kernel uses.
//
// Grouped order ("TensorCore_GEMM_with_TMA", §2.3 kernel, GROUP_M = 8; the
// TVM TIRx chapter's step 6 scheduler uses the same l2_group_size = 8): tile
// indices are cut into groups of `group_m` tile rows times all tile columns;
// inside a group the index runs down the rows of one column, then moves to the
// next column.  Neighbouring indices therefore share B column panels and a
// small set of A row panels, which keeps both in L2.  The last group may have
// fewer than `group_m` rows.
//
// XCD-aware workgroup numbering (MI355X-specific): the dispatcher hands
// workgroups to the 8 XCDs round-robin (workgroup w runs on XCD w % 8), and
// each XCD has its own L2.  Renumbering w so that each XCD owns one contiguous
// range of logical ids puts tiles that are neighbours in the grouped order on
// the same XCD, so they share that XCD's L2.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GT_HD __host__ __device__
#else
#define GT_HD
#endif

namespace gt {

constexpr int kNumXcd = 8;

struct TileCoord {
  int64_t tm;
  int64_t tn;
};

GT_HD inline TileCoord grouped_tile(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t group_m) {
  const int64_t per_group = group_m * tiles_n;
  const int64_t group = t / per_group;
  const int64_t first_m = group * group_m;
  const int64_t rows_here = (tiles_m - first_m < group_m) ? (tiles_m - first_m) : group_m;
  const int64_t within = t - group * per_group;
  TileCoord c;
  c.tm = first_m + within % rows_here;
  c.tn = within / rows_here;
  return c;
}

// The same mapping in 32-bit arithmetic, for grids of fewer than 2^31 tiles
// (a 64-bit division is a long instruction sequence on the GPU).
GT_HD inline TileCoord grouped_tile32(uint32_t t, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m) {
  const uint32_t per_group = group_m * tiles_n;
  const uint32_t group = t / per_group;
  const uint32_t first_m = group * group_m;
  const uint32_t rows_here = (tiles_m - first_m < group_m) ? (tiles_m - first_m) : group_m;
  const uint32_t within = t - group * per_group;
  const uint32_t tn = within / rows_here;
  TileCoord c;
  c.tm = first_m + (within - tn * rows_here);
  c.tn = tn;
  return c;
}

// The grouped mapping as the kernel computes it: in 32-bit arithmetic when
// every intermediate fits (fewer than 2^30 tiles and group_m * tiles_n below
// 2^31), else in 64-bit.
GT_HD inline TileCoord tile_of(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t group_m) {
  if (tiles_m * tiles_n < (int64_t{1} << 30) && group_m * tiles_n < (int64_t{1} << 31))
    return grouped_tile32(static_cast<uint32_t>(t), static_cast<uint32_t>(tiles_m), static_cast<uint32_t>(tiles_n),
                          static_cast<uint32_t>(group_m));
  return grouped_tile(t, tiles_m, tiles_n, group_m);
}

// Logical id of hardware workgroup `w` in a grid of `grid` workgroups.  The
// renumbering is a bijection on [0, grid) when grid % kNumXcd == 0, and the
// identity otherwise.
GT_HD inline int64_t xcd_logical_id(int64_t w, int64_t grid) {
  if (grid % kNumXcd != 0) return w;
  return (w % kNumXcd) * (grid / kNumXcd) + w / kNumXcd;
}

}  // namespace gt
