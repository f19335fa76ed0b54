// Ragged tile mapping shared by the grouped GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct Tile {
  int g;
  int64_t row0;
  int M;   // valid rows in this tile (0: block has no work)
  int nt;  // N-tile index
};

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin by id
constexpr int kCus = 256; // MI355X compute units

// Maps blockIdx.x to a (group, row tile, N tile).  The tile list runs over the
// groups in order; inside a group it is row-tile major (consecutive tiles share
// A rows) or, with n_major, N-tile major (consecutive tiles share one weight
// tile: for groups whose weights outweigh their rows).  Each XCD takes one
// contiguous band of the list, keeping a band's operands in that XCD's L2.
// Wave 0 builds the per-group row-tile prefix from the device-side offsets;
// the result goes through LDS.
template <int BM>
__device__ __forceinline__ Tile find_tile(const int32_t* __restrict__ goff, int G, int64_t dense_M, int64_t max_rows,
                          int n_tiles, int* s_info, bool n_major = false) {
  Tile tl;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int total_m, incl = 0, local = 0, g0 = 0, gpl = 1;
    int gs[4], gm[4];  // start and rows of this lane's groups, kept for the owner search
    if (goff == nullptr) {
      total_m = (int)((dense_M + BM - 1) / BM);
    } else {
      gpl = (G + 63) / 64;  // groups per lane (<= 4: at most 256 groups)
      g0 = lane * gpl;
      // every offset load goes out before any is used (groups clamped to
      // G - 1, dropped afterwards): under the per-group branch each load got
      // a wait of its own
      int lo[4], hi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = g0 + q < G ? g0 + q : G - 1;
        lo[q] = goff[g];
        hi[q] = goff[g + 1];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool own = q < gpl && g0 + q < G;
        gs[q] = own ? lo[q] : 0;
        gm[q] = own ? hi[q] - lo[q] : 0;
        local += (gm[q] + BM - 1) / BM;
      }
      incl = local;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_up(incl, m, 64);
        if (lane >= m) incl += o;
      }
      total_m = __shfl(incl, 63, 64);
    }
    const int64_t total = (int64_t)total_m * n_tiles;
    const int64_t band = (total + kXcds - 1) / kXcds;
    const int64_t b = blockIdx.x;
    const int64_t i = b / kXcds;
    const int64_t L = (b % kXcds) * band + i;
    const bool work = i < band && L < total;
    const int mt = work ? (int)(L / n_tiles) : -1;
    if (lane == 0) {
      s_info[0] = -1;
      s_info[3] = work ? (int)(L % n_tiles) : 0;
      if (work && goff == nullptr) {
        s_info[0] = 0;
        s_info[1] = mt * BM;
        const int64_t rem = dense_M - (int64_t)mt * BM;
        s_info[2] = rem < BM ? (int)rem : BM;
      }
    }
    if (work && goff != nullptr) {
      // group g owns list entries [pre n_tiles, (pre + tiles) n_tiles) in
      // either order, which is also the row-tile range [pre, pre + tiles)
      int pre = incl - local;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = g0 + q;
        const int Mg = gm[q];
        const int tiles = (Mg + BM - 1) / BM;  // 0 past this lane's groups
        if (mt >= pre && mt < pre + tiles) {
          int r = mt - pre;
          if (n_major) {
            const int64_t l = L - (int64_t)pre * n_tiles;
            r = (int)(l % tiles);
            s_info[3] = (int)(l / tiles);
          }
          s_info[0] = g;
          s_info[1] = gs[q] + r * BM;
          s_info[2] = (Mg - r * BM) < BM ? (Mg - r * BM) : BM;
        }
        pre += tiles;
      }
    }
  }
  __syncthreads();
  tl.g = s_info[0];
  tl.row0 = s_info[1];
  tl.M = tl.g < 0 ? 0 : s_info[2];
  tl.nt = s_info[3];
  if (tl.row0 >= max_rows) tl.M = 0;
  else if (tl.row0 + tl.M > max_rows) tl.M = (int)(max_rows - tl.row0);
  return tl;
}

// Blocks to launch for a tile bound: every XCD band must be coverable.
static inline int64_t grid_blocks(int64_t bound_m_tiles, int n_tiles) {
  const int64_t bound = bound_m_tiles * n_tiles;
  return (bound + 2 * kXcds - 1) / kXcds * kXcds;
}

}  // namespace moe
