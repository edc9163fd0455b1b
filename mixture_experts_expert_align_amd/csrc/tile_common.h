// Tile bookkeeping shared by the LDS-tiled grouped GEMMs (bf16 and MXFP8):
// the XOR-swizzled LDS row layout, and the mapping of a workgroup to its
// (expert, weight tile, route tile) in an XCD-aware order.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace tile {

constexpr int NXCD = 8;
constexpr int kXcdChunk = 32;
enum Order { kWeightMajor = 0, kRouteMajor = 1 };

template <int BK>
__device__ __forceinline__ int lds_off(int row, int c) {
  constexpr int CH = BK / 8;  // 16-byte chunks per row
  // chunk c of row r lives at chunk c ^ f(r); f spreads 8 consecutive rows
  // over the 128-byte bank period for the reads of 8 lanes
  constexpr int RPW = 256 / (BK * 2) > 0 ? 256 / (BK * 2) : 1;   // rows per 256-byte bank window
  const int x = (row / RPW) & (CH - 1);
  return row * BK + ((c ^ x) << 3);
}

// Workgroup -> (expert, first weight row, first route row).
struct TileCoord {
  int expert, col0;
  int64_t row0;   // contiguous: sorted position; batched: slab row e*max_tokens + r0;
                  // rows: first row of the tile
  int mlo;        // route rows [mlo, nvalid) of the tile exist (the rest are padding)
  int nvalid;
};

__host__ __device__ inline int64_t padded_blocks(int64_t nlog) {
  const int64_t unit = (int64_t)NXCD * kXcdChunk;
  return (nlog + unit - 1) / unit * unit;
}

// Block b (blockIdx.x, or a virtual block of a grid-stride loop whose grid
// size is a multiple of 8, so that b % 8 is still the block's XCD).
template <int BM, int BN, int ORDER>
__device__ __forceinline__ bool tile_coord(const GemmArgs& g, int ncol, int64_t nlog, TileCoord& tc,
                                           int64_t b = -1) {
  const RowMap& rm = g.rows;
  // block b runs on XCD b % 8 as that XCD's (b / 8)-th block
  if (b < 0) b = blockIdx.x;
  const int64_t k = b / NXCD;
  int64_t L = b;
  if (rm.layout == 0) {
    const int64_t total = (int64_t)rm.num_post[0] / BM * ncol;
    if (ORDER == kWeightMajor) {
      // full rounds of 8 chunks; the tiles left after them are split evenly
      // over the 8 XCDs so that none idles through the last round
      const int64_t full = total / (NXCD * kXcdChunk);
      const int64_t x = b % NXCD;
      if (k < full * kXcdChunk) {
        L = ((k / kXcdChunk) * NXCD + x) * kXcdChunk + (k % kXcdChunk);
      } else {
        const int64_t c2 = (total - full * NXCD * kXcdChunk + NXCD - 1) / NXCD;
        const int64_t kk = k - full * kXcdChunk;
        if (kk >= c2) return false;
        L = full * NXCD * kXcdChunk + x * c2 + kk;
      }
    }
    if (L >= total) return false;
    // expert e owns logical tiles [offsets[e]/BM*ncol, offsets[e+1]/BM*ncol)
    int lo = 0, hi = g.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)rm.offsets[mid] / BM * ncol <= L) lo = mid; else hi = mid - 1;
    }
    const int64_t t0 = rm.offsets[lo] / BM;
    const int64_t ne = rm.offsets[lo + 1] / BM - t0;
    const int64_t local = L - t0 * ncol;
    tc.expert = lo;
    if (ORDER == kRouteMajor) {
      tc.col0 = (int)(local % ncol) * BN;
      tc.row0 = (t0 + local / ncol) * BM;
    } else {
      tc.col0 = (int)(local / ne) * BN;
      tc.row0 = (t0 + local % ne) * BM;
    }
    // the expert's run holds counts[lo] routes, then padding to a tile
    tc.mlo = 0;
    tc.nvalid = (int)max<int64_t>(0, min<int64_t>(BM, rm.counts[lo] - (tc.row0 - rm.offsets[lo])));
    return true;
  }
  if (L >= nlog) return false;
  const int tpe = (rm.max_tokens + BM - 1) / BM;
  const int e = (int)(L / ((int64_t)ncol * tpe));
  const int local = (int)(L - (int64_t)e * ncol * tpe);
  const int r0 = (ORDER == kRouteMajor ? local / ncol : local % tpe) * BM;
  const int cnt = min(rm.counts[e], rm.max_tokens);
  if (r0 >= cnt) return false;
  tc.expert = e;
  tc.col0 = (ORDER == kRouteMajor ? local % ncol : local / tpe) * BN;
  tc.row0 = (int64_t)e * rm.max_tokens + r0;
  tc.mlo = 0;
  tc.nvalid = min(BM, cnt - r0);
  return true;
}

}  // namespace tile
}  // namespace moe
