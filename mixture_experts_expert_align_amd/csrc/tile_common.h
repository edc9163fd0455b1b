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

// Transposed operand slots (row = contraction index, 256 outputs of 2 bytes
// a row): logical 16-byte chunk c of row r sits at physical chunk
// wt_phys(r, c) = c ^ 2 (r & 3) ^ 8 bit1(c).  The first term puts the 4 rows
// one transposing read touches (r .. r+3 from a multiple of 4) on distinct
// chunks, so a group of 16 lanes covers 32 banks once; the second puts the
// lane groups 0-15 and 16-31, whose outputs differ in bit 1 of the chunk, on
// opposite halves of the 64 banks (with the first term alone all four groups
// met in one half: counters showed more bank-conflict cycles than LDS-active
// ones).  It is a bijection on the chunks of a row; wt_logical inverts it.
__device__ __forceinline__ int wt_phys(int r, int c) { return c ^ ((r & 3) << 1) ^ (((c >> 1) & 1) << 3); }
__device__ __forceinline__ int wt_logical(int r, int p) {
  const int u = p ^ ((r & 3) << 1);
  return u ^ (((u >> 1) & 1) << 3);
}
__device__ __forceinline__ int wt_off(int r, int col) { return r * 256 + (wt_phys(r, col >> 3) << 3) + (col & 7); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// MFMA row-operand fragment (32 outputs x 8 consecutive contraction values
// per lane) of a transposed weight slot: outputs j0 .. j0+31, contraction
// c0 + 8 (lane / 32) .. +7.  ds_read_b64_tr_b16 (gfx950): in each group of
// 16 lanes, destination lane 4a+b receives element b of the 8 bytes read by
// lanes a, a+4, a+8 and a+12; source lane L points at row c + L / 4, outputs
// j + 4 (L % 4) .. +3, so destination lane D holds output j + D at rows
// c .. c+3.  Two reads give 8 rows.
__device__ __forceinline__ bf16x8 wt_frag(const uint16_t* slot, int j0, int c0, int lane) {
  const int gq = lane >> 4, L = lane & 15;
  const int j = j0 + 16 * (gq & 1) + 4 * (L & 3);
  const int c = c0 + 8 * (gq >> 1) + (L >> 2);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(slot + wt_off(c, j)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(slot + wt_off(c + 4, j)));
  const v4i16 v8[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v8);
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
