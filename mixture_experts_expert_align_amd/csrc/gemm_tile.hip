// LDS-tiled grouped GEMM (bf16 in, fp32 accumulate) for the two matmuls of
// the expert computation ("Fused MoE Modular Kernel", apply(): matmul with
// W1, act + mul, matmul with W2, unpermute) when experts hold many rows.
//
// A workgroup computes BN weight rows x BM route rows of one expert, stepping
// through the contraction in BK-wide slices staged in LDS (double buffered;
// 16-byte chunks XOR-swizzled so the 32-row fragment reads of an MFMA hit
// distinct banks).  The waves form a WN x WM grid; each owns (BN/WN) weight
// rows x (BM/WM) routes as tiles of v_mfma_f32_32x32x16_bf16 with the weight
// rows in the MFMA row operand, so a lane's accumulators hold 4 consecutive
// output features of one route and the epilogue writes 8-byte runs.  Inside
// a slice the fragments of the next 16-wide k step are read from LDS while
// the MFMAs of the current one run.
//
// W1 (kGateUp): the BN weight rows are BN/2 gate rows and the BN/2 matching up
// rows; each wave holds gate and up values of the same (feature, route) in
// registers and forms silu(gate) * up before the only store (bf16 z, row =
// sorted position).  Route rows are gathered through the route list (token =
// flat slot / topk) while loading; padding routes load zeros.
// W2 (kDown): the epilogue writes each real route's row to its (token, slot)
// row of y (the per-(token, slot) buffer of the Cake MegaMoE EP16 page,
// section 3); padding rows are dropped.
//
// Tile order (expert-major in both):
//  kWeightMajor (contiguous format): inside an expert, weight tile major and
//    route tile minor, so the route tiles of one expert reuse a weight tile
//    from L2 one after another.  The hardware deals workgroups to the 8 XCDs
//    round robin; the logical order is handed to the XCDs in chunks of
//    kXcdChunk consecutive tiles, round robin, so each XCD's L2 sees runs of
//    neighbouring tiles while a skewed expert load still spreads over all
//    XCDs.
//  kRouteMajor (batched format, many small experts, weight-bandwidth bound):
//    inside an expert, route tile major and weight tile minor, in plain block
//    order: workgroups in flight read different weight tiles of one expert
//    while sharing its route tile, and when the weight-tile count is a
//    multiple of 8 the route tiles of one weight tile land on the same XCD.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace tile {

constexpr int NXCD = 8;
constexpr int kXcdChunk = 8;
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
  int64_t row0;   // contiguous: sorted position; batched: slab row e*max_tokens + r0
  int nvalid;     // route rows of the tile that exist (the rest are padding)
};

__host__ __device__ inline int64_t padded_blocks(int64_t nlog) {
  const int64_t unit = (int64_t)NXCD * kXcdChunk;
  return (nlog + unit - 1) / unit * unit;
}

template <int BM, int BN, int ORDER>
__device__ __forceinline__ bool tile_coord(const GemmArgs& g, int ncol, int64_t nlog, TileCoord& tc) {
  const RowMap& rm = g.rows;
  // block b runs on XCD b % 8 as that XCD's (b / 8)-th block
  const int64_t b = blockIdx.x;
  const int64_t k = b / NXCD;
  const int64_t L = ORDER == kRouteMajor ? b : ((k / kXcdChunk) * NXCD + (b % NXCD)) * kXcdChunk + (k % kXcdChunk);
  if (L >= nlog) return false;
  if (rm.layout == 0) {
    const int64_t total = (int64_t)rm.num_post[0] / BM * ncol;
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
    tc.nvalid = (int)max<int64_t>(0, min<int64_t>(BM, rm.counts[lo] - (tc.row0 - rm.offsets[lo])));
    return true;
  }
  const int tpe = (rm.max_tokens + BM - 1) / BM;
  const int e = (int)(L / ((int64_t)ncol * tpe));
  const int local = (int)(L - (int64_t)e * ncol * tpe);
  const int r0 = (ORDER == kRouteMajor ? local / ncol : local % tpe) * BM;
  const int cnt = min(rm.counts[e], rm.max_tokens);
  if (r0 >= cnt) return false;
  tc.expert = e;
  tc.col0 = (ORDER == kRouteMajor ? local % ncol : local / tpe) * BN;
  tc.row0 = (int64_t)e * rm.max_tokens + r0;
  tc.nvalid = min(BM, cnt - r0);
  return true;
}

template <int EPI, int BM, int BN, int BK, int WN, int WM, int OCC, int ORDER>
__global__ void __launch_bounds__(64 * WN * WM, OCC) gemm_tile_bf16_kernel(GemmArgs g, int ncol,
                                                                           int64_t nlog) {
  constexpr int NT = 64 * WN * WM;
  constexpr int CH = BK / 8;
  constexpr int TW = BN / WN / 32;   // weight tiles per wave
  constexpr int TX = BM / WM / 32;   // route tiles per wave
  static_assert(EPI != kEpiGateUp || TW % 2 == 0, "gate/up pairs need an even tile count");
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sX[2][BM * BK];

  TileCoord tc;
  if (!tile_coord<BM, BN, ORDER>(g, ncol, nlog, tc)) return;
  const RowMap& rm = g.rows;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave / WM;
  const int wm = wave % WM;
  const int K = g.kdim;

  // ---- global -> register staging: 16-byte chunk c = tid + NT*i -> row c/CH, chunk c%CH.
  // Buffer loads with per-lane byte offsets and the slice's byte offset in
  // the scalar operand; a padding route gets an offset past the buffer, which
  // the range check turns into zeros.
  constexpr int WCH = BN * CH / NT;   // weight chunks per thread
  constexpr int XCH = BM * CH / NT;   // route chunks per thread
  static_assert(WCH * NT == BN * CH && XCH * NT == BM * CH, "tile / thread mismatch");
  const int kc = tid % CH;
  const uint16_t* wexp = static_cast<const uint16_t*>(g.w) + (int64_t)tc.expert * g.w_expert_stride;
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride * 2);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
  uint32_t ow[WCH], ox[XCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int n = (tid + NT * i) / CH;
    int wrow;
    if (EPI == kEpiGateUp) {
      const int f = tc.col0 / 2 + (n % (BN / 2));
      const bool up = n >= BN / 2;
      wrow = g.w1_order == 0 ? (up ? g.I + f : f) : (32 * (f >> 4) + (f & 15) + (up ? 16 : 0));
    } else {
      wrow = tc.col0 + n;
    }
    ow[i] = (uint32_t)((wrow * K + kc * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int m = (tid + NT * i) / CH;
    int64_t row = -1;
    if (rm.layout == 0) {
      if (EPI == kEpiGateUp) {
        const int sid = rm.sorted_ids[tc.row0 + m];
        if (sid != rm.sentinel) row = sid / rm.topk;
      } else {
        row = tc.row0 + m;
      }
    } else if (m < tc.nvalid) {
      row = tc.row0 + m;
    }
    ox[i] = row >= 0 ? (uint32_t)((row * g.act_ld + kc * 8) * 2) : 0x80000000u;
  }

  // Two register sets: slice t lives in set t % 2 from its load to its LDS
  // store two slices later, so each load has two slices of MFMA work to
  // arrive.
  i32x4 rw[2][WCH], rx[2][XCH];
  const int nk = K / BK;
  auto gload = [&](int set, int kt) {
    const int kb = min(kt, nk - 1) * BK * 2;   // past the end: repeat the last slice (unused)
#pragma unroll
    for (int i = 0; i < WCH; ++i) rw[set][i] = __builtin_amdgcn_raw_buffer_load_b128(wr, ow[i], kb, 0);
#pragma unroll
    for (int i = 0; i < XCH; ++i) rx[set][i] = __builtin_amdgcn_raw_buffer_load_b128(ar, ox[i], kb, 0);
  };
  auto sstore = [&](int buf, int set) {
#pragma unroll
    for (int i = 0; i < WCH; ++i)
      *reinterpret_cast<i32x4*>(&sW[buf][lds_off<BK>((tid + NT * i) / CH, kc)]) = rw[set][i];
#pragma unroll
    for (int i = 0; i < XCH; ++i)
      *reinterpret_cast<i32x4*>(&sX[buf][lds_off<BK>((tid + NT * i) / CH, kc)]) = rx[set][i];
  };

  // ---- this wave's MFMA tiles.  kGateUp: weight tiles [0, TW/2) are gate
  // rows of the wave's features, tiles [TW/2, TW) the matching up rows.
  int wrow_l[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (EPI == kEpiGateUp) {
      constexpr int FW = BN / 2 / WN;   // features per wave
      wrow_l[i] = (i < TW / 2 ? 0 : BN / 2) + wn * FW + 32 * (i % (TW / 2)) + (lane & 31);
    } else {
      wrow_l[i] = wn * (BN / WN) + 32 * i + (lane & 31);
    }
  }
  const int xrow_l = wm * (BM / WM) + (lane & 31);
  // a wave whose route rows all lie past the tile's valid rows holds only
  // padding: it skips its fragment reads and MFMAs (its accumulators stay 0,
  // what zero-filled padding rows would give) but still stages and meets
  // the barriers; a wave-uniform branch
  const bool wlive = __builtin_amdgcn_readfirstlane(wm) * (BM / WM) < tc.nvalid;

  f32x16 acc[TW][TX];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TX; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  bf16x8 fw[2][TW], fx[2][TX];
  auto fload = [&](int fb, int buf, int s) {
    const int c = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TW; ++i)
      fw[fb][i] = as_bf16x8(*reinterpret_cast<const i32x4*>(&sW[buf][lds_off<BK>(wrow_l[i], c)]));
#pragma unroll
    for (int j = 0; j < TX; ++j)
      fx[fb][j] = as_bf16x8(*reinterpret_cast<const i32x4*>(&sX[buf][lds_off<BK>(xrow_l + 32 * j, c)]));
  };
  auto compute = [&](int buf) {
    if (!wlive) return;
    fload(0, buf, 0);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) fload((s + 1) & 1, buf, s + 1);
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TX; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s & 1][i], fx[s & 1][j], acc[i][j], 0, 0, 0);
    }
  };
  // slice kt (LDS buffer and register set kt % 2, literals at each call):
  // multiply it, store slice kt+1 (register set (kt+1) % 2) to the other
  // buffer, refill that set with slice kt+3
  auto step = [&](int p, int kt) {
    compute(p);
    __builtin_amdgcn_sched_barrier(0);
    sstore(p ^ 1, p ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    gload(p ^ 1, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };

  gload(0, 0);
  gload(1, 1);
  sstore(0, 0);
  gload(0, 2);
  lds_barrier();
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    step(0, kt);
    step(1, kt + 1);
  }
  if (kt < nk) compute(0);

  // ---- epilogue.  acc[i][j][r]: weight row (tile i) 8*(r/4) + 4*(lane/32) + r%4,
  // route wm*(BM/WM) + 32*j + lane%32.  Registers 4h..4h+3 are 4 consecutive rows.
  uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
  for (int j = 0; j < TX; ++j) {
    const int m = wm * (BM / WM) + 32 * j + (lane & 31);
    if (rm.layout != 0 && m >= tc.nvalid) continue;   // contiguous: padding rows of z are written (zeros)
    int64_t orow;
    if (EPI == kEpiGateUp || rm.layout != 0) {
      orow = tc.row0 + m;
    } else {
      const int sid = rm.sorted_ids[tc.row0 + m];
      if (sid == rm.sentinel) continue;
      orow = sid;
    }
    uint16_t* o = out + orow * g.out_ld;
    if (EPI == kEpiGateUp) {
      constexpr int FW = BN / 2 / WN;
#pragma unroll
      for (int i = 0; i < TW / 2; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = f32_to_bf16_rne(silu_f32(acc[i][j][4 * h + r]) * acc[i + TW / 2][j][4 * h + r]);
          const int f = tc.col0 / 2 + wn * FW + 32 * i + 8 * h + 4 * (lane >> 5);
          *reinterpret_cast<uint2*>(o + f) = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
    } else {
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = f32_to_bf16_rne(acc[i][j][4 * h + r]);
          const int n = tc.col0 + wn * (BN / WN) + 32 * i + 8 * h + 4 * (lane >> 5);
          *reinterpret_cast<uint2*>(o + n) = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
    }
  }
}

// Grid and launch of one tile configuration.
template <int EPI, int BM, int BN, int BK, int WN, int WM, int OCC, int ORDER>
hipError_t launch(const GemmArgs& g, hipStream_t s) {
  const int ncol = EPI == kEpiGateUp ? g.nfeat / (BN / 2) : g.nfeat / BN;
  int64_t nrow;
  if (g.rows.layout == 0) nrow = g.max_tiles * 128 / BM;   // plan tiles are 128 routes
  else nrow = (int64_t)g.E * ((g.rows.max_tokens + BM - 1) / BM);
  const int64_t nlog = nrow * ncol;
  dim3 grid((unsigned)(ORDER == kRouteMajor ? nlog : padded_blocks(nlog)));
  hipLaunchKernelGGL((gemm_tile_bf16_kernel<EPI, BM, BN, BK, WN, WM, OCC, ORDER>), grid,
                     dim3(64 * WN * WM), 0, s, g, ncol, nlog);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  // contiguous: 128 routes x 256 weight rows, 8 waves of 64x64, two
  // workgroups per CU; batched: 128 x 128, 4 waves of 64x64, route-major
  if (g.rows.layout == 0) return launch<EPI, 128, 256, 32, 4, 2, 2, kWeightMajor>(g, s);
  return launch<EPI, 128, 128, 64, 2, 2, 1, kRouteMajor>(g, s);
}

}  // namespace tile

// Plan tiles are 128 routes (block_m).
hipError_t launch_gemm_tile_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.epi == kEpiGateUp) return tile::launch_layout<kEpiGateUp>(g, s);
  return tile::launch_layout<kEpiDown>(g, s);
}

}  // namespace moe
