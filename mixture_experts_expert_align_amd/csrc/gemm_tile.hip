// LDS-tiled grouped GEMM (bf16 in, fp32 accumulate) for the two matmuls of
// the expert computation ("Fused MoE Modular Kernel", apply(): matmul with
// W1, act + mul, matmul with W2, unpermute) when experts hold many rows.
//
// A workgroup computes BN weight rows x BM route rows of one expert, stepping
// through the contraction in BK-wide slices.  The slices reach LDS by buffer
// loads that write LDS themselves (no registers, no LDS store instructions).
// In LDS the 16-byte chunks of a row are XOR-swizzled so the 32-row fragment
// reads of an MFMA hit distinct banks; one such load writes the 64 lanes' 16
// bytes to 1 KB of LDS at a wave-uniform address, lane i at byte 16 i, so
// each lane fetches the chunk that the swizzle places at its position.  The
// waves form a WN x WM grid; each owns (BN/WN) weight rows x (BM/WM) routes
// as tiles of v_mfma_f32_32x32x16_bf16 with the weight rows in the MFMA row
// operand, so a lane's accumulators hold 4 consecutive output features of
// one route and the epilogue writes 8-byte runs.
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
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_common.h"

namespace moe {
namespace tile {

// Epilogue.  acc[i][j][r]: weight row (tile i) 8*(r/4) + 4*(lane/32) + r%4,
// route wm*(BM/WM) + 32*j + lane%32; registers 4h..4h+3 are 4 consecutive
// rows, i.e. 4 consecutive output features of one route.  The tile's bf16
// outputs are first laid out row by row in LDS (the staging ring is free by
// then), 16-byte chunks XOR-swizzled by row so that both the writes from the
// accumulators (one chunk of 32 rows per instruction) and the row reads
// spread over the banks; then each row's segment of the output goes out in
// 16-byte stores, whole segments per group of lanes, instead of 8-byte
// pieces of 32 rows per store instruction.
// ROUTES: the launch may take the contiguous format, whose W2 rows go to the
// routes' (token, slot) rows (false for the rows layout of training).
template <int EPI, int BM, int BN, int WN, int WM, int NT, int TW, int TX, bool ROUTES>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const TileCoord& tc,
                                              const f32x16 (&acc)[TW][TX], int wn, int wm, int lane,
                                              uint16_t* stage) {
  constexpr int OUTF = EPI == kEpiGateUp ? BN / 2 : BN;   // output features per route row
  constexpr int NCH = OUTF / 8;                            // 16-byte chunks per row
  static_assert(NCH <= 64 && (NCH & (NCH - 1)) == 0, "row segment: a power of two of at most 64 chunks");
  const RowMap& rm = g.rows;
  // element offset of chunk c of row m
  auto chunk_at = [](int m, int c) { return (m * NCH + (c ^ (m & (NCH - 1)))) * 8; };
  // contiguous W2: the destination rows of the rows this thread writes out,
  // requested before the staging so their latency hides behind it
  constexpr int RPP = NT / NCH;   // rows per pass of the workgroup
  constexpr int NP = BM / RPP;    // passes
  static_assert(BM % RPP == 0, "whole passes");
  const bool lookup = ROUTES && EPI != kEpiGateUp && rm.layout == 0;
  int sid[NP];
  if (lookup) {
#pragma unroll
    for (int p = 0; p < NP; ++p) sid[p] = rm.sorted_ids[tc.row0 + threadIdx.x / NCH + RPP * p];
  }
#pragma unroll
  for (int j = 0; j < TX; ++j) {
    const int m = wm * (BM / WM) + 32 * j + (lane & 31);
    const bool pad = m >= tc.nvalid;   // contiguous W1: padding rows of z are zeros
    if (EPI == kEpiGateUp) {
      constexpr int FW = BN / 2 / WN;
#pragma unroll
      for (int i = 0; i < TW / 2; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = pad ? 0u : f32_to_bf16_rne(silu_f32(acc[i][j][4 * h + r]) * acc[i + TW / 2][j][4 * h + r]);
          const int f = wn * FW + 32 * i + 8 * h + 4 * (lane >> 5);
          *reinterpret_cast<uint2*>(stage + chunk_at(m, f / 8) + (f & 7)) =
              make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
    } else {
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = f32_to_bf16_rne(acc[i][j][4 * h + r]);
          const int f = wn * (BN / WN) + 32 * i + 8 * h + 4 * (lane >> 5);
          *reinterpret_cast<uint2*>(stage + chunk_at(m, f / 8) + (f & 7)) =
              make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
    }
  }
  lds_barrier();
  uint16_t* out = static_cast<uint16_t*>(g.out);
  const int col = EPI == kEpiGateUp ? tc.col0 / 2 : tc.col0;
  const int c = threadIdx.x % NCH;
  auto put = [&](int m, int64_t orow) {
    *reinterpret_cast<i32x4*>(out + orow * g.out_ld + col + 8 * c) =
        *reinterpret_cast<const i32x4*>(stage + chunk_at(m, c));
  };
  if (lookup) {
#pragma unroll
    for (int p = 0; p < NP; ++p)   // W2: each route to its (token, slot) row, padding rows dropped
      if (sid[p] != rm.sentinel) put(threadIdx.x / NCH + RPP * p, sid[p]);
  } else {
    for (int m = threadIdx.x / NCH; m < BM; m += RPP) {
      if (rm.layout != 0 && (m < tc.mlo || m >= tc.nvalid)) continue;   // batched / rows: only the tile's own rows
      put(m, tc.row0 + m);
    }
  }
}

// Per-lane byte offsets of the slice loads.  Block b of a slot (b = wave +
// NW * i) holds rows RPB*b .. RPB*b + RPB-1 of its region; lane l lands on
// row RPB*b + l/CH, physical chunk l%CH, which holds logical chunk
// (l%CH) ^ x(row).  W1 tiles hold BN/2 gate rows then the BN/2 matching up
// rows; route rows are gathered through the route list (token = flat slot /
// topk) for W1, read in position order for W2, or taken from the expert's
// slab for the batched format; a padding route (or a batched row past its
// expert's count) gets an offset past the buffer, which loads zeros.
template <int EPI, int BM, int BN, int BK, int NW, bool WT>
__device__ __forceinline__ void load_offsets(const GemmArgs& g, const TileCoord& tc, int wave, int lane,
                                             uint32_t (&ow)[BN / (512 / BK) / NW],
                                             uint32_t (&ox)[BM / (512 / BK) / NW]) {
  constexpr int CH = BK / 8;
  constexpr int RPB = 64 / CH;
  constexpr int RPW = 256 / (BK * 2) > 0 ? 256 / (BK * 2) : 1;
  constexpr int LW = BN / RPB / NW;
  constexpr int LX = BM / RPB / NW;
  const RowMap& rm = g.rows;
  const int K = g.kdim;
  if (WT) {
    // weights stored with the output index contiguous: the slot holds BK
    // contraction rows of BN outputs; block b = rows 2b, 2b+1 (BN = 256:
    // 512 bytes a row), lane l -> row 2b + l / 32, physical chunk l % 32,
    // holding logical chunk wt_logical(row, l % 32); the slice's first row
    // comes in through the instruction offset
    static_assert(!WT || BN * 2 == 512, "transposed weight rows of 512 bytes");
#pragma unroll
    for (int i = 0; i < LW; ++i) {
      const int r = 2 * (wave + NW * i) + lane / 32;
      const int c = wt_logical(r, lane % 32);
      ow[i] = (uint32_t)(((int64_t)r * g.nfeat + tc.col0 + 8 * c) * 2);
    }
  } else
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int n = (wave + NW * i) * RPB + lane / CH;
    const int c = (lane % CH) ^ ((n / RPW) & (CH - 1));
    int wrow;
    if (EPI == kEpiGateUp) {
      const int f = tc.col0 / 2 + (n % (BN / 2));
      wrow = w1_row(f, n >= BN / 2, g.I, g.w1_order);
    } else {
      wrow = tc.col0 + n;
    }
    ow[i] = (uint32_t)((wrow * K + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < LX; ++i) {
    const int m = (wave + NW * i) * RPB + lane / CH;
    const int c = (lane % CH) ^ ((m / RPW) & (CH - 1));
    int64_t row = -1;
    if (rm.layout != 0) {
      if (m >= tc.mlo && m < tc.nvalid) row = tc.row0 + m;   // rows outside the tile's own are never read
    } else if (EPI == kEpiGateUp) {
      const int sid = rm.sorted_ids[tc.row0 + m];
      if (sid != rm.sentinel) row = sid / rm.topk;
    } else {
      row = tc.row0 + m;
    }
    ox[i] = row >= 0 ? (uint32_t)((row * g.act_ld + c * 8) * 2) : 0x80000000u;
  }
}

// LDS rows of a wave's fragments: weight row of tile i (W1: gate tiles, then
// the matching up tiles) and the first route row of its route tiles.
template <int EPI, int BM, int BN, int WN, int WM>
__device__ __forceinline__ void frag_rows(int wn, int wm, int lane, int (&wrow_l)[BN / WN / 32], int& xrow_l) {
  constexpr int TW = BN / WN / 32;
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (EPI == kEpiGateUp) {
      constexpr int FW = BN / 2 / WN;
      wrow_l[i] = (i < TW / 2 ? 0 : BN / 2) + wn * FW + 32 * (i % (TW / 2)) + (lane & 31);
    } else {
      wrow_l[i] = wn * (BN / WN) + 32 * i + (lane & 31);
    }
  }
  xrow_l = wm * (BM / WM) + (lane & 31);
}

// The kernel.  Its ring of slice buffers is split by operand and the slice
// hand-off sits in the last k step (prefill: 256 routes x 256 weight rows,
// K = 4096 for W1; batched: 128 x 128):
//  * Weights are requested two slices ahead (3 slots), routes one ahead
//    (2 slots): for 256 x 256 tiles 3 x 32 KB + 2 x 32 KB = 160 KB, all of
//    the LDS; for 128 x 128 tiles 80 KB, two workgroups per CU.  Weight rows
//    come from HBM (each weight tile serves only the few route tiles of its
//    expert) and have the longer way; route rows mostly hit L2.
//  * Slice kt's last k step begins with the wait for slice kt+1 and the
//    barrier; right after it the freed slots are refilled (routes of slice
//    kt+2, weights of slice kt+3) and the first fragments of slice kt+1 are
//    read while the MFMAs of that last step run, so the MFMA pipe has work
//    across the barrier instead of waiting for the first reads of a slice.
//  * Fragment reads and MFMAs of a step are interleaved one to one
//    (scheduling groups), so the next step's reads overlap this step's
//    MFMAs instead of being issued after them into the same registers.
//  * Waits count only weight loads as younger than the loads they wait for:
//    a wave skips its route blocks made only of padding, so its route loads
//    per slice are not a fixed number.
//  * A wave whose route rows are all padding runs the same loop without
//    fragment reads and MFMAs (its own copy of the loop, so the live copy
//    has no branches around its MFMAs).
template <int BM, int BN, int BK>
struct SplitRing {
  static constexpr int WS = 3, RS = 2;              // weight / route slots
  static constexpr int WSLOT = BN * BK, RSLOT = BM * BK;
  static constexpr int Elems = WS * WSLOT + RS * RSLOT;   // uint16 elements of LDS
};

// One tile: BN weight rows from tc.col0 times the route rows [mlo, nvalid)
// of the BM from tc.row0, through the epilogue.  smem: SplitRing::Elems
// elements; the caller meets a barrier before it reuses them.
template <int EPI, int BM, int BN, int BK, int WN, int WM, bool WT = false, bool ROUTES = true>
__device__ __forceinline__ void split_tile(const GemmArgs& g, const TileCoord& tc, uint16_t* smem) {
  constexpr int NW = WN * WM;
  constexpr int CH = BK / 8;
  constexpr int RPB = 64 / CH;
  constexpr int LW = BN / RPB / NW;          // weight loads per wave per slice
  constexpr int LX = BM / RPB / NW;          // route loads per wave per slice
  static_assert(LW * NW * RPB == BN && LX * NW * RPB == BM, "blocks / waves mismatch");
  static_assert(2 * LW < 64, "wait counts");
  using Ring = SplitRing<BM, BN, BK>;
  constexpr int WS = Ring::WS, RS = Ring::RS;
  constexpr int WSLOT = Ring::WSLOT, RSLOT = Ring::RSLOT;
  constexpr int TW = BN / WN / 32;
  constexpr int TX = BM / WM / 32;
  constexpr int NSTEP = BK / 16;
  static_assert(EPI != kEpiGateUp || TW % 2 == 0, "gate/up pairs need an even tile count");
  uint16_t* const wbase = smem;
  uint16_t* const rbase = smem + WS * WSLOT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave / WM;
  const int wm = wave % WM;
  const uint16_t* wexp = static_cast<const uint16_t*>(g.w) + (int64_t)tc.expert * g.w_expert_stride;
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride * 2);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
  uint32_t ow[LW], ox[LX];
  load_offsets<EPI, BM, BN, BK, NW, WT>(g, tc, wave, lane, ow, ox);
  static_assert(!WT || EPI == kEpiDown, "transposed weights: plain outputs");
  // per slice, the weight loads advance BK elements along a row, or BK rows
  const int wstep = WT ? BK * g.nfeat * 2 : BK * 2;
  const int nk = g.kdim / BK;
  // A route block whose rows are all padding is not loaded: its LDS rows keep
  // stale values, which reach only those rows' own outputs (an MFMA output
  // column depends on its route row alone), and the epilogue drops them or
  // writes zeros in their place.
  bool xload[LX];
#pragma unroll
  for (int i = 0; i < LX; ++i)
    xload[i] = __builtin_amdgcn_readfirstlane(
                   (int)((wave + NW * i) * RPB < tc.nvalid && (wave + NW * i + 1) * RPB > tc.mlo)) != 0;
  auto issue_w = [&](int kt) {
    uint16_t* slot = wbase + (kt % WS) * WSLOT;
#pragma unroll
    for (int i = 0; i < LW; ++i) lds_load16(wr, slot + (wave + NW * i) * RPB * BK, ow[i], kt * wstep);
    issue_order();
  };
  auto issue_r = [&](int kt) {
    uint16_t* slot = rbase + (kt % RS) * RSLOT;
#pragma unroll
    for (int i = 0; i < LX; ++i)
      if (xload[i]) lds_load16(ar, slot + (wave + NW * i) * RPB * BK, ox[i], kt * BK * 2);
    issue_order();
  };
  int wrow_l[TW], xrow_l;
  frag_rows<EPI, BM, BN, WN, WM>(wn, wm, lane, wrow_l, xrow_l);
  f32x16 acc[TW][TX];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TX; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  bf16x8 fw[2][TW], fx[2][TX];
  // fragments of k step s of slice kt into buffer fb
  auto fload = [&](int fb, int kt, int s) {
    const uint16_t* ws = wbase + (kt % WS) * WSLOT;
    const uint16_t* rs = rbase + (kt % RS) * RSLOT;
    const int c = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TW; ++i)
      fw[fb][i] = WT ? wt_frag(ws, wn * (BN / WN) + 32 * i, 16 * s, lane)
                     : as_bf16x8(*reinterpret_cast<const i32x4*>(&ws[lds_off<BK>(wrow_l[i], c)]));
#pragma unroll
    for (int j = 0; j < TX; ++j)
      fx[fb][j] = as_bf16x8(*reinterpret_cast<const i32x4*>(&rs[lds_off<BK>(xrow_l + 32 * j, c)]));
  };
  auto mma = [&](int fb) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
      for (int j = 0; j < TX; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[fb][i], fx[fb][j], acc[i][j], 0, 0, 0);
  };
  // one fragment read, one MFMA, and so on; the MFMAs (or reads) past the
  // pairs last
  auto interleave = [&]() {
    constexpr int NDS = (WT ? 2 : 1) * TW + TX;   // LDS reads per k step
    constexpr int NP = NDS < TW * TX ? NDS : TW * TX;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    }
    if (TW * TX > NP) __builtin_amdgcn_sched_group_barrier(0x008, TW * TX - NP, 0);
    if (NDS > NP) __builtin_amdgcn_sched_group_barrier(0x100, NDS - NP, 0);
  };

  // prologue: weights 0, routes 0 and 1, weights 1 and 2; wait for slice 0
  issue_w(0);
  issue_r(0);
  if (nk > 1) { issue_r(1); issue_w(1); }
  if (nk > 2) issue_w(2);
  if (nk > 2) wait_vm<2 * LW>();
  else if (nk > 1) wait_vm<LW>();
  else wait_vm<0>();
  lds_barrier();

  // Slice kt.  MODE 2: slices kt+2 and kt+3 exist (routes of kt+2 and
  // weights of kt+3 are requested); 1: only kt+2; 0: only kt+1; -1: kt is
  // the last slice.  LIVE: the wave computes.
  auto slice = [&](int kt, auto mode, auto live) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool LIVE = decltype(live)::value;
    if (LIVE) {
#pragma unroll
      for (int s = 0; s + 1 < NSTEP; ++s) {
        fload((s + 1) & 1, kt, s + 1);
        mma(s & 1);
        interleave();
      }
    }
    if (MODE >= 0) {
      // slice kt+1 has landed once only the weights of slice kt+2 (issued
      // after its routes) may still be in flight
      if (MODE >= 1) wait_vm<LW>();
      else wait_vm<0>();
      lds_barrier();   // every wave's slice kt+1 is in; nobody reads slice kt's slots any more
      if (MODE >= 1) issue_r(kt + 2);
      if (MODE >= 2) issue_w(kt + 3);
      if (LIVE) {
        fload(0, kt + 1, 0);
        mma((NSTEP - 1) & 1);
        interleave();
      }
    } else if (LIVE) {
      mma((NSTEP - 1) & 1);
    }
  };
  auto run = [&](auto live) {
    if (decltype(live)::value) fload(0, 0, 0);
    int kt = 0;
    for (; kt + 3 < nk; ++kt) slice(kt, std::integral_constant<int, 2>(), live);
    if (kt + 2 < nk) slice(kt++, std::integral_constant<int, 1>(), live);
    if (kt + 1 < nk) slice(kt++, std::integral_constant<int, 0>(), live);
    slice(kt, std::integral_constant<int, -1>(), live);
  };
  // a wave whose route rows all lie outside the tile's valid rows holds only
  // padding: it loads and meets the barriers but computes nothing (its
  // accumulators stay 0, what zero-filled padding rows would give)
  if (wm * (BM / WM) < tc.nvalid && (wm + 1) * (BM / WM) > tc.mlo) run(std::true_type());
  else run(std::false_type());

  wait_vm<0>();
  lds_barrier();
  static_assert(BM * (EPI == kEpiGateUp ? BN / 2 : BN) <= Ring::Elems, "epilogue tile fits the LDS");
  tile_epilogue<EPI, BM, BN, WN, WM, 64 * WN * WM, TW, TX, ROUTES>(g, tc, acc, wn, wm, lane, smem);
}

template <int EPI, int BM, int BN, int BK, int WN, int WM, int OCC, int ORDER>
__global__ void __launch_bounds__(64 * WN * WM, OCC) gemm_tile_split_bf16_kernel(GemmArgs g, int ncol,
                                                                                int64_t nlog) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SplitRing<BM, BN, BK>::Elems];
  TileCoord tc;
  if (!tile_coord<BM, BN, ORDER>(g, ncol, nlog, tc)) return;
  split_tile<EPI, BM, BN, BK, WN, WM, false, ORDER == kWeightMajor>(g, tc, smem);
}

// Training forward (page "Cake deterministic MoE grouped GEMM",
// introduction): y[r] = W[e] x[r] for the rows r of group e, rows grouped by
// expert in x (layout 2: the route rows of a tile are rows of x, and the
// outputs go to the same rows of y).  A logical tile is BM rows of x from r0
// times BN features of y; it runs the contraction once per group its rows
// meet, each time with only that group's rows live (rows of other groups
// load nothing and are not written), so every output element comes from one
// pass with a fixed contraction order.  The (row tile, column tile) grid is
// cut into blocks of kRowBlock row tiles x kColBlock column tiles, one block
// per XCD chunk, row-block major: the 32 tiles an XCD runs together share
// kRowBlock row tiles of x and kColBlock weight tiles in its L2 (x and W
// are each far larger than the Infinity Cache, so an order that streams one
// of them per column or row tile would read it from HBM again each time).
constexpr int kRowBlock = 4, kColBlock = 8;
static_assert(kRowBlock * kColBlock == kXcdChunk, "a block fills one XCD chunk");

// The groups of rows a rows-layout launch multiplies: group e is rows
// [offsets[e], offsets[e+1]) of the R rows of the activation matrix
// (clamped to [0, R]; the groups follow each other).
struct RowGroups {
  const int32_t* offsets;
  int32_t E;
  int64_t R;
  __device__ int64_t clampr(int64_t v) const { return min<int64_t>(max<int64_t>(v, 0), R); }
  __device__ int64_t start(int e) const { return clampr(offsets[e]); }
  __device__ int64_t end(int e) const { return max(clampr(offsets[e + 1]), start(e)); }
  // rows of later groups begin at or after this
  __device__ int64_t next_start(int e) const { return end(e); }
  // the first group with rows past r0
  __device__ int first(int64_t r0) const {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (end(mid) > r0) hi = mid; else lo = mid + 1;
    }
    return lo;
  }
};

template <int EPI, int BM, int BN, int BK, int WN, int WM, int OCC, bool WT>
__global__ void __launch_bounds__(64 * WN * WM, OCC) gemm_tile_rows_kernel(GemmArgs g, RowGroups grp, int64_t nrt,
                                                                          int64_t nct) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[SplitRing<BM, BN, BK>::Elems];
  // block b runs on XCD b % 8 as that XCD's (b / 8)-th block: chunk
  // (k / 32) * 8 + b % 8, tile k % 32 of it
  const int64_t b = blockIdx.x;
  const int64_t k = b / NXCD;
  const int64_t chunk = (k / kXcdChunk) * NXCD + b % NXCD;
  const int t = (int)(k % kXcdChunk);
  const int64_t ncb = (nct + kColBlock - 1) / kColBlock;
  const int64_t rt = (chunk / ncb) * kRowBlock + t / kColBlock;
  const int64_t ct = (chunk % ncb) * kColBlock + t % kColBlock;
  if (rt >= nrt || ct >= nct) return;
  const int64_t r0 = rt * BM, r1 = min<int64_t>(r0 + BM, grp.R);
  int e = grp.first(r0);
  TileCoord tc;
  tc.col0 = (int)ct * BN;
  tc.row0 = r0;
  if (grp.next_start(e) >= r1 || e + 1 >= grp.E) {
    // the common case, one group at most in the tile: one pass, outside the
    // loop (inside it the compiler keeps more values live and spills)
    const int64_t s0 = max(grp.start(e), r0), s1 = min(grp.end(e), r1);
    if (s1 <= s0) return;   // no row of any group
    tc.expert = e;
    tc.mlo = (int)(s0 - r0);
    tc.nvalid = (int)(s1 - r0);
    split_tile<EPI, BM, BN, BK, WN, WM, WT, false>(g, tc, smem);
    return;
  }
  bool first = true;
  for (; e < grp.E; ++e) {
    const int64_t a = grp.start(e), z = grp.end(e);
    if (a >= r1) break;
    const int64_t s0 = max(a, r0), s1 = min(z, r1);
    if (s1 <= s0) continue;
    if (!first) lds_barrier();   // the previous pass's epilogue has read its LDS
    first = false;
    tc.expert = e;
    tc.mlo = (int)(s0 - r0);
    tc.nvalid = (int)(s1 - r0);
    split_tile<EPI, BM, BN, BK, WN, WM, WT, false>(g, tc, smem);
  }
}

// 256 rows x 256 weight rows per tile (W1: 128 features of gate and up)
constexpr int kRowsBM = 256, kRowsBN = 256;

template <int EPI, bool WT>
hipError_t launch_rows(const GemmArgs& g, const RowGroups& grp, hipStream_t s) {
  constexpr int BM = kRowsBM, BN = kRowsBN;
  const int fpt = EPI == kEpiGateUp ? BN / 2 : BN;   // output features per tile
  if (g.rows.layout != 2 || g.nfeat % fpt || g.kdim % 64) return hipErrorInvalidValue;
  if (grp.R <= 0) return hipSuccess;
  const int64_t nrt = (grp.R + BM - 1) / BM, nct = g.nfeat / fpt;
  const int64_t nchunk = (nrt + kRowBlock - 1) / kRowBlock * ((nct + kColBlock - 1) / kColBlock);
  const int64_t grid = (nchunk + NXCD - 1) / NXCD * NXCD * kXcdChunk;
  hipLaunchKernelGGL((gemm_tile_rows_kernel<EPI, BM, BN, 64, 4, 4, 4, WT>), dim3((unsigned)grid), dim3(1024), 0, s,
                     g, grp, nrt, nct);
  return hipGetLastError();
}

template <int EPI, int BM, int BN, int BK, int WN, int WM, int OCC, int ORDER>
hipError_t launch_split(const GemmArgs& g, hipStream_t s) {
  const int ncol = EPI == kEpiGateUp ? g.nfeat / (BN / 2) : g.nfeat / BN;
  int64_t nlog;
  if (g.rows.layout == 0) {
    if (BM != kTileRoutesContiguous) return hipErrorInvalidValue;   // a tile is one plan tile of routes
    nlog = g.max_tiles * ncol;
  } else {
    nlog = (int64_t)g.E * ((g.rows.max_tokens + BM - 1) / BM) * ncol;
  }
  const int64_t grid = ORDER == kRouteMajor ? nlog : padded_blocks(nlog);
  hipLaunchKernelGGL((gemm_tile_split_bf16_kernel<EPI, BM, BN, BK, WN, WM, OCC, ORDER>), dim3((unsigned)grid),
                     dim3(64 * WN * WM), 0, s, g, ncol, nlog);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_layout(const GemmArgs& g, hipStream_t s) {
  // both formats on the split ring: contiguous 256 routes x 256 weight rows,
  // 16 waves of 64x64 (160 KB of LDS, one workgroup per CU), weight-major
  // in XCD chunks; batched 128 x 128, 4 waves of 64x64 (80 KB, two per CU),
  // route-major
  if (g.rows.layout == 0) return launch_split<EPI, 256, 256, 64, 4, 4, 4, kWeightMajor>(g, s);
  return launch_split<EPI, 128, 128, 64, 2, 2, 2, kRouteMajor>(g, s);
}

}  // namespace tile

// 256 rows x 256 features, the contiguous tile shape
hipError_t launch_tile_rows_bf16(const GemmArgs& g, const int32_t* offsets, int64_t R, bool wt, hipStream_t s) {
  using namespace tile;
  if (g.epi != kEpiDown) return hipErrorInvalidValue;
  const RowGroups grp{offsets, g.E, R};
  return wt ? launch_rows<kEpiDown, true>(g, grp, s) : launch_rows<kEpiDown, false>(g, grp, s);
}

hipError_t launch_gemm_tile_bf16(const GemmArgs& g, hipStream_t s) {
  if (g.epi == kEpiGateUp) return tile::launch_layout<kEpiGateUp>(g, s);
  return tile::launch_layout<kEpiDown>(g, s);
}

}  // namespace moe
