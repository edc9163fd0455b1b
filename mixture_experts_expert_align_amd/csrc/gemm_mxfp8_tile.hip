// LDS-tiled grouped GEMM with MXFP8 weights and activations (E4M3 codes,
// one UE8M0 scale per 32 values along the contraction) — the matmuls of the
// page "Cake MegaMoE EP16 backend for BF16 activations and MXFP8 weights"
// (section 2: the block-32 format; section 3: a weight tile is loaded once and
// reused for every row segment of its expert).
//
// A workgroup of NW waves computes 32 NW weight rows x 64 routes of one
// expert (NW = 4: 128 rows, two workgroups per CU).  Each 128-wide
// contraction step (one v_mfma_scale_f32_16x16x128_f8f6f4) of both
// operands — weight codes 32 NW x 128 B and route codes 64 x 128 B — reaches
// LDS by buffer loads that write LDS directly, into a ring of 3 step slots:
// step kt+3 is requested once step kt's slot is free, so every load has two
// steps of work to land in.  The scale words come with each step, or, where
// the contraction allows, 4 steps at a time into a ring of their own (from
// row-major scale arrays, or as contiguous blocks from grouped ones: see
// MxTile).  Workgroups are ordered
// weight-major inside an expert and handed to the XCDs in chunks (the bf16
// tile kernel's order), so an expert with more than 64 routes reads each
// weight tile from HBM once and its other route tiles find it in L2.
//
// Operand layout of the scaled MFMA (measured on gfx950 with an in-bounds
// probe of the builtin): lane l (row l % 16, group g = l / 16) holds
// k = 16g .. 16g+15 in bytes 0-15 and k = 64+16g .. 64+16g+15 in bytes 16-31,
// and its scale byte is the scale of the 32-wide k block g.  In LDS each
// 128-byte row keeps its 16-byte chunks XOR-swizzled by (row / 2) & 7, so the
// 16 rows a fragment read touches fall on distinct banks.
//
// Wave w owns weight rows 32w .. 32w+31 as two 16-row tiles and all 64
// routes as four 16-route groups (8 MFMAs per step).  Once a tile is done the
// workgroup moves on to the tile one grid further along, so the launch stays
// at two workgroups per CU however many tiles there are.
//   kGateUp: the tile's 32 NW rows are the gate and up rows of 16 NW features,
//            wave w holding gate (tile 0) and up (tile 1) of features
//            16w .. 16w+15; z = silu(gate) * up is staged in LDS and each
//            thread then quantises one (route, 32-feature block) to E4M3 codes
//            and a UE8M0 scale (the same rule as the weights).
//   kDown:   the tile's bf16 outputs are staged in LDS and leave as whole
//            256-byte row segments of each route's (token, slot) row of y.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_common.h"

namespace moe {
namespace {

using tile::TileCoord;

constexpr int kBM = kTileRoutesMxfp8;   // routes per tile (the plan's block size)
constexpr int kSlots = 3;

// NW waves, 32 weight rows each: BN = 32 NW weight rows per tile.  One step
// slot (bytes): weight codes, route codes and, unless GS, the step's scale
// words of the weight rows and of the routes; each region a whole number of
// KB.
// GS (grouped scales, when a row's scale bytes are a multiple of 16): the
// scale words of kGroup steps travel together, one 16-byte load per lane
// (16 consecutive scale bytes of one row) into a ring of their own, instead
// of one 4-byte load per lane and step.  A scale load touches one cache line
// per lane whatever its width, so the 4-byte form costs the address and data
// path as much per load as a 1 KB code block; in a read loop with this
// kernel's mix of loads it held the weight stream at 5.4 TB/s against 5.9
// with the grouped form.
constexpr int kGroup = 4;     // steps per scale group (16 bytes of a row)
constexpr int kSSlots = 2;    // scale group slots
template <int NW, bool GS>
struct MxTile {
  static constexpr int BN = 32 * NW;
  static constexpr int WCode = 0;
  static constexpr int XCode = WCode + BN * 128;
  static constexpr int WScale = XCode + kBM * 128;
  static constexpr int XScale = WScale + (BN * 4 + 1023) / 1024 * 1024;
  static constexpr int Slot = GS ? WScale : XScale + 1024;
  // GS: one scale group slot (weight rows' 16 bytes, then the routes'), and
  // where the ring of them starts
  static constexpr int SSlot = (BN + kBM) * 16;
  static constexpr int SRing = kSlots * Slot;
  // W2: the tile's 64 destination rows (sorted ids), after the scale ring;
  // Lds: the W2 kernel's LDS, Rows: the W1 kernel's
  static constexpr int Rows = SRing + (GS ? kSSlots * SSlot : 0);
  static constexpr int Lds = Rows + kBM * 4;
  // loads per wave per step: weight code blocks, route code blocks and,
  // unless GS, one 256-byte block of scale words (GS: one 1 KB block of
  // scale words on the first step of each group, scale waves only)
  static constexpr int LW = BN / 8 / NW;
  static constexpr int LX = kBM / 8 / NW;
  static constexpr int Loads = LW + LX + (GS ? 0 : 1);
  static_assert(LW * 8 * NW == BN && LX * 8 * NW == kBM, "code blocks per wave");
  static_assert(BN / 64 + 1 <= NW, "every scale block has a wave");
};
static_assert(kBM == 64, "route scale words fill one 256-byte block");

// byte offset of logical 16-byte chunk c of a 128-byte row
__device__ __forceinline__ int chunk_off(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

// The tile's end.  acc[t][c][r]: weight row 32 wave + 16 t + 4 q + r, route
// 16 c + l16.  The operand slots are free (the caller has waited for every
// load and met a barrier), so both epilogues stage the tile there.  orow
// (W2): the tile's route rows' destination rows, in LDS.
template <int EPI, int NW, int SMEM, bool PK>
__device__ __forceinline__ void mx_epilogue(const GemmArgs& g, const TileCoord& tc, const f32x4 (&acc)[2][4],
                                            uint8_t* smem, const int32_t* orow) {
  constexpr int kBN = 32 * NW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int q = lane >> 4;
  if (EPI == kEpiGateUp) {
    // z[route][feature] (fp32, rows of 132 floats so the float4 reads of
    // consecutive routes fall on different banks)
    constexpr int kZs = 132;
    static_assert(kBM * kZs * 4 <= SMEM && kBN / 2 <= kZs - 4, "z fits the LDS");
    float* zs = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        zs[(16 * c + l16) * kZs + 16 * wave + 4 * q + r] = silu_f32(acc[0][c][r]) * acc[1][c][r];
    lds_barrier();
    // thread: route m, 32-feature block b of the tile's BN/2 features
    const int m = threadIdx.x & (kBM - 1);
    const int b = threadIdx.x / kBM;
    if (b < kBN / 64 && m < tc.nvalid) {
      float z[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(zs + m * kZs + 32 * b + 4 * i);
        z[4 * i] = v.x; z[4 * i + 1] = v.y; z[4 * i + 2] = v.z; z[4 * i + 3] = v.w;
      }
      float bm = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) bm = fmaxf(bm, fabsf(z[i]));
      const uint32_t sc = mx_scale_code(bm);
      const float inv = mx_inv_scale(sc);
      uint32_t w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w[i] = e4m3_pack4(z[4 * i] * inv, z[4 * i + 1] * inv, z[4 * i + 2] * inv, z[4 * i + 3] * inv);
      const int64_t pos = tc.row0 + m;
      const int f = tc.col0 / 2 + 32 * b;   // first feature of the block
      uint8_t* o = static_cast<uint8_t*>(g.out) + pos * g.out_ld + f;
      *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(o + 16) = make_uint4(w[4], w[5], w[6], w[7]);
      // PK: z's scales grouped like the weights' (16 bytes a row per group)
      const int j = f / 32;
      g.out_scale[PK ? (int64_t)(j / 16) * g.scale_group + pos * 16 + j % 16 : pos * (g.out_ld / 32) + j] =
          (uint8_t)sc;
    }
  } else {
    // bf16 rows of the tile's kBN outputs per route, laid out in LDS row by
    // row (16-byte chunk c of row m at c ^ (m % NCH), so the 8-byte writes
    // from the accumulators and the row reads spread over the banks), then
    // written out as whole row segments: each store instruction covers 4
    // rows of 256 bytes instead of 16 rows of 32
    constexpr int NCH = kBN / 8;   // 16-byte chunks per row
    static_assert(kBM * kBN * 2 <= SMEM && (NCH & (NCH - 1)) == 0 && NCH <= 64, "W2 staging");
    uint16_t* st = reinterpret_cast<uint16_t*>(smem);
    auto chunk_at = [](int m, int c) { return (m * NCH + (c ^ (m & (NCH - 1)))) * 8; };
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m = 16 * c + l16;
        const int f = 32 * wave + 16 * t + 4 * q;
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(acc[t][c][r]);
        *reinterpret_cast<uint2*>(st + chunk_at(m, f / 8) + (f & 7)) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    lds_barrier();
    uint16_t* out = static_cast<uint16_t*>(g.out);
    const int c = threadIdx.x % NCH;
    for (int m = threadIdx.x / NCH; m < tc.nvalid; m += 64 * NW / NCH)
      *reinterpret_cast<i32x4*>(out + (int64_t)orow[m] * g.out_ld + tc.col0 + 8 * c) =
          *reinterpret_cast<const i32x4*>(st + chunk_at(m, c));
  }
}

// PK (with GS): the scale arrays are grouped (moe_pack_mxfp8_scales for the
// weights, the same layout for the activations), so a group's 16 bytes of
// 64 consecutive rows are one contiguous KiB.
template <int EPI, int NW, bool GS, bool PK>
__device__ __forceinline__ void mxfp8_tile(const GemmArgs& g, const TileCoord& tc, uint8_t* smem) {
  static_assert(!PK || GS, "grouped arrays are loaded a group at a time");
  using T = MxTile<NW, GS>;
  constexpr int kNW = NW;
  constexpr int kBN = T::BN;
  constexpr int kWCode = T::WCode, kXCode = T::XCode, kWScale = T::WScale, kXScale = T::XScale, kSlot = T::Slot;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int q = lane >> 4;
  const int K = g.kdim;                  // contraction length = code bytes per row
  const int KS = K / 32;                 // scale bytes per row
  const int nk = K / 128;

  const uint8_t* wexp = static_cast<const uint8_t*>(g.w) + (int64_t)tc.expert * g.w_expert_stride;
  const uint8_t* wsexp = g.w_scale + (int64_t)tc.expert * (g.w_expert_stride / 32);
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride);
  const __amdgpu_buffer_rsrc_t wsr = buffer_rsrc(wsexp, g.w_expert_stride / 32);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
  const __amdgpu_buffer_rsrc_t asr = buffer_rsrc(g.act_scale, g.act_bytes / 32);

  // global row of the tile's weight row n
  auto wrow_of = [&](int n) {
    if (EPI == kEpiGateUp) return w1_row(tc.col0 / 2 + 16 * (n >> 5) + (n & 15), ((n >> 4) & 1) != 0, g.I, g.w1_order);
    return tc.col0 + n;
  };
  // route m's sorted position, or -1 for padding
  auto pos_of = [&](int m) { return m < tc.nvalid ? (int64_t)tc.row0 + m : (int64_t)-1; };

  // Per step every wave issues T::Loads loads into the step's slot: LW
  // blocks of weight codes (block b = 8 rows x 128 B, lane i -> row 8b + i/8,
  // physical chunk i % 8), LX blocks of route codes, and one 256-byte block
  // of scale words (waves 0 .. BN/64-1: weight rows 64w .. 64w+63; wave
  // BN/64: the 64 routes; later waves repeat weight blocks from 0, the same
  // bytes to the same place).  GS: the scale blocks are 1 KB (16 bytes of
  // each row: kGroup steps), loaded on the first step of each group into
  // group slot (step / kGroup) % kSSlots, by waves 0 .. BN/64 only.
  constexpr int LW = T::LW, LX = T::LX;
  constexpr int kWsBlocks = kBN / 64;
  uint32_t ow[LW], ox[LX], osc;
#pragma unroll
  for (int j = 0; j < LW; ++j) {
    const int n = 8 * (wave + kNW * j) + (lane >> 3);
    ow[j] = (uint32_t)(wrow_of(n) * K + (((lane & 7) ^ ((n >> 1) & 7)) << 4));
  }
#pragma unroll
  for (int j = 0; j < LX; ++j) {
    const int m = 8 * (wave + kNW * j) + (lane >> 3);
    const int64_t pos = pos_of(m);
    ox[j] = pos >= 0 ? (uint32_t)(pos * g.act_ld + (((lane & 7) ^ ((m >> 1) & 7)) << 4)) : 0x80000000u;
  }
  const bool xscale_wave = wave == kWsBlocks;
  const int sblk = wave < kWsBlocks ? wave : (wave - kWsBlocks - 1) % kWsBlocks;
  if (xscale_wave) {
    const int64_t pos = pos_of(lane);
    osc = pos >= 0 ? (uint32_t)(pos * (PK ? 16 : g.act_ld / 32)) : 0x80000000u;
  } else {
    osc = (uint32_t)(wrow_of(64 * sblk + lane) * (PK ? 16 : KS));
  }
  // PK: bytes between groups, the weights' (rows of the expert's matrix x
  // 16) and the activations'
  const int wgroup = PK ? (int)(g.w_expert_stride / K) * 16 : 0;
  const int xgroup = PK ? (int)g.scale_group : 0;
  // GS: whether this wave loads scale groups (waves past BN/64 do not)
  const bool sc_wave = !GS || wave <= kWsBlocks;
  // W2: the last wave brings the tile's 64 sorted ids (the routes'
  // destination rows) into LDS with step 0, so the epilogue does not wait
  // for them; a route past the tile's valid rows is never written
  int32_t* const orow = reinterpret_cast<int32_t*>(smem + T::Rows);
  const __amdgpu_buffer_rsrc_t sidr = buffer_rsrc(g.rows.sorted_ids + tc.row0, kBM * 4);
  auto issue = [&](int st) {
    uint8_t* slot = smem + (st % kSlots) * kSlot;
    if (EPI == kEpiDown && st == 0 && wave == kNW - 1) lds_load4(sidr, orow, (uint32_t)(4 * lane), 0);
#pragma unroll
    for (int j = 0; j < LW; ++j) lds_load16(wr, slot + kWCode + (wave + kNW * j) * 1024, ow[j], st * 128);
#pragma unroll
    for (int j = 0; j < LX; ++j) lds_load16(ar, slot + kXCode + (wave + kNW * j) * 1024, ox[j], st * 128);
    if (!GS) {
      if (xscale_wave) lds_load4(asr, slot + kXScale, osc, st * 4);
      else lds_load4(wsr, slot + kWScale + sblk * 256, osc, st * 4);
    } else if (sc_wave && st % kGroup == 0) {
      uint8_t* ss = smem + T::SRing + (st / kGroup % kSSlots) * T::SSlot;
      if (xscale_wave) lds_load16(asr, ss + kBN * 16, osc, PK ? st / kGroup * xgroup : st * 4);
      else lds_load16(wsr, ss + sblk * 1024, osc, PK ? st / kGroup * wgroup : st * 4);
    }
    issue_order();
  };
  constexpr int kLoads = T::Loads;   // per wave per step, scale groups aside
  // wait until step st has landed, step st+1 (the only younger one) in flight
  auto wait_before = [&](int st1) {
    if (GS && sc_wave && st1 % kGroup == 0) wait_vm<kLoads + 1>();
    else wait_vm<kLoads>();
  };

  f32x4 acc[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[t][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // fragments of one step: weight tiles, route groups, scale bytes (in the
  // low byte; the builtin takes the scale from byte 0 with opsel 0)
  i32x8 fa[2][2], fb[2][4];
  int sa[2][2], sb[2][4];
  // scale word of LDS row r (weight rows, then BN + route rows) at step st
  auto scale_word = [&](const uint8_t* slot, int r, int st) {
    if (GS) {
      const uint8_t* ss = smem + T::SRing + (st / kGroup % kSSlots) * T::SSlot;
      return *reinterpret_cast<const uint32_t*>(ss + 16 * r + 4 * (st % kGroup));
    }
    return *reinterpret_cast<const uint32_t*>(slot + (r < kBN ? kWScale + 4 * r : kXScale + 4 * (r - kBN)));
  };
  auto fload = [&](int buf, int st) {
    const uint8_t* slot = smem + (st % kSlots) * kSlot;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 32 * wave + 16 * t + l16;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(slot + kWCode + chunk_off(r, q));
      const i32x4 hi = *reinterpret_cast<const i32x4*>(slot + kWCode + chunk_off(r, 4 + q));
      fa[buf][t] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sa[buf][t] = (int)(scale_word(slot, r, st) >> (8 * q));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = 16 * c + l16;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(slot + kXCode + chunk_off(r, q));
      const i32x4 hi = *reinterpret_cast<const i32x4*>(slot + kXCode + chunk_off(r, 4 + q));
      fb[buf][c] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      sb[buf][c] = (int)(scale_word(slot, kBN + r, st) >> (8 * q));
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[t][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[buf][t], fb[buf][c], acc[t][c], 0, 0, 0,
                                                                    sa[buf][t], 0, sb[buf][c]);
  };

  // prologue: steps 0, 1, 2 requested; wait for step 0 (steps 1 and 2 open
  // no scale group)
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  if (nk > 2) wait_vm<2 * kLoads>();
  else if (nk > 1) wait_vm<kLoads>();
  else wait_vm<0>();
  lds_barrier();
  fload(0, 0);
  // step kt multiplies fragment set B (its parity; the loop is unrolled by two
  // so that every register index is known at compile time)
  auto step = [&](int kt, auto b) {
    constexpr int B = decltype(b)::value;
    mma(B);
    if (kt + 1 < nk) {
      // step kt+1 has landed once only step kt+2's loads may still fly;
      // after the barrier nobody reads step kt's slot any more
      if (kt + 2 < nk) wait_before(kt + 2);
      else wait_vm<0>();
      lds_barrier();
      if (kt + 3 < nk) issue(kt + 3);
      fload(B ^ 1, kt + 1);
    }
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, std::integral_constant<int, 0>());
    if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>());
  }
  wait_vm<0>();
  lds_barrier();

  mx_epilogue<EPI, NW, kSlots * kSlot, PK>(g, tc, acc, smem, orow);
}

// WPC workgroups per CU (each ring takes 3 slots of LDS) walk the tiles in
// grid-stride order.  The grid is sized for the worst routing the plan
// allows (an expert-parallel share may hold only a small part of the
// routes), so the walk stops at the tiles the align step actually laid out
// instead of dispatching a workgroup for every possible one.
template <int EPI, int NW, int WPC, bool GS, bool PK>
__global__ void __launch_bounds__(64 * NW, NW * WPC / 4) gemm_tile_mxfp8_kernel(GemmArgs g, int ncol, int64_t nlog) {
  using T = MxTile<NW, GS>;
  // W1 has no destination rows to keep
  __shared__ __attribute__((aligned(1024))) uint8_t smem[EPI == kEpiDown ? T::Lds : T::Rows];
  const int64_t total = (int64_t)g.rows.num_post[0] / kBM * ncol;
  const int64_t vend = tile::padded_blocks(total < nlog ? total : nlog);
  for (int64_t v = blockIdx.x; v < vend; v += gridDim.x) {
    TileCoord tc;
    if (!tile::tile_coord<kBM, T::BN, tile::kWeightMajor>(g, ncol, nlog, tc, v)) continue;
    mxfp8_tile<EPI, NW, GS, PK>(g, tc, smem);
    lds_barrier();   // the epilogue's LDS reads are done before the next tile's loads land
  }
}

// NW waves per workgroup, WPC workgroups per CU (the grid: WPC per CU, a
// multiple of the 8 XCDs)
template <int EPI, int NW, int WPC, bool GS, bool PK>
hipError_t launch_tile_mxfp8_gs(const GemmArgs& g, hipStream_t s) {
  using T = MxTile<NW, GS>;
  static_assert(WPC * T::Lds <= 160 * 1024, "workgroups per CU fit the LDS");
  if (g.rows.layout != 0) return hipErrorInvalidValue;
  const int ncol = EPI == kEpiGateUp ? g.nfeat / (T::BN / 2) : g.nfeat / T::BN;
  const int64_t nlog = g.max_tiles * ncol;
  const int64_t grid = std::min<int64_t>(tile::padded_blocks(nlog), 256 * WPC);
  hipLaunchKernelGGL((gemm_tile_mxfp8_kernel<EPI, NW, WPC, GS, PK>), dim3((unsigned)grid), dim3(64 * NW), 0, s, g,
                     ncol, nlog);
  return hipGetLastError();
}

// Grouped scales need 16 consecutive scale bytes of a row to be one aligned
// 16-byte load: weight and activation rows whose scale bytes are a multiple
// of 16 (contraction a multiple of 512) and 16-byte aligned scale arrays.
// Grouped arrays (g.scale_group > 0) meet all of that by construction (the
// plan and the entry points check it).
template <int EPI, int NW, int WPC>
hipError_t launch_tile_mxfp8_nw(const GemmArgs& g, hipStream_t s) {
  if (g.scale_group) return launch_tile_mxfp8_gs<EPI, NW, WPC, true, true>(g, s);
  const bool gs = g.kdim % 512 == 0 && g.act_ld % 512 == 0 &&
                  ((reinterpret_cast<uintptr_t>(g.w_scale) | reinterpret_cast<uintptr_t>(g.act_scale)) & 15) == 0;
  return gs ? launch_tile_mxfp8_gs<EPI, NW, WPC, true, false>(g, s)
            : launch_tile_mxfp8_gs<EPI, NW, WPC, false, false>(g, s);
}

// 4 waves and 128 weight rows per tile, two workgroups per CU (78 KB of LDS
// each): measured 2-4% faster on the EP16 share than 8 waves and 256 rows
// with one workgroup per CU (the two workgroups' barriers interleave)
template <int EPI>
hipError_t launch_tile_mxfp8(const GemmArgs& g, hipStream_t s) {
  return launch_tile_mxfp8_nw<EPI, 4, 2>(g, s);
}

}  // namespace

hipError_t launch_gemm_tile_mxfp8(const GemmArgs& g, hipStream_t s) {
  return g.epi == kEpiGateUp ? launch_tile_mxfp8<kEpiGateUp>(g, s) : launch_tile_mxfp8<kEpiDown>(g, s);
}

}  // namespace moe
