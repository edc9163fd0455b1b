// Streaming grouped GEMMs for experts that hold few rows (decode batches,
// and one rank's local-expert share of a large layer).
//
// With few rows per expert the matmuls are bound by reading the active
// experts' weights from HBM once.  Each wave owns a strip of weight rows and
// the whole contraction: the weight rows go from HBM straight into the row
// operand of the MFMA (16 rows x the contraction slice, each lane reading a
// contiguous run of one row, no LDS), and the expert's routed tokens (up to
// 16 per pass for bf16, 64 for MXFP8) sit in the other operand, read from
// L2.  The Mixture-of-Experts kernel engineering on SageMaker page ("Swap-AB
// for WGMMA utilization") swaps A and B so the weight's large N dimension
// fills Hopper's fixed 64-row slot; on gfx950 both MFMA slots are 16 wide,
// so what carries over is only that the weight rows occupy the row slot and
// stream without staging.
//
// The contraction is split among the four 16-lane groups of a wave and among
// the MFMA's own k slots in any fixed way, provided both operands use the
// same split: lane group q reads elements [base + 32q, base + 32q + 32) of
// each step (a contiguous 64-byte bf16 run or a 32-byte E4M3 MX block).
//
// Grid: (feature strips, active experts).  The active-expert list comes from
// the align step, so the grid depends only on the plan; workgroups whose
// slot is past the number of active experts leave at once.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ i32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ i32x4 ld16nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

// W row index of intermediate feature f (gate, or up when up = true).
__device__ __forceinline__ int w1_row(int f, bool up, int I, int order) {
  return order == 0 ? (up ? I + f : f) : (32 * (f >> 4) + (f & 15) + (up ? 16 : 0));
}

// ------------------------------------------------------------------ bf16 --
// Each wave: two 16-row weight tiles t0/t1.  kGateUp: 16 features (gate
// rows, then up rows).  kDown: 32 features (two tiles of 16).
template <int EPI>
__global__ void __launch_bounds__(NT) gemm_stream_bf16_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const RowMap& rm = g.rows;
  const int slot = blockIdx.y;
  if (slot >= rm.active[g.max_active]) return;
  const int e = rm.active[slot];
  const int cnt = rm.counts[e];
  const int pos0 = rm.offsets[e];
  const int K = g.kdim;
  const int q = lane >> 4;   // k lane group
  const int l16 = lane & 15;

  const uint16_t* wexp = static_cast<const uint16_t*>(g.w) + (int64_t)e * g.w_expert_stride;
  int f0, r0, r1;
  if (EPI == kEpiGateUp) {
    f0 = (blockIdx.x * 4 + wave) * 16;
    r0 = w1_row(f0 + l16, false, g.I, g.w1_order);
    r1 = w1_row(f0 + l16, true, g.I, g.w1_order);
  } else {
    f0 = (blockIdx.x * 4 + wave) * 32;
    r0 = f0 + l16;
    r1 = f0 + 16 + l16;
  }
  const uint16_t* w0 = wexp + (int64_t)r0 * K + 32 * q;
  const uint16_t* w1 = wexp + (int64_t)r1 * K + 32 * q;
  const uint16_t* act = static_cast<const uint16_t*>(g.act);
  uint16_t* out = static_cast<uint16_t*>(g.out);
  const i32x4 zero = {0, 0, 0, 0};

  for (int tg = 0; tg * 16 < cnt; ++tg) {
    const int tk = tg * 16 + l16;
    const bool tv = tk < cnt;
    const int pos = pos0 + tk;
    const uint16_t* pa = nullptr;
    if (tv) {
      if (EPI == kEpiGateUp) pa = act + (int64_t)(rm.sorted_ids[pos] / rm.topk) * g.act_ld;
      else pa = act + (int64_t)pos * g.act_ld;
      pa += 32 * q;
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    i32x4 a0[2][4], a1[2][4], b[2][4];
    auto load = [&](int st, int k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0[st][j] = ld16nt(w0 + k + 8 * j);
        a1[st][j] = ld16nt(w1 + k + 8 * j);
        b[st][j] = pa ? ld16(pa + k + 8 * j) : zero;
      }
    };
    auto mma = [&](int st) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0[st][j]), as_bf16x8(b[st][j]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1[st][j]), as_bf16x8(b[st][j]), acc1, 0, 0, 0);
      }
    };
    const int nsteps = K / 128;
    load(0, 0);
    int k = 0;
    for (int it = 0; it + 1 < nsteps; it += 2) {
      load(1, k + 128);
      mma(0);
      if (it + 2 < nsteps) load(0, k + 256);
      mma(1);
      k += 256;
    }
    if (nsteps & 1) mma(0);

    // acc[r]: weight row (tile row) 4*q + r, token column l16
    if (tv) {
      if (EPI == kEpiGateUp) {
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(silu_f32(acc0[r]) * acc1[r]);
        uint2 v = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        *reinterpret_cast<uint2*>(out + (int64_t)pos * g.out_ld + f0 + 4 * q) = v;
      } else {
        const int64_t orow = rm.sorted_ids[pos];
        uint32_t h0[4], h1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          h0[r] = f32_to_bf16_rne(acc0[r]);
          h1[r] = f32_to_bf16_rne(acc1[r]);
        }
        *reinterpret_cast<uint2*>(out + orow * g.out_ld + f0 + 4 * q) =
            make_uint2(h0[0] | (h0[1] << 16), h0[2] | (h0[3] << 16));
        *reinterpret_cast<uint2*>(out + orow * g.out_ld + f0 + 16 + 4 * q) =
            make_uint2(h1[0] | (h1[1] << 16), h1[2] | (h1[3] << 16));
      }
    }
  }
}

// ----------------------------------------------------------------- MXFP8 --
// v_mfma_scale_f32_16x16x128_f8f6f4, one 128-wide contraction step per
// instruction.  Operand layout (measured on gfx950 with an in-bounds probe of
// the builtin): in lane l (row l % 16, group g = l / 16) bytes 0-15 hold
// k = 16g .. 16g+15 and bytes 16-31 hold k = 64+16g .. 64+16g+15, and the
// lane's scale byte is the scale of the 32-wide k block g.  Read in memory
// order, a k step therefore needs, per lane, the 16 bytes at k0 + 16g and the
// 16 at k0 + 64 + 16g, plus the scale of MX block k0/32 + g: each MX block
// of the weight and activation rows lines up with exactly one scale.
// A pass covers 64 tokens (four 16-token column tiles) so each weight
// fragment feeds four MFMAs.  Each wave: 32 features.
//   kGateUp: tiles (gate f0..+15, up f0..+15, gate f0+16..+31, up f0+16..+31);
//            the epilogue quantises silu(gate)*up of the 32 features of each
//            token as one MX block (E4M3 codes + UE8M0 scale).
//   kDown:   tiles (f0..+15, f0+16..+31); bf16 y rows per (token, slot).
template <int EPI>
__global__ void __launch_bounds__(NT) gemm_stream_mxfp8_kernel(GemmArgs g) {
  constexpr int NTILE = EPI == kEpiGateUp ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const RowMap& rm = g.rows;
  const int slot = blockIdx.y;
  if (slot >= rm.active[g.max_active]) return;
  const int e = rm.active[slot];
  const int cnt = rm.counts[e];
  const int pos0 = rm.offsets[e];
  const int K = g.kdim;
  const int KB = K / 32;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int f0 = (blockIdx.x * 4 + wave) * 32;

  const uint8_t* wexp = static_cast<const uint8_t*>(g.w) + (int64_t)e * g.w_expert_stride;
  const uint8_t* wsexp = g.w_scale + (int64_t)e * (g.w_expert_stride / 32);
  const uint8_t* wp[NTILE];
  const uint8_t* wsp[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    int row;
    if (EPI == kEpiGateUp) row = w1_row(f0 + 16 * (t >> 1) + l16, (t & 1) != 0, g.I, g.w1_order);
    else row = f0 + 16 * t + l16;
    wp[t] = wexp + (int64_t)row * K + 16 * q;
    wsp[t] = wsexp + (int64_t)row * KB + q;
  }
  const uint8_t* act = static_cast<const uint8_t*>(g.act);

  for (int tg = 0; tg * 64 < cnt; ++tg) {
    const uint8_t* pa[4];
    const uint8_t* psa[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int tk = tg * 64 + 16 * c + l16;
      if (tk < cnt) {
        const int64_t pos = pos0 + tk;
        pa[c] = act + pos * g.act_ld + 16 * q;
        psa[c] = g.act_scale + pos * (g.act_ld / 32) + q;
      } else {
        pa[c] = nullptr;
        psa[c] = nullptr;
      }
    }
    f32x4 acc[NTILE][4];
#pragma unroll
    for (int t = 0; t < NTILE; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[t][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int k = 0; k < K; k += 128) {
      const int kb = k / 32;
      i32x8 wa[NTILE];
      int wsc[NTILE];
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        const i32x4 lo = ld16nt(wp[t] + k);
        const i32x4 hi = ld16nt(wp[t] + k + 64);
        wa[t] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        wsc[t] = wsp[t][kb];
      }
      i32x8 xb[4];
      int xsc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (pa[c]) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(pa[c] + k);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(pa[c] + k + 64);
          xb[c] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          xsc[c] = psa[c][kb];
        } else {
          xb[c] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
          xsc[c] = 0;
        }
      }
#pragma unroll
      for (int t = 0; t < NTILE; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[t][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wa[t], xb[c], acc[t][c], 0, 0, 0, wsc[t], 0, xsc[c]);
    }

    // acc[t][c][r]: weight row 4*q + r of tile t, token tg*64 + 16*c + l16
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int tk = tg * 64 + 16 * c + l16;
      const bool tv = tk < cnt;   // uniform per 16-lane column group only
      const int64_t pos = pos0 + tk;
      if (EPI == kEpiGateUp) {
        float z[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[r] = silu_f32(acc[0][c][r]) * acc[1][c][r];
          z[4 + r] = silu_f32(acc[2][c][r]) * acc[3][c][r];
        }
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(z[r]));
        // the 32 features of this token live in lanes l16, l16+16, l16+32, l16+48
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const uint32_t sc = mx_scale_code(m);
        const float inv = mx_inv_scale(sc);
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          w0 |= e4m3_encode(z[r] * inv) << (8 * r);
          w1 |= e4m3_encode(z[4 + r] * inv) << (8 * r);
        }
        if (tv) {
          uint8_t* o = static_cast<uint8_t*>(g.out) + pos * g.out_ld;
          *reinterpret_cast<uint32_t*>(o + f0 + 4 * q) = w0;
          *reinterpret_cast<uint32_t*>(o + f0 + 16 + 4 * q) = w1;
          if (q == 0) g.out_scale[pos * (g.out_ld / 32) + f0 / 32] = (uint8_t)sc;
        }
      } else if (tv) {
        const int64_t orow = rm.sorted_ids[pos];
        uint16_t* o = static_cast<uint16_t*>(g.out) + orow * g.out_ld;
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
          uint32_t h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(acc[t][c][r]);
          *reinterpret_cast<uint2*>(o + f0 + 16 * t + 4 * q) =
              make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_stream_bf16(const GemmArgs& g, hipStream_t s) {
  const int per_block = g.epi == kEpiGateUp ? 64 : 128;
  dim3 grid(g.nfeat / per_block, (unsigned)g.max_active);
  if (g.epi == kEpiGateUp)
    hipLaunchKernelGGL(gemm_stream_bf16_kernel<kEpiGateUp>, grid, dim3(NT), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_stream_bf16_kernel<kEpiDown>, grid, dim3(NT), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_stream_mxfp8(const GemmArgs& g, hipStream_t s) {
  dim3 grid(g.nfeat / 128, (unsigned)g.max_active);
  if (g.epi == kEpiGateUp)
    hipLaunchKernelGGL(gemm_stream_mxfp8_kernel<kEpiGateUp>, grid, dim3(NT), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_stream_mxfp8_kernel<kEpiDown>, grid, dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
