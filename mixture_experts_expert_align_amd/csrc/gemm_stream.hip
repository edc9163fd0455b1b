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
// Which k each lane feeds the MFMA may follow any fixed assignment as long
// as both operands use the same one, so the loads are laid out for memory:
// the lanes of one load instruction cover a contiguous run of each of 16
// weight rows.
//
// Grid: (feature strips, active experts).  The active-expert list comes from
// the align step, so the grid depends only on the plan; workgroups whose
// slot is past the number of active experts leave at once.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int NT = 256;
constexpr int kBufferFlags = 0x00020000;   // raw buffer, 32-bit data format (CDNA3/4 word 3)

__device__ __forceinline__ i32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ i32x4 ld16nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

// W row index of intermediate feature f (gate, or up when up = true).
__device__ __forceinline__ int w1_row(int f, bool up, int I, int order) {
  return order == 0 ? (up ? I + f : f) : (32 * (f >> 4) + (f & 15) + (up ? 16 : 0));
}

// ------------------------------------------------------------------ bf16 --
// A workgroup owns 16 output features of one expert and KS waves split the
// contraction into KS equal runs; each wave streams its run of the weight
// rows with a three-deep register pipeline, the partial sums meet in LDS and
// wave 0 adds them in wave order (a fixed order, so every run gives the same
// bits) before the epilogue.  Splitting the contraction keeps each
// workgroup's task short, so the last wave of workgroups on the chip is short
// too; with a whole contraction per workgroup the tail of the grid left much
// of the chip idle.
//   kGateUp: two 16-row tiles: the gate rows and the matching up rows of the
//            16 features; epilogue z = silu(gate) * up, bf16, row = position.
//   kDown:   one 16-row tile of W2; epilogue writes y rows per (token, slot).
// Per lane and 128-wide step, lane group q takes the four 16-byte pieces at
// k + 8q + 32j (j = 0..3) of its row: the four groups of one load
// instruction read 64 contiguous bytes of each of 16 rows.
template <int EPI, int KS>
__global__ void __launch_bounds__(64 * KS) gemm_stream_bf16_kernel(GemmArgs g) {
  constexpr int NTL = EPI == kEpiGateUp ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const RowMap& rm = g.rows;
  const int slot = blockIdx.y;
  if (slot >= rm.active[g.max_active]) return;
  const int e = rm.active[slot];
  const int cnt = rm.counts[e];
  const int pos0 = rm.offsets[e];
  const int K = g.kdim;
  const int KW = K / KS;                      // contraction run of this wave
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int kbase = wave * KW + 8 * q;
  const int f0 = blockIdx.x * 16;

  // Buffer loads: the expert's weights and the activations as two buffer
  // resources, per-lane 32-bit byte offsets, the step's k in the scalar
  // offset.  A lane without a token gets an offset past the buffer's size,
  // which the hardware's range check turns into zeros.
  const uint16_t* wexp = static_cast<const uint16_t*>(g.w) + (int64_t)e * g.w_expert_stride;
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc((void*)wexp, 0, (int)min<int64_t>(g.w_expert_stride * 2, 0x7fffffff),
                                        kBufferFlags);
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.act, 0, (int)min<int64_t>(g.act_bytes, 0x7fffffff), kBufferFlags);
  uint32_t wo[NTL];
  if (EPI == kEpiGateUp) {
    wo[0] = (uint32_t)(w1_row(f0 + l16, false, g.I, g.w1_order) * K + kbase) * 2u;
    wo[NTL - 1] = (uint32_t)(w1_row(f0 + l16, true, g.I, g.w1_order) * K + kbase) * 2u;
  } else {
    wo[0] = (uint32_t)((f0 + l16) * K + kbase) * 2u;
  }
  uint16_t* out = static_cast<uint16_t*>(g.out);
  __shared__ f32x4 red[KS][NTL][64];
  const int nsteps = KW / 128;

  for (int tg = 0; tg * 16 < cnt; ++tg) {
    const int tk = tg * 16 + l16;
    const bool tv = tk < cnt;
    const int pos = pos0 + tk;
    uint32_t ao = 0x80000000u;               // past the end: loads return 0
    if (tv) {
      const int64_t row = EPI == kEpiGateUp ? rm.sorted_ids[pos] / rm.topk : pos;
      ao = (uint32_t)((row * g.act_ld + kbase) * 2);
    }
    f32x4 acc[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    i32x4 a[3][NTL][4], b[3][4];
    auto load = [&](int st, int k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t = 0; t < NTL; ++t)
          a[st][t][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, wo[t] + 64 * j, 2 * k, 0);
        b[st][j] = __builtin_amdgcn_raw_buffer_load_b128(ar, ao + 64 * j, 2 * k, 0);
      }
    };
    auto mma = [&](int st) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < NTL; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[st][t][j]), as_bf16x8(b[st][j]),
                                                           acc[t], 0, 0, 0);
    };
    load(0, 0);
    if (nsteps > 1) load(1, 128);
    for (int it = 0; it < nsteps; it += 3) {
      if (it + 2 < nsteps) load(2, 128 * (it + 2));
      mma(0);
      if (it + 3 < nsteps) load(0, 128 * (it + 3));
      if (it + 1 < nsteps) mma(1);
      if (it + 4 < nsteps) load(1, 128 * (it + 4));
      if (it + 2 < nsteps) mma(2);
    }

#pragma unroll
    for (int t = 0; t < NTL; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        f32x4 sum = red[0][t][lane];
        for (int w = 1; w < KS; ++w) sum += red[w][t][lane];
        acc[t] = sum;
      }
      // acc[t][r]: weight row 4*q + r of tile t, token column l16
      if (tv) {
        uint32_t h[4];
        int64_t o;
        if (EPI == kEpiGateUp) {
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(silu_f32(acc[0][r]) * acc[NTL - 1][r]);
          o = (int64_t)pos * g.out_ld;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(acc[0][r]);
          o = (int64_t)rm.sorted_ids[pos] * g.out_ld;
        }
        *reinterpret_cast<uint2*>(out + o + f0 + 4 * q) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
    __syncthreads();
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

// Waves per workgroup: as many as divide the contraction into runs that are
// whole 128-wide steps, up to 4 for W1 and 8 for W2 (the fastest shapes
// measured for the decode workload).
template <int EPI>
static hipError_t launch_stream_bf16(const GemmArgs& g, hipStream_t s, int max_ks) {
  dim3 grid(g.nfeat / 16, (unsigned)g.max_active);
  int ks = max_ks;
  while (ks > 1 && g.kdim % (128 * ks)) ks >>= 1;
  switch (ks) {
    case 8: hipLaunchKernelGGL((gemm_stream_bf16_kernel<EPI, 8>), grid, dim3(512), 0, s, g); break;
    case 4: hipLaunchKernelGGL((gemm_stream_bf16_kernel<EPI, 4>), grid, dim3(256), 0, s, g); break;
    case 2: hipLaunchKernelGGL((gemm_stream_bf16_kernel<EPI, 2>), grid, dim3(128), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_stream_bf16_kernel<EPI, 1>), grid, dim3(64), 0, s, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_stream_bf16(const GemmArgs& g, hipStream_t s) {
  return g.epi == kEpiGateUp ? launch_stream_bf16<kEpiGateUp>(g, s, 4)
                             : launch_stream_bf16<kEpiDown>(g, s, 8);
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
