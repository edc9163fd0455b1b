// Streaming grouped GEMMs for experts that hold few rows (decode batches,
// and one rank's local-expert share of a large layer).
//
// With few rows per expert the matmuls are bound by reading the active
// experts' weights from HBM once.  Each wave owns a strip of weight rows and
// the whole contraction: the weight rows go from HBM straight into the row
// operand of the MFMA (16 rows x the contraction slice, each lane reading a
// contiguous run of one row, no LDS), and the expert's routed tokens sit in
// the other operand: up to 16 per pass for bf16, read from L2; 64 per pass
// for MXFP8, staged once per workgroup in LDS and shared by its waves.  The Mixture-of-Experts kernel engineering on SageMaker page ("Swap-AB
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

__device__ __forceinline__ i32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const i32x4*>(p); }

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
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride * 2);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
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
//
// A workgroup owns four 16-row weight tiles of one expert, one per wave; each
// wave streams its tile over the whole contraction straight from HBM into
// registers, one stage (two 128-wide steps) ahead.  The 64 routed token rows
// of a pass (four 16-token column tiles) are staged in LDS a stage at a time
// (double buffered) and shared by the four waves, so activations cross L2
// once per workgroup.  The barriers between stages wait only for LDS
// operations, so the weight loads stay in flight across them.
//   kGateUp: tiles (gate f0..+15, up f0..+15, gate f0+16..+31, up f0+16..+31),
//            32 features = one MX block of z per token: the epilogue gathers
//            the four tiles in LDS and quantises silu(gate)*up (E4M3 codes +
//            UE8M0 scale).
//   kDown:   tiles f0 + 16t, 64 features; bf16 y rows per (token, slot).
constexpr int kMxTok = 64;                 // tokens per pass

// LDS byte offset of 16-byte chunk c of staged token row r (rows of ROW
// bytes, ROW a multiple of 128): the chunk index is XOR-ed with a function of
// the row that stays inside the row, chosen so the 16 rows one lane group
// reads at a chunk cover all 16 chunk slots of a 256-byte bank window (rows
// of 128 bytes: two rows per window, 8 XOR values; wider rows: r % 16).
template <int ROW>
__device__ __forceinline__ int mx_lds(int r, int c) {
  constexpr int RPW = ROW >= 256 ? 1 : 256 / ROW;            // rows per 256-byte window
  constexpr int XM = (ROW / 16 < 16 ? ROW / 16 : 16) - 1;   // XOR range inside a row
  return r * ROW + ((c ^ ((r / RPW) & XM)) << 4);
}

// STEPS: 128-wide steps per stage (2, or 1 for an odd step count), dividing
// the contraction's step count, so every stage is full and the loop has no
// per-step tests.  (Four steps per stage need more than the 256 registers
// that keep two workgroups on a CU.)
template <int EPI, int STEPS>
__global__ void __launch_bounds__(256, 2) gemm_stream_mxfp8_kernel(GemmArgs g) {
  constexpr int kRow = 128 * STEPS;          // bytes of one token row per stage
  constexpr int kChunks = kRow / 16;         // 16-byte chunks per staged row
  constexpr int kStage = kMxTok * kRow;      // bytes of one staged stage
  constexpr int kRowsPerPass = 256 / kChunks;
  constexpr int kLoads = kMxTok / kRowsPerPass;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;          // = weight tile
  const int tid = threadIdx.x;
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
  const int f0 = blockIdx.x * (EPI == kEpiGateUp ? 32 : 64);

  const uint8_t* wexp = static_cast<const uint8_t*>(g.w) + (int64_t)e * g.w_expert_stride;
  const uint8_t* wsexp = g.w_scale + (int64_t)e * (g.w_expert_stride / 32);
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride);
  const __amdgpu_buffer_rsrc_t wsr = buffer_rsrc(wsexp, g.w_expert_stride / 32);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
  const __amdgpu_buffer_rsrc_t asr = buffer_rsrc(g.act_scale, g.act_bytes / 32);
  int row;
  if (EPI == kEpiGateUp) row = w1_row(f0 + 16 * (wave >> 1) + l16, (wave & 1) != 0, g.I, g.w1_order);
  else row = f0 + 16 * wave + l16;
  const uint32_t wo = (uint32_t)(row * K + 16 * q);
  const uint32_t wso = (uint32_t)(row * KB + q);

  // staged activations (two stages) and their scales; the epilogue reuses
  // the first stage buffer for the four waves' accumulators
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kStage];
  __shared__ uint32_t sBs[2][kMxTok * STEPS];             // 4 scale bytes per token per step
  f32x4* sOut = reinterpret_cast<f32x4*>(&sB[0][0]);      // [tile][column tile][lane]
  static_assert(16 * 64 * sizeof(f32x4) <= 2 * kStage, "epilogue buffer");
  const int nstages = K / kRow;

  // staging: thread tid moves chunk tid % kChunks of rows tid / kChunks +
  // kRowsPerPass * i (i < kLoads) and, for tid < 64 * STEPS, one scale word
  // (token tid / STEPS, step tid % STEPS)
  const int srow = tid / kChunks, schk = tid % kChunks;
  for (int tg = 0; tg * kMxTok < cnt; ++tg) {
    uint32_t xo[kLoads], xso = 0x80000000u;    // past the end: loads return 0
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int t = tg * kMxTok + srow + kRowsPerPass * i;
      xo[i] = t < cnt ? (uint32_t)((int64_t)(pos0 + t) * g.act_ld + 16 * schk) : 0x80000000u;
    }
    if (tid < kMxTok * STEPS) {
      const int tt = tg * kMxTok + tid / STEPS;
      if (tt < cnt) xso = (uint32_t)((int64_t)(pos0 + tt) * (g.act_ld / 32) + 4 * (tid % STEPS));
    }
    i32x4 pb[kLoads];
    uint32_t pbs = 0;
    // stage numbers are uniform; readfirstlane tells the compiler so, and
    // keeps the scalar offsets of the loads in scalar registers
    auto bload = [&](int stage) {
      const int kb = __builtin_amdgcn_readfirstlane(stage * kRow);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) pb[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, xo[i], kb, 0);
      if (tid < kMxTok * STEPS) pbs = __builtin_amdgcn_raw_buffer_load_b32(asr, xso, kb >> 5, 0);
    };
    auto bstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        *reinterpret_cast<i32x4*>(&sB[buf][mx_lds<kRow>(srow + kRowsPerPass * i, schk)]) = pb[i];
      if (tid < kMxTok * STEPS) sBs[buf][tid] = pbs;
    };

    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // weight fragments of two stages
    i32x8 wa[2][STEPS];
    int wsc[2][STEPS];
    auto aload = [&](int p, int stage) {
#pragma unroll
      for (int sub = 0; sub < STEPS; ++sub) {
        const int k = __builtin_amdgcn_readfirstlane(128 * (stage * STEPS + sub));
        const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(wr, wo, k, 0);
        const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(wr, wo + 64, k, 0);
        wa[p][sub] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        wsc[p][sub] = (int)(uint32_t)__builtin_amdgcn_raw_buffer_load_b8(wsr, wso, k >> 5, 0);
      }
    };
    auto mma = [&](int p) {
#pragma unroll
      for (int sub = 0; sub < STEPS; ++sub) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int tr = 16 * c + l16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(&sB[p][mx_lds<kRow>(tr, 8 * sub + q)]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(&sB[p][mx_lds<kRow>(tr, 8 * sub + 4 + q)]);
          const i32x8 xb = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const int xs = (sBs[p][tr * STEPS + sub] >> (8 * q)) & 0xff;
          acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[p][sub], xb, acc[c], 0, 0, 0,
                                                                   wsc[p][sub], 0, xs);
        }
      }
    };
    // One stage with stage parity p (a literal at each call).  On entry the
    // activations of stage stg+1 are in registers (fetched a stage earlier)
    // and the weights of stage stg are on their way.  The stage stores the
    // activations of stg+1 to LDS, fetches the activations of stg+2 and the
    // weights of stg+1, then multiplies stage stg.  The scheduling barriers
    // keep this order, so each load has a whole stage to arrive.  The fetch
    // of stage stg+2 may run past the contraction (the last two stages): it
    // reads bytes of the next row or, past the buffer, zeros, and is never
    // stored.
    auto body = [&](int p, int stg) {
      bstore(p ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      bload(stg + 2);
      aload(p ^ 1, stg + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(p);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
    };

    // prologue, issuing in the loop's order (activations before weights) so
    // the waits in the loop stay partial
    bload(0);
    bstore(0);
    bload(1);
    aload(0, 0);
    lds_barrier();
    int stg = 0;
    while (true) {
      if (stg + 1 >= nstages) { mma(0); break; }
      body(0, stg++);
      if (stg + 1 >= nstages) { mma(1); break; }
      body(1, stg++);
    }
    lds_barrier();

    // acc[c][r]: weight row 4*q + r of this wave's tile, token tg*64 + 16*c + l16
#pragma unroll
    for (int c = 0; c < 4; ++c) sOut[(wave * 4 + c) * 64 + lane] = acc[c];
    lds_barrier();
    if (EPI == kEpiGateUp) {
      // wave c finishes column tile c: 16 tokens x 32 features
      const int c = wave;
      const f32x4 g0 = sOut[(0 * 4 + c) * 64 + lane], u0 = sOut[(1 * 4 + c) * 64 + lane];
      const f32x4 g1 = sOut[(2 * 4 + c) * 64 + lane], u1 = sOut[(3 * 4 + c) * 64 + lane];
      float z[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = silu_f32(g0[r]) * u0[r];
        z[4 + r] = silu_f32(g1[r]) * u1[r];
      }
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(z[r]));
      // the 32 features of a token live in lanes l16, l16+16, l16+32, l16+48
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
      const int tk = tg * kMxTok + 16 * c + l16;
      if (tk < cnt) {
        const int64_t pos = pos0 + tk;
        uint8_t* o = static_cast<uint8_t*>(g.out) + pos * g.out_ld;
        *reinterpret_cast<uint32_t*>(o + f0 + 4 * q) = w0;
        *reinterpret_cast<uint32_t*>(o + f0 + 16 + 4 * q) = w1;
        if (q == 0) g.out_scale[pos * (g.out_ld / 32) + f0 / 32] = (uint8_t)sc;
      }
    } else {
      // wave c writes column tile c: 16 tokens x 64 features
      const int c = wave;
      const int tk = tg * kMxTok + 16 * c + l16;
      if (tk < cnt) {
        const int64_t orow = rm.sorted_ids[pos0 + tk];
        uint16_t* o = static_cast<uint16_t*>(g.out) + orow * g.out_ld;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 v = sOut[(t * 4 + c) * 64 + lane];
          uint32_t h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(v[r]);
          *reinterpret_cast<uint2*>(o + f0 + 16 * t + 4 * q) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
      }
    }
    lds_barrier();
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

template <int EPI>
static hipError_t launch_mxfp8(const GemmArgs& g, hipStream_t s) {
  const dim3 grid(g.nfeat / (EPI == kEpiGateUp ? 32 : 64), (unsigned)g.max_active);
  const int nsteps = g.kdim / 128;
  if (nsteps % 2 == 0)
    hipLaunchKernelGGL((gemm_stream_mxfp8_kernel<EPI, 2>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_stream_mxfp8_kernel<EPI, 1>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_stream_mxfp8(const GemmArgs& g, hipStream_t s) {
  return g.epi == kEpiGateUp ? launch_mxfp8<kEpiGateUp>(g, s) : launch_mxfp8<kEpiDown>(g, s);
}

}  // namespace moe
