// Streaming grouped GEMM with MXFP8 weights and activations for experts that
// hold few rows (one rank's local-expert share of a large layer): the page
// "Cake MegaMoE EP16 backend for BF16 activations and MXFP8 weights" runs
// this share with block-32 E4M3 codes and UE8M0 scales on both operands.
//
// The matmuls are bound by reading the active experts' weights from HBM
// once: each wave's 16 weight rows go from HBM straight into the row operand
// of the scaled MFMA, no LDS; the expert's routed tokens, already gathered
// and quantised in sorted order, are staged in LDS 64 at a time and shared
// by the workgroup's waves.
//
// Grid: (feature strips, active experts).  The active-expert list comes from
// the align step, so the grid depends only on the plan; workgroups whose
// slot is past the number of active experts leave at once.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

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
// A workgroup of 8 waves owns 128 weight rows of one expert, 16 per wave, and
// the expert's routed tokens, 64 per pass.  Weights stream from HBM straight
// into registers, CS 128-wide steps ahead (CS register sets, one per step of
// a chunk).  The tokens' codes and scales are staged in LDS a chunk of CS
// steps at a time (two buffers), by buffer loads that write LDS directly, so
// staging costs no registers and the waves meet at a barrier once per chunk.
// The compiler does not track those loads, so the wait before each chunk's
// barrier is explicit, counted from a fixed issue order: a chunk issues one
// weight-scale load (a 16-step group), then in each step the 2 weight loads
// of the step CS ahead, and after its barrier the CS + 1 staging loads of the
// chunk after next.
//   kGateUp: wave w holds the gate (w even) or up (w odd) rows of features
//            f0 + 16 (w / 2) .. +15; z = silu(gate) * up per token, quantised
//            per 32 features (one MX block = waves 4b .. 4b+3) in the
//            epilogue, which gathers the tiles in LDS.
//   kDown:   wave w holds rows f0 + 16 w .. +15 and writes them as bf16 y rows
//            per (token, slot) straight from its accumulators.
constexpr int kMxTok = 64;                       // tokens per pass
constexpr int kMxWaves = 8;
constexpr int kMxStepA = kMxTok * 128;           // token code bytes per step
constexpr int kMxStepAS = kMxTok * 4;            // token scale bytes per step (one wave's slot)

// CS: steps per chunk (4, 2 or 1, dividing the contraction's step count);
// the weights stream CS steps ahead.  TT: 16-row weight tiles per wave (2
// for W1: each staged activation fragment then feeds two MFMAs, and the
// workgroup's 256 weight rows amortise the activation staging, which costs
// the address unit as many lane requests per byte as the weights do).
template <int EPI, int CS, int TT>
__global__ void __launch_bounds__(64 * kMxWaves, 4) gemm_stream_mxfp8_kernel(GemmArgs g) {
  constexpr int kChunk = CS * kMxStepA + kMxWaves * kMxStepAS;   // one LDS buffer
  // the W1 epilogue gathers every wave's accumulators ([wave][tile][token tile][lane])
  constexpr int kOutBytes = EPI == kEpiGateUp ? kMxWaves * TT * 4 * 64 * 16 : 0;
  constexpr int kLds = 2 * kChunk > kOutBytes ? 2 * kChunk : kOutBytes;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const RowMap& rm = g.rows;
  // work item (slot, feature block): the hardware deals blocks to the 8 XCDs
  // round robin (block b on XCD b % 8); each XCD takes a contiguous range of
  // the items of the active slots, so the feature blocks of one expert share
  // an XCD and its L2 serves them the expert's staged activation rows
  const int nfb = g.nfeat / ((EPI == kEpiGateUp ? 64 : 128) * TT);
  const int64_t items = (int64_t)nfb * rm.active[g.max_active];
  const int64_t per_xcd = (items + 7) / 8;
  const int64_t k = blockIdx.x / 8;
  const int64_t item = (blockIdx.x % 8) * per_xcd + k;
  if (k >= per_xcd || item >= items) return;
  const int slot = (int)(item / nfb);
  const int e = rm.active[slot];
  const int cnt = rm.counts[e];
  const int pos0 = rm.offsets[e];
  const int K = g.kdim;
  const int KB = K / 32;
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int f0 = (int)(item % nfb) * (EPI == kEpiGateUp ? 64 : 128) * TT;
  const int nsteps = K / 128;
  const int nchunks = nsteps / CS;

  const uint8_t* wexp = static_cast<const uint8_t*>(g.w) + (int64_t)e * g.w_expert_stride;
  const uint8_t* wsexp = g.w_scale + (int64_t)e * (g.w_expert_stride / 32);
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride);
  const __amdgpu_buffer_rsrc_t wsr = buffer_rsrc(wsexp, g.w_expert_stride / 32);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
  const __amdgpu_buffer_rsrc_t asr = buffer_rsrc(g.act_scale, g.act_bytes / 32);
  // tile tt of wave w: W1 gate (w even) or up (w odd) rows of features
  // f0 + 16 (TT (w / 2) + tt) + l16; W2 rows f0 + 16 (TT w + tt) + l16
  uint32_t wo[TT], wso[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int row = EPI == kEpiGateUp
                        ? w1_row(f0 + 16 * (TT * (wave >> 1) + tt) + l16, (wave & 1) != 0, g.I, g.w1_order)
                        : f0 + 16 * (TT * wave + tt) + l16;
    wo[tt] = (uint32_t)(row * K + 16 * q);     // lane: row l16, bytes 16q of a step (+64)
    wso[tt] = (uint32_t)(row * KB + 16 * q);
  }
  // weight scales, 16 steps at a time: lane (row l16, group q) loads the 4
  // words of steps 4q .. 4q+3 of a 16-step group (16 bytes), and each step
  // takes its word from the lane that holds it (one load per chunk instead
  // of one per step: every load instruction costs the address unit 64 lane
  // requests, whatever its width)
  const int ngroups = (nsteps + 15) / 16;

  __shared__ __attribute__((aligned(16))) uint8_t sA[kLds];
  // within a buffer: step sub's codes at sub * kMxStepA, laid out [token tile
  // c][half j][lane] (1 KB blocks: lane i holds token 16c + i % 16, bytes
  // 64j + 16 (i / 16) of the step), then one 256-byte slot per wave: wave w
  // loads the scale words of all 64 tokens for step w % CS (waves past CS
  // load copies, so every wave issues the same loads and none is masked)

  for (int tg = 0; tg * kMxTok < cnt; ++tg) {
    // this wave stages block (c, j) = (wave / 2, wave % 2) of every step and
    // the scale words of step wave % CS; past the count: zeros
    const int tk = tg * kMxTok + 16 * (wave >> 1) + l16;
    const uint32_t xo = tk < cnt ? (uint32_t)((int64_t)(pos0 + tk) * g.act_ld + 64 * (wave & 1) + 16 * q) : 0x80000000u;
    const int ts = tg * kMxTok + lane;
    const uint32_t xso = ts < cnt ? (uint32_t)((int64_t)(pos0 + ts) * (g.act_ld / 32)) : 0x80000000u;
    const int ssub = wave % CS;
    // CS + 1 loads per wave: chunk ch into buffer buf
    auto stage = [&](int ch, int buf) {
      uint8_t* base = sA + buf * kChunk;
#pragma unroll
      for (int sub = 0; sub < CS; ++sub)
        lds_load16(ar, base + sub * kMxStepA + wave * 1024, xo, (ch * CS + sub) * 128);
      lds_load4(asr, base + CS * kMxStepA + wave * kMxStepAS, xso, (ch * CS + ssub) * 4);
    };
    // 2 TT loads: the weights of step st into register set i
    i32x8 wa[CS][TT];
    auto wload = [&](int i, int st) {
      const int k = st * 128;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(wr, wo[tt], k, 0);
        const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(wr, wo[tt] + 64, k, 0);
        wa[i][tt] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
    };
    // TT loads: the scale words of 16-step group gi (past the end: the last)
    i32x4 scur[TT], snext[TT];   // the current chunk's group, the next chunk's
    auto sload = [&](int gi) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        snext[tt] = __builtin_amdgcn_raw_buffer_load_b128(wsr, wso[tt], 64 * min(gi, ngroups - 1), 0);
    };
    f32x4 acc[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[tt][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
    auto mma = [&](int i, int buf, int sub, int st) {
      const uint8_t* base = sA + buf * kChunk;
      // step st is word st % 4 of the lanes of group q = (st % 16) / 4
      const int w4 = st & 3;
      uint32_t wsw[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int word = w4 == 0 ? scur[tt][0] : w4 == 1 ? scur[tt][1] : w4 == 2 ? scur[tt][2] : scur[tt][3];
        wsw[tt] = (uint32_t)__shfl(word, l16 + 16 * ((st & 15) >> 2));
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 xl = *reinterpret_cast<const i32x4*>(base + sub * kMxStepA + (2 * c) * 1024 + 16 * lane);
        const i32x4 xh = *reinterpret_cast<const i32x4*>(base + sub * kMxStepA + (2 * c + 1) * 1024 + 16 * lane);
        const i32x8 xb = (i32x8){xl[0], xl[1], xl[2], xl[3], xh[0], xh[1], xh[2], xh[3]};
        const uint32_t xsw =   // wave sub's slot holds step sub
            *reinterpret_cast<const uint32_t*>(base + CS * kMxStepA + sub * kMxStepAS + 4 * (16 * c + l16));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[tt][c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wa[i][tt], xb, acc[tt][c], 0, 0, 0, (int)(wsw[tt] >> (8 * q)), 0, (int)(xsw >> (8 * q)));
      }
    };
    // the CS steps of chunk ch (LDS buffer buf): multiply step s, then load
    // the weights of step s + CS into the freed register set (past the end:
    // the last step again, unused)
    auto chunk = [&](int ch, int buf) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) scur[tt] = snext[tt];   // loaded a chunk ago
      sload(((ch + 1) * CS) / 16);
      issue_order();
#pragma unroll
      for (int sub = 0; sub < CS; ++sub) {
        mma(sub, buf, sub, ch * CS + sub);
        wload(sub, min((ch + 1) * CS + sub, nsteps - 1));
        // also: one step's token fragments live at a time
        issue_order();
      }
    };

    // prologue: chunk 0 staged, the weights of steps 0 .. CS-1 loaded, chunk 1
    // staged (the loop's issue order: weights, then the next staging)
    stage(0, 0);
    issue_order();
    sload(0);
    issue_order();
#pragma unroll
    for (int sub = 0; sub < CS; ++sub) {
      wload(sub, min(sub, nsteps - 1));
      issue_order();
    }
    stage(min(1, nchunks - 1), 1);
    issue_order();
    // chunk 0's loads are older than the scale groups' (TT), the weights'
    // (2 TT CS) and chunk 1's (CS + 1)
    wait_vm<TT + 2 * TT * CS + CS + 1>();
    lds_barrier();
    for (int ch = 0; ch + 1 < nchunks; ++ch) {
      const int buf = ch & 1;
      chunk(ch, buf);
      // chunk ch+1's staging loads are older than the TT scale groups and
      // the 2 TT CS weight loads of this chunk; then every wave's share is in
      // place and chunk ch is read
      wait_vm<TT + 2 * TT * CS>();
      lds_barrier();
      stage(min(ch + 2, nchunks - 1), buf);   // past the end: reloads the last chunk, unused
      issue_order();
    }
    chunk(nchunks - 1, (nchunks - 1) & 1);
    // drain the remaining (unused) loads before LDS is reused
    wait_vm<0>();
    lds_barrier();

    // acc[tt][c][r]: weight row 4*q + r of this wave's tile tt, token
    // tg*64 + 16*c + l16
    if (EPI == kEpiGateUp) {
      f32x4* sOut = reinterpret_cast<f32x4*>(sA);      // [wave][tile][token tile][lane]
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) sOut[((wave * TT + tt) * 4 + c) * 64 + lane] = acc[tt][c];
      lds_barrier();
      // units (MX block b = features f0 + 32 b .. +31, token tile c): 8 TT
      // of them, wave w finishes units w + 8 v (v < TT), unit u being
      // (b, c) = (u / 4, u % 4).  The gate rows of features 32 b + 16 h +
      // (0..15) are tile h' of wave gw and the up rows tile h' of wave gw + 1,
      // with (gw, h') = (4 b + 2 h, 0) for TT = 1 and (2 b, h) for TT = 2.
#pragma unroll
      for (int v = 0; v < TT; ++v) {
      const int unit = wave + kMxWaves * v;
      const int c = unit & 3, b = unit >> 2;
      auto tile = [&](int h, int up) {
        const int gw = TT == 1 ? 4 * b + 2 * h : 2 * b;
        const int ht = TT == 1 ? 0 : h;
        return sOut[(((gw + up) * TT + ht) * 4 + c) * 64 + lane];
      };
      const f32x4 g0 = tile(0, 0), u0 = tile(0, 1);
      const f32x4 g1 = tile(1, 0), u1 = tile(1, 1);
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
      const uint32_t w0 = e4m3_pack4(z[0] * inv, z[1] * inv, z[2] * inv, z[3] * inv);
      const uint32_t w1 = e4m3_pack4(z[4] * inv, z[5] * inv, z[6] * inv, z[7] * inv);
      const int t = tg * kMxTok + 16 * c + l16;
      if (t < cnt) {
        const int64_t pos = pos0 + t;
        uint8_t* o = static_cast<uint8_t*>(g.out) + pos * g.out_ld;
        const int fb = f0 + 32 * b;
        *reinterpret_cast<uint32_t*>(o + fb + 4 * q) = w0;
        *reinterpret_cast<uint32_t*>(o + fb + 16 + 4 * q) = w1;
        if (q == 0) g.out_scale[pos * (g.out_ld / 32) + fb / 32] = (uint8_t)sc;
      }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = tg * kMxTok + 16 * c + l16;
        if (t < cnt) {
          const int64_t orow = rm.sorted_ids[pos0 + t];
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            uint16_t* o = static_cast<uint16_t*>(g.out) + orow * g.out_ld + f0 + 16 * (TT * wave + tt) + 4 * q;
            uint32_t h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(acc[tt][c][r]);
            *reinterpret_cast<uint2*>(o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
          }
        }
      }
    }
    lds_barrier();
  }
}

}  // namespace

template <int EPI>
static hipError_t launch_mxfp8(const GemmArgs& g, hipStream_t s) {
  const int nsteps = g.kdim / 128;
  // W1: two tiles per wave (128 features per workgroup) and chunks of 2
  // steps when the features divide; W2 keeps one tile and chunks of 2 steps:
  // with more, its epilogue's registers no longer fit the 128 that let two
  // workgroups share a CU
  // one block per (slot, feature block) work item of the largest possible
  // slot count, rounded up to the 8 XCDs
  auto blocks = [&](int feats) { return dim3((unsigned)((((int64_t)g.nfeat / feats) * g.max_active + 7) / 8 * 8)); };
  if (EPI == kEpiGateUp && g.nfeat % 128 == 0 && nsteps % 2 == 0) {
    hipLaunchKernelGGL((gemm_stream_mxfp8_kernel<kEpiGateUp, 2, 2>), blocks(128), dim3(64 * kMxWaves), 0, s, g);
    return hipGetLastError();
  }
  const dim3 grid = blocks(EPI == kEpiGateUp ? 64 : 128);
  if (EPI == kEpiGateUp && nsteps % 4 == 0)
    hipLaunchKernelGGL((gemm_stream_mxfp8_kernel<kEpiGateUp, 4, 1>), grid, dim3(64 * kMxWaves), 0, s, g);
  else if (nsteps % 2 == 0)
    hipLaunchKernelGGL((gemm_stream_mxfp8_kernel<EPI, 2, 1>), grid, dim3(64 * kMxWaves), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_stream_mxfp8_kernel<EPI, 1, 1>), grid, dim3(64 * kMxWaves), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_stream_mxfp8(const GemmArgs& g, hipStream_t s) {
  return g.epi == kEpiGateUp ? launch_mxfp8<kEpiGateUp>(g, s) : launch_mxfp8<kEpiDown>(g, s);
}

}  // namespace moe
