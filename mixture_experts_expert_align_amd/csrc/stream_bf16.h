// The bf16 streaming strip shared by the two-launch streaming GEMMs and the
// single-launch expert computation: a group of waves computes 16 output
// features of one expert for all of its routed rows, weights streamed from
// HBM straight into the MFMA row operand.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// KS waves (wave = 0 .. ks-1 here) own 16 output features of one expert
// and split the contraction into ks equal runs; each wave streams its run of
// the weight rows with a three-deep register pipeline, the partial sums
// meet in LDS and wave 0 adds them in wave order (a fixed order, so every
// run gives the same bits) before the epilogue.  Splitting the contraction
// keeps each task short, so the last wave of work on the chip is short too;
// with a whole contraction per workgroup the tail of the grid left much of
// the chip idle.
//   kGateUp: two 16-row tiles: the gate rows and the matching up rows of the
//            16 features; epilogue z = silu(gate) * up, bf16, row = position.
//   kDown:   one 16-row tile of W2; epilogue writes y rows per (token, slot).
// Per lane and 128-wide step, lane group q takes the four 16-byte pieces at
// k + 8q + 32j (j = 0..3) of its row: the four groups of one load
// instruction read 64 contiguous bytes of each of 16 rows.
// red: LDS for ks x (2 or 1 tiles) x 64 f32x4.  Every thread of the
// workgroup calls this with the same slot (the barriers are workgroup-wide).
//
// SPLIT (kGateUp only): the strip's gate and up tiles go to two groups of ks
// waves (ut = 0 gate, 1 up) instead of each wave streaming both: half the
// registers per wave, and the same partial sums added in the same order, so
// the same bits.  red keeps the [ks][2][64] layout; the gate group's wave 0
// writes z.
// COH: the row map, and for W2 the activations (z), were written earlier in
// the same launch by other workgroups, maybe on another XCD, whose L2 is not
// kept coherent with this one: they are read with device-coherent loads
// (sc1), and W1 writes z with device-coherent stores, so producer and
// consumer need no L2 write-back or invalidate between them.
template <bool COH>
__device__ __forceinline__ int rd_rows(const int32_t* p) {
  return COH ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
}

// The routed rows of one active-expert slot: the expert, its number of
// rows and its first sorted position.
struct SlotRows {
  int e, cnt, pos0;
};

// False when the slot is past the number of active experts.
template <bool COH>
__device__ __forceinline__ bool slot_rows(const GemmArgs& g, int slot, SlotRows& r) {
  const RowMap& rm = g.rows;
  if (slot >= rd_rows<COH>(rm.active + g.max_active)) return false;
  r.e = rd_rows<COH>(rm.active + slot);
  r.cnt = rd_rows<COH>(rm.counts + r.e);
  r.pos0 = rd_rows<COH>(rm.offsets + r.e);
  return true;
}

// row_of(tk): the sorted id (flat slot t*topk+j) at position pos0 + tk.
template <int EPI, bool SPLIT = false, bool COH = false, typename RowOf>
__device__ __forceinline__ void stream_bf16_strip(const GemmArgs& g, const SlotRows& sr, RowOf row_of, int f0,
                                                  int wave, int ks, f32x4* red, int ut = 0) {
  constexpr int NT = EPI == kEpiGateUp ? 2 : 1;               // tiles of the strip
  constexpr int NTL = EPI == kEpiGateUp && !SPLIT ? 2 : 1;     // tiles this wave streams
  constexpr int kActPolicy = EPI == kEpiDown && COH ? 16 : 0;  // sc1
  const int lane = threadIdx.x & 63;
  const RowMap& rm = g.rows;
  const int e = sr.e;
  const int cnt = sr.cnt;
  const int pos0 = sr.pos0;
  const int K = g.kdim;
  const int KW = K / ks;                      // contraction run of this wave
  const int q = lane >> 4;
  const int l16 = lane & 15;
  const int kbase = wave * KW + 8 * q;
  // Buffer loads: the expert's weights and the activations as two buffer
  // resources, per-lane 32-bit byte offsets, the step's k in the scalar
  // offset.  A lane without a token gets an offset past the buffer's size,
  // which the hardware's range check turns into zeros.
  const uint16_t* wexp = static_cast<const uint16_t*>(g.w) + (int64_t)e * g.w_expert_stride;
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wexp, g.w_expert_stride * 2);
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(g.act, g.act_bytes);
  uint32_t wo[NTL];
  if (EPI == kEpiGateUp && SPLIT) {
    wo[0] = (uint32_t)(w1_row(f0 + l16, ut != 0, g.I, g.w1_order) * K + kbase) * 2u;
  } else if (EPI == kEpiGateUp) {
    wo[0] = (uint32_t)(w1_row(f0 + l16, false, g.I, g.w1_order) * K + kbase) * 2u;
    wo[NTL - 1] = (uint32_t)(w1_row(f0 + l16, true, g.I, g.w1_order) * K + kbase) * 2u;
  } else {
    wo[0] = (uint32_t)((f0 + l16) * K + kbase) * 2u;
  }
  uint16_t* out = static_cast<uint16_t*>(g.out);
  const int nsteps = KW / 128;

  for (int tg = 0; tg * 16 < cnt; ++tg) {
    const int tk = tg * 16 + l16;
    const bool tv = tk < cnt;
    const int pos = pos0 + tk;
    uint32_t ao = 0x80000000u;               // past the end: loads return 0
    if (tv) {
      const int64_t row = EPI == kEpiGateUp ? row_of(tk) / rm.topk : pos;
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
        b[st][j] = __builtin_amdgcn_raw_buffer_load_b128(ar, ao + 64 * j, 2 * k, kActPolicy);
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
    for (int t = 0; t < NTL; ++t) red[(wave * NT + (SPLIT ? ut : t)) * 64 + lane] = acc[t];
    __syncthreads();
    if (wave == 0 && (!SPLIT || ut == 0)) {
      f32x4 fin[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 sum = red[t * 64 + lane];
        for (int w = 1; w < ks; ++w) sum += red[(w * NT + t) * 64 + lane];
        fin[t] = sum;
      }
      // fin[t][r]: weight row 4*q + r of tile t, token column l16
      if (tv) {
        uint32_t h[4];
        int64_t o;
        if (EPI == kEpiGateUp) {
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(silu_f32(fin[0][r]) * fin[NT - 1][r]);
          o = (int64_t)pos * g.out_ld;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(fin[0][r]);
          o = (int64_t)row_of(tk) * g.out_ld;
        }
        const uint64_t v = (uint64_t)(h[0] | (h[1] << 16)) | ((uint64_t)(h[2] | (h[3] << 16)) << 32);
        uint64_t* dst = reinterpret_cast<uint64_t*>(out + o + f0 + 4 * q);
        if (EPI == kEpiGateUp && COH)
          __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe
