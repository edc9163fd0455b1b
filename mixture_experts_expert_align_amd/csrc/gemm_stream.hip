// Streaming grouped GEMMs with bf16 weights for experts that hold few rows
// (decode batches), one launch per matmul; the strip itself is in
// stream_bf16.h, shared with the single-launch path.
//
// With few rows per expert the matmuls are bound by reading the active
// experts' weights from HBM once.  Each wave owns a strip of weight rows and
// the whole contraction: the weight rows go from HBM straight into the row
// operand of the MFMA (16 rows x the contraction slice, each lane reading a
// contiguous run of one row, no LDS), and the expert's routed tokens sit in
// the other operand, up to 16 per pass, read from L2.  The page
// "Mixture-of-Experts kernel engineering on SageMaker" ("Swap-AB
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
#include "stream_bf16.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ bf16 --
// Grid (I or K / 16 feature strips, active-expert slots); KS waves per strip.
template <int EPI, int KS>
__global__ void __launch_bounds__(64 * KS) gemm_stream_bf16_kernel(GemmArgs g) {
  __shared__ f32x4 red[KS * (EPI == kEpiGateUp ? 2 : 1) * 64];
  SlotRows sr;
  if (!slot_rows<false>(g, blockIdx.y, sr)) return;
  const int32_t* sid = g.rows.sorted_ids + sr.pos0;
  stream_bf16_strip<EPI>(g, sr, [&](int tk) { return sid[tk]; }, blockIdx.x * 16, threadIdx.x >> 6, KS, red);
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

}  // namespace moe
