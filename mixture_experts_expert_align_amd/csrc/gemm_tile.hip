// LDS-tiled grouped GEMM (bf16 in, fp32 accumulate) for the two matmuls of
// the expert computation ("Fused MoE Modular Kernel", apply(): matmul with
// W1, act + mul, matmul with W2, unpermute).
//
// One workgroup computes a 128 x 128 tile: 128 rows of one expert (a tile of
// the padded sorted routes, or of a batched expert slab) against 128 weight
// rows, stepping through the contraction in 64-wide slices.  Both slices are
// staged in LDS (double buffered, 16-byte chunks XOR-swizzled by row so that
// the MFMA fragment reads of 32 rows hit distinct banks) and multiplied with
// v_mfma_f32_32x32x16_bf16; four waves each own a 64 x 64 quarter.
//
// W1 (epilogue kGateUp): the 128 weight rows are 64 gate rows and the 64
// matching up rows, so each wave holds gate and up values of the same
// (row, feature) in the same register and forms silu(gate) * up before the
// only store (bf16 z, row = sorted position).  A rows are gathered through
// the route list (token = flat slot / topk) while loading; padding routes
// load zeros.
// W2 (epilogue kDown): the epilogue writes each real route's row straight to
// its (token, slot) row of y (the per-(token, slot) buffer of the Cake
// MegaMoE EP16 page, section 3); padding rows are dropped.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;

__device__ __forceinline__ int swz(int row, int kc) { return row * BK + ((kc ^ (row & 7)) << 3); }

template <int EPI>
__global__ void __launch_bounds__(NT) gemm_tile_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const RowMap& rm = g.rows;

  // ---- which rows / expert
  int expert;
  int64_t row0;       // first row: sorted position (contiguous) or slab row e*max_tokens + r0
  int nrows_valid;    // batched: rows of this tile below the count
  if (rm.layout == 0) {
    const int t = blockIdx.y;
    if ((int64_t)t * BM >= rm.num_post[0]) return;
    expert = rm.block_expert[t];
    row0 = (int64_t)t * BM;
    nrows_valid = BM;
  } else {
    const int tpe = (rm.max_tokens + BM - 1) / BM;
    expert = blockIdx.y / tpe;
    const int r0 = (blockIdx.y - expert * tpe) * BM;
    const int cnt = min(rm.counts[expert], rm.max_tokens);
    if (r0 >= cnt) return;
    row0 = (int64_t)expert * rm.max_tokens + r0;
    nrows_valid = min(BM, cnt - r0);
  }
  const int col0 = blockIdx.x * (EPI == kEpiGateUp ? BN / 2 : BN);
  const int K = g.kdim;

  // ---- this thread's global rows: chunk c = tid + 256*i -> row c/8, 16B chunk c%8
  const int kc = tid & 7;
  const uint16_t* pa[4];
  const uint16_t* pb[4];
  const uint16_t* act = static_cast<const uint16_t*>(g.act);
  const uint16_t* wexp = static_cast<const uint16_t*>(g.w) + (int64_t)expert * g.w_expert_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const uint16_t* p = nullptr;
    if (rm.layout == 0) {
      if (EPI == kEpiGateUp) {
        const int sid = rm.sorted_ids[row0 + r];
        if (sid != rm.sentinel) p = act + (int64_t)(sid / rm.topk) * g.act_ld;
      } else {
        p = act + (row0 + r) * g.act_ld;
      }
    } else if (r < nrows_valid) {
      p = act + (row0 + r) * g.act_ld;
    }
    pa[i] = p ? p + kc * 8 : nullptr;
    int wrow;
    if (EPI == kEpiGateUp) {
      const int f = col0 + (r & 63);
      const bool up = r >= 64;
      wrow = g.w1_order == 0 ? (up ? g.I + f : f) : (32 * (f >> 4) + (f & 15) + (up ? 16 : 0));
    } else {
      wrow = col0 + r;
    }
    pb[i] = wexp + (int64_t)wrow * K + kc * 8;
  }

  i32x4 ra[4], rb[4];
  const i32x4 zero = {0, 0, 0, 0};
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = pa[i] ? *reinterpret_cast<const i32x4*>(pa[i] + k0) : zero;
      rb[i] = *reinterpret_cast<const i32x4*>(pb[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<i32x4*>(&sA[buf][swz(r, kc)]) = ra[i];
      *reinterpret_cast<i32x4*>(&sB[buf][swz(r, kc)]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // B columns (weight rows) of this wave's two MFMA tiles
  int ncol[2];
  if (EPI == kEpiGateUp) {
    ncol[0] = wn * 32 + (lane & 31);        // gate
    ncol[1] = 64 + wn * 32 + (lane & 31);   // matching up
  } else {
    ncol[0] = wn * 64 + (lane & 31);
    ncol[1] = wn * 64 + 32 + (lane & 31);
  }
  const int arow0 = wm * 64 + (lane & 31);

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kcf = 2 * s + (lane >> 5);
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = arow0 + mi * 32;
        fa[mi] = as_bf16x8(*reinterpret_cast<const i32x4*>(&sA[buf][swz(r, kcf)]));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        fb[ni] = as_bf16x8(*reinterpret_cast<const i32x4*>(&sB[buf][swz(ncol[ni], kcf)]));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  acc[mi][ni][r] is row wm*64 + mi*32 + 8*(r/4) + 4*(lane/32) + r%4
  // of the tile, weight column ncol[ni].
  uint16_t* out = static_cast<uint16_t*>(g.out);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (EPI == kEpiGateUp) {
        if (rl >= nrows_valid) continue;
        const float z = silu_f32(acc[mi][0][r]) * acc[mi][1][r];
        out[(row0 + rl) * g.out_ld + col0 + wn * 32 + (lane & 31)] = (uint16_t)f32_to_bf16_rne(z);
      } else {
        int64_t orow;
        if (rm.layout == 0) {
          const int sid = rm.sorted_ids[row0 + rl];
          if (sid == rm.sentinel) continue;
          orow = sid;
        } else {
          if (rl >= nrows_valid) continue;
          orow = row0 + rl;
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          out[orow * g.out_ld + col0 + wn * 64 + ni * 32 + (lane & 31)] =
              (uint16_t)f32_to_bf16_rne(acc[mi][ni][r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_tile_bf16(const GemmArgs& g, hipStream_t s) {
  const int ncolt = g.epi == kEpiGateUp ? g.nfeat / (BN / 2) : g.nfeat / BN;
  int64_t nrowt;
  if (g.rows.layout == 0) nrowt = g.max_tiles;
  else nrowt = (int64_t)g.E * ((g.rows.max_tokens + BM - 1) / BM);
  dim3 grid(ncolt, (unsigned)nrowt);
  if (g.epi == kEpiGateUp)
    hipLaunchKernelGGL(gemm_tile_bf16_kernel<kEpiGateUp>, grid, dim3(NT), 0, s, g);
  else
    hipLaunchKernelGGL(gemm_tile_bf16_kernel<kEpiDown>, grid, dim3(NT), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
