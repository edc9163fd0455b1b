// Bandwidth-bound kernels: the top-k weighted reductions and the MXFP8
// codec.
//
// Reductions ("Fused MoE Modular Kernel", section "TopKWeightAndReduce"):
// every output element is a float32 sum in a fixed order (ascending top-k
// slot for the contiguous format; ascending (expert, row) for the batched
// format via the CSR list the align step builds), one fused multiply-add per
// term, rounded once to bf16.  No atomics, so every run gives the same bits;
// an empty sum stays +0.0 (the convention of the Cake deterministic grouped
// GEMM page, section 2).
//
// Codec (page "Cake MegaMoE EP16 backend for BF16 activations and MXFP8
// weights", section 2): one thread per 32-element block: block max, scale
// code, then E4M3 round-to-nearest-even of each element over the scale.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int NT = 256;
constexpr int kBatch = 8;   // reduce terms whose loads are issued together

__device__ __forceinline__ void fma8(float* acc, float w, i32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = (uint32_t)v[i];
    acc[2 * i] = fmaf(w, bf16_to_f32(u & 0xffffu), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, bf16_to_f32(u >> 16), acc[2 * i + 1]);
  }
}

__device__ __forceinline__ i32x4 pack8(const float* acc) {
  i32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (int)(f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16));
  return o;
}

// One workgroup per token and span of NT * cpt chunks of 8 columns: the
// token's slots are read once per thread, then each thread reduces up to cpt
// (<= kChunks) chunks of its columns — more per thread for many tokens (the
// slot reads amortised), one for few (more workgroups in flight).  Slots go
// in batches of kBatch: all ids,
// then all map entries, then every valid slot's row, then the FMAs in
// ascending slot order (the same sum as one slot at a time, without a chain
// of dependent loads per slot).
constexpr int kChunks = 4;

__global__ void __launch_bounds__(NT) reduce_contiguous_kernel(const uint16_t* __restrict__ y,
                                                               const int32_t* __restrict__ ids,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ emap, int G,
                                                               uint16_t* __restrict__ out, int64_t M,
                                                               int topk, int64_t K, int E,
                                                               int32_t* __restrict__ sync_zero,
                                                               int64_t sync_lines, int cpt) {
  if (sync_zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int64_t i = threadIdx.x; i < sync_lines; i += NT) sync_zero[32 * i] = 0;
  const int64_t t = blockIdx.x;
  const int64_t K8 = K / 8;
  const int64_t cbeg = (int64_t)blockIdx.y * NT * cpt + threadIdx.x;
  float acc[kChunks][8];
#pragma unroll
  for (int u = 0; u < kChunks; ++u)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
  for (int j0 = 0; j0 < topk; j0 += kBatch) {
    const int64_t s0 = t * topk + j0;
    int id[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) id[q] = j0 + q < topk ? ids[s0 + q] : -1;
    if (emap) {
#pragma unroll
      for (int q = 0; q < kBatch; ++q) id[q] = (id[q] >= 0 && id[q] < G) ? emap[id[q]] : -1;   // global -> local
    }
    float wt[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) wt[q] = id[q] >= 0 && id[q] < E ? w[s0 + q] : 0.f;
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int64_t c = cbeg + (int64_t)NT * u;
      if (u >= cpt || c >= K8) break;
      i32x4 v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (id[q] >= 0 && id[q] < E) v[q] = *reinterpret_cast<const i32x4*>(y + (s0 + q) * K + 8 * c);
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (id[q] >= 0 && id[q] < E) fma8(acc[u], wt[q], v[q]);
    }
  }
#pragma unroll
  for (int u = 0; u < kChunks; ++u) {
    const int64_t c = cbeg + (int64_t)NT * u;
    if (u < cpt && c < K8) *reinterpret_cast<i32x4*>(out + t * K + 8 * c) = pack8(acc[u]);
  }
}

// With an expert map (one rank's share of the experts: most slots belong to
// experts held elsewhere) the per-token chain of dependent loads (ids, then
// the map, then the rows) dominates, so a workgroup takes kMapTok tokens at
// once.  Wave tt resolves token tt: lane j loads id and weight of slot j
// together, maps the id, and the local slots are compacted in ascending slot
// order into LDS (a ballot).  Then thread c owns 8-column chunk c of all
// kMapTok tokens: the first kMapBatch terms of every token are loaded
// together and added, the rest (tokens with more local slots) kMapBatch at a
// time.  Same terms, order and arithmetic as reduce_contiguous_kernel, so the
// same bits.  Workgroup size: the chunks of a row rounded up to waves, at
// least kMapTok waves.
constexpr int kMapTok = 4;
constexpr int kMapBatch = 2;
constexpr int kMapMaxTopk = 64;

__global__ void __launch_bounds__(1024) reduce_map_kernel(const uint16_t* __restrict__ y,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ emap, int G,
                                                          uint16_t* __restrict__ out, int64_t M, int topk,
                                                          int64_t K, int E, int32_t* __restrict__ sync_zero,
                                                          int64_t sync_lines) {
  __shared__ int s_row[kMapTok * kMapMaxTopk];
  __shared__ float s_w[kMapTok * kMapMaxTopk];
  __shared__ int s_n[kMapTok];
  if (sync_zero && blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < sync_lines; i += blockDim.x) sync_zero[32 * i] = 0;
  const int64_t t0 = (int64_t)blockIdx.x * kMapTok;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < kMapTok) {
    const int64_t t = t0 + wave;
    bool valid = false;
    float wt = 0.f;
    if (t < M && lane < topk) {
      const int64_t sl = t * topk + lane;
      int id = ids[sl];
      wt = w[sl];
      if (emap) id = (id >= 0 && id < G) ? emap[id] : -1;   // global -> local
      valid = id >= 0 && id < E;
    }
    const uint64_t mask = __ballot(valid);
    if (valid) {
      const int r = __popcll(mask & ((1ull << lane) - 1ull));
      s_row[wave * kMapMaxTopk + r] = (int)(t * topk + lane);
      s_w[wave * kMapMaxTopk + r] = wt;
    }
    if (lane == 0) s_n[wave] = __popcll(mask);
  }
  __syncthreads();
  const int64_t c = threadIdx.x;
  if (c >= K / 8) return;
  float acc[kMapTok][8];
  int n[kMapTok];
#pragma unroll
  for (int tt = 0; tt < kMapTok; ++tt) {
    n[tt] = s_n[tt];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[tt][q] = 0.f;
  }
  auto add = [&](int tt, int q0) {
    i32x4 v[kMapBatch];
#pragma unroll
    for (int q = 0; q < kMapBatch; ++q)
      if (q0 + q < n[tt])
        v[q] = *reinterpret_cast<const i32x4*>(y + (int64_t)s_row[tt * kMapMaxTopk + q0 + q] * K + 8 * c);
#pragma unroll
    for (int q = 0; q < kMapBatch; ++q)
      if (q0 + q < n[tt]) fma8(acc[tt], s_w[tt * kMapMaxTopk + q0 + q], v[q]);
  };
  {
    // the first kMapBatch terms of every token, all loads issued first
    i32x4 v[kMapTok][kMapBatch];
#pragma unroll
    for (int tt = 0; tt < kMapTok; ++tt)
#pragma unroll
      for (int q = 0; q < kMapBatch; ++q)
        if (q < n[tt]) v[tt][q] = *reinterpret_cast<const i32x4*>(y + (int64_t)s_row[tt * kMapMaxTopk + q] * K + 8 * c);
#pragma unroll
    for (int tt = 0; tt < kMapTok; ++tt)
#pragma unroll
      for (int q = 0; q < kMapBatch; ++q)
        if (q < n[tt]) fma8(acc[tt], s_w[tt * kMapMaxTopk + q], v[tt][q]);
  }
#pragma unroll
  for (int tt = 0; tt < kMapTok; ++tt)
    for (int q0 = kMapBatch; q0 < n[tt]; q0 += kMapBatch) add(tt, q0);
#pragma unroll
  for (int tt = 0; tt < kMapTok; ++tt)
    if (t0 + tt < M) *reinterpret_cast<i32x4*>(out + (t0 + tt) * K + 8 * c) = pack8(acc[tt]);
}

// The same layout for the batched format's CSR list of each output token.
__global__ void __launch_bounds__(NT) reduce_csr_kernel(const uint16_t* __restrict__ y,
                                                        const float* __restrict__ w,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ rows,
                                                        uint16_t* __restrict__ out, int64_t n_out,
                                                        int64_t K, int cpt) {
  const int64_t t = blockIdx.x;
  const int64_t K8 = K / 8;
  const int64_t cbeg = (int64_t)blockIdx.y * NT * cpt + threadIdx.x;
  float acc[kChunks][8];
#pragma unroll
  for (int u = 0; u < kChunks; ++u)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
  const int b = offsets[t], e = offsets[t + 1];
  for (int i0 = b; i0 < e; i0 += kBatch) {
    int64_t r[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) r[q] = i0 + q < e ? rows[i0 + q] : -1;
    float wt[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) wt[q] = r[q] >= 0 ? w[r[q]] : 0.f;
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int64_t c = cbeg + (int64_t)NT * u;
      if (u >= cpt || c >= K8) break;
      i32x4 v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (r[q] >= 0) v[q] = *reinterpret_cast<const i32x4*>(y + r[q] * K + 8 * c);
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (r[q] >= 0) fma8(acc[u], wt[q], v[q]);
    }
  }
#pragma unroll
  for (int u = 0; u < kChunks; ++u) {
    const int64_t c = cbeg + (int64_t)NT * u;
    if (u < cpt && c < K8) *reinterpret_cast<i32x4*>(out + t * K + 8 * c) = pack8(acc[u]);
  }
}

// Quantise one 32-element block held in v[0..31].
__device__ __forceinline__ void quantize_block(const float* v, uint8_t* codes, uint8_t* scale) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  const uint32_t sc = mx_scale_code(m);
  const float inv = mx_inv_scale(sc);
  i32x4 o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* q = v + 16 * h + 4 * i;
      o[h][i] = (int)e4m3_pack4(q[0] * inv, q[1] * inv, q[2] * inv, q[3] * inv);
    }
  reinterpret_cast<i32x4*>(codes)[0] = o[0];
  reinterpret_cast<i32x4*>(codes)[1] = o[1];
  *scale = (uint8_t)sc;
}

__global__ void __launch_bounds__(NT) quantize_kernel(const void* __restrict__ x, int x_dtype,
                                                      int64_t rows, int64_t cols,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t nb = cols / 32;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= rows * nb) return;
  const int64_t r = idx / nb;
  const int64_t b = idx - r * nb;
  float v[32];
  if (x_dtype == 0) {
    const float* p = static_cast<const float*>(x) + r * cols + b * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = reinterpret_cast<const float4*>(p)[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(x) + r * cols + b * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x4 q = reinterpret_cast<const i32x4*>(p)[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_to_f32((uint32_t)q[j] & 0xffffu);
        v[8 * i + 2 * j + 1] = bf16_to_f32((uint32_t)q[j] >> 16);
      }
    }
  }
  quantize_block(v, codes + r * cols + b * 32, scales + r * nb + b);
}

// One wave per sorted position p < num_post (a grid-stride loop over the
// positions, so the grid is bounded whatever the plan's capacity): the
// wave reads its route's token row once (sorted id / topk, a scalar load)
// and each lane quantises blocks lane, lane + 64, ... of the row.
__global__ void __launch_bounds__(NT) quantize_gather_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ num_post, int topk, int sentinel, int64_t K,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t scale_group) {
  const int nb = (int)(K / 32);
  const int lane = threadIdx.x & 63;
  const int nwaves = (int)gridDim.x * (NT / 64);
  const int npos = num_post[0];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (int p = (int)blockIdx.x * (NT / 64) + wave; p < npos; p += nwaves) {
    const int sid = __builtin_amdgcn_readfirstlane(sorted_ids[p]);
    if (sid == sentinel) continue;   // padding rows are never read by the W1 kernel
    const uint16_t* row = x + (int64_t)(sid / topk) * K;
    // up to four blocks per lane at a time, all their loads issued first
    for (int b0 = lane; b0 < nb; b0 += 4 * 64) {
      i32x4 q[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (b0 + 64 * u < nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) q[u][i] = reinterpret_cast<const i32x4*>(row + (b0 + 64 * u) * 32)[i];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + 64 * u;
        if (b >= nb) break;
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j] = bf16_to_f32((uint32_t)q[u][i][j] & 0xffffu);
            v[8 * i + 2 * j + 1] = bf16_to_f32((uint32_t)q[u][i][j] >> 16);
          }
        uint8_t* sc = scale_group ? scales + (int64_t)(b / 16) * scale_group + (int64_t)p * 16 + b % 16
                                  : scales + (int64_t)p * nb + b;
        quantize_block(v, codes + (int64_t)p * K + b * 32, sc);
      }
    }
  }
}

// Scale arrays row-major -> grouped: thread i moves 16-byte piece i of the
// source, piece g of row r of matrix m (rows of ng pieces), to
// m * rows * ng * 16 + g * rows * 16 + r * 16 in dst.  Sources rows are
// read in order, so each wave reads 1 KB of them contiguously.
__global__ void __launch_bounds__(NT) pack_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int64_t rows, int64_t ng, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const int64_t g = i % ng;
    const int64_t mr = i / ng;   // m * rows + r
    const int64_t m = mr / rows, r = mr - m * rows;
    const i32x4 v = reinterpret_cast<const i32x4*>(src)[i];
    reinterpret_cast<i32x4*>(dst)[(m * ng + g) * rows + r] = v;
  }
}

// p[i * stride] = 0 for i < n: clears counters where a caller cannot rely on
// the previous call having left them zero (and where hipMemsetAsync would
// put a memset node into a captured graph).
__global__ void __launch_bounds__(NT) zero_words_kernel(int32_t* __restrict__ p, int64_t n, int64_t stride) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i < n) p[i * stride] = 0;
}

inline unsigned nblocks(int64_t n) { return (unsigned)((n + NT - 1) / NT); }

// Chunks per thread of the reduces: as many (up to kChunks) as keep about
// 2048 workgroups (eight per CU) in the grid.

// TopKWeightAndReduceNaiveBatched in one launch: workgroup t owns output
// token t and all of its columns (K <= 8 * kRT: one 8-column chunk per
// thread).  It walks the E * mt (expert, row) entries in ascending order,
// kScanChunk at a time, each thread 16 consecutive entries in runs of 4: a
// run of four valid rows of one expert (r < count[e]) is one 16-byte map load
// (all of a thread's loads issued before any is used), a run past the count
// reads nothing, and a run at a count or slab edge is read entry by entry, so
// rows past the count are never read.  A workgroup-wide exclusive scan of the
// per-thread match counts places the rows whose map entry is t in LDS in
// ascending order; they are added into the fp32 accumulators, kBatch rows'
// loads issued together, one multiply-add per row in order — the order and
// the arithmetic of the list-based reduce, so the same bits.  Workgroup 0
// also counts the valid rows whose map entry lies outside {-1} U [0, n_out)
// and writes the count to status.
constexpr int kRT = 1024;                  // threads of the one-launch reduce
constexpr int kPerThread = 16;
constexpr int kScanChunk = kPerThread * kRT;   // 64 KB of LDS list

// exclusive prefix sum of v over the kRT threads; total gets the sum
__device__ __forceinline__ int block_exclusive_scan(int v, int& total, int* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kRT / 64; ++w) {
    const int tw = sh[w];
    if (w < wave) before += tw;
    sum += tw;
  }
  total = sum;
  __syncthreads();   // sh is free again
  return before + x - v;
}

__global__ void __launch_bounds__(kRT) reduce_batched_kernel(const uint16_t* __restrict__ y,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ row_token,
                                                             const float* __restrict__ w, int mt, int E,
                                                             uint16_t* __restrict__ out, int n_out, int K,
                                                             int32_t* __restrict__ status, int vec_map) {
  __shared__ int32_t list[kScanChunk];
  __shared__ int32_t sh[kRT / 64];
  __shared__ int32_t scnt[kReduceBatchedMaxE];   // valid rows per expert, min(counts[e], mt)
  for (int e = threadIdx.x; e < E; e += kRT) scnt[e] = min(max(counts[e], 0), mt);
  __syncthreads();
  const int t = blockIdx.x;
  const int K8 = K / 8;
  const uint32_t R = (uint32_t)E * (uint32_t)mt;   // < 2^31
  const int c = threadIdx.x;                       // this thread's 8-column chunk
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  int invalid = 0;
  constexpr int NR = kPerThread / 4;
  for (uint32_t base = 0; base < R; base += kScanChunk) {
    const uint32_t i0 = base + (uint32_t)threadIdx.x * kPerThread;
    uint32_t e = i0 / (uint32_t)mt, r = i0 - e * (uint32_t)mt;
    i32x4 v[NR];
    uint32_t full = 0, edge = 0;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      v[j] = (i32x4){-1, -1, -1, -1};
      const uint32_t i = i0 + 4 * j;
      if (i < R) {
        const uint32_t cnt = (uint32_t)scnt[e];
        if (vec_map && r + 4 <= cnt) {
          v[j] = *reinterpret_cast<const i32x4*>(row_token + i);
          full |= 1u << j;
        } else if (!(r >= cnt && r + 4 <= (uint32_t)mt)) {
          edge |= 1u << j;
        }
      }
      r += 4;
      while (r >= (uint32_t)mt) { r -= mt; ++e; }
    }
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (!(edge >> j & 1)) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t iq = i0 + 4 * j + q;
        const uint32_t eq = iq / (uint32_t)mt, rq = iq - eq * (uint32_t)mt;
        if (iq < R && rq < (uint32_t)scnt[eq]) v[j][q] = row_token[iq];   // -1 stays: not a row
      }
    }
    uint32_t mask = 0;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (!((full | edge) >> j & 1)) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int tok = v[j][q];
        if (tok == t) mask |= 1u << (4 * j + q);
        if (t == 0 && tok != -1 && (tok < 0 || tok >= n_out)) ++invalid;
      }
    }
    int total;
    int pos = block_exclusive_scan(__builtin_popcount(mask), total, sh);
    for (uint32_t m = mask; m; m &= m - 1) list[pos++] = (int32_t)(i0 + __builtin_ctz(m));
    __syncthreads();
    if (c < K8) {
      for (int j0 = 0; j0 < total; j0 += kBatch) {
        int64_t rr[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) rr[q] = j0 + q < total ? list[j0 + q] : -1;
        float wt[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) wt[q] = rr[q] >= 0 ? w[rr[q]] : 0.f;
        i32x4 yv[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
          if (rr[q] >= 0) yv[q] = *reinterpret_cast<const i32x4*>(y + rr[q] * K + 8 * c);
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
          if (rr[q] >= 0) fma8(acc, wt[q], yv[q]);
      }
    }
    __syncthreads();   // the list is read before the next chunk writes it
  }
  if (c < K8) *reinterpret_cast<i32x4*>(out + (int64_t)t * K + 8 * c) = pack8(acc);
  if (t == 0) {
    int tot;
    block_exclusive_scan(invalid, tot, sh);
    if (threadIdx.x == 0) status[0] = tot;
  }
}

inline int reduce_cpt(int64_t rows, int64_t K8) {
  int cpt = 1;
  while (cpt < kChunks && rows * ((K8 + NT * 2 * cpt - 1) / (NT * 2 * cpt)) >= 2048) cpt *= 2;
  return cpt;
}

}  // namespace

hipError_t launch_reduce_contiguous(const uint16_t* y, const int32_t* ids, const float* w,
                                    const int32_t* expert_map, int32_t G, uint16_t* out, int64_t M,
                                    int32_t topk, int64_t K, int32_t E, int32_t* sync_zero,
                                    int64_t sync_lines, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (expert_map && K / 8 <= 1024 && topk <= kMapMaxTopk) {
    const int64_t nth = std::max<int64_t>(64 * kMapTok, (K / 8 + 63) / 64 * 64);
    hipLaunchKernelGGL(reduce_map_kernel, dim3((unsigned)((M + kMapTok - 1) / kMapTok)), dim3((unsigned)nth), 0, s,
                       y, ids, w, expert_map, G, out, M, topk, K, E, sync_zero, sync_lines);
    return hipGetLastError();
  }
  const int cpt = reduce_cpt(M, K / 8);
  const dim3 grid((unsigned)M, (unsigned)((K / 8 + NT * cpt - 1) / (NT * cpt)));
  hipLaunchKernelGGL(reduce_contiguous_kernel, grid, dim3(NT), 0, s, y, ids, w, expert_map, G, out, M,
                     topk, K, E, sync_zero, sync_lines, cpt);
  return hipGetLastError();
}

hipError_t launch_reduce_csr(const uint16_t* y, const float* w, const int32_t* offsets,
                             const int32_t* rows, uint16_t* out, int64_t n_out, int64_t K,
                             hipStream_t s) {
  if (n_out == 0) return hipSuccess;
  const int cpt = reduce_cpt(n_out, K / 8);
  const dim3 grid((unsigned)n_out, (unsigned)((K / 8 + NT * cpt - 1) / (NT * cpt)));
  hipLaunchKernelGGL(reduce_csr_kernel, grid, dim3(NT), 0, s, y, w, offsets, rows, out, n_out, K, cpt);
  return hipGetLastError();
}

hipError_t launch_reduce_batched(const uint16_t* y, const int32_t* counts, const int32_t* row_token,
                                 const float* w, int32_t mt, int32_t E, uint16_t* out, int64_t n_out,
                                 int64_t K, int32_t* status, hipStream_t s) {
  if (n_out == 0) return hipSuccess;
  if (K / 8 > kRT || E > kReduceBatchedMaxE || (int64_t)E * mt >= (1ll << 31) || n_out >= (1ll << 31))
    return hipErrorInvalidValue;
  // the map is read 16 bytes at a time where that is aligned
  const int vec_map = (reinterpret_cast<uintptr_t>(row_token) & 15) == 0;
  hipLaunchKernelGGL(reduce_batched_kernel, dim3((unsigned)n_out), dim3(kRT), 0, s, y, counts, row_token, w, mt, E,
                     out, (int)n_out, (int)K, status, vec_map);
  return hipGetLastError();
}

hipError_t launch_zero_words(int32_t* p, int64_t n, int64_t stride, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3(nblocks(n)), dim3(NT), 0, s, p, n, stride);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s) {
  hipLaunchKernelGGL(quantize_kernel, dim3(nblocks(rows * (cols / 32))), dim3(NT), 0, s, x, x_dtype,
                     rows, cols, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_gather_mxfp8(const uint16_t* x, const int32_t* sorted_ids,
                                        const int32_t* num_post, int32_t topk, int32_t sentinel,
                                        int64_t capacity, int64_t K, uint8_t* codes,
                                        uint8_t* scales, int64_t scale_group, hipStream_t s) {
  // a wave per position, up to eight workgroups per CU
  if (capacity <= 0) return hipSuccess;
  const int64_t need = (capacity + NT / 64 - 1) / (NT / 64);
  const int64_t wgs = need < 2048 ? need : 2048;
  hipLaunchKernelGGL(quantize_gather_kernel, dim3((unsigned)wgs), dim3(NT), 0, s, x, sorted_ids, num_post, topk,
                     sentinel, K, codes, scales, scale_group);
  return hipGetLastError();
}

hipError_t launch_pack_mxfp8_scales(const uint8_t* src, uint8_t* dst, int64_t mats, int64_t rows, int64_t cols,
                                    hipStream_t s) {
  const int64_t n = mats * rows * (cols / 512);   // 16-byte pieces
  if (n == 0) return hipSuccess;
  const int64_t wgs = std::min<int64_t>((n + NT - 1) / NT, 8192);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)wgs), dim3(NT), 0, s, src, dst, rows, cols / 512, n);
  return hipGetLastError();
}

}  // namespace moe
