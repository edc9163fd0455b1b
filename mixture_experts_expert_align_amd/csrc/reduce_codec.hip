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
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int NT = 256;

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

__global__ void __launch_bounds__(NT) reduce_contiguous_kernel(const uint16_t* __restrict__ y,
                                                               const int32_t* __restrict__ ids,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ emap, int G,
                                                               uint16_t* __restrict__ out, int64_t M,
                                                               int topk, int64_t K, int E,
                                                               int32_t* __restrict__ sync_zero,
                                                               int64_t sync_lines) {
  if (sync_zero && blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < sync_lines; i += NT) sync_zero[32 * i] = 0;
  const int64_t K8 = K / 8;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= M * K8) return;
  const int64_t t = idx / K8;
  const int64_t c = (idx - t * K8) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < topk; ++j) {
    const int64_t s = t * topk + j;
    int id = ids[s];
    if (emap) id = (id >= 0 && id < G) ? emap[id] : -1;   // global -> local (-1: held elsewhere)
    if (id < 0 || id >= E) continue;
    const i32x4 v = *reinterpret_cast<const i32x4*>(y + s * K + c);
    fma8(acc, w[s], v);
  }
  *reinterpret_cast<i32x4*>(out + t * K + c) = pack8(acc);
}

__global__ void __launch_bounds__(NT) reduce_csr_kernel(const uint16_t* __restrict__ y,
                                                        const float* __restrict__ w,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ rows,
                                                        uint16_t* __restrict__ out, int64_t n_out,
                                                        int64_t K) {
  const int64_t K8 = K / 8;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= n_out * K8) return;
  const int64_t t = idx / K8;
  const int64_t c = (idx - t * K8) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int b = offsets[t], e = offsets[t + 1];
  for (int i = b; i < e; ++i) {
    const int64_t r = rows[i];
    const i32x4 v = *reinterpret_cast<const i32x4*>(y + r * K + c);
    fma8(acc, w[r], v);
  }
  *reinterpret_cast<i32x4*>(out + t * K + c) = pack8(acc);
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
      uint32_t wd = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) wd |= e4m3_encode(v[16 * h + 4 * i + b] * inv) << (8 * b);
      o[h][i] = (int)wd;
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

__global__ void __launch_bounds__(NT) quantize_gather_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ num_post, int topk, int sentinel, int64_t capacity, int64_t K,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = K / 32;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= capacity * nb) return;
  const int64_t p = idx / nb;
  if (p >= num_post[0]) return;
  const int sid = sorted_ids[p];
  if (sid == sentinel) return;   // padding rows are never read by the W1 kernel
  const int64_t b = idx - p * nb;
  const uint16_t* src = x + (int64_t)(sid / topk) * K + b * 32;
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const i32x4 q = reinterpret_cast<const i32x4*>(src)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_to_f32((uint32_t)q[j] & 0xffffu);
      v[8 * i + 2 * j + 1] = bf16_to_f32((uint32_t)q[j] >> 16);
    }
  }
  quantize_block(v, codes + p * K + b * 32, scales + p * nb + b);
}

inline unsigned nblocks(int64_t n) { return (unsigned)((n + NT - 1) / NT); }

}  // namespace

hipError_t launch_reduce_contiguous(const uint16_t* y, const int32_t* ids, const float* w,
                                    const int32_t* expert_map, int32_t G, uint16_t* out, int64_t M,
                                    int32_t topk, int64_t K, int32_t E, int32_t* sync_zero,
                                    int64_t sync_lines, hipStream_t s) {
  hipLaunchKernelGGL(reduce_contiguous_kernel, dim3(nblocks(M * (K / 8))), dim3(NT), 0, s, y, ids, w,
                     expert_map, G, out, M, topk, K, E, sync_zero, sync_lines);
  return hipGetLastError();
}

hipError_t launch_reduce_csr(const uint16_t* y, const float* w, const int32_t* offsets,
                             const int32_t* rows, uint16_t* out, int64_t n_out, int64_t K,
                             hipStream_t s) {
  hipLaunchKernelGGL(reduce_csr_kernel, dim3(nblocks(n_out * (K / 8))), dim3(NT), 0, s, y, w, offsets,
                     rows, out, n_out, K);
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
                                        uint8_t* scales, hipStream_t s) {
  hipLaunchKernelGGL(quantize_gather_kernel, dim3(nblocks(capacity * (K / 32))), dim3(NT), 0, s, x,
                     sorted_ids, num_post, topk, sentinel, capacity, K, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
