// Permute step of the expert computation ("Fused MoE Modular Kernel",
// apply(), step 1): a stable counting sort of the flat routes t*topk+j by
// expert, each expert's run padded to the GEMM tile size.
//
// histogram -> exclusive scan of the padded counts -> stable scatter.  The
// scatter is stable (ascending flat index inside an expert) because routes
// are taken in index order: in the multi-block path each workgroup owns a
// contiguous chunk and starts at the scanned count of the chunks before it;
// inside a workgroup the waves take their 64 routes in turn, and inside a
// wave a lane's rank among the lanes with the same key comes from ballots.
// Integer-only, so the result is the same on every run.
//
// Small problems (R <= kAlignSmallMaxR) run as one workgroup in one launch
// (decode batches are launch-latency bound); larger ones as three launches:
// per-chunk histograms (stored bucket-major), a scan of each bucket over
// the chunks plus the bucket layout, and the scatter, whose workgroups also
// write the padding sentinels and the tile owners — two launches when the
// histogram matrix is small enough for every scatter workgroup to scan it.
#include "align_device.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(1024) align_small_kernel(AlignArgs a) {
  __shared__ int s_cnt[kAlignMaxBuckets];
  __shared__ int s_off[kAlignMaxBuckets + 1];
  __shared__ int s_tmp[17];
  __shared__ int s_invalid;
  align_workgroup(a, s_cnt, s_off, s_tmp, &s_invalid);
}

// Multi-block path, launch 1: per-chunk histograms, bucket-major:
// block_hist[e * nblocks + b] (row nb: invalid ids).
__global__ void __launch_bounds__(256) align_hist_kernel(AlignArgs a) {
  __shared__ int s_cnt[kAlignMaxBuckets + 1];
  for (int e = threadIdx.x; e <= a.nb; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * a.chunk;
  const int64_t end = min(a.R, begin + a.chunk);
  int inv = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += blockDim.x) {
    const KeyRead kr = read_key(a, i);
    if (kr.valid) atomicAdd(&s_cnt[kr.key], 1);
    inv += kr.invalid;
  }
  if (inv) atomicAdd(&s_cnt[a.nb], inv);
  __syncthreads();
  for (int e = threadIdx.x; e <= a.nb; e += blockDim.x) a.block_hist[(int64_t)e * a.nblocks + blockIdx.x] = s_cnt[e];
}

// Launch 2: each bucket's histogram row scanned over the chunks (in place:
// each chunk's starting rank), a wave per bucket, then the bucket layout.
// A wave takes kScanBatch of its buckets at a time and issues their loads
// together, so it waits for memory once per batch rather than once per
// bucket.
constexpr int kScanBatch = 8;
__global__ void __launch_bounds__(1024) align_scan_kernel(AlignArgs a) {
  __shared__ int s_cnt[kAlignMaxBuckets + 1];
  __shared__ int s_off[kAlignMaxBuckets + 1];
  __shared__ int s_tmp[17];
  const int lane = __lane_id();
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int e0 = wave; e0 <= a.nb; e0 += nwaves * kScanBatch) {
    int run[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) run[u] = 0;
    for (int b0 = 0; b0 < a.nblocks; b0 += kWave) {
      const int b = b0 + lane;
      int v[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        const int e = e0 + u * nwaves;
        v[u] = (e <= a.nb && b < a.nblocks) ? a.block_hist[(int64_t)e * a.nblocks + b] : 0;
      }
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        const int e = e0 + u * nwaves;
        int x = v[u];
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
          const int y = __shfl_up(x, d);
          if (lane >= d) x += y;
        }
        if (e <= a.nb && b < a.nblocks) a.block_hist[(int64_t)e * a.nblocks + b] = run[u] + x - v[u];
        run[u] += __shfl(x, kWave - 1);
      }
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const int e = e0 + u * nwaves;
      if (lane == 0 && e <= a.nb) s_cnt[e] = run[u];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.status[0] = s_cnt[a.nb];
  bucket_layout(a, s_cnt, s_off, s_tmp);
}

// Launch 3: each chunk scatters its routes from its starting ranks; the
// workgroups also write the padding and the tile owners.
__global__ void __launch_bounds__(256) align_scatter_kernel(AlignArgs a) {
  __shared__ int s_cur[kAlignMaxBuckets];
  for (int e = threadIdx.x; e < a.nb; e += blockDim.x)
    s_cur[e] = a.offsets[e] + a.block_hist[(int64_t)e * a.nblocks + blockIdx.x];
  __syncthreads();
  const int64_t begin = (int64_t)blockIdx.x * a.chunk;
  const int64_t end = min(a.R, begin + a.chunk);
  scatter_range(a, begin, end, s_cur);
  const int nwaves = blockDim.x / kWave;
  pad_and_owners(a, (int64_t)blockIdx.x * nwaves + threadIdx.x / kWave, (int64_t)gridDim.x * nwaves,
                 (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x, a.offsets,
                 a.counts);
}

// Launches 2 and 3 in one, when the histogram matrix is small (at most
// kAlignFuseMaxBuckets buckets and kAlignFuseMaxEntries entries, kFusePer a
// thread, all loaded together): every scatter workgroup sums the matrix
// itself — per bucket the total and the counts of the chunks before its own,
// integer LDS atomics, exact in any order — and lays the buckets out in its
// LDS; the first workgroup also publishes the layout and the invalid count.
// Padding and tile owners come from the LDS layout, so no workgroup reads
// what another one writes.
constexpr int kAlignFuseMaxBuckets = 1024;
constexpr int kFusePer = 16;
constexpr int64_t kAlignFuseMaxEntries = 256 * kFusePer;
__global__ void __launch_bounds__(256) align_scan_scatter_kernel(AlignArgs a) {
  __shared__ int s_cnt[kAlignFuseMaxBuckets + 1];
  __shared__ int s_off[kAlignFuseMaxBuckets + 1];
  __shared__ int s_cur[kAlignFuseMaxBuckets + 1];
  __shared__ int s_tmp[17];
  const int me = blockIdx.x;
  for (int e = threadIdx.x; e <= a.nb; e += blockDim.x) {
    s_cnt[e] = 0;
    s_cur[e] = 0;
  }
  const int n = (a.nb + 1) * a.nblocks;
  int v[kFusePer];
#pragma unroll
  for (int q = 0; q < kFusePer; ++q) {
    const int i = threadIdx.x + 256 * q;
    v[q] = i < n ? a.block_hist[i] : 0;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kFusePer; ++q) {
    if (v[q]) {
      const int i = threadIdx.x + 256 * q;
      const int e = i / a.nblocks, b = i - e * a.nblocks;   // row e: bucket (nb: invalid ids), column b: chunk
      atomicAdd(&s_cnt[e], v[q]);
      if (b < me) atomicAdd(&s_cur[e], v[q]);
    }
  }
  __syncthreads();
  const bool first = me == 0;
  if (first && threadIdx.x == 0) a.status[0] = s_cnt[a.nb];
  bucket_layout(a, s_cnt, s_off, s_tmp, first);   // ends with a barrier
  for (int e = threadIdx.x; e < a.nb; e += blockDim.x) s_cur[e] += s_off[e];
  __syncthreads();
  const int64_t begin = (int64_t)me * a.chunk;
  const int64_t end = min(a.R, begin + a.chunk);
  scatter_range(a, begin, end, s_cur);
  const int nwaves = blockDim.x / kWave;
  pad_and_owners(a, (int64_t)me * nwaves + threadIdx.x / kWave, (int64_t)gridDim.x * nwaves,
                 (int64_t)me * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x, s_off, s_cnt);
}

}  // namespace

hipError_t launch_align(const AlignArgs& args, hipStream_t s) {
  AlignArgs a = args;
  a.nbits = align_key_bits(a.nb);
  if (a.nblocks == 0) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  // chunks of a multiple of 256 routes, one per workgroup
  const int64_t per = (a.R + a.nblocks - 1) / a.nblocks;
  a.chunk = (int32_t)((per + 255) / 256 * 256);
  hipLaunchKernelGGL(align_hist_kernel, dim3(a.nblocks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nb <= kAlignFuseMaxBuckets && (int64_t)(a.nb + 1) * a.nblocks <= kAlignFuseMaxEntries) {
    hipLaunchKernelGGL(align_scan_scatter_kernel, dim3(a.nblocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(1024), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(a.nblocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
