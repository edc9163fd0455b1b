// Device-side pieces of the permute step ("Fused MoE Modular Kernel",
// apply(), step 1), shared by the align kernels and the single-launch
// expert computation: key reading (with the expert map), a workgroup scan,
// the bucket layout, padding and tile owners, and the stable scatter.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

struct KeyRead {
  int key;
  bool valid;    // a route of a bucket
  bool invalid;  // read, not -1, out of range
};

__device__ __forceinline__ KeyRead read_key(const AlignArgs& a, int64_t i) {
  KeyRead r{-1, false, false};
  if (a.group_count) {
    const int64_t g = i / a.rows_per_group;
    const int64_t row = i - g * a.rows_per_group;
    if (row >= a.group_count[g]) return r;  // masked row: never read
  }
  int k = a.keys[i];
  if (a.key_map) {
    if (k >= 0 && k < a.key_range) {
      k = a.key_map[k];
    } else if (k != -1) {
      r.invalid = true;    // outside {-1} U [0, key_range)
      return r;
    }
  }
  r.key = k;
  r.valid = k >= 0 && k < a.nb;
  r.invalid = !r.valid && k != -1;
  return r;
}

// Exclusive scan over the workgroup (blockDim.x a multiple of 64, <= 1024).
// s_tmp needs 17 ints.  Returns the exclusive prefix; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = __lane_id();
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) s_tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int t = s_tmp[w];
      s_tmp[w] = run;
      run += t;
    }
    s_tmp[16] = run;
  }
  __syncthreads();
  const int res = x - v + s_tmp[wave];
  *total = s_tmp[16];
  __syncthreads();
  return res;
}

// Largest e with s_off[e] <= pos (s_off non-decreasing, s_off[0] = 0).
__device__ __forceinline__ int find_bucket(const int* s_off, int nb, int pos) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_off[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// From per-bucket counts in s_cnt: offsets (in s_off, nb+1 ints) and, when
// publish is set, offsets, counts, the active list and the padded total in
// memory.  Run by one workgroup.
__device__ void bucket_layout(const AlignArgs& a, int* s_cnt, int* s_off, int* s_tmp, bool publish = true) {
  const int nb = a.nb;
  const int nt = blockDim.x;
  const int per = (nb + nt - 1) / nt;
  const int e0 = min(nb, (int)threadIdx.x * per);
  const int e1 = min(nb, e0 + per);
  int psum = 0, asum = 0;
  for (int e = e0; e < e1; ++e) {
    const int c = s_cnt[e];
    psum += (c + a.B - 1) / a.B * a.B;
    asum += c > 0;
  }
  int total, n_active;
  int pbase = block_exclusive_scan(psum, s_tmp, &total);
  int abase = block_exclusive_scan(asum, s_tmp, &n_active);
  for (int e = e0; e < e1; ++e) {
    const int c = s_cnt[e];
    s_off[e] = pbase;
    if (publish) {
      a.offsets[e] = pbase;
      a.counts[e] = c;
      if (c > 0) a.active[abase++] = e;
    }
    pbase += (c + a.B - 1) / a.B * a.B;
  }
  if (threadIdx.x == 0) {
    s_off[nb] = total;
    if (publish) {
      a.offsets[nb] = total;
      a.num_post[0] = total;
      a.active[a.max_active] = n_active;
    }
  }
  if (publish)
    for (int64_t i = n_active + threadIdx.x; i < a.max_active; i += nt) a.active[i] = -1;
  __syncthreads();
}

// Padding sentinels and tile owners, from offsets (nb+1) and counts, in
// global memory or LDS: bucket e's padding [offsets[e] + counts[e],
// offsets[e+1]) and tiles [offsets[e] / B, offsets[e+1] / B); past the total,
// sentinels and owner -1.  Work item w of nw: buckets w, w + nw, ... one
// wave each, and a grid-stride share of the tail.
__device__ void pad_and_owners(const AlignArgs& a, int64_t w, int64_t nw, int64_t gtid, int64_t gsize,
                               const int* offsets, const int* counts) {
  const int lane = __lane_id();
  for (int64_t e = w; e < a.nb; e += nw) {
    const int off = offsets[e], c = counts[e], end = offsets[e + 1];
    for (int64_t p = off + c + lane; p < end; p += kWave) a.sorted[p] = a.sentinel;
    for (int64_t t = off / a.B + lane; t < end / a.B; t += kWave) a.block_bucket[t] = (int32_t)e;
  }
  const int64_t total = offsets[a.nb];
  for (int64_t p = total + gtid; p < a.capacity; p += gsize) a.sorted[p] = a.sentinel;
  for (int64_t t = total / a.B + gtid; t < a.max_tiles; t += gsize) a.block_bucket[t] = -1;
}

// Place routes [begin, end) in index order; s_cur[e] is the next free
// position of bucket e and is advanced.  Waves take turns.  first (optional):
// this thread's key of the first block, read before.
__device__ void scatter_range(const AlignArgs& a, int64_t begin, int64_t end, int* s_cur,
                              const KeyRead* first = nullptr) {
  const int nt = blockDim.x;
  const int wave = threadIdx.x / kWave;
  const int nwaves = nt / kWave;
  for (int64_t base = begin; base < end; base += nt) {
    const int64_t i = base + threadIdx.x;
    KeyRead kr{-1, false, false};
    if (i < end) kr = (first && base == begin) ? *first : read_key(a, i);
    int rank, gsize;
    bool last;
    wave_match_rank(kr.key, kr.valid, a.nbits, rank, gsize, last);
    // only the waves that hold keys of this block take a turn
    const int nturns = (int)min<int64_t>(nwaves, (end - base + kWave - 1) / kWave);
    for (int w = 0; w < nturns; ++w) {
      if (w == wave && kr.valid) {
        const int b0 = s_cur[kr.key];
        a.sorted[b0 + rank] = (int32_t)i;
        if (last) s_cur[kr.key] = b0 + gsize;
      }
      __syncthreads();
    }
  }
}

// The whole align in one workgroup (blockDim.x a multiple of 64, <= 1024):
// s_cnt and s_off need nb and nb + 1 ints, s_tmp 17, s_invalid 1.  Ends
// with every global write of the workgroup issued (not yet visible to other
// workgroups: a caller that publishes them fences first).
__device__ void align_workgroup(const AlignArgs& a, int* s_cnt, int* s_off, int* s_tmp, int* s_invalid) {
  for (int e = threadIdx.x; e < a.nb; e += blockDim.x) s_cnt[e] = 0;
  if (threadIdx.x == 0) *s_invalid = 0;
  __syncthreads();
  int inv = 0;
  KeyRead k0{-1, false, false};   // this thread's key of the first block, kept for the scatter
  for (int64_t i = threadIdx.x; i < a.R; i += blockDim.x) {
    const KeyRead kr = read_key(a, i);
    if (i == threadIdx.x) k0 = kr;
    if (kr.valid) atomicAdd(&s_cnt[kr.key], 1);
    inv += kr.invalid;
  }
  if (inv) atomicAdd(s_invalid, inv);
  __syncthreads();
  if (threadIdx.x == 0) a.status[0] = *s_invalid;
  bucket_layout(a, s_cnt, s_off, s_tmp);   // ends with a barrier
  // padding and tile owners from the layout in LDS (s_cnt still holds the counts)
  pad_and_owners(a, threadIdx.x / kWave, blockDim.x / kWave, threadIdx.x, blockDim.x, s_off, s_cnt);
  __syncthreads();
  for (int e = threadIdx.x; e < a.nb; e += blockDim.x) s_cnt[e] = s_off[e];
  __syncthreads();
  scatter_range(a, 0, a.R, s_cnt, &k0);
}

}  // namespace
}  // namespace moe
