// The expert computation for small layers in one launch (page "Cake MegaMoE
// EP16 backend for BF16 activations and MXFP8 weights", section 4, session
// handling: each run is one model kernel for FC1, SwiGLU and FC2 plus one
// kernel for the ordered top-k reduce), for bf16 weights on the contiguous
// format.
//
// A workgroup takes a ticket from a device counter when it starts and does
// the work of that ticket:
//   ticket 0                 the permute step (align) of all routes, in this
//                            one workgroup;
//   next max_active*P1/C1    W1 + SiLU-and-mul: C1 consecutive strips of one
//                            slot (expert) each, slots in order;
//   next max_active*P2/C2    W2 + unpermute: C2 consecutive strips of one slot.
// A W1 chunk waits until the align is published; a W2 chunk waits until the
// align is published and all P1 W1 strips of its slot have been published.
// Tickets are handed out in order as workgroups start, so every chunk a
// workgroup waits for already belongs to a running workgroup that itself
// waits only for earlier tickets: the waits end whatever order the hardware
// dispatches workgroups in.  Each wait is also bounded: after about a second
// it gives up and counts a time-out in status[1], so no wave can spin
// forever.
//
// The eight XCDs keep separate L2 caches that are not coherent with each
// other.  Agent-scope release/acquire would write back or invalidate a whole
// L2 per publish or wait, under the feet of every workgroup streaming on
// that XCD; measured that way (one strip per ticket) the launch ran three
// times slower than the two-launch path.  Instead the data that crosses
// workgroups inside the launch goes through device-coherent accesses (sc1):
// the row map's reads, and z's stores (W1) and loads (W2).  Publishing is
// then: every wave waits until its stores are done (vmcnt 0), a barrier, one
// relaxed increment; waiting is relaxed polling.  Only the align, whose
// stores are the shared permute code's ordinary ones, publishes with a
// release (one L2 write-back per call); it also writes one 16-byte record
// per slot (expert, rows, first position), so a chunk learns its slot in one
// load rather than a chain of three.  Each counter has a 128-byte line of
// its own.  A ticket still costs a claim and a poll, each a round trip to
// memory (measured with one strip per ticket: 24 thousand tickets, three
// times slower than the two-launch path), so it covers a chunk of strips,
// sized so that each phase keeps about a thousand chunks (one strip for
// small layers, where latency matters most).  The ordered reduce that
// follows the launch puts the counters back to zero for the next call.
//
// The matmul strips are the ones the two-launch streaming path uses
// (stream_bf16.h), with the same split of each contraction and the same
// summation order, so both paths give the same bits.
#include "align_device.h"
#include "stream_bf16.h"

namespace moe {
namespace {

constexpr int kFusedWaves = 8;
constexpr int kSpinLimit = 1 << 20;   // polls (each at least a global round trip)
constexpr int kRowCache = 256;        // a chunk's sorted ids kept in LDS

// LDS: the align's bucket arrays, or the strips' partial sums
constexpr int kFusedAlignInts = 2 * kFusedMaxExperts + 1 + 17 + 1;
constexpr int kFusedRedBytes = kFusedWaves * 2 * 64 * 16;
constexpr int kFusedLds = kFusedAlignInts * 4 > kFusedRedBytes ? kFusedAlignInts * 4 : kFusedRedBytes;

__device__ __forceinline__ int load_relaxed(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(0): this wave's loads and stores are done (gfx9 encoding;
// expcnt and lgkmcnt left alone)
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0070 | 0x0f00); }

// Thread 0 polls (device-coherent loads) until *p >= target, or the limit
// (a time-out is counted); then the workgroup goes on together.
__device__ void wait_at_least(const int32_t* p, int target, int32_t* timeouts) {
  if (threadIdx.x == 0) {
    int n = 0;
    while (load_relaxed(p) < target) {
      if (++n > kSpinLimit) {
        atomicAdd(timeouts, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// Every wave's (device-coherent) stores done, then one increment of *p by n.
// RELEASE: also write this XCD's L2 back first, for ordinary stores.
template <bool RELEASE>
__device__ void publish_add(int32_t* p, int n) {
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (RELEASE)
      __hip_atomic_fetch_add(p, n, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_fetch_add(p, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The slot's record (one device-coherent 16-byte load); false when the slot
// is past the active experts.
__device__ __forceinline__ bool slot_record(const FusedArgs& f, int slot, SlotRows& r) {
  const int32_t* rec = f.sync + kSyncLine * sync_counter_lines(f.max_active);
  const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rec, 16 * f.max_active);
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rr, 16 * slot, 0, 16);   // sc1
  r.e = v[0];
  r.cnt = v[1];
  r.pos0 = v[2];
  return v[3] != 0;
}

// The first kRowCache sorted ids of the slot, read once per chunk into LDS
// (each is a device-coherent round trip to memory); the lookup the strips
// use: LDS, or memory past the cache.
__device__ __forceinline__ auto cache_rows(const GemmArgs& g, const SlotRows& sr, int* s_rows) {
  const int32_t* sid = g.rows.sorted_ids + sr.pos0;
  const int n = sr.cnt < kRowCache ? sr.cnt : kRowCache;
  for (int i = threadIdx.x; i < n; i += blockDim.x) s_rows[i] = load_relaxed(sid + i);
  __syncthreads();
  return [=](int tk) { return tk < kRowCache ? s_rows[tk] : load_relaxed(sid + tk); };
}

// 8 waves and at most 128 registers, so two workgroups share a CU and one's
// start (ticket, poll) overlaps the other's streaming.
__global__ void __launch_bounds__(64 * kFusedWaves, 4) fused_stream_bf16_kernel(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) char smem[kFusedLds];
  __shared__ int s_ticket;
  __shared__ int s_rows[kRowCache];
  int32_t* sync = f.sync;
  if (threadIdx.x == 0) s_ticket = atomicAdd(&sync[kSyncTicket], 1);
  __syncthreads();
  const int64_t t = s_ticket;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
  int32_t* timeouts = f.align.status + 1;

  if (t == 0) {
    int* s_cnt = reinterpret_cast<int*>(smem);
    int* s_off = s_cnt + f.align.nb;
    int* s_tmp = s_off + f.align.nb + 1;
    align_workgroup(f.align, s_cnt, s_off, s_tmp, s_tmp + 17);
    __syncthreads();
    const int na = f.align.active[f.max_active];
    for (int64_t s = threadIdx.x; s < f.max_active; s += blockDim.x) {
      i32x4 r = {0, 0, 0, 0};
      if (s < na) {
        const int e = f.align.active[s];
        r = (i32x4){e, f.align.counts[e], f.align.offsets[e], 1};
      }
      reinterpret_cast<i32x4*>(sync + kSyncLine * sync_counter_lines(f.max_active))[s] = r;
    }
    publish_add<true>(&sync[kSyncAligned], 1);
  } else if (t <= f.n1c) {
    const int64_t i0 = (t - 1) * f.c1;          // first strip of the chunk
    const int slot = (int)(i0 / f.p1);
    const int p0 = (int)(i0 % f.p1);
    wait_at_least(&sync[kSyncAligned], 1, timeouts);
    SlotRows sr;
    if (slot_record(f, slot, sr)) {
      const auto row_of = cache_rows(f.w1, sr, s_rows);
      // wave: strip h, tile ut (gate / up), contraction run wave % ks1
      const int h = wave / (2 * f.ks1);
      const int ut = (wave / f.ks1) & 1;
      f32x4* red = reinterpret_cast<f32x4*>(smem) + h * f.ks1 * 2 * 64;
      for (int p = p0; p < p0 + f.c1; ++p)
        stream_bf16_strip<kEpiGateUp, true, true>(f.w1, sr, row_of, 16 * (f.ns1 * p + h), wave % f.ks1,
                                                  f.ks1, red, ut);
      publish_add<false>(&sync[kSyncSlots + kSyncLine * slot], f.c1);
    }
  } else if (t <= f.n1c + f.n2c) {
    const int64_t i0 = (t - 1 - f.n1c) * f.c2;
    const int slot = (int)(i0 / f.p2);
    const int p0 = (int)(i0 % f.p2);
    wait_at_least(&sync[kSyncAligned], 1, timeouts);
    SlotRows sr;
    if (slot_record(f, slot, sr)) {
      wait_at_least(&sync[kSyncSlots + kSyncLine * slot], f.p1, timeouts);
      const auto row_of = cache_rows(f.w2, sr, s_rows);
      const int h = wave / f.ks2;
      f32x4* red = reinterpret_cast<f32x4*>(smem) + h * f.ks2 * 64;
      for (int p = p0; p < p0 + f.c2; ++p)
        stream_bf16_strip<kEpiDown, false, true>(f.w2, sr, row_of, 16 * (f.ns2 * p + h), wave % f.ks2,
                                                 f.ks2, red);
    }
  }
}

}  // namespace

// Strips per ticket: a power of two dividing the strips of a slot (so a
// chunk never spans two slots), at most 16, and small enough that the phase
// keeps about 1024 chunks (two per workgroup slot on 256 CUs at two
// workgroups each).
static int32_t chunk_strips(int64_t strips, int32_t per_slot) {
  int32_t c = 1;
  while (c < 16 && per_slot % (2 * c) == 0 && strips / (2 * c) >= 1024) c *= 2;
  return c;
}

// Waves per contraction: as many as divide it into runs of whole 128-wide
// steps, up to 4 for W1 and 8 for W2 (as the two-launch path, so the sums
// are the same); a W1 strip takes twice that (gate and up tiles); the other
// waves of the 8 take further strips of the same slot.
hipError_t launch_fused_stream_bf16(FusedArgs f, hipStream_t s) {
  f.align.nbits = align_key_bits(f.align.nb);
  f.ks1 = 4;
  while (f.ks1 > 1 && f.w1.kdim % (128 * f.ks1)) f.ks1 >>= 1;
  f.ks2 = 8;
  while (f.ks2 > 1 && f.w2.kdim % (128 * f.ks2)) f.ks2 >>= 1;
  f.ns1 = kFusedWaves / (2 * f.ks1);
  f.ns2 = kFusedWaves / f.ks2;
  f.p1 = f.w1.nfeat / (16 * f.ns1);
  f.p2 = f.w2.nfeat / (16 * f.ns2);
  f.c1 = chunk_strips(f.max_active * f.p1, f.p1);
  f.c2 = chunk_strips(f.max_active * f.p2, f.p2);
  f.n1c = f.max_active * f.p1 / f.c1;
  f.n2c = f.max_active * f.p2 / f.c2;
  f.nitems = 1 + f.n1c + f.n2c;
  hipLaunchKernelGGL(fused_stream_bf16_kernel, dim3((unsigned)f.nitems), dim3(64 * kFusedWaves), 0, s, f);
  return hipGetLastError();
}

}  // namespace moe
