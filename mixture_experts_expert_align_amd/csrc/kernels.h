// Host-side launchers of the gfx950 kernels, used by the C ABI layer
// (moe_api.hip).  Each returns hipSuccess or the launch error; none
// allocates or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- align ----
// Stable counting sort of R flat keys into nb buckets.  With key_map, a key
// k in [0, key_range) is first replaced by key_map[k] (-1: skipped, not an
// error) and a key outside {-1} U [0, key_range) is invalid.  Key i is valid
// when the (mapped) key is in [0, nb) and, if group_count is given,
// (i % rows_per_group) < group_count[i / rows_per_group] (the batched
// format's valid rows).  Keys other than -1 that are out of range count in
// status[0] (keys of rows masked out by group_count are never read).
struct AlignArgs {
  const int32_t* keys;
  const int32_t* key_map;      // optional: keys in [0, key_range) are replaced by key_map[key]
  int32_t key_range;
  int64_t R;
  int32_t nb;
  int32_t B;                   // each bucket's run is padded to a multiple of B
  const int32_t* group_count;  // optional
  int32_t rows_per_group;
  int32_t* counts;             // [nb]
  int32_t* offsets;            // [nb+1]
  int32_t* sorted;             // [capacity]  values: flat index i, or sentinel
  int32_t* block_bucket;       // [max_tiles]
  int32_t* num_post;           // [1]
  int32_t* active;             // [max_active+1]
  int32_t* status;             // [>=1]
  int32_t* block_hist;         // [nblocks * nb]  (multi-block path)
  int64_t capacity;
  int64_t max_tiles;
  int64_t max_active;
  int32_t sentinel;
  int32_t nblocks;             // 0: single-block path; else chunks (<= kAlignMaxBlocks)
  int32_t chunk;               // set by launch_align: keys per chunk
  int32_t nbits;               // set by align_key_bits: bits of a bucket index
};

// Bits a bucket index in [0, nb) needs (the scatter's per-bit ballots).
inline int32_t align_key_bits(int32_t nb) {
  int32_t n = 0;
  while ((1 << n) < nb) ++n;
  return n;
}

constexpr int kAlignSmallMaxR = 8192;    // single-workgroup path up to this R
constexpr int kAlignChunk = 1024;        // keys per workgroup in the multi-block path (at least)
constexpr int kAlignMaxBlocks = 1024;    // workgroups of the multi-block path (at most)
constexpr int kAlignMaxBuckets = 8192;   // LDS-resident bucket counters

hipError_t launch_align(const AlignArgs& a, hipStream_t s);

// ---------------------------------------------------------------- gemms ----
enum Epilogue { kEpiGateUp = 0, kEpiDown = 1 };

// Rows a GEMM works on: the routes of each expert in sorted (align) order for
// the contiguous format, or rows r < count[e] of each expert's slab for the
// batched format.
struct RowMap {
  int32_t layout;              // 0 contiguous, 1 batched, 2 rows (grouped rows of the
                               // activation matrix, outputs to the same rows)
  const int32_t* sorted_ids;   // contiguous
  const int32_t* block_expert; // contiguous (tile path)
  const int32_t* num_post;     // contiguous
  const int32_t* offsets;      // contiguous (stream path)
  const int32_t* counts;       // contiguous: routes per expert; batched: valid rows
  const int32_t* active;       // contiguous (stream path)
  int32_t topk;
  int32_t sentinel;
  int32_t max_tokens;          // batched
};

struct GemmArgs {
  int32_t epi;
  RowMap rows;
  // activations: W1 reads x (contiguous, gathered by token) or the batched
  // slab; W2 reads z in position order
  const void* act;
  const uint8_t* act_scale;    // MXFP8 only
  int64_t act_ld;              // elements per activation row
  int64_t act_bytes;           // size of the activation buffer
  // weights
  const void* w;
  const uint8_t* w_scale;      // MXFP8 only
  int64_t w_expert_stride;     // elements per expert
  int32_t kdim;                // contraction length
  int32_t nfeat;               // W1: I; W2: K
  int32_t I;
  int32_t w1_order;            // 0 halves, 1 interleave16
  int32_t E;
  int64_t max_tiles;           // contiguous tile grid
  int64_t max_active;          // stream grid
  // outputs
  void* out;                   // W1: z; W2: y rows
  uint8_t* out_scale;          // W1 MXFP8: z scales
  int64_t out_ld;
  // MXFP8 with grouped scales (moe_pack_mxfp8_scales): bytes between the
  // 16-byte groups of the activation scales and of W1's output scales (their
  // rows x 16); the weight scales are grouped per expert.  0: every scale
  // array row-major.
  int64_t scale_group;
};

// Routes per plan tile of the tiled kernels: the contiguous format's align
// pads each expert's run to a multiple of kTileRoutesContiguous, which is
// the route count of one contiguous tile; the batched tiles hold 128 rows.
constexpr int kTileRoutesContiguous = 256;
constexpr int kTileRowsBatched = 128;
// The MXFP8 tiles hold 64 routes (the align pads each expert's run to 64)
// and 128 weight rows.
constexpr int kTileRoutesMxfp8 = 64;

hipError_t launch_gemm_tile_bf16(const GemmArgs& g, hipStream_t s);
// rows layout (2): y rows = W[e] x rows for the groups offsets[e] ..
// offsets[e+1] of R rows; 256 x 256 tiles (nfeat % 256 == 0, kdim % 64 == 0).
// wt: W[e] is stored [kdim, nfeat] (output index contiguous) and is read
// transposed: y rows = W[e]^T x rows.
hipError_t launch_tile_rows_bf16(const GemmArgs& g, const int32_t* offsets, int64_t R, bool wt, hipStream_t s);
hipError_t launch_gemm_stream_bf16(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_stream_mxfp8(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_tile_mxfp8(const GemmArgs& g, hipStream_t s);

// -------------------------------------------------------- single launch ----
// Align, W1 + SiLU-and-mul and W2 + unpermute of the bf16 streaming path in
// one launch (work items taken from a device ticket counter; see fused.hip).
constexpr int kFusedMaxExperts = 2048;   // the align's bucket arrays live in LDS
// The sync area, in int32 words: one 128-byte line per counter (they are
// polled and incremented by different workgroups at once) — [0] ticket,
// [32] align published, [64 + 32 s] W1 strips published for slot s — then
// one record per slot, int4 {expert, rows, first position, 1}, or zeros for
// a slot past the active experts (written by the align).  The counters are
// zero before the first call and the reduce that follows each call zeroes
// them again.
constexpr int kSyncLine = 32;
enum { kSyncTicket = 0, kSyncAligned = kSyncLine, kSyncSlots = 2 * kSyncLine };
__host__ __device__ inline int64_t sync_counter_lines(int64_t max_active) { return 2 + max_active; }
__host__ __device__ inline int64_t sync_words(int64_t max_active) { return kSyncLine * sync_counter_lines(max_active) + 4 * max_active; }

struct FusedArgs {
  AlignArgs align;             // single-workgroup align (nblocks 0)
  GemmArgs w1, w2;             // as for the two streaming launches
  int32_t* sync;               // [sync_words(max_active)]
  int64_t max_active;
  // set by the launcher
  int32_t ks1, ks2;            // waves per W1 / W2 strip
  int32_t ns1, ns2;            // strips per workgroup
  int32_t p1, p2;              // strips per slot
  int32_t c1, c2;              // strips per ticket
  int64_t n1c, n2c;            // W1 / W2 tickets
  int64_t nitems;              // workgroups of the launch
};

hipError_t launch_fused_stream_bf16(FusedArgs f, hipStream_t s);

// ------------------------------------------------------------- training ----
// Deterministic ragged grouped GEMMs (see train.hip): group e is rows
// [offsets[e], offsets[e+1]) of x [R, K] and dy [R, N]; w is [E, N, K].
enum TrainMode { kTrainForward = 0, kTrainDgrad = 1, kTrainWgrad = 2 };

struct TrainArgs {
  int32_t mode;
  const uint16_t* x;           // forward, wgrad
  const uint16_t* dy;          // dgrad, wgrad
  const uint16_t* w;           // forward, dgrad
  const int32_t* offsets;      // [E+1]
  void* out;                   // y [R,N] bf16 / dx [R,K] bf16 / dW [E,N,K] fp32
  int64_t R;
  int32_t N, K, E;
  int32_t accumulate;          // wgrad: add into out instead of writing it
};

hipError_t launch_train(const TrainArgs& t, hipStream_t s);

// --------------------------------------------------------------- reduce ----
// out[t] = sum over slots j (ascending) whose id (mapped through expert_map
// when given: ids in [0, G)) is a local expert in [0, E) of w[t,j] * y[t*topk+j]
// sync_zero (optional): word 32 i is zeroed for i < sync_lines (the
// single-launch path's counters, for the next call).
hipError_t launch_reduce_contiguous(const uint16_t* y, const int32_t* ids, const float* w,
                                    const int32_t* expert_map, int32_t G, uint16_t* out, int64_t M,
                                    int32_t topk, int64_t K, int32_t E, int32_t* sync_zero,
                                    int64_t sync_lines, hipStream_t s);
// out[t] = sum over CSR list of t (ascending) of w[row] * y[row]
// out[t] = sum over the valid rows (e, r) of the batched format (r <
// min(counts[e], mt)) with row_token == t, ascending (e, r), of w * y, one
// workgroup per token scanning the map itself (K <= 8192, E <=
// kReduceBatchedMaxE, whose counts it keeps in LDS: 64 KB of row list + the
// counts fit two workgroups per CU); status[0] = valid rows mapping outside
// {-1} U [0, n_out)
constexpr int kReduceBatchedMaxE = 4080;
hipError_t launch_reduce_batched(const uint16_t* y, const int32_t* counts, const int32_t* row_token,
                                 const float* w, int32_t mt, int32_t E, uint16_t* out, int64_t n_out,
                                 int64_t K, int32_t* status, hipStream_t s);
hipError_t launch_reduce_csr(const uint16_t* y, const float* w, const int32_t* offsets,
                             const int32_t* rows, uint16_t* out, int64_t n_out, int64_t K,
                             hipStream_t s);

// p[i * stride] = 0 for i < n (a fill kernel, capturable in a graph).
hipError_t launch_zero_words(int32_t* p, int64_t n, int64_t stride, hipStream_t s);

// ---------------------------------------------------------------- codec ----
hipError_t launch_quantize_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s);
// MXFP8 rows of x gathered in sorted order: row p <- x[sorted_ids[p] / topk]
// for the positions p < num_post[0] that hold a route (padding positions are
// skipped: the W1 kernels never read them).  Scales row-major [capacity,
// K/32], or with scale_group > 0 grouped: byte j of row p at
// (j / 16) * scale_group + p * 16 + j % 16.
hipError_t launch_quantize_gather_mxfp8(const uint16_t* x, const int32_t* sorted_ids,
                                        const int32_t* num_post, int32_t topk, int32_t sentinel,
                                        int64_t capacity, int64_t K, uint8_t* codes,
                                        uint8_t* scales, int64_t scale_group, hipStream_t s);
// mats matrices of rows x cols/32 scale bytes, row-major -> grouped per
// matrix (byte j of row r at (j / 16) * rows * 16 + r * 16 + j % 16)
hipError_t launch_pack_mxfp8_scales(const uint8_t* src, uint8_t* dst, int64_t mats, int64_t rows, int64_t cols,
                                    hipStream_t s);

}  // namespace moe
