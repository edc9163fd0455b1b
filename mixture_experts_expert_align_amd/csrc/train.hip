// Deterministic grouped GEMMs for training a MoE layer (page "Cake
// deterministic MoE grouped GEMM", introduction: a ragged bf16 grouped GEMM
// whose forward, dgrad and wgrad give the same bits on every run, and whose
// fp32 weight gradient is added into the fp32 main_grad inside the kernel,
// the same bits as out.add_(dW), section 1).
//
// Rows are grouped by expert: group e is rows [offsets[e], offsets[e+1]) of
// x [R, K] and dy [R, N]; W is [E, N, K].
//   forward  y[r]  = W[e] x[r]                      ([R, N] bf16)
//   dgrad    dx[r] = W[e]^T dy[r]                   ([R, K] bf16)
//   wgrad    dW[e] = sum over the group's rows of dy[r] x[r]^T
//                    ([E, N, K] fp32, written, or added to the fp32 buffer)
//
// One kernel body computes C[i][j] = sum_c A(i, c) B(j, c) for a tile of C,
// the contraction in slices staged in LDS (two buffers; each slice loaded
// into registers two slices ahead of its LDS store), waves of 64 x 64 as
// 2 x 2 tiles of v_mfma_f32_32x32x16_bf16: 128 x 256 tiles of eight waves
// for forward and dgrad, 128 x 128 tiles of four waves for wgrad.  Each operand
// is stored either with c contiguous (x and W for the forward, dy for dgrad)
// or with its own index contiguous (W for dgrad, dy and x for wgrad): MFMA
// wants 8 consecutive c per lane, so the second kind is staged transposed —
// a thread loads two rows of c (16 bytes of 8 consecutive i each), pairs up
// the values of the same i, and writes 8 four-byte words, each at its i row.
//
// Determinism: every output element is computed by one workgroup, whose
// MFMAs add the contraction in a fixed order; nothing is split across
// workgroups and no atomics touch floating point.  The accumulate adds the
// finished fp32 sum to the buffer once (a plain fp32 add), so it equals the
// overwrite followed by out.add_.  An empty group's sum stays +0.0 (the
// accumulators start at +0.0), which turns a -0.0 in the buffer into +0.0
// (section 2).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_common.h"

namespace moe {
namespace train {

// A tile configuration: C tile BI x BJ, contraction slice BC, WN x WM waves
// of 64 x 64.
template <int BI_, int BJ_, int BC_, int WN_, int WM_>
struct Tile {
  static constexpr int BI = BI_, BJ = BJ_, BC = BC_, WN = WN_, WM = WM_;
  static constexpr int NT = 64 * WN * WM;
  static constexpr int CH = BC / 8;            // 16-byte chunks per LDS row
  static constexpr int RPW = 256 / (BC * 2);   // LDS rows per 256-byte bank window
};
// forward and dgrad: 8 waves, 128 x 256, two workgroups per CU (128 VGPRs)
using RowsTile = Tile<128, 256, 32, 4, 2>;
// wgrad (both operands staged transposed): 4 waves, 128 x 128 and 64-wide
// slices, whose 128-byte LDS rows keep the transposed stores at 2-way bank
// conflicts (64-byte rows reach 8-way) and whose registers fit without spills
using WgradTile = Tile<128, 128, 64, 2, 2>;

constexpr int kNumXcd = 8;    // workgroups are dealt to the XCDs round robin
constexpr int kXcdRun = 8;    // consecutive logical tiles one XCD takes

// chunk c of LDS row `row`, XOR-swizzled.  (row / RPW) puts the 8
// consecutive rows one 128-byte quarter of an MFMA fragment read touches in
// distinct banks; (row / 16), constant over such 8 rows, spreads the
// transposed stores, whose 16 lanes of one c pair write rows 8 apart (with
// the first term alone they met in 2 chunks, an 8-way bank conflict).
template <class T>
__device__ __forceinline__ int lds_off(int row, int c) {
  const int x = ((row / T::RPW) ^ (row / 16)) & (T::CH - 1);
  return row * T::BC + ((c ^ x) << 3);
}

// An operand of C: element (i, c) at byte offset 2 * (i * ld + c) (c
// contiguous) or 2 * (c * ld + i) (i contiguous) from `base`, valid for
// ilo <= i < ihi and c < nc; the others load zeros (an offset past the end,
// which the buffer range check turns into 0).
struct Operand {
  const uint16_t* base;
  int64_t bytes;      // readable bytes from base (range check)
  int32_t ld;         // elements between consecutive rows of storage
  int32_t ilo, ihi;   // valid i
  int32_t nc;         // valid c
};

constexpr uint32_t kPast = 0x80000000u;   // an offset past every buffer

// Each stager keeps two register sets: slice t is loaded into set t % 2 two
// slices before its LDS store, so each load has two slices of MFMAs to land.

// c-contiguous operand: EXT rows x CH chunks, NU per thread.
template <class T, int EXT>
struct RowStager {
  static constexpr int CH = T::CH, NT = T::NT;
  static constexpr int NU = EXT * CH / NT;
  static_assert(NU * NT == EXT * CH, "rows x chunks must fill the threads");
  // unit u of this thread: row (tid + NT u) / CH, chunk (tid + NT u) % CH
  // (recomputed where used: registers are the scarce resource here)
  i32x4 v[2][NU];
  uint32_t off[NU];
  __device__ void setup(const Operand& o, int i0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int q = threadIdx.x + NT * u;
      const int i = i0 + q / CH;
      off[u] = i >= o.ilo && i < o.ihi ? (uint32_t)(((int64_t)i * o.ld + 8 * (q % CH)) * 2) : kPast;
    }
  }
  __device__ void load(int set, const __amdgpu_buffer_rsrc_t& r, const Operand&, int c0) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
      v[set][u] = __builtin_amdgcn_raw_buffer_load_b128(r, off[u] == kPast ? kPast : off[u] + 2 * c0, 0, 0);
  }
  __device__ void store(int set, uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int q = threadIdx.x + NT * u;
      *reinterpret_cast<i32x4*>(lds + lds_off<T>(q / CH, q % CH)) = v[set][u];
    }
  }
};

// i-contiguous operand: a block is two c rows (2p, 2p+1) x 8 consecutive i,
// NB = (BC / 2) (EXT / 8) blocks; block b = thread + NT u takes i chunk
// b % (EXT / 8) of c pair b / (EXT / 8), so the lanes of one c pair read
// contiguous bytes of one c row.  With fewer blocks than threads the
// remaining threads stage nothing.
template <class T, int EXT>
struct ColStager {
  static constexpr int NT = T::NT;
  static constexpr int NCX = EXT / 8;                 // i chunks
  static constexpr int NB = (T::BC / 2) * NCX;
  static constexpr int NU = (NB + NT - 1) / NT;
  // block u of this thread: b = tid + NT u, c pair b / NCX, i chunk b % NCX
  // (recomputed where used)
  i32x4 v[2][NU][2];
  uint32_t ioff[NU];   // kPast when the block stages nothing or its i are invalid
  __device__ void setup(const Operand& o, int i0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = threadIdx.x + NT * u;
      const int i = i0 + 8 * (b % NCX);    // i-contiguous extents are multiples of 8
      ioff[u] = b < NB && i >= o.ilo && i < o.ihi ? (uint32_t)(2 * i) : kPast;
    }
  }
  __device__ void load(int set, const __amdgpu_buffer_rsrc_t& r, const Operand& o, int c0) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int p = (threadIdx.x + NT * u) / NCX;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = c0 + 2 * p + h;
        const uint32_t off = ioff[u] != kPast && c < o.nc ? (uint32_t)((int64_t)c * o.ld * 2) + ioff[u] : kPast;
        v[set][u][h] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
      }
    }
  }
  // word t of block u: (i = 8 ic + t; c = 2p, 2p+1) -> LDS row i, element 2p
  __device__ void store(int set, uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = threadIdx.x + NT * u;
      if (NB % NT != 0 && b >= NB) continue;   // this thread stages no block u
      const int p = b / NCX, ic = b % NCX;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t a = (uint32_t)v[set][u][0][t / 2], w2 = (uint32_t)v[set][u][1][t / 2];
        const uint32_t w = (t & 1) ? ((a >> 16) | (w2 & 0xffff0000u)) : ((a & 0xffffu) | (w2 << 16));
        *reinterpret_cast<uint32_t*>(lds + lds_off<T>(8 * ic + t, (2 * p) / 8) + (2 * p) % 8) = w;
      }
    }
  }
};

template <class T, bool ACOL, bool BCOL>
struct Stagers {
  typename std::conditional<ACOL, ColStager<T, T::BI>, RowStager<T, T::BI>>::type a;
  typename std::conditional<BCOL, ColStager<T, T::BJ>, RowStager<T, T::BJ>>::type b;
};

// C tile [i0, i0+BI) x [j0, j0+BJ) over the contraction [0, nc): returns
// the accumulators.  acc[tw][tx][r]: j = 64 wn + 32 tw + 8 (r/4) + 4 (lane/32)
// + r%4, i = 64 wm + 32 tx + lane%32 (wave = WM wn + wm).
template <class T, bool ACOL, bool BCOL>
__device__ __forceinline__ void tile_mma(const Operand& A, const Operand& B, int i0, int j0, int nc,
                                         uint16_t (*sA)[T::BI * T::BC], uint16_t (*sB)[T::BJ * T::BC],
                                         f32x16 (&acc)[2][2]) {
  constexpr int BC = T::BC;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave / T::WM, wm = wave % T::WM;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A.base, A.bytes);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(B.base, B.bytes);
  Stagers<T, ACOL, BCOL> st;
  st.a.setup(A, i0);
  st.b.setup(B, j0);
#pragma unroll
  for (int tw = 0; tw < 2; ++tw)
#pragma unroll
    for (int tx = 0; tx < 2; ++tx)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tw][tx][r] = 0.0f;
  const int ns = (nc + BC - 1) / BC;
  if (ns == 0) return;
  const int jrow = 64 * wn + (lane & 31);
  const int irow = 64 * wm + (lane & 31);

  // set `set` <- slice kt (past the end: the last slice again, unused)
  auto gload = [&](int set, int kt) {
    const int c0 = BC * min(kt, ns - 1);
    st.a.load(set, ra, A, c0);
    st.b.load(set, rb, B, c0);
  };
  auto sstore = [&](int buf, int set) {
    st.a.store(set, sA[buf]);
    st.b.store(set, sB[buf]);
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int k = 0; k < BC / 16; ++k) {
      const int c = 2 * k + (lane >> 5);
      bf16x8 fb[2], fa[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fb[t] = as_bf16x8(*reinterpret_cast<const i32x4*>(&sB[buf][lds_off<T>(jrow + 32 * t, c)]));
        fa[t] = as_bf16x8(*reinterpret_cast<const i32x4*>(&sA[buf][lds_off<T>(irow + 32 * t, c)]));
      }
#pragma unroll
      for (int tw = 0; tw < 2; ++tw)
#pragma unroll
        for (int tx = 0; tx < 2; ++tx)
          acc[tw][tx] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tw], fa[tx], acc[tw][tx], 0, 0, 0);
    }
  };
  // slice kt sits in LDS buffer p (= kt % 2): multiply it, store slice kt+1
  // (register set p ^ 1) to the other buffer, refill that set with kt+3
  auto step = [&](int p, int kt) {
    compute(p);
    __builtin_amdgcn_sched_barrier(0);
    sstore(p ^ 1, p ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    gload(p ^ 1, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
  };

  gload(0, 0);
  gload(1, 1);
  sstore(0, 0);
  gload(0, 2);
  lds_barrier();
  int kt = 0;
  for (; kt + 2 <= ns; kt += 2) {
    step(0, kt);
    step(1, kt + 1);
  }
  if (kt < ns) compute(0);
  lds_barrier();   // every wave is done with LDS before it is reused
}

// Group e's rows, clamped to [0, R] (a malformed offsets array reads no row
// outside the buffers).
__device__ __forceinline__ void group_rows(const TrainArgs& t, int e, int& a, int& b) {
  a = min(max(t.offsets[e], 0), (int)t.R);
  b = min(max(t.offsets[e + 1], a), (int)t.R);
}

// forward / dgrad: C rows are rows r of x / dy, C columns the n / k of the
// output; a 128-row tile loops over the groups it meets.
template <int MODE>
__global__ void __launch_bounds__(RowsTile::NT, 4) train_rows_kernel(TrainArgs t) {
  using T = RowsTile;
  constexpr int BI = T::BI, BJ = T::BJ;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][T::BI * T::BC];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][T::BJ * T::BC];
  const int ncol = MODE == kTrainForward ? t.N : t.K;   // output columns
  // Logical tiles in column-tile-major order (the row tiles of one weight
  // column tile in a row), dealt to the 8 XCDs in runs of kXcdRun: block b
  // runs on XCD b % 8 as its (b / 8)-th block, so each XCD's L2 serves one
  // weight tile to kXcdRun consecutive row tiles (of one group, mostly).
  const int64_t rt = (t.R + BI - 1) / BI;
  const int64_t nlog = rt * ((ncol + BJ - 1) / BJ);
  const int64_t bk = blockIdx.x / kNumXcd;
  const int64_t L = ((bk / kXcdRun) * kNumXcd + blockIdx.x % kNumXcd) * kXcdRun + bk % kXcdRun;
  if (L >= nlog) return;
  const int r0 = (int)(L % rt) * BI;
  const int j0 = (int)(L / rt) * BJ;
  const int nc = MODE == kTrainForward ? t.K : t.N;     // contraction
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave / T::WM, wm = wave % T::WM;
  // first group with rows past r0
  int lo = 0, hi = t.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (min(max(t.offsets[mid + 1], 0), (int)t.R) > r0) hi = mid; else lo = mid + 1;
  }
  uint16_t* out = static_cast<uint16_t*>(t.out);
  for (int e = lo; e < t.E; ++e) {
    int a, b;
    group_rows(t, e, a, b);
    if (a >= r0 + BI) break;
    const int s0 = max(a, r0), s1 = min(b, r0 + BI);
    if (s1 <= s0) continue;
    // A: rows [r0, r0 + 128) of x or dy, valid only inside the group
    Operand A;
    const uint16_t* arows = MODE == kTrainForward ? t.x : t.dy;
    A.base = arows + (int64_t)r0 * nc;
    A.bytes = (int64_t)(s1 - r0) * nc * 2;
    A.ld = nc;
    A.ilo = s0 - r0;
    A.ihi = s1 - r0;
    A.nc = nc;
    // B(j, c): forward W[e][n = j][k = c] (c contiguous); dgrad W[e][n = c][k = j]
    Operand B;
    B.base = t.w + (int64_t)e * t.N * t.K;
    B.bytes = (int64_t)t.N * t.K * 2;
    B.ld = t.K;
    B.ilo = 0;
    B.ihi = ncol;
    B.nc = nc;
    f32x16 acc[2][2];
    tile_mma<T, false, MODE == kTrainDgrad>(A, B, 0, j0, nc, sA, sB, acc);
#pragma unroll
    for (int tx = 0; tx < 2; ++tx) {
      const int r = r0 + 64 * wm + 32 * tx + (lane & 31);
      if (r < s0 || r >= s1) continue;
      uint16_t* o = out + (int64_t)r * ncol;
#pragma unroll
      for (int tw = 0; tw < 2; ++tw)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = f32_to_bf16_rne(acc[tw][tx][4 * h + q]);
          const int j = j0 + 64 * wn + 32 * tw + 8 * h + 4 * (lane >> 5);
          if (j < ncol)   // a partial last column tile
            *reinterpret_cast<uint2*>(o + j) = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
        }
    }
  }
}

// wgrad: C = dW[e] tile [n0, n0+128) x [k0, k0+128), contraction over the
// group's rows: A(n, r) = dy[r][n], B(k, r) = x[r][k], both i-contiguous.
__global__ void __launch_bounds__(WgradTile::NT, 2) train_wgrad_kernel(TrainArgs t) {
  using T = WgradTile;
  constexpr int BI = T::BI, BJ = T::BJ;
  // the two operand buffers, then (after the contraction) the fp32 C tile
  constexpr int kRing = 2 * (T::BI + T::BJ) * T::BC;   // uint16 elements
  static_assert(kRing * 2 >= BI * BJ * 4, "the C tile fits the operand buffers");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kRing];
  auto sA = reinterpret_cast<uint16_t(*)[T::BI * T::BC]>(smem);
  auto sB = reinterpret_cast<uint16_t(*)[T::BJ * T::BC]>(smem + 2 * T::BI * T::BC);
  // blocks (n tile, k tile) with k fastest, per group: dealt round robin,
  // XCD x sees the k tiles congruent to x mod 8 for every n tile, so those x
  // slices stay in its L2 (runs of 8 consecutive k tiles per XCD measured
  // slower: every XCD then cycles through all the x slices)
  const int kt = (t.K + BJ - 1) / BJ;
  const int n0 = (int)(blockIdx.x / kt) * BI;
  const int k0 = (int)(blockIdx.x % kt) * BJ;
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave / T::WM, wm = wave % T::WM;
  int a, b;
  group_rows(t, e, a, b);
  const int m = b - a;
  Operand A, B;
  A.base = t.dy + (int64_t)a * t.N;
  A.bytes = (int64_t)m * t.N * 2;
  A.ld = t.N;
  A.ilo = 0;
  A.ihi = t.N;
  A.nc = m;
  B.base = t.x + (int64_t)a * t.K;
  B.bytes = (int64_t)m * t.K * 2;
  B.ld = t.K;
  B.ilo = 0;
  B.ihi = t.K;
  B.nc = m;
  f32x16 acc[2][2];
  tile_mma<T, true, true>(A, B, n0, k0, m, sA, sB, acc);
  // Epilogue through LDS (tile_mma's last barrier freed it): the C tile is
  // laid out row by row (16-byte chunks of 4 k, XOR-swizzled by row so the
  // writes from the accumulators — one chunk of 32 rows per instruction —
  // and the row reads spread over the banks); then each row's 512-byte
  // segment is read from main_grad, added and written back by 32 lanes,
  // every thread's loads of the previous values issued together.
  constexpr int NCH = BJ / 4;                  // 16-byte chunks per C row
  float* stage = reinterpret_cast<float*>(smem);
  auto chunk_at = [](int r, int c) { return (r * NCH + (c ^ (r & (NCH - 1)))) * 4; };
#pragma unroll
  for (int tx = 0; tx < 2; ++tx) {
    const int r = 64 * wm + 32 * tx + (lane & 31);
#pragma unroll
    for (int tw = 0; tw < 2; ++tw)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int c = (64 * wn + 32 * tw + 8 * h + 4 * (lane >> 5)) / 4;
        *reinterpret_cast<f32x4*>(stage + chunk_at(r, c)) =
            (f32x4){acc[tw][tx][4 * h], acc[tw][tx][4 * h + 1], acc[tw][tx][4 * h + 2], acc[tw][tx][4 * h + 3]};
      }
  }
  lds_barrier();
  float* out = static_cast<float*>(t.out) + (int64_t)e * t.N * t.K;
  constexpr int RPP = T::NT / NCH;             // rows per pass of the workgroup
  constexpr int NP = BI / RPP;                 // passes
  const int c = threadIdx.x % NCH;
  const int k = k0 + 4 * c;
  f32x4 prev[NP];
  if (t.accumulate) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = threadIdx.x / NCH + RPP * p;
      if (k < t.K) prev[p] = *reinterpret_cast<const f32x4*>(out + (int64_t)(n0 + r) * t.K + k);
    }
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = threadIdx.x / NCH + RPP * p;
    if (k >= t.K) continue;   // a partial last column tile
    f32x4 v = *reinterpret_cast<const f32x4*>(stage + chunk_at(r, c));
    if (t.accumulate) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = prev[p][q] + v[q];
    }
    *reinterpret_cast<f32x4*>(out + (int64_t)(n0 + r) * t.K + k) = v;
  }
}


// wgrad on the split ring (N and K multiples of 256): a workgroup owns the
// 256 x 256 tile [n0, n0+256) x [k0, k0+256) of dW[e] and runs the
// contraction over the group's rows in slices of 64.  Both operands hold the
// contraction along their rows (x[r][k], dy[r][n], r in the group), so both
// reach LDS in memory order — 64 rows of 256 outputs, 512 bytes a row,
// chunks XOR-swizzled by row — and both are read transposed
// (ds_read_b64_tr_b16): the MFMA rows are k (from x), the columns n (from
// dy), so a lane's accumulators hold 4 consecutive k of one n.  Each
// operand's buffer descriptor ends at the group's last row, so the rows of a
// partial last slice read zeros through the range check.  x is requested two
// slices ahead in 3 slots, dy one ahead in 2, as the inference tiles do with
// weights and routes (160 KB, one workgroup per CU); every load count is
// fixed.  The fp32 tile leaves through LDS in two halves of 128 rows of n,
// each row's 1 KB segment read, added (accumulate) and written by 64
// threads.  Tiles: per group, blocks of 4 n tiles x 8 k tiles, one block per
// XCD chunk (the tiles an XCD runs together share 4 column blocks of dy and
// 8 of x in its L2).
constexpr int kWgB = 256;              // output tile, both ways
constexpr int kWgBK = 64;              // contraction rows per slice
constexpr int kWgSlot = kWgBK * kWgB;  // uint16 elements per slot
constexpr int kWgNBlk = 4, kWgKBlk = 8;
static_assert(kWgNBlk * kWgKBlk == tile::kXcdChunk, "a block fills one XCD chunk");

__global__ void __launch_bounds__(1024, 4) train_wgrad_tile_kernel(TrainArgs t, int nnt, int nkt) {
  constexpr int NW = 16, WM = 4;           // waves: 4 along k x 4 along n, 64 x 64 each
  constexpr int LW = 2, LX = 2;            // 1 KB loads per wave per slice, each operand
  constexpr int NSTEP = kWgBK / 16;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[5 * kWgSlot];
  uint16_t* const wbase = smem;                 // 3 slots of x^T
  uint16_t* const rbase = smem + 3 * kWgSlot;   // 2 slots of dy^T

  const int64_t b = blockIdx.x;
  const int64_t kx = b / tile::NXCD;
  const int64_t chunk = (kx / tile::kXcdChunk) * tile::NXCD + b % tile::NXCD;
  const int tt = (int)(kx % tile::kXcdChunk);
  const int nnb = (nnt + kWgNBlk - 1) / kWgNBlk, nkb = (nkt + kWgKBlk - 1) / kWgKBlk;
  const int64_t cpg = (int64_t)nnb * nkb;
  const int64_t e = chunk / cpg;
  if (e >= t.E) return;
  const int lc = (int)(chunk % cpg);
  const int ntile = (lc / nkb) * kWgNBlk + tt / kWgKBlk;
  const int ktile = (lc % nkb) * kWgKBlk + tt % kWgKBlk;
  if (ntile >= nnt || ktile >= nkt) return;
  const int n0 = ntile * kWgB, k0 = ktile * kWgB;
  int a, z;
  group_rows(t, (int)e, a, z);
  const int m = z - a;
  const int nk = (m + kWgBK - 1) / kWgBK;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave / WM, wm = wave % WM;
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(t.x + (int64_t)a * t.K, (int64_t)m * t.K * 2);
  const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(t.dy + (int64_t)a * t.N, (int64_t)m * t.N * 2);
  // block i of this wave: slot rows 2 (wave + 16 i) and +1; lane l -> row
  // 2 (wave + 16 i) + l / 32, physical chunk l % 32 (logical chunk
  // wt_logical(row, l % 32))
  uint32_t ow[LW], orr[LX];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int r = 2 * (wave + NW * i) + lane / 32;
    const int c = tile::wt_logical(r, lane % 32);
    ow[i] = (uint32_t)(((int64_t)r * t.K + k0 + 8 * c) * 2);
    orr[i] = (uint32_t)(((int64_t)r * t.N + n0 + 8 * c) * 2);
  }
  const int wstep = kWgBK * t.K * 2, rstep = kWgBK * t.N * 2;   // bytes per slice
  auto issue_w = [&](int kt) {
    uint16_t* slot = wbase + (kt % 3) * kWgSlot;
#pragma unroll
    for (int i = 0; i < LW; ++i) lds_load16(wr, slot + (wave + NW * i) * 512, ow[i], kt * wstep);
    issue_order();
  };
  auto issue_r = [&](int kt) {
    uint16_t* slot = rbase + (kt % 2) * kWgSlot;
#pragma unroll
    for (int i = 0; i < LX; ++i) lds_load16(rr, slot + (wave + NW * i) * 512, orr[i], kt * rstep);
    issue_order();
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  bf16x8 fw[2][2], fx[2][2];
  auto fload = [&](int fb, int kt, int st) {
    const uint16_t* ws = wbase + (kt % 3) * kWgSlot;
    const uint16_t* rs = rbase + (kt % 2) * kWgSlot;
#pragma unroll
    for (int i = 0; i < 2; ++i) fw[fb][i] = tile::wt_frag(ws, wn * 64 + 32 * i, 16 * st, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) fx[fb][j] = tile::wt_frag(rs, wm * 64 + 32 * j, 16 * st, lane);
  };
  auto mma = [&](int fb) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[fb][i], fx[fb][j], acc[i][j], 0, 0, 0);
  };
  // 8 LDS reads and 4 MFMAs a step: read, MFMA in pairs, then the reads left
  auto interleave = [&]() {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  };

  if (nk > 0) {
    // prologue: x^T 0, dy^T 0 and 1, x^T 1 and 2; wait for slice 0 (the
    // count leaves only x^T loads outstanding, as in the inference tiles)
    issue_w(0);
    issue_r(0);
    if (nk > 1) { issue_r(1); issue_w(1); }
    if (nk > 2) issue_w(2);
    if (nk > 2) wait_vm<2 * LW>();
    else if (nk > 1) wait_vm<LW>();
    else wait_vm<0>();
    lds_barrier();
    // slice kt; MODE 2: slices kt+2 and kt+3 exist, 1: only kt+2, 0: only
    // kt+1, -1: kt is the last
    auto slice = [&](int kt, auto mode) {
      constexpr int MODE = decltype(mode)::value;
#pragma unroll
      for (int st = 0; st + 1 < NSTEP; ++st) {
        fload((st + 1) & 1, kt, st + 1);
        mma(st & 1);
        interleave();
      }
      if (MODE >= 0) {
        if (MODE >= 1) wait_vm<LW>();   // slice kt+1 is in; x^T of kt+2 may fly
        else wait_vm<0>();
        lds_barrier();                  // nobody reads slice kt's slots any more
        if (MODE >= 1) issue_r(kt + 2);
        if (MODE >= 2) issue_w(kt + 3);
        fload(0, kt + 1, 0);
        mma((NSTEP - 1) & 1);
        interleave();
      } else {
        mma((NSTEP - 1) & 1);
      }
    };
    fload(0, 0, 0);
    int kt = 0;
    for (; kt + 3 < nk; ++kt) slice(kt, std::integral_constant<int, 2>());
    if (kt + 2 < nk) slice(kt++, std::integral_constant<int, 1>());
    if (kt + 1 < nk) slice(kt++, std::integral_constant<int, 0>());
    slice(kt, std::integral_constant<int, -1>());
    wait_vm<0>();
    lds_barrier();
  }

  // epilogue: acc[i][j][4q + h]: k = wn 64 + 32 i + 8 q + 4 (lane / 32) + h,
  // n = wm 64 + 32 j + lane % 32.  Half hf stages the n rows [128 hf,
  // 128 hf + 128) as fp32 rows of 256 k, 16-byte chunk c of row r at
  // c ^ (r & 63).
  float* stage = reinterpret_cast<float*>(smem);
  float* out = static_cast<float*>(t.out) + (e * t.N + n0) * (int64_t)t.K + k0;
  const int c = threadIdx.x % 64;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    if (wm / 2 == hf) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = (wm - 2 * hf) * 64 + 32 * j + (lane & 31);
            const int kc = (wn * 64 + 32 * i + 8 * q + 4 * (lane >> 5)) / 4;
            *reinterpret_cast<f32x4*>(stage + r * 256 + ((kc ^ (r & 63)) << 2)) =
                (f32x4){acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
    }
    lds_barrier();
    f32x4 prev[8];
    if (t.accumulate) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int r = threadIdx.x / 64 + 16 * p;
        prev[p] = *reinterpret_cast<const f32x4*>(out + (int64_t)(128 * hf + r) * t.K + 4 * c);
      }
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = threadIdx.x / 64 + 16 * p;
      f32x4 v = *reinterpret_cast<const f32x4*>(stage + r * 256 + ((c ^ (r & 63)) << 2));
      if (t.accumulate) {
#pragma unroll
        for (int h = 0; h < 4; ++h) v[h] = prev[p][h] + v[h];
      }
      *reinterpret_cast<f32x4*>(out + (int64_t)(128 * hf + r) * t.K + 4 * c) = v;
    }
    lds_barrier();   // the half's reads are done before the next half is staged
  }
}

}  // namespace train

// Forward and dgrad on the inference tile kernel (rows layout: 256 rows of
// x or dy by 256 output features per tile, both operands loaded straight
// into LDS; for dgrad W[e] is read transposed from LDS) when the output
// width (N for the forward, K for dgrad) is a multiple of 256.
static bool rows_on_tiles(const TrainArgs& t) {
  return (t.mode == kTrainForward && t.N % 256 == 0) || (t.mode == kTrainDgrad && t.K % 256 == 0);
}

static hipError_t launch_rows_tiles(const TrainArgs& t, hipStream_t s) {
  const bool fwd = t.mode == kTrainForward;
  const int nc = fwd ? t.K : t.N;      // contraction
  const int nout = fwd ? t.N : t.K;    // output features
  GemmArgs g = {};
  g.epi = kEpiDown;
  g.rows.layout = 2;
  g.act = fwd ? t.x : t.dy;
  g.act_ld = nc;
  g.act_bytes = t.R * nc * 2;
  g.w = t.w;
  g.w_expert_stride = (int64_t)t.N * t.K;
  g.kdim = nc;
  g.nfeat = nout;
  g.E = t.E;
  g.out = t.out;
  g.out_ld = nout;
  return launch_tile_rows_bf16(g, t.offsets, t.R, !fwd, s);
}

hipError_t launch_train(const TrainArgs& t, hipStream_t s) {
  using namespace train;
  if (rows_on_tiles(t)) return launch_rows_tiles(t, s);
  if (t.mode == kTrainWgrad && t.N % kWgB == 0 && t.K % kWgB == 0) {
    const int nnt = t.N / kWgB, nkt = t.K / kWgB;
    const int64_t cpg = (int64_t)((nnt + kWgNBlk - 1) / kWgNBlk) * ((nkt + kWgKBlk - 1) / kWgKBlk);
    const int64_t nchunk = (t.E * cpg + tile::NXCD - 1) / tile::NXCD * tile::NXCD;
    hipLaunchKernelGGL(train_wgrad_tile_kernel, dim3((unsigned)(nchunk * tile::kXcdChunk)), dim3(1024), 0, s, t, nnt,
                       nkt);
    return hipGetLastError();
  }
  if (t.mode == kTrainWgrad) {
    using W = WgradTile;
    hipLaunchKernelGGL(train_wgrad_kernel, dim3((t.N / W::BI) * ((t.K + W::BJ - 1) / W::BJ), t.E),
                       dim3(W::NT), 0, s, t);
  } else {
    if (t.R == 0) return hipSuccess;
    const int ncol = t.mode == kTrainForward ? t.N : t.K;
    using T = RowsTile;
    const int64_t nlog = (t.R + T::BI - 1) / T::BI * ((ncol + T::BJ - 1) / T::BJ);
    const int64_t unit = (int64_t)kNumXcd * kXcdRun;
    const dim3 grid((unsigned)((nlog + unit - 1) / unit * unit));
    if (t.mode == kTrainForward)
      hipLaunchKernelGGL(train_rows_kernel<kTrainForward>, grid, dim3(T::NT), 0, s, t);
    else
      hipLaunchKernelGGL(train_rows_kernel<kTrainDgrad>, grid, dim3(T::NT), 0, s, t);
  }
  return hipGetLastError();
}

}  // namespace moe
