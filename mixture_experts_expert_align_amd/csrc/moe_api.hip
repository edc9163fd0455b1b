// The C ABI declared in include/moe_mi355x.h: validation, planning,
// workspace layout and the launch sequences.  Host code, plus the one device
// array that moe_apply_contiguous_static uses as its workspace; it enqueues
// kernels on the caller's stream and never allocates or synchronises.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_mi355x.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int64_t kAlign = 256;
inline int64_t up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return p && ((uintptr_t)p & 3u) == 0; }
// MXFP8 weights, with row-major or grouped scale arrays
inline bool is_mxfp8(const moe_problem& P) { return P.w_dtype == MOE_W_MXFP8 || P.w_dtype == MOE_W_MXFP8_GROUPED; }

int fail(moe_plan* plan, int code, const char* msg) {
  if (plan) snprintf(plan->reason, sizeof(plan->reason), "%s", msg);
  return code;
}

struct AlignLayout {
  int64_t counts, offsets, sorted, block_bucket, num_post, active, status, scratch, end;
};

AlignLayout layout_align(int64_t base, int64_t nb, int64_t capacity, int64_t max_tiles,
                         int64_t max_active, int64_t nblocks) {
  AlignLayout L;
  int64_t o = base;
  L.counts = o;       o = up(o + 4 * nb, kAlign);
  L.offsets = o;      o = up(o + 4 * (nb + 1), kAlign);
  L.sorted = o;       o = up(o + 4 * capacity, kAlign);
  L.block_bucket = o; o = up(o + 4 * max_tiles, kAlign);
  L.num_post = o;     o = up(o + 4, kAlign);
  L.active = o;       o = up(o + 4 * (max_active + 1), kAlign);
  L.status = o;       o = up(o + 16, kAlign);
  L.scratch = o;      o = up(o + 4 * nblocks * (nb + 1), kAlign);
  L.end = o;
  return L;
}

int64_t align_nblocks(int64_t R) {
  if (R <= kAlignSmallMaxR) return 0;
  const int64_t n = (R + kAlignChunk - 1) / kAlignChunk;
  return n < kAlignMaxBlocks ? n : kAlignMaxBlocks;
}

template <typename T>
T* at(void* base, int64_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

AlignArgs align_args(const moe_plan* p, const int32_t* keys, const int32_t* expert_map, void* ws13) {
  AlignArgs a{};
  a.keys = keys;
  a.key_map = expert_map;
  a.key_range = (int32_t)p->prob.global_experts;
  a.R = p->routes;
  a.nb = (int32_t)p->prob.E;
  a.B = p->block_m;
  a.counts = at<int32_t>(ws13, p->off_counts);
  a.offsets = at<int32_t>(ws13, p->off_offsets);
  a.sorted = at<int32_t>(ws13, p->off_sorted_ids);
  a.block_bucket = at<int32_t>(ws13, p->off_block_expert);
  a.num_post = at<int32_t>(ws13, p->off_num_post_padded);
  a.active = at<int32_t>(ws13, p->off_active);
  a.status = at<int32_t>(ws13, p->off_status);
  a.block_hist = at<int32_t>(ws13, p->off_align_scratch);
  a.capacity = p->sorted_capacity;
  a.max_tiles = p->max_tiles;
  a.max_active = p->max_active;
  a.sentinel = (int32_t)p->routes;
  a.nblocks = (int32_t)p->align_blocks;
  return a;
}

}  // namespace

// ------------------------------------------------ the allocation-free call ----
// The workspaces of moe_apply_contiguous_static: one array per GPU, held from
// the library's load until the process ends.  Host code never uses the
// array's name as an address (in host code it names a host-side stand-in);
// it takes the device address hipGetSymbolAddress returns for the current
// device, once per device.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, or nullptr.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported problem";
    case MOE_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

void moe_struct_sizes(int64_t* problem, int64_t* plan, int64_t* weights) {
  if (problem) *problem = sizeof(moe_problem);
  if (plan) *plan = sizeof(moe_plan);
  if (weights) *weights = sizeof(moe_weights);
}

const char* moe_plan_reason(const moe_plan* plan) { return plan ? plan->reason : ""; }

int moe_plan_init(moe_plan* plan, const moe_problem* prob) {
  if (!plan || !prob) return MOE_EINVAL;
  memset(plan, 0, sizeof(*plan));
  plan->prob = *prob;
  plan->abi_version = MOE_ABI_VERSION;
  const moe_problem& P = *prob;
  if (P.M <= 0 || P.K <= 0 || P.I <= 0 || P.E <= 0)
    return fail(plan, MOE_EINVAL, "M, K, I and E must be positive");
  if (P.layout != MOE_LAYOUT_CONTIGUOUS && P.layout != MOE_LAYOUT_BATCHED)
    return fail(plan, MOE_EINVAL, "unknown layout");
  if (P.w_dtype != MOE_W_BF16 && !is_mxfp8(P))
    return fail(plan, MOE_EINVAL, "unknown weight dtype");
  if (P.w1_order != MOE_W1_HALVES && P.w1_order != MOE_W1_INTERLEAVE16)
    return fail(plan, MOE_EINVAL, "unknown W1 row order");
  if (P.variant < MOE_VARIANT_AUTO || P.variant > MOE_VARIANT_FUSED)
    return fail(plan, MOE_EINVAL, "unknown variant");
  const bool contiguous = P.layout == MOE_LAYOUT_CONTIGUOUS;
  if (contiguous) {
    if (P.global_experts != 0 && (P.global_experts < P.E || P.global_experts >= (1ll << 31)))
      return fail(plan, MOE_EINVAL, "global_experts must be 0 or in [E, 2^31)");
    const int64_t id_space = P.global_experts ? P.global_experts : P.E;
    if (P.topk <= 0 || P.topk > id_space)
      return fail(plan, MOE_EINVAL, "topk must be in [1, E] (or [1, global_experts])");
  } else {
    if (P.max_tokens <= 0) return fail(plan, MOE_EINVAL, "max_tokens must be positive");
    if (P.global_experts != 0) return fail(plan, MOE_EINVAL, "the batched format takes local experts only");
  }
  const int64_t R = contiguous ? P.M * P.topk : P.E * P.max_tokens;
  // flat slot ids, positions and the sentinel are int32; rows are addressed
  // in 64-bit, so only these ranges matter
  if (R >= (1ll << 31) - 1 || P.M >= (1ll << 31) || P.E > kAlignMaxBuckets)
    return fail(plan, MOE_EINVAL, "routes or experts past the 32-bit index range");
  if (P.w1_order == MOE_W1_INTERLEAVE16 && P.I % 16)
    return fail(plan, MOE_EINVAL, "the 16-row interleave needs I % 16 == 0");

  int variant = P.variant;
  if (is_mxfp8(P)) {
    if (!contiguous)
      return fail(plan, MOE_EUNSUPPORTED, "MXFP8 weights are built for the contiguous format only");
    if (variant == MOE_VARIANT_FUSED)
      return fail(plan, MOE_EUNSUPPORTED, "MXFP8 weights have no single-launch kernel");
    if (P.K % 128 || P.I % 128)
      return fail(plan, MOE_EUNSUPPORTED, "MXFP8 kernels need K % 128 == 0 and I % 128 == 0");
    if (2 * P.I * P.K >= (1ll << 31))
      return fail(plan, MOE_EUNSUPPORTED, "MXFP8 kernels address one expert with 32-bit offsets");
    // the tiles (128 weight rows: 64 W1 features, 128 W2 rows, covered by
    // the checks above) unless the streaming kernels are asked for
    if (variant == MOE_VARIANT_AUTO) variant = MOE_VARIANT_TILE;
    if (P.w_dtype == MOE_W_MXFP8_GROUPED) {
      if (variant != MOE_VARIANT_TILE)
        return fail(plan, MOE_EUNSUPPORTED, "grouped MXFP8 scales are read by the tile kernels only");
      if (P.K % 512 || P.I % 512)
        return fail(plan, MOE_EUNSUPPORTED, "grouped MXFP8 scales need K % 512 == 0 and I % 512 == 0");
    }
    if (variant == MOE_VARIANT_TILE) {
      snprintf(plan->reason, sizeof(plan->reason),
               "tile (MXFP8): 128 weight rows x 64 routes per workgroup, both operands staged in LDS");
    } else {
      snprintf(plan->reason, sizeof(plan->reason),
               "stream (MXFP8): weight rows streamed into scaled MFMA, 64 tokens per pass");
    }
  } else {
    if (variant == MOE_VARIANT_AUTO) {
      // small layers (all weights within 1 GiB, at most 32 rows per expert
      // that can hold a route, one-workgroup align): one launch plus the
      // reduce, where launch latency is most of the time; few rows per
      // expert: the two streaming launches; otherwise the tiles
      const int64_t slots = P.E < R ? P.E : R;
      const bool small = 6 * P.E * P.I * P.K <= (1ll << 30) && R <= 32 * slots && R <= kAlignSmallMaxR &&
                         P.E <= kFusedMaxExperts && P.K % 128 == 0 && P.I % 128 == 0;
      variant = !contiguous ? MOE_VARIANT_TILE
                : small     ? MOE_VARIANT_FUSED
                : P.M <= 16 ? MOE_VARIANT_STREAM
                            : MOE_VARIANT_TILE;
    }
    if (variant == MOE_VARIANT_STREAM || variant == MOE_VARIANT_FUSED) {
      if (!contiguous) return fail(plan, MOE_EUNSUPPORTED, "the streaming kernels take the contiguous format only");
      if (P.K % 128 || P.I % 128)
        return fail(plan, MOE_EUNSUPPORTED, "streaming kernels need K % 128 == 0 and I % 128 == 0");
      // 32-bit buffer offsets: one expert's W1 and the activation buffers
      if (4 * P.I * P.K >= (1ll << 31) || 2 * P.M * P.K >= (1ll << 31))
        return fail(plan, MOE_EUNSUPPORTED, "streaming kernels address one expert with 32-bit offsets");
      if (variant == MOE_VARIANT_FUSED) {
        if (R > kAlignSmallMaxR || P.E > kFusedMaxExperts)
          return fail(plan, MOE_EUNSUPPORTED, "the single-launch kernel needs M*topk <= 8192 and E <= 2048");
        snprintf(plan->reason, sizeof(plan->reason),
                 "fused: align, W1 and W2 streaming strips in one launch (device work queue), then the reduce");
      } else {
        snprintf(plan->reason, sizeof(plan->reason),
                 "stream: M <= 16 rows per expert, weights streamed into the MFMA row operand");
      }
    } else {
      // 32-bit buffer offsets: one expert's W1, the activation rows and z
      const int64_t act_rows = contiguous ? P.M : P.E * P.max_tokens;
      if (4 * P.I * P.K >= (1ll << 31) || 2 * act_rows * P.K >= (1ll << 31) ||
          2 * (contiguous ? R + P.E * kTileRoutesContiguous : act_rows) * P.I >= (1ll << 31))
        return fail(plan, MOE_EUNSUPPORTED, "tiled kernels address one expert and the activations with 32-bit offsets");
      if (contiguous) {
        if (P.K % 256 || P.I % 128)
          return fail(plan, MOE_EUNSUPPORTED, "contiguous tiled kernels need K % 256 == 0 and I % 128 == 0");
        snprintf(plan->reason, sizeof(plan->reason),
                 "tile: 256 weight rows x 256 routes per workgroup, slices loaded straight into LDS");
      } else {
        if (P.K % 128 || P.I % 64)
          return fail(plan, MOE_EUNSUPPORTED, "batched tiled kernels need K % 128 == 0 and I % 64 == 0");
        snprintf(plan->reason, sizeof(plan->reason),
                 "tile: 128 weight rows x 128 rows per workgroup, route-tile-major order");
      }
    }
  }
  plan->variant = variant;
  plan->block_m = variant != MOE_VARIANT_TILE   ? 16
                  : !contiguous                  ? kTileRowsBatched
                  : is_mxfp8(P)                  ? kTileRoutesMxfp8
                                                 : kTileRoutesContiguous;
  plan->reduce_kind = contiguous ? MOE_REDUCE_NOOP : MOE_REDUCE_NAIVE_BATCHED;
  plan->routes = R;
  const int64_t B = plan->block_m;
  if (contiguous) {
    plan->max_active = P.E < R ? P.E : R;
    plan->max_tiles = (R + plan->max_active * (B - 1)) / B;
    plan->sorted_capacity = plan->max_tiles * B;
    plan->align_blocks = variant == MOE_VARIANT_FUSED ? 0 : align_nblocks(R);
  } else {
    plan->max_active = P.E;
    plan->max_tiles = 0;
    plan->sorted_capacity = 0;
    plan->align_blocks = 0;
  }
  if (plan->max_tiles > 65535 || plan->max_active > 65535)
    return fail(plan, MOE_EUNSUPPORTED, "grid too large");
  if (contiguous && (variant != MOE_VARIANT_TILE || is_mxfp8(P))) {
    // the streaming and MXFP8 kernels read z (and for MXFP8 the gathered
    // activation codes) through one buffer resource with 32-bit offsets,
    // whose range check stops at 2^31 - 1 bytes: rows past it would read 0
    const int64_t zbytes = plan->sorted_capacity * P.I * (is_mxfp8(P) ? 1 : 2);
    const int64_t xqbytes = is_mxfp8(P) ? plan->sorted_capacity * P.K : 0;
    if (zbytes >= (1ll << 31) - 1 || xqbytes >= (1ll << 31) - 1)
      return fail(plan, MOE_EUNSUPPORTED,
                  "streaming/MXFP8 kernels address z and the gathered activations with 32-bit offsets");
  }

  AlignLayout L = layout_align(0, P.E, plan->sorted_capacity, plan->max_tiles, plan->max_active,
                               plan->align_blocks);
  plan->off_counts = L.counts;
  plan->off_offsets = L.offsets;
  plan->off_sorted_ids = L.sorted;
  plan->off_block_expert = L.block_bucket;
  plan->off_num_post_padded = L.num_post;
  plan->off_active = L.active;
  plan->off_status = L.status;
  plan->off_align_scratch = L.scratch;
  int64_t o = L.end;
  const int64_t zrows = contiguous ? plan->sorted_capacity : P.E * P.max_tokens;
  plan->off_z = o;
  if (is_mxfp8(P)) {
    o = up(o + zrows * P.I, kAlign);
    plan->off_z_scale = o;
    o = up(o + zrows * (P.I / 32), kAlign);
    plan->off_xq = o;
    o = up(o + zrows * P.K, kAlign);
    plan->off_xq_scale = o;
    o = up(o + zrows * (P.K / 32), kAlign);
  } else {
    o = up(o + zrows * P.I * 2, kAlign);
    plan->off_z_scale = plan->off_xq = plan->off_xq_scale = -1;
  }
  if (variant == MOE_VARIANT_FUSED) {
    plan->off_sync = o;
    o = up(o + 4 * sync_words(plan->max_active), kAlign);
  } else {
    plan->off_sync = -1;
  }
  plan->ws13_bytes = o;
  plan->ws2_bytes = contiguous ? up(R * P.K * 2, kAlign) : 0;
  plan->out_rows = contiguous ? P.M : P.E * P.max_tokens;
  plan->out_cols = P.K;
  return MOE_OK;
}

// An expert map is given exactly when the plan's ids are global.
static bool map_ok(const moe_plan* plan, const int32_t* expert_map) {
  return plan->prob.global_experts ? aligned4(expert_map) : expert_map == nullptr;
}

int moe_align_permute(const moe_plan* plan, const int32_t* topk_ids, const int32_t* expert_map,
                      void* ws13, void* stream) {
  if (!plan || plan->abi_version != MOE_ABI_VERSION) return MOE_EINVAL;
  if (plan->prob.layout != MOE_LAYOUT_CONTIGUOUS) return MOE_EINVAL;
  if (!aligned4(topk_ids) || !aligned16(ws13) || !map_ok(plan, expert_map)) return MOE_EINVAL;
  AlignArgs a = align_args(plan, topk_ids, expert_map, ws13);
  return launch_align(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

static GemmArgs gemm_common(const moe_plan* p, void* ws13) {
  GemmArgs g{};
  const moe_problem& P = p->prob;
  g.rows.layout = P.layout;
  g.rows.sorted_ids = at<int32_t>(ws13, p->off_sorted_ids);
  g.rows.block_expert = at<int32_t>(ws13, p->off_block_expert);
  g.rows.num_post = at<int32_t>(ws13, p->off_num_post_padded);
  g.rows.offsets = at<int32_t>(ws13, p->off_offsets);
  g.rows.counts = at<int32_t>(ws13, p->off_counts);
  g.rows.active = at<int32_t>(ws13, p->off_active);
  g.rows.topk = (int32_t)P.topk;
  g.rows.sentinel = (int32_t)p->routes;
  g.rows.max_tokens = (int32_t)P.max_tokens;
  g.I = (int32_t)P.I;
  g.w1_order = P.w1_order;
  g.E = (int32_t)P.E;
  g.max_tiles = p->max_tiles;
  g.max_active = p->max_active;
  return g;
}

static bool contiguous_args_ok(const moe_plan* plan, const moe_weights* w) {
  if (!plan || plan->abi_version != MOE_ABI_VERSION || !w) return false;
  const moe_problem& P = plan->prob;
  if (P.layout != MOE_LAYOUT_CONTIGUOUS) return false;
  if (!aligned16(w->w1) || !aligned16(w->w2)) return false;
  if (P.w_dtype == MOE_W_MXFP8 && (!aligned4(w->w1_scale) || !aligned4(w->w2_scale))) return false;
  if (P.w_dtype == MOE_W_MXFP8_GROUPED && (!aligned16(w->w1_scale) || !aligned16(w->w2_scale))) return false;
  return true;
}

static GemmArgs w1_args(const moe_plan* plan, const moe_weights* w, void* ws13) {
  const moe_problem& P = plan->prob;
  GemmArgs g = gemm_common(plan, ws13);
  g.epi = kEpiGateUp;
  g.w = w->w1;
  g.w_scale = w->w1_scale;
  g.w_expert_stride = 2 * P.I * P.K;
  g.kdim = (int32_t)P.K;
  g.nfeat = (int32_t)P.I;
  g.out = at<void>(ws13, plan->off_z);
  g.out_ld = P.I;
  return g;
}

static GemmArgs w2_args(const moe_plan* plan, const moe_weights* w, void* ws13, void* ws2) {
  const moe_problem& P = plan->prob;
  GemmArgs g = gemm_common(plan, ws13);
  g.epi = kEpiDown;
  g.w = w->w2;
  g.w_scale = w->w2_scale;
  g.w_expert_stride = P.K * P.I;
  g.kdim = (int32_t)P.I;
  g.nfeat = (int32_t)P.K;
  g.act = at<void>(ws13, plan->off_z);
  g.act_ld = P.I;
  g.act_bytes = plan->sorted_capacity * P.I * 2;
  g.out = ws2;
  g.out_ld = P.K;
  return g;
}

// Grouped MXFP8 scales: bytes between the 16-byte groups of the gathered
// activations' and z's scale arrays (sorted_capacity rows each); 0 for
// row-major scales.
static int64_t scale_group(const moe_plan* plan) {
  return plan->prob.w_dtype == MOE_W_MXFP8_GROUPED ? plan->sorted_capacity * 16 : 0;
}

static int gate_up_act(const moe_plan* plan, const void* a, const moe_weights* w, void* ws13,
                       hipStream_t s) {
  const moe_problem& P = plan->prob;
  GemmArgs g = w1_args(plan, w, ws13);
  if (is_mxfp8(P)) {
    uint8_t* xq = at<uint8_t>(ws13, plan->off_xq);
    uint8_t* xqs = at<uint8_t>(ws13, plan->off_xq_scale);
    g.scale_group = scale_group(plan);
    if (launch_quantize_gather_mxfp8(static_cast<const uint16_t*>(a), g.rows.sorted_ids,
                                     g.rows.num_post, (int32_t)P.topk, g.rows.sentinel,
                                     plan->sorted_capacity, P.K, xq, xqs, g.scale_group, s) != hipSuccess)
      return MOE_EHIP;
    g.act = xq;
    g.act_scale = xqs;
    g.act_ld = P.K;
    g.act_bytes = plan->sorted_capacity * P.K;
    g.out_scale = at<uint8_t>(ws13, plan->off_z_scale);
    const hipError_t e = plan->variant == MOE_VARIANT_TILE ? launch_gemm_tile_mxfp8(g, s) : launch_gemm_stream_mxfp8(g, s);
    return e == hipSuccess ? MOE_OK : MOE_EHIP;
  }
  g.act = a;
  g.act_ld = P.K;
  g.act_bytes = P.M * P.K * 2;
  hipError_t e = plan->variant != MOE_VARIANT_TILE ? launch_gemm_stream_bf16(g, s)
                                                     : launch_gemm_tile_bf16(g, s);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

static int down_unpermute(const moe_plan* plan, const moe_weights* w, void* ws13, void* ws2,
                          hipStream_t s) {
  const moe_problem& P = plan->prob;
  GemmArgs g = w2_args(plan, w, ws13, ws2);
  hipError_t e;
  if (is_mxfp8(P)) {
    g.act_scale = at<uint8_t>(ws13, plan->off_z_scale);
    g.scale_group = scale_group(plan);
    g.act_bytes = plan->sorted_capacity * P.I;
    e = plan->variant == MOE_VARIANT_TILE ? launch_gemm_tile_mxfp8(g, s) : launch_gemm_stream_mxfp8(g, s);
  } else {
    e = plan->variant != MOE_VARIANT_TILE ? launch_gemm_stream_bf16(g, s)
                                            : launch_gemm_tile_bf16(g, s);
  }
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_gate_up_act(const moe_plan* plan, const void* a, const moe_weights* w, void* ws13,
                    void* stream) {
  if (!contiguous_args_ok(plan, w) || !aligned16(a) || !aligned16(ws13)) return MOE_EINVAL;
  return gate_up_act(plan, a, w, ws13, (hipStream_t)stream);
}

int moe_down_unpermute(const moe_plan* plan, const moe_weights* w, void* ws13, void* ws2,
                       void* stream) {
  if (!contiguous_args_ok(plan, w) || !aligned16(ws13) || !aligned16(ws2)) return MOE_EINVAL;
  return down_unpermute(plan, w, ws13, ws2, (hipStream_t)stream);
}

// The launches of moe_apply_contiguous (arguments already validated).
static int apply_contiguous(const moe_plan* plan, const void* a, const int32_t* topk_ids,
                            const float* topk_weights, const moe_weights* w, void* out, void* ws13,
                            void* ws2, hipStream_t s) {
  const moe_problem& P = plan->prob;
  AlignArgs al = align_args(plan, topk_ids, w->expert_map, ws13);
  if (plan->variant == MOE_VARIANT_FUSED) {
    FusedArgs f{};
    f.align = al;
    f.w1 = w1_args(plan, w, ws13);
    f.w1.act = a;
    f.w1.act_ld = P.K;
    f.w1.act_bytes = P.M * P.K * 2;
    f.w2 = w2_args(plan, w, ws13, ws2);
    f.sync = at<int32_t>(ws13, plan->off_sync);
    f.max_active = plan->max_active;
    if (launch_fused_stream_bf16(f, s) != hipSuccess) return MOE_EHIP;
  } else {
    if (launch_align(al, s) != hipSuccess) return MOE_EHIP;
    int st = gate_up_act(plan, a, w, ws13, s);
    if (st != MOE_OK) return st;
    st = down_unpermute(plan, w, ws13, ws2, s);
    if (st != MOE_OK) return st;
  }
  const bool fused = plan->variant == MOE_VARIANT_FUSED;
  hipError_t e = launch_reduce_contiguous(static_cast<const uint16_t*>(ws2), topk_ids, topk_weights,
                                          w->expert_map, (int32_t)P.global_experts,
                                          static_cast<uint16_t*>(out), P.M, (int32_t)P.topk, P.K,
                                          (int32_t)P.E,
                                          fused ? at<int32_t>(ws13, plan->off_sync) : nullptr,
                                          fused ? sync_counter_lines(plan->max_active) : 0, s);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

static bool apply_args_ok(const moe_plan* plan, const void* a, const int32_t* topk_ids,
                          const float* topk_weights, const moe_weights* w, const void* out) {
  return contiguous_args_ok(plan, w) && map_ok(plan, w->expert_map) && aligned16(a) &&
         aligned4(topk_ids) && aligned4(topk_weights) && aligned16(out);
}

int moe_apply_contiguous(const moe_plan* plan, const void* a, const int32_t* topk_ids,
                         const float* topk_weights, const moe_weights* w, void* out, void* ws13,
                         void* ws2, void* stream) {
  if (!apply_args_ok(plan, a, topk_ids, topk_weights, w, out) || !aligned16(ws13) || !aligned16(ws2))
    return MOE_EINVAL;
  return apply_contiguous(plan, a, topk_ids, topk_weights, w, out, ws13, ws2, (hipStream_t)stream);
}

int moe_apply_contiguous_static(const moe_plan* plan, const void* a, const int32_t* topk_ids,
                                const float* topk_weights, const moe_weights* w, void* out,
                                void* stream) {
  if (!apply_args_ok(plan, a, topk_ids, topk_weights, w, out)) return MOE_EINVAL;
  const int64_t ws2_off = up(plan->ws13_bytes, kAlign);
  if (plan->ws13_bytes <= 0 || ws2_off + plan->ws2_bytes > (int64_t)MOE_STATIC_SCRATCH_BYTES)
    return MOE_EUNSUPPORTED;
  uint8_t* base = static_cast<uint8_t*>(scratch_on_current_device());
  if (!base) return MOE_EHIP;
  hipStream_t s = (hipStream_t)stream;
  void* ws13 = base;
  void* ws2 = base + ws2_off;
  // The array keeps whatever the previous call (of any plan) left in it.
  // Every buffer the kernels read is written earlier in the same call,
  // except the single-launch variant's work-queue counters and the status
  // words it counts into: clear those first, with a kernel rather than a
  // memset node, so the call stays capturable.
  if (launch_zero_words(at<int32_t>(ws13, plan->off_status), 4, 1, s) != hipSuccess) return MOE_EHIP;
  if (plan->variant == MOE_VARIANT_FUSED &&
      launch_zero_words(at<int32_t>(ws13, plan->off_sync), sync_counter_lines(plan->max_active), kSyncLine,
                        s) != hipSuccess)
    return MOE_EHIP;
  return apply_contiguous(plan, a, topk_ids, topk_weights, w, out, ws13, ws2, s);
}

int moe_apply_batched(const moe_plan* plan, const void* a, const int32_t* expert_num_tokens,
                      const moe_weights* w, void* y, void* ws13, void* stream) {
  if (!plan || plan->abi_version != MOE_ABI_VERSION || !w) return MOE_EINVAL;
  const moe_problem& P = plan->prob;
  if (P.layout != MOE_LAYOUT_BATCHED) return MOE_EINVAL;
  if (!aligned16(a) || !aligned4(expert_num_tokens) || !aligned16(y) || !aligned16(ws13) ||
      !aligned16(w->w1) || !aligned16(w->w2))
    return MOE_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g1 = gemm_common(plan, ws13);
  g1.rows.counts = expert_num_tokens;
  g1.epi = kEpiGateUp;
  g1.act = a;
  g1.act_ld = P.K;
  g1.act_bytes = P.E * P.max_tokens * P.K * 2;
  g1.w = w->w1;
  g1.w_expert_stride = 2 * P.I * P.K;
  g1.kdim = (int32_t)P.K;
  g1.nfeat = (int32_t)P.I;
  g1.out = at<void>(ws13, plan->off_z);
  g1.out_ld = P.I;
  GemmArgs g2 = g1;
  g2.epi = kEpiDown;
  g2.act = at<void>(ws13, plan->off_z);
  g2.act_ld = P.I;
  g2.act_bytes = P.E * P.max_tokens * P.I * 2;
  g2.w = w->w2;
  g2.w_expert_stride = P.K * P.I;
  g2.kdim = (int32_t)P.I;
  g2.nfeat = (int32_t)P.K;
  g2.out = y;
  g2.out_ld = P.K;
  if (launch_gemm_tile_bf16(g1, s) != hipSuccess) return MOE_EHIP;
  if (launch_gemm_tile_bf16(g2, s) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

int moe_topk_reduce_contiguous(const moe_plan* plan, const void* y, const int32_t* topk_ids,
                               const float* topk_weights, const int32_t* expert_map, void* out,
                               void* stream) {
  if (!plan || plan->abi_version != MOE_ABI_VERSION) return MOE_EINVAL;
  const moe_problem& P = plan->prob;
  if (P.layout != MOE_LAYOUT_CONTIGUOUS) return MOE_EINVAL;
  if (!aligned16(y) || !aligned4(topk_ids) || !aligned4(topk_weights) || !aligned16(out) ||
      !map_ok(plan, expert_map))
    return MOE_EINVAL;
  hipError_t e = launch_reduce_contiguous(static_cast<const uint16_t*>(y), topk_ids, topk_weights,
                                          expert_map, (int32_t)P.global_experts,
                                          static_cast<uint16_t*>(out), P.M, (int32_t)P.topk, P.K,
                                          (int32_t)P.E, nullptr, 0, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

static AlignLayout batched_reduce_layout(const moe_plan* p, int64_t n_out) {
  const int64_t R = p->prob.E * p->prob.max_tokens;
  const int64_t max_active = n_out < R ? n_out : R;
  // the first 256 bytes hold the status word (out-of-range tokens seen)
  return layout_align(kAlign, n_out, R, R, max_active, align_nblocks(R));
}

int64_t moe_naive_batched_ws_bytes(const moe_plan* plan, int64_t n_out) {
  if (!plan || plan->prob.layout != MOE_LAYOUT_BATCHED || n_out <= 0 || n_out > kAlignMaxBuckets)
    return -1;
  return batched_reduce_layout(plan, n_out).end;
}

int moe_topk_reduce_naive_batched(const moe_plan* plan, const void* y,
                                  const int32_t* expert_num_tokens, const int32_t* row_token,
                                  const float* row_weight, int64_t n_out, void* out, void* ws,
                                  void* stream) {
  if (!plan || plan->abi_version != MOE_ABI_VERSION) return MOE_EINVAL;
  const moe_problem& P = plan->prob;
  if (P.layout != MOE_LAYOUT_BATCHED || n_out <= 0 || n_out > kAlignMaxBuckets) return MOE_EINVAL;
  if (!aligned16(y) || !aligned4(expert_num_tokens) || !aligned4(row_token) ||
      !aligned4(row_weight) || !aligned16(out) || !aligned16(ws))
    return MOE_EINVAL;
  const int64_t R = P.E * P.max_tokens;
  hipStream_t s = (hipStream_t)stream;
  if (P.K <= 8192 && P.E <= kReduceBatchedMaxE) {
    // one launch: each token's workgroup finds its rows itself
    const hipError_t e = launch_reduce_batched(static_cast<const uint16_t*>(y), expert_num_tokens, row_token,
                                               row_weight, (int32_t)P.max_tokens, (int32_t)P.E,
                                               static_cast<uint16_t*>(out), n_out, P.K, at<int32_t>(ws, 0), s);
    return e == hipSuccess ? MOE_OK : MOE_EHIP;
  }
  AlignLayout L = batched_reduce_layout(plan, n_out);
  AlignArgs a{};
  a.keys = row_token;
  a.R = R;
  a.nb = (int32_t)n_out;
  a.B = 1;
  a.group_count = expert_num_tokens;
  a.rows_per_group = (int32_t)P.max_tokens;
  a.counts = at<int32_t>(ws, L.counts);
  a.offsets = at<int32_t>(ws, L.offsets);
  a.sorted = at<int32_t>(ws, L.sorted);
  a.block_bucket = at<int32_t>(ws, L.block_bucket);
  a.num_post = at<int32_t>(ws, L.num_post);
  a.active = at<int32_t>(ws, L.active);
  a.status = at<int32_t>(ws, 0);
  a.block_hist = at<int32_t>(ws, L.scratch);
  a.capacity = R;
  a.max_tiles = R;
  a.max_active = n_out < R ? n_out : R;
  a.sentinel = (int32_t)R;
  a.nblocks = (int32_t)align_nblocks(R);
  if (launch_align(a, s) != hipSuccess) return MOE_EHIP;
  hipError_t e = launch_reduce_csr(static_cast<const uint16_t*>(y), row_weight, a.offsets, a.sorted,
                                   static_cast<uint16_t*>(out), n_out, P.K, s);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_quantize_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  if (rows <= 0 || cols <= 0 || cols % 32 || (x_dtype != 0 && x_dtype != 1)) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !scales) return MOE_EINVAL;
  hipError_t e = launch_quantize_mxfp8(x, x_dtype, rows, cols, codes, scales, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_pack_mxfp8_scales(const uint8_t* src, uint8_t* dst, int64_t mats, int64_t rows, int64_t cols,
                          void* stream) {
  if (mats <= 0 || rows <= 0 || cols <= 0 || cols % 512) return MOE_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return MOE_EINVAL;
  const int64_t bytes = mats * rows * (cols / 32);
  if (bytes / mats / rows != cols / 32) return MOE_EINVAL;   // overflow
  // the buffers must not overlap
  if ((uintptr_t)src < (uintptr_t)dst + bytes && (uintptr_t)dst < (uintptr_t)src + bytes) return MOE_EINVAL;
  hipError_t e = launch_pack_mxfp8_scales(src, dst, mats, rows, cols, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}


// ------------------------------------------------------------- training ----

static int grouped_ok(const moe_grouped_problem* p, const int32_t* offsets) {
  if (!p || !aligned4(offsets)) return MOE_EINVAL;
  if (p->E < 1 || p->E > 65535 || p->R < 0 || p->R >= (1ll << 31) || p->N <= 0 || p->K <= 0)
    return MOE_EINVAL;
  if (p->N % 128 || p->K % 128) return MOE_EUNSUPPORTED;
  const int64_t wide = p->N > p->K ? p->N : p->K;
  if (p->R * wide * 2 >= (1ll << 31) || p->N * p->K * 2 >= (1ll << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static TrainArgs train_args(const moe_grouped_problem* p, int mode, const int32_t* offsets, void* out) {
  TrainArgs t{};
  t.mode = mode;
  t.offsets = offsets;
  t.out = out;
  t.R = p->R;
  t.N = (int32_t)p->N;
  t.K = (int32_t)p->K;
  t.E = (int32_t)p->E;
  return t;
}

int moe_grouped_forward(const moe_grouped_problem* p, const void* x, const void* w,
                        const int32_t* group_offsets, void* y, void* stream) {
  const int st = grouped_ok(p, group_offsets);
  if (st != MOE_OK) return st;
  if (p->R > 0 && (!aligned16(x) || !aligned16(w) || !aligned16(y))) return MOE_EINVAL;
  TrainArgs t = train_args(p, kTrainForward, group_offsets, y);
  t.x = static_cast<const uint16_t*>(x);
  t.w = static_cast<const uint16_t*>(w);
  return launch_train(t, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_grouped_dgrad(const moe_grouped_problem* p, const void* dy, const void* w,
                      const int32_t* group_offsets, void* dx, void* stream) {
  const int st = grouped_ok(p, group_offsets);
  if (st != MOE_OK) return st;
  if (p->R > 0 && (!aligned16(dy) || !aligned16(w) || !aligned16(dx))) return MOE_EINVAL;
  TrainArgs t = train_args(p, kTrainDgrad, group_offsets, dx);
  t.dy = static_cast<const uint16_t*>(dy);
  t.w = static_cast<const uint16_t*>(w);
  return launch_train(t, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_grouped_wgrad(const moe_grouped_problem* p, const void* dy, const void* x,
                      const int32_t* group_offsets, float* dw, int accumulate, void* stream) {
  const int st = grouped_ok(p, group_offsets);
  if (st != MOE_OK) return st;
  if (!aligned16(dw) || (accumulate != 0 && accumulate != 1)) return MOE_EINVAL;
  if (p->R > 0 && (!aligned16(dy) || !aligned16(x))) return MOE_EINVAL;
  TrainArgs t = train_args(p, kTrainWgrad, group_offsets, dw);
  t.dy = static_cast<const uint16_t*>(dy);
  t.x = static_cast<const uint16_t*>(x);
  t.accumulate = accumulate;
  return launch_train(t, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
