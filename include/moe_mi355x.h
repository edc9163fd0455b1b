/*
 * moe_mi355x.h — C ABI of the fused-MoE expert computation for one AMD
 * MI355X (gfx950).
 *
 * What it computes is the expert side of the vLLM modular kernel: the steps
 * of FusedMoEExpertsModular::apply() listed on the page "Fused MoE Modular
 * Kernel" (section "FusedMoEExpertsModular / apply()"): permute the routes by
 * expert, multiply by W1 (gate and up projections), SiLU-and-mul, optionally
 * quantise the intermediate, multiply by W2, unpermute, and apply the top-k
 * weights with a reduction.  Inputs follow that page's two activation formats
 * (introduction): contiguous (M,K) activations with (M,topk) ids and weights,
 * id -1 meaning a skipped slot; and batched (E,max_tokens,K) activations with
 * expert_num_tokens[E].
 *
 * Conventions shared by every call:
 *  - Pointers marked "device" are HIP device (or managed) memory; "host"
 *    pointers are ordinary host memory.  Every buffer is owned by the caller;
 *    the library never allocates, frees, or keeps a pointer after returning.
 *  - Dense tensors are row-major with the last index contiguous; element
 *    types are named per argument.  bf16 is the upper half of an IEEE
 *    binary32; E4M3 is the OCP FP8 E4M3FN format; UE8M0 is a biased power-of
 *    two exponent byte (value 2^(code-127)).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *    call only enqueues kernels on it: no host synchronisation, no device
 *    allocation.  Grid sizes depend only on the plan, so calls can be
 *    captured in a HIP graph.
 *  - Return value: MOE_OK (0) or an error code.  On an error nothing has been
 *    enqueued, except MOE_EHIP (a launch failed; earlier kernels of the same
 *    call may have been enqueued).  No C++ exception crosses this boundary.
 *  - Device buffers of activations, weights, outputs and workspaces must be
 *    16-byte aligned; the 4-byte element arrays (topk ids and weights,
 *    expert_num_tokens, the batched row map, group offsets, the expert map)
 *    and the MXFP8 scale arrays need 4-byte alignment.  (Scale arrays that
 *    are 16-byte aligned, with K and I multiples of 512, let the MXFP8 tile
 *    kernels load four contraction steps of scale words at once.)
 *  - Calls are reentrant; a plan is immutable after moe_plan_init.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

/* Status codes. */
enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null/misaligned pointer, bad size or enum value   */
  MOE_EUNSUPPORTED = 2,  /* valid but not built; the plan's reason says why   */
  MOE_EHIP = 3           /* a kernel launch failed                            */
};

/* Activation format (page "Fused MoE Modular Kernel", introduction and
 * FusedMoEActivationFormat in "activation_formats()"). */
enum { MOE_LAYOUT_CONTIGUOUS = 0, MOE_LAYOUT_BATCHED = 1 };

/* Expert weight element type. */
enum {
  MOE_W_BF16 = 0,
  /* E4M3 codes plus one UE8M0 scale per 32 consecutive elements along the
   * contraction dimension (K for W1, I for W2), scale exponent
   * ceil(log2(blockmax/448)) + 127 clamped to [0,254], 0 for an all-zero block
   * (page "Cake MegaMoE EP16 backend for BF16 activations and MXFP8 weights",
   * section 2, the new scale rule). */
  MOE_W_MXFP8 = 1,
  /* MOE_W_MXFP8 with the scale arrays grouped: in each expert's matrix of
   * rows x cols/32 scale bytes, byte j of row r sits at
   * (j / 16) * rows * 16 + r * 16 + j % 16.  For every 4 contraction steps of
   * 128, the 16 scale bytes of each row lie side by side.
   * moe_pack_mxfp8_scales writes this layout from the row-major one, once,
   * as the weights are loaded (the same page, section 2, packs the scale
   * arrays for its GEMM at that point).  The tile kernels then load the
   * scale words of 4 steps of 64 rows as one contiguous KiB, instead of one
   * 16-byte piece from each of 64 rows.  Needs K and I multiples of 512,
   * the contiguous format, the tile variant and 16-byte-aligned scale
   * arrays. */
  MOE_W_MXFP8_GROUPED = 2
};

/* Row order of W1 [E, 2I, K]. */
enum {
  MOE_W1_HALVES = 0,        /* rows [0,I) gate, rows [I,2I) up                 */
  MOE_W1_INTERLEAVE16 = 1   /* blocks of 32 rows: 16 gate rows, then the 16
                               matching up rows (same page, section 2)          */
};

/* Kernel family (chosen by moe_plan_init unless forced). */
enum {
  MOE_VARIANT_AUTO = -1,
  MOE_VARIANT_TILE = 0,     /* LDS-tiled grouped GEMM: both operands staged     */
  MOE_VARIANT_STREAM = 1,   /* few rows per expert: weight rows streamed from
                               HBM straight into the MFMA row operand, the few
                               token rows in the other operand                  */
  /* the streaming path of moe_apply_contiguous in two launches: one kernel
   * runs the permute, W1 + SiLU-and-mul and W2 + unpermute as work items
   * taken from a device ticket counter (a W2 item waits for its expert's W1
   * items), then the ordered reduce (page "Cake MegaMoE EP16 backend for
   * BF16 activations and MXFP8 weights", section 4: one model kernel plus one
   * ordered top-k reduce per run).  bf16 weights, contiguous format,
   * M*topk <= 8192, E <= 2048; same results, bit for bit, as
   * MOE_VARIANT_STREAM.  AUTO picks it for small layers (all weights within
   * 1 GiB, at most 32 routes per expert).  The stage entry points run the
   * two-launch streaming kernels on such a plan. */
  MOE_VARIANT_FUSED = 2
};

/* Which TopKWeightAndReduce the caller's finalize must apply (page "Fused MoE
 * Modular Kernel", section "TopKWeightAndReduce"). */
enum {
  MOE_REDUCE_NOOP = 0,          /* apply() already reduced (contiguous)         */
  MOE_REDUCE_CONTIGUOUS = 1,
  MOE_REDUCE_NAIVE_BATCHED = 2  /* batched: call moe_topk_reduce_naive_batched */
};

typedef struct moe_problem {
  int64_t M;           /* contiguous: tokens; batched: output tokens          */
  int64_t K;           /* hidden size                                         */
  int64_t I;           /* intermediate size (W1 has 2I rows)                  */
  int64_t E;           /* experts held by this GPU                            */
  int64_t topk;        /* contiguous: slots per token; batched: ignored       */
  int64_t max_tokens;  /* batched: rows per expert slab; contiguous: ignored  */
  /* contiguous: 0 when topk_ids hold local expert ids in [0,E); otherwise
   * the number G >= E of global expert ids, and topk_ids hold global ids in
   * [0,G) that moe_weights.expert_map maps to local ones (an expert-parallel
   * share: page "Fused MoE Modular Kernel", "How To Add a
   * FusedMoEExpertsModular Type", supports_expert_map(); page "DeepGEMM Mega
   * MoE as an EP implementation", introduction: global ids, unmasked
   * weights).  Batched: must be 0. */
  int64_t global_experts;
  int32_t layout;      /* MOE_LAYOUT_*                                        */
  int32_t w_dtype;     /* MOE_W_*                                             */
  int32_t w1_order;    /* MOE_W1_*                                            */
  int32_t variant;     /* MOE_VARIANT_* (AUTO lets the plan choose)           */
} moe_problem;

typedef struct moe_weights {
  const void* w1;          /* device. bf16 or E4M3 [E, 2I, K]                  */
  const uint8_t* w1_scale; /* device. UE8M0 [E, 2I, K/32] (MXFP8 only)         */
  const void* w2;          /* device. bf16 or E4M3 [E, K, I]                   */
  const uint8_t* w2_scale; /* device. UE8M0 [E, K, I/32] (MXFP8 only)          */
  /* device. int32 [global_experts] when prob.global_experts > 0 (else NULL):
   * the local id in [0,E) of each global expert, -1 for an expert this GPU
   * does not hold.  Slots whose expert maps to -1 are skipped (whatever their
   * weight); global ids outside {-1} U [0,G) and map entries outside
   * {-1} U [0,E) are skipped and counted as invalid. */
  const int32_t* expert_map;
} moe_weights;

/* A plan: validated sizes, the chosen kernels and the workspace layout.  The
 * offsets are byte offsets inside ws13 and are documented so that tests can
 * inspect the intermediate results; callers otherwise treat ws13/ws2 as
 * opaque.  (Workspaces as in "workspace_shapes()": the plan states their
 * sizes, the caller allocates them once at the largest size it needs.) */
typedef struct moe_plan {
  moe_problem prob;
  int32_t abi_version;
  int32_t variant;         /* MOE_VARIANT_TILE, _STREAM or _FUSED             */
  int32_t block_m;         /* align tile size B: expert runs padded to it     */
  int32_t reduce_kind;     /* MOE_REDUCE_*                                    */
  int64_t routes;          /* R: M*topk (contiguous) or E*max_tokens (batched)*/
  int64_t sorted_capacity; /* positions in sorted_ids (worst case over routings)*/
  int64_t max_tiles;       /* sorted_capacity / block_m                       */
  int64_t max_active;      /* min(E, R): experts that can hold a route        */
  int64_t align_blocks;    /* blocks of the multi-block align path (0: single)*/
  int64_t ws13_bytes;      /* size of workspace 13                            */
  int64_t ws2_bytes;       /* size of workspace 2                             */
  int64_t out_rows, out_cols;
  /* ws13 sub-buffers (int32 unless noted) */
  int64_t off_counts;      /* [E]    routes per expert                         */
  int64_t off_offsets;     /* [E+1]  padded exclusive scan of counts            */
  int64_t off_sorted_ids;  /* [sorted_capacity] flat slot t*topk+j, or R       */
  int64_t off_block_expert;/* [max_tiles] owner expert of each tile, or -1     */
  int64_t off_num_post_padded; /* [1] offsets[E]                              */
  int64_t off_active;      /* [max_active+1] experts with routes, ascending;
                              element max_active holds their number            */
  int64_t off_status;      /* [4] [0]: ids outside {-1} U [0,E) seen;
                              [1] (MOE_VARIANT_FUSED): waits that timed out,
                              summed over calls (non-zero: the outputs of
                              some call are undefined)                         */
  int64_t off_align_scratch; /* per-block histograms of the multi-block path  */
  int64_t off_z;           /* intermediate silu(gate)*up rows, in sorted
                              order: bf16 [sorted_capacity, I], or E4M3
                              [sorted_capacity, I] for MXFP8 (batched: rows
                              e*max_tokens + r)                                */
  int64_t off_z_scale;     /* MXFP8: UE8M0 [rows of z, I/32]; MOE_W_MXFP8_GROUPED:
                              grouped as the weights' ([I/512][rows][16])      */
  int64_t off_xq;          /* MXFP8: E4M3 activations gathered in sorted order
                              [sorted_capacity, K]                              */
  int64_t off_xq_scale;    /* MXFP8: UE8M0 [sorted_capacity, K/32];
                              MOE_W_MXFP8_GROUPED: [K/512][sorted_capacity][16]*/
  int64_t off_sync;        /* MOE_VARIANT_FUSED: the work queue, int32 words:
                              counters at 32*i for i < 2 + max_active (ticket,
                              align published, W1 strips done per slot), then
                              int4 [max_active] slot records.  The counters
                              must be zero before the first call on this ws13
                              (allocate it zero-filled) and are zero again
                              after every moe_apply_contiguous call; -1 for
                              other variants.  Calls that share a ws13 must
                              not overlap.                                     */
  char reason[192];        /* why this variant / why unsupported              */
} moe_plan;

/* ABI version of the loaded library; compare with MOE_ABI_VERSION to catch a
 * stale shared object (page "Cake deterministic MoE grouped GEMM", review
 * follow-up: a prebuilt library whose argument list no longer matches). */
int moe_abi_version(void);

/* Static string for a status code, the readable companion of the plan's
 * reason field (page "Cake deterministic MoE grouped GEMM", section 1 and
 * its closing lessons: the plan records why a path was not taken, in a
 * diagnostic field meant for callers and tests).  Never NULL; unknown codes
 * give "unknown status".  The string is owned by the library. */
const char* moe_status_string(int status);

/* sizeof(moe_problem), sizeof(moe_plan) and sizeof(moe_weights) as compiled
 * into the library, for bindings that lay the structs out themselves (the
 * same concern as moe_abi_version: page "Cake deterministic MoE grouped
 * GEMM", review follow-up, a binding whose view of the arguments no longer
 * matches the library).  Each pointer may be NULL. */
void moe_struct_sizes(int64_t* problem, int64_t* plan, int64_t* weights);

/* Validate `prob` (host) and fill `plan` (host): the workspace sizes of page
 * "Fused MoE Modular Kernel", section "workspace_shapes()" (the caller
 * allocates ws13 and ws2 of the sizes the plan states, once, at the largest
 * size it needs), and the reduce kind of section
 * "finalize_weight_and_reduce_impl()".  Chooses the kernel variant when
 * prob->variant is AUTO (bf16 contiguous: FUSED for small layers — all
 * weights within 1 GiB, at most 32 routes per expert slot, R <= 8192,
 * E <= 2048, K and I multiples of 128 — else STREAM for M <= 16, else TILE; batched and MXFP8: TILE), the align
 * tile size, the workspace sizes and the reduce kind (NOOP for contiguous,
 * NAIVE_BATCHED for batched).  Errors: MOE_EINVAL for null pointers,
 * non-positive sizes, topk > E, global_experts neither 0 nor in [E, 2^31),
 * bad enum values or index ranges past 2^31;
 * MOE_EUNSUPPORTED (with plan->reason set) for shapes no kernel is built
 * for: the bf16 tiled kernels need K % 256 == 0 and I % 128 == 0
 * (contiguous format) or K % 128 == 0 and I % 64 == 0 (batched format), the
 * streaming kernels and both MXFP8 families K % 128 == 0 and I % 128 == 0. */
int moe_plan_init(moe_plan* plan, const moe_problem* prob);

/* plan->reason: why moe_plan_init chose this kernel family, or why it
 * refused the problem (page "Cake deterministic MoE grouped GEMM", section 1:
 * the plan's accumulate_reason says why the fused route was not taken; the
 * closing lessons: such a field serves both callers and tests).  `plan` is
 * host memory; returns "" for NULL.  The string lives inside the plan. */
const char* moe_plan_reason(const moe_plan* plan);

/* Permute (page "Fused MoE Modular Kernel", apply() step 1): group the flat
 * routes t*topk+j of `topk_ids` (device, int32 [M, topk]) by expert.  Writes
 * into ws13 (device, plan->ws13_bytes): counts, offsets (each expert's run
 * padded to block_m), sorted_ids (ascending flat order within an expert;
 * padding holds R = M*topk), block_expert (-1 past the last run),
 * num_post_padded, the active-expert list and the status word.  Ids outside
 * {-1} U [0,E) are skipped and counted in status[0].  expert_map: device
 * int32 [global_experts] as in moe_weights (ids are then global and mapped
 * first), or NULL when plan->prob.global_experts == 0 (MOE_EINVAL if one is
 * given without the other).  Contiguous plans only. */
int moe_align_permute(const moe_plan* plan, const int32_t* topk_ids, const int32_t* expert_map,
                      void* ws13, void* stream);

/* The whole expert computation on the contiguous format (page "Fused MoE
 * Modular Kernel", apply(); reduce kind NOOP: the top-k weighted sum is done
 * here).  a: device bf16 [M, K]; topk_ids: device int32 [M, topk];
 * topk_weights: device float32 [M, topk]; w: host struct of device pointers;
 * out: device bf16 [M, K] — out[t] = bf16(sum_j w[t,j] * y[t,j]) summed in
 * ascending j in float32, +0.0 for a token with no valid slot; ws13, ws2:
 * device, plan->ws13_bytes and plan->ws2_bytes.  ws2 receives the per-(token,
 * slot) W2 outputs y (bf16 [M*topk, K]; rows of skipped slots untouched). */
int moe_apply_contiguous(const moe_plan* plan, const void* a, const int32_t* topk_ids,
                         const float* topk_weights, const moe_weights* w, void* out,
                         void* ws13, void* ws2, void* stream);

/* Bytes of the library's own workspace array used by
 * moe_apply_contiguous_static (one per GPU). */
#define MOE_STATIC_SCRATCH_BYTES (64ll << 20)

/* moe_apply_contiguous for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results (bit for bit) as moe_apply_contiguous, but
 * ws13 and ws2 live in an array inside the library: MOE_STATIC_SCRATCH_BYTES
 * of device memory per GPU, held from the library's load until the process
 * ends.  The call allocates and frees nothing.  Limit: the plan's ws13
 * (rounded up to 256 bytes) plus ws2 must fit in MOE_STATIC_SCRATCH_BYTES,
 * else MOE_EUNSUPPORTED and nothing is enqueued (e.g. the decode batch
 * M=4 K=4096 I=8192 E=64 top-8 needs about 8.7 MB; a prefill batch of 8192
 * tokens does not fit).  Every call on one GPU uses that GPU's one array:
 * calls that overlap in time on one GPU (two streams, two host threads)
 * race and give undefined results; calls ordered on one stream are safe.
 * The status words of ws13 (invalid ids, time-outs) are cleared at the start
 * of each call and are not visible to the caller.  Errors as for
 * moe_apply_contiguous, plus MOE_EHIP when the array's device address
 * cannot be obtained. */
int moe_apply_contiguous_static(const moe_plan* plan, const void* a, const int32_t* topk_ids,
                                const float* topk_weights, const moe_weights* w, void* out,
                                void* stream);

/* The two matmul stages of moe_apply_contiguous on their own, for callers
 * that time or overlap them (contiguous plans; moe_align_permute must have
 * filled ws13 first, on the same stream).
 * moe_gate_up_act: matmul with W1, SiLU-and-mul, and for MXFP8 weights the
 * quantisation of the gathered activations and of the intermediate ("Fused
 * MoE Modular Kernel", apply() steps 2-4).  Writes z into ws13.
 * moe_down_unpermute: matmul with W2 and unpermute (steps 5-6): writes each
 * route's row to its (token, slot) row of ws2 (bf16 [M*topk, K]).
 * Arguments as for moe_apply_contiguous (w->expert_map is not read: the
 * routes come from moe_align_permute). */
int moe_gate_up_act(const moe_plan* plan, const void* a, const moe_weights* w, void* ws13,
                    void* stream);
int moe_down_unpermute(const moe_plan* plan, const moe_weights* w, void* ws13, void* ws2,
                       void* stream);

/* The expert computation on the batched format (page "Fused MoE Modular
 * Kernel", introduction: batched activations with expert_num_tokens; reduce
 * kind NAIVE_BATCHED).  a: device bf16 [E, max_tokens, K];
 * expert_num_tokens: device int32 [E] (each in [0, max_tokens]); y: device
 * bf16 [E, max_tokens, K] — y[e, r] = W2_e(silu(W1g_e a[e,r]) * W1u_e
 * a[e,r]) for r < expert_num_tokens[e]; rows past the count are neither read
 * nor written.  ws13: device, plan->ws13_bytes. */
int moe_apply_batched(const moe_plan* plan, const void* a, const int32_t* expert_num_tokens,
                      const moe_weights* w, void* y, void* ws13, void* stream);

/* TopKWeightAndReduceContiguous on its own (page "Fused MoE Modular
 * Kernel", section "TopKWeightAndReduce": the contiguous policy weights each
 * (token, slot) row and sums the slots of a token; page "Cake MegaMoE EP16
 * backend for BF16 activations and MXFP8 weights", section 3: the ordered
 * Top-K reduce over the per-(token, slot) buffer).  y: device bf16 [M*topk, K], row
 * t*topk+j is slot (t, j); out: device bf16 [M, K]; expert_map as for
 * moe_align_permute; same arithmetic as the reduce inside
 * moe_apply_contiguous. */
int moe_topk_reduce_contiguous(const moe_plan* plan, const void* y, const int32_t* topk_ids,
                               const float* topk_weights, const int32_t* expert_map, void* out,
                               void* stream);

/* Bytes of workspace moe_topk_reduce_naive_batched needs for n_out tokens
 * (page "Fused MoE Modular Kernel", workspace_shapes(): the kernel reports
 * its workspace sizes and the caller allocates them).  -1 for a NULL plan,
 * a plan of the contiguous layout, or n_out outside [1, 8192]. */
int64_t moe_naive_batched_ws_bytes(const moe_plan* plan, int64_t n_out);

/* TopKWeightAndReduceNaiveBatched (page "Fused MoE Modular Kernel", section
 * "TopKWeightAndReduce"): out[tok] = bf16(sum of row_weight[e,r] * y[e,r]
 * over valid rows (r < expert_num_tokens[e]) with row_token[e,r] == tok),
 * summed in float32 in ascending (e, r) order; tokens no row maps to get
 * +0.0.  y: device bf16 [E, max_tokens, K]; expert_num_tokens: device int32
 * [E]; row_token: device int32 [E, max_tokens] (valid rows in [0, n_out));
 * row_weight: device float32 [E, max_tokens]; out: device bf16 [n_out, K];
 * ws: device, moe_naive_batched_ws_bytes(plan, n_out).  Invalid rows' map
 * entries are never read; a valid row mapping to -1 is skipped; valid rows
 * mapping elsewhere outside [0, n_out) are skipped and counted in the first
 * int32 of ws (written by every call). */
int moe_topk_reduce_naive_batched(const moe_plan* plan, const void* y,
                                  const int32_t* expert_num_tokens, const int32_t* row_token,
                                  const float* row_weight, int64_t n_out, void* out, void* ws,
                                  void* stream);

/* MXFP8 codec on its own (page "Cake MegaMoE EP16 backend for BF16
 * activations and MXFP8 weights", section 2): each row of x (device, [rows,
 * cols], float32 if x_dtype == 0, bf16 if x_dtype == 1) is cut into blocks of
 * 32 columns; codes (device, uint8 [rows, cols]) get the E4M3 encoding
 * (round to nearest even) of x / 2^(s-127) and scales (device, uint8 [rows,
 * cols/32]) the scale code s of the rule above.  cols % 32 must be 0.  This is
 * how MXFP8 weights are produced for moe_apply_*. */
int moe_quantize_mxfp8(const void* x, int x_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* Scale arrays for MOE_W_MXFP8_GROUPED (page "Cake MegaMoE EP16 backend for
 * BF16 activations and MXFP8 weights", section 2: the scales are packed for
 * the GEMM once, when the weights are loaded).  src (device, 16-byte
 * aligned) holds mats matrices of rows x cols/32 UE8M0 bytes, row-major, as
 * moe_quantize_mxfp8 writes them (W1: mats = E, rows = 2I, cols = K; W2: E,
 * K, I); dst (device, the same size, 16-byte aligned, not overlapping src)
 * receives each matrix grouped as MOE_W_MXFP8_GROUPED describes.  cols % 512 must be 0.  Enqueues
 * one kernel on the stream; allocates nothing and does not synchronise.
 * MOE_EINVAL for a null or misaligned pointer or a bad size. */
int moe_pack_mxfp8_scales(const uint8_t* src, uint8_t* dst, int64_t mats, int64_t rows, int64_t cols,
                          void* stream);

/* ---------------------------------------------------------------------------
 * Training grouped GEMMs (page "Cake deterministic MoE grouped GEMM":
 * introduction — a ragged bf16 grouped GEMM for training whose forward,
 * dgrad and wgrad give the same bits on every run; section 1 — the fp32
 * weight gradient added into the fp32 main_grad inside the kernel, the same
 * bits as out.add_(dW); section 2 — an empty group's sum is +0.0).
 *
 * Rows are grouped by expert: group e is rows [group_offsets[e],
 * group_offsets[e+1]) of x [R, K] and dy [R, N] (row-major bf16); W is
 * [E, N, K] bf16 (expert e's forward maps K features to N).  group_offsets:
 * device int32 [E+1], non-decreasing from 0 to R (entries are clamped to
 * [0, R], so a malformed array reads no row outside the buffers but gives
 * undefined results).  bf16 products accumulate in fp32 in a fixed order; no
 * result depends on the run.  Each call launches one kernel on `stream`,
 * allocates nothing and does not synchronise.  With R = 0 the row matrices
 * (x, dy, y, dx) and w may be NULL.  Errors: MOE_EINVAL (null or
 * misaligned pointer: 16 bytes for the matrices, 4 for group_offsets; E
 * outside [1, 65535]; R outside [0, 2^31); N or K not positive),
 * MOE_EUNSUPPORTED (N or K not a multiple of 128, or R * max(N, K) * 2 or
 * N * K * 2 bytes at or past 2^31), MOE_EHIP (launch failure).
 * ------------------------------------------------------------------------- */
typedef struct moe_grouped_problem {
  int64_t R;   /* rows over all groups                                      */
  int64_t N;   /* forward output features                                   */
  int64_t K;   /* forward contraction                                       */
  int64_t E;   /* groups (experts)                                          */
} moe_grouped_problem;

/* Forward (page "Cake deterministic MoE grouped GEMM", introduction):
 * y[r] = W[e] x[r] for the rows r of group e: y device bf16 [R, N]. */
int moe_grouped_forward(const moe_grouped_problem* p, const void* x, const void* w,
                        const int32_t* group_offsets, void* y, void* stream);

/* dgrad (page "Cake deterministic MoE grouped GEMM", introduction):
 * dx[r] = W[e]^T dy[r]: dx device bf16 [R, K]. */
int moe_grouped_dgrad(const moe_grouped_problem* p, const void* dy, const void* w,
                      const int32_t* group_offsets, void* dx, void* stream);

/* wgrad (page "Cake deterministic MoE grouped GEMM", sections 1 and 2):
 * dW[e] = sum over the rows r of group e of dy[r] x[r]^T, fp32.
 * dw: device float32 [E, N, K]; accumulate = 0 writes dW (+0.0 for an empty
 * group), accumulate = 1 adds it: dw[e] = dw[e] + dW[e] in one fp32 add per
 * element, bit for bit what the overwrite followed by dw.add_(dW) gives (an
 * empty group adds +0.0, which turns -0.0 into +0.0). */
int moe_grouped_wgrad(const moe_grouped_problem* p, const void* dy, const void* x,
                      const int32_t* group_offsets, float* dw, int accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
