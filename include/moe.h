/*
 * moe.h - C ABI of the single-GPU mixture-of-experts (MoE) layer hot path on
 * MI355X (gfx950): top-k router, capacity-bounded permutation into per-expert
 * buckets (viewable as P per-rank send buffers), SwiGLU experts as a grouped
 * GEMM, and the gate-weighted inverse permutation (combine).
 *
 * Sources (pages, cited by title and section):
 *   [EP-glossary]   "Expert Parallelism" (klaylearn.com glossary): router scores,
 *                   top-k choice and combine weights; permute, run local experts
 *                   on buckets, restore order and weight.
 *   [EP-inferensys] "Expert Parallelism" (inferensys.com glossary): top-k gating;
 *                   expert capacity = cf * k * T / E; overflowing tokens dropped
 *                   and passed through unchanged; pre-allocated contiguous
 *                   buffers of maximum capacity.
 *   [EP-guide]      "Expert Parallelism" (infra.bea.ai guide), section 2 "The
 *                   Dispatch Pattern": router -> dispatch -> local experts ->
 *                   combine -> weighted sum.
 *   [EP-A2A]        "Expert Parallelism & All-to-All" (neelmishra.github.io):
 *                   "All-to-all: the distributed transpose" (combine is the exact
 *                   inverse permutation; gate-weighted sum into the residual),
 *                   "Why fixed-size buffers matter here" (C = cf * k * T / E;
 *                   drops on overflow, padding on underflow), "Why MoE forces a
 *                   new axis" (E/P whole experts per device).
 *
 * Conventions for every entry point:
 *  - Every array argument is a caller-owned, contiguous, row-major DEVICE
 *    pointer unless stated otherwise. The library never allocates, frees or
 *    keeps memory between calls; scratch memory is the caller's `workspace`.
 *    Two calls whose work may overlap on the device (different streams) need
 *    separate workspaces; calls ordered on one stream may share one.
 *  - bf16 arrays hold IEEE bfloat16 bit patterns; fp32 arrays hold IEEE binary32.
 *    `dtype` selects the element type of x, weights, buckets, h, y and out;
 *    logits, gates are always fp32, indices and counts int32, totals int64.
 *  - Weight layouts are [out, in]: W_router [E, d], W_gate and W_up [E, d_ff, d],
 *    W_down [E, d, d_ff].
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous: outputs are valid once the caller synchronises the stream.
 *    No call synchronises or copies device memory to the host.
 *  - Argument errors are detected on the host before any HIP call, and then no
 *    output is touched. A HIP launch failure returns MOE_ERR_HIP; its message
 *    is available from moe_last_error() on the same thread.
 *  - T == 0 returns MOE_OK and enqueues nothing. Capacity overflow is not an
 *    error: it drops copies. Inputs must be finite (NaN/Inf give unspecified
 *    routing).
 *  - Limits (else MOE_ERR_UNSUPPORTED): d and d_ff multiples of 8 (fp32: of 4),
 *    E <= 4096, k <= 32, T * k < 2^31, E * C < 2^31, and per expert
 *    (C + 256) * max(d, d_ff) * 4 < 2^31 and d * d_ff * 4 < 2^31 bytes.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,
  MOE_ERR_UNSUPPORTED = -2,
  MOE_ERR_WORKSPACE = -3,
  MOE_ERR_HIP = -4
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Indices into moe_stats_t.totals. */
enum {
  MOE_TOTAL_DROPPED = 0,        /* k*T - sum(kept): copies dropped on overflow */
  MOE_TOTAL_FULLY_DROPPED = 1,  /* tokens whose k copies were all dropped */
  MOE_TOTAL_PADDED_ROWS = 2,    /* E*C - sum(kept): unused bucket rows */
  MOE_TOTAL_OFFRANK_BYTES = 3,  /* sum over p != 0 of send_count[p] * d * elem bytes */
  MOE_NUM_TOTALS = 4
};

/* Optional outputs of moe_layer_forward. Each pointer is caller-owned device
 * memory of the size given, or NULL, in which case the layer keeps that array
 * in the workspace. */
typedef struct {
  int32_t* topk_idx;     /* [T, k] chosen experts, best first */
  float* topk_w;         /* [T, k] gate weights */
  int32_t* slot;         /* [T, k] row in the expert's bucket, -1 = dropped */
  int32_t* src;          /* [E, C] copy id t*k+j held by each bucket row, -1 = padding */
  int32_t* routed_count; /* [E] copies routed to each expert */
  int32_t* kept_count;   /* [E] min(routed, C) */
  int32_t* send_count;   /* [P] kept rows in each rank's send buffer */
  int64_t* totals;       /* [MOE_NUM_TOTALS] */
  void* buckets;         /* [E, C, d] dtype; rank p's send buffer is experts
                            [p*E/P, (p+1)*E/P), a contiguous slice */
  int32_t* instance;     /* [T, k] replica instance of each copy (replicated layer only) */
  /* The expert activations, kept for moe_layer_backward_saved (plain layer
   * only; the replicated layer ignores them): g = X_e W_gate[e]^T, u = X_e
   * W_up[e]^T and h = silu(g) * u, each [E, C, d_ff] dtype, rows < kept_count
   * written (the others left as they were), all three or none. Where GEMM 1
   * runs on 256- or 320-row tiles with d % 128 == 0 it writes the rounded g
   * and u beside h, and the layer's output is unchanged; elsewhere g and u
   * come from two plain grouped GEMMs and h from their rounded values, as
   * the backward recomputes them. */
  void* g;
  void* u;
  void* h;
} moe_stats_t;

/* Expert capacity C = ceil(cf * k * T / E), evaluated in IEEE double as
 * ((cf * k) * T) / E ([EP-inferensys] capacity entry; [EP-A2A] "Why
 * fixed-size buffers matter here"). Host only; touches no device state.
 * Errors: T < 0, E < 1, k < 1, cf not finite or <= 0, NULL C_out. */
int moe_capacity(int64_t T, int32_t E, int32_t k, float cf, int64_t* C_out);

/* Bytes of workspace moe_layer_forward needs for these sizes (host only). */
int moe_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf,
                       int32_t P, moe_dtype_t dtype, size_t* bytes);

/* The whole layer ([EP-guide] section 2; [EP-glossary]):
 *   logits = x W_router^T (+ router_bias)                      fp32 [T, E]
 *   topk_idx, topk_w = top-k of logits (ties: lower index first), softmax of
 *                      the k chosen logits
 *   C = moe_capacity(T, E, k, cf); slot = stable token-order rank of each copy
 *   among its expert's copies, dropped (-1) if >= C
 *   buckets[e, s] = x[t] for each kept copy (t, j) of expert e at slot s
 *   h = silu(X_e W_gate[e]^T) * (X_e W_up[e]^T);  y = h W_down[e]^T  (rows < kept)
 *   out[t] = x[t] + sum_j [slot >= 0] topk_w[t,j] * y[idx[t,j], slot[t,j]];
 *   a token with every copy dropped is copied through bit for bit.
 * x [T, d], out [T, d] (must not overlap x), router_bias [E] fp32 or NULL,
 * P >= 1 with E % P == 0 (send-buffer view only; no communication).
 * max_ranks: 0 (or >= P) for plain top-k; otherwise each token's experts are
 * limited to max_ranks of the P ranks, chosen as in moe_route.
 * stats may be NULL. workspace must hold moe_workspace_size() bytes, 256-byte
 * aligned. */
int moe_layer_forward(const void* x, const void* W_router, const float* router_bias,
                      const void* W_gate, const void* W_up, const void* W_down,
                      int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf,
                      int32_t P, int32_t max_ranks, moe_dtype_t dtype, void* out,
                      moe_stats_t* stats, void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass of the layer ([EP-A2A] "The bandwidth bill": the backward
 * runs the dispatch and the combine again, in reverse; "All-to-all: the
 * distributed transpose": the combine is the gate-weighted inverse of the
 * dispatch). Given the forward's inputs (as for moe_layer_forward) and
 * dout = dLoss/dout [T, d] (dtype), writes
 *   dx [T, d] dtype; dW_router [E, d] dtype; d_bias [E] fp32 (may be NULL);
 *   dW_gate, dW_up [E, d_ff, d] and dW_down [E, d, d_ff] dtype,
 * the chain rule through the forward with the top-k choice and the capacity
 * drops held fixed: a dropped copy passes no gradient to its expert, but its
 * gate still does through the softmax; a fully dropped token gets dx = dout.
 * Routing, capacity and the expert activations are recomputed from the
 * inputs (no forward state is kept). Sums run in fp32 in a fixed order, so
 * results are deterministic. dx must not overlap x or dout. Gradients are
 * written, not accumulated. workspace: moe_backward_workspace_size() bytes,
 * 256-byte aligned. Errors as moe_layer_forward. */
int moe_backward_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf,
                                int32_t P, moe_dtype_t dtype, size_t* bytes);
int moe_layer_backward(const void* x, const void* W_router, const float* router_bias,
                       const void* W_gate, const void* W_up, const void* W_down, const void* dout,
                       int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                       int32_t max_ranks, moe_dtype_t dtype, void* dx, void* dW_router,
                       float* d_bias, void* dW_gate, void* dW_up, void* dW_down, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The backward pass from the forward's kept state: as moe_layer_backward,
 * but the routing (topk_idx, topk_w), the buckets and the activations g, u, h
 * come from `saved`, the stats of a moe_layer_forward call on the same inputs
 * that kept them (all six pointers non-NULL), instead of being recomputed;
 * the counts and slots are derived again from topk_idx. The results equal
 * moe_layer_backward's bit for bit. Errors as moe_layer_backward, and a NULL
 * saved array. */
int moe_layer_backward_saved(const void* x, const void* W_router, const float* router_bias,
                             const void* W_gate, const void* W_up, const void* W_down, const void* dout,
                             int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf, int32_t P,
                             int32_t max_ranks, moe_dtype_t dtype, const moe_stats_t* saved, void* dx,
                             void* dW_router, float* d_bias, void* dW_gate, void* dW_up, void* dW_down,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Hot-expert replication ([EP-guide] section 6 "Optimizations", "Expert
 * Replication": a popular expert is replicated on several devices and its
 * tokens may go to either copy, for better balance and fewer drops at the
 * cost of memory; [EP-vs-TP] "Expert parallelism pays in all-to-all
 * dispatch": a load balancer re-places experts under skew). The pages give
 * no policy; the readings taken:
 *  - moe_replica_plan (host only): r[e] = 1 for every expert, then each of
 *    `extra` more replicas goes to the expert with the highest routed[e]/r[e]
 *    (exact integer comparison, lowest index on a tie).
 *  - moe_layer_forward_replicated: expert e has replicas[e] >= 1 instances of
 *    capacity C each (C = moe_capacity of the unreplicated layer); instance i
 *    = inst_off[e] + j for replica j, inst_off the exclusive prefix sum.
 *    The copies of expert e, in stable token order, are dealt to its
 *    replicas in turn: copy q goes to replica q mod r at slot q div r, and is
 *    dropped iff that slot is >= C. Replica j of expert e sits on rank
 *    (e / (E/P) + j) mod P for the send counts.
 *  The output is that of the unreplicated layer in which expert e has
 *  capacity replicas[e] * C. replicas is [E] int32 device memory summing to
 *  R (E <= R <= 4096; results are unspecified otherwise, instances are
 *  clamped to R - 1). stats: topk_idx, topk_w as before; slot = row in the
 *  copy's instance; instance [T, k]; src [R, C]; routed_count [E];
 *  kept_count [R]; send_count [P]; totals; buckets [R, C, d].
 *  workspace: moe_replicated_workspace_size() bytes, 256-byte aligned. */
int moe_replica_plan(const int32_t* routed_count, int32_t E, int32_t extra, int32_t* replicas);
int moe_replicated_workspace_size(int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf,
                                  int32_t P, int32_t R, moe_dtype_t dtype, size_t* bytes);
int moe_layer_forward_replicated(const void* x, const void* W_router, const float* router_bias,
                                 const void* W_gate, const void* W_up, const void* W_down,
                                 int64_t T, int64_t d, int64_t d_ff, int32_t E, int32_t k, float cf,
                                 int32_t P, int32_t max_ranks, const int32_t* replicas, int32_t R,
                                 moe_dtype_t dtype, void* out, moe_stats_t* stats, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Router stage ([EP-inferensys] gating-network entry): logits on the matrix
 * cores, then top-k (with the rank limit P, max_ranks) and gates as in moe_route. logits_out [T, E] fp32 may be
 * NULL; otherwise it receives the scores (bias included). The scores are
 * summed over slices of d in a fixed order, so results do not depend on
 * scheduling. workspace: moe_router_workspace_size() bytes, 256-byte aligned. */
int moe_router_workspace_size(int64_t T, int64_t d, int32_t E, moe_dtype_t dtype, size_t* bytes);
int moe_router(const void* x, const void* W_router, const float* router_bias, int64_t T,
               int64_t d, int32_t E, int32_t k, int32_t P, int32_t max_ranks,
               moe_dtype_t dtype, int32_t* topk_idx, float* topk_w, float* logits_out,
               void* workspace, size_t workspace_bytes, void* stream);

/* Top-k and gates from given fp32 logits [T, E]: per token the k experts in
 * order of score descending, then index ascending (+0 == -0); gates
 * w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), evaluated in fp64, rounded to
 * fp32.
 * Rank limit ([EP-A2A] "The bandwidth bill", node-limited routing; [EP-vs-TP]
 * "Expert parallelism pays in all-to-all dispatch", at most 4 nodes per token
 * in DeepSeek-V3): with 0 < max_ranks < P, rank p owning experts
 * [p E/P, (p+1) E/P), a rank's score is its best expert score, the max_ranks
 * best ranks are allowed (lower rank first on a tie) and the top k is taken
 * over their experts only. max_ranks = 0 or >= P: no limit.
 * Errors: P < 1 or E % P != 0, max_ranks < 0, or max_ranks * E/P < k
 * (MOE_ERR_INVALID_ARG); a limit with P > 64 (MOE_ERR_UNSUPPORTED). */
int moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t P, int32_t max_ranks,
              int32_t* topk_idx, float* topk_w, void* stream);

/* Permutation stage ([EP-inferensys] capacity and memory entries; [EP-A2A]
 * "Why fixed-size buffers matter here"): from topk_idx [T, k] computes
 * routed/kept counts, slot [T, k], src [E, C], buckets [E, C, d] (kept rows
 * only; padding rows are not written), send_count [P] and totals. C is given
 * (normally moe_capacity()). Any of src, send_count, totals may be NULL.
 * A topk_idx entry outside [0, E) is dropped (slot -1, counted in no
 * expert), so no index given by a caller reaches outside the buckets.
 * workspace: moe_permute_workspace_size() bytes. */
int moe_permute_workspace_size(int64_t T, int32_t E, size_t* bytes);
int moe_permute(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E,
                int32_t k, int64_t C, int32_t P, moe_dtype_t dtype, void* buckets,
                int32_t* slot, int32_t* src, int32_t* routed_count, int32_t* kept_count,
                int32_t* send_count, int64_t* totals, void* workspace, size_t workspace_bytes,
                void* stream);

/* moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments, results and errors as moe_permute; its
 * scratch (what moe_permute_workspace_size() gives, at most 16 MiB) is a
 * static buffer inside the library, one per GPU, held until the process
 * ends. Larger T x E are rejected with MOE_ERR_UNSUPPORTED before any work is
 * enqueued. The call allocates nothing. Every call on one GPU uses that GPU's
 * buffer: calls whose work may overlap on the device (different streams, or
 * different host threads without ordering) race and give unspecified
 * results; calls ordered on one stream are safe. */
int moe_permute_static(const void* x, const int32_t* topk_idx, int64_t T, int64_t d, int32_t E,
                       int32_t k, int64_t C, int32_t P, moe_dtype_t dtype, void* buckets,
                       int32_t* slot, int32_t* src, int32_t* routed_count, int32_t* kept_count,
                       int32_t* send_count, int64_t* totals, void* stream);

/* Expert stage ([EP-guide] section 1, three matrices per expert; [EP-A2A]
 * "Tensor parallelism for experts", gate/up/down): for every expert e and
 * bucket row s < kept_count[e]:
 *   h[e, s] = silu(buckets[e, s] W_gate[e]^T) * (buckets[e, s] W_up[e]^T)
 *   y[e, s] = h[e, s] W_down[e]^T
 * Rows >= kept_count[e] are neither read for results nor written. bf16 runs
 * on the matrix cores with fp32 accumulation, h and y rounded to bf16.
 * kept_count [E] int32 device memory; each count is taken clamped to [0, C]
 * (a count above C processes the C rows of the bucket, a negative one none),
 * so the call never reads or writes outside buckets [E, C, d], h [E, C, d_ff]
 * and y [E, C, d]. Weights are [E, d_ff, d] (W_gate, W_up) and [E, d, d_ff]
 * (W_down). Errors as for the layer, plus E * C >= 2^31 (MOE_ERR_UNSUPPORTED).
 * workspace: moe_grouped_gemm_workspace_size() bytes. */
int moe_grouped_gemm_workspace_size(int32_t E, int64_t C, size_t* bytes);
int moe_grouped_gemm(const void* buckets, const int32_t* kept_count, const void* W_gate,
                     const void* W_up, const void* W_down, int32_t E, int64_t C, int64_t d,
                     int64_t d_ff, moe_dtype_t dtype, void* h, void* y, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Combine stage ([EP-A2A] "All-to-all: the distributed transpose"):
 *   out[t] = x[t] + sum_j [slot[t,j] >= 0] topk_w[t,j] * y[topk_idx[t,j], slot[t,j]]
 * summed in fp32 over j ascending and rounded once; tokens with every slot -1
 * are copied bit for bit ([EP-inferensys] capacity entry). y is [E, C, d].
 * A copy counts as kept only when 0 <= slot[t,j] < C and 0 <= topk_idx[t,j]
 * < E; any other copy is treated as dropped, so no index reaches outside y.
 * x, out [T, d]; topk_idx, slot [T, k] int32; topk_w [T, k] fp32. */
int moe_combine(const void* x, const void* y, const int32_t* topk_idx, const float* topk_w,
                const int32_t* slot, int64_t T, int64_t d, int32_t E, int32_t k, int64_t C,
                moe_dtype_t dtype, void* out, void* stream);

/* Stages of moe_layer_forward (and of moe_layer_forward_replicated, whose
 * ROUTE stage also ranks each expert's copies and deals them to instances),
 * in launch order. */
enum {
  MOE_STAGE_ROUTER = 0,   /* scores on the matrix cores */
  MOE_STAGE_ROUTE = 1,    /* top-k and gates */
  MOE_STAGE_SLOTS = 2,    /* scan over token tiles, capacity, counts, GEMM tile maps, slots and drop
                             mask (and the tile histogram when top-k did not build it) */
  MOE_STAGE_SCATTER = 3,  /* row copies into the buckets (with short tile histograms also the scan and
                             slots: one kernel, the SLOTS stage then empty) */
  MOE_STAGE_GATE_UP = 4,  /* grouped GEMM 1 with the SwiGLU product */
  MOE_STAGE_DOWN = 5,     /* grouped GEMM 2 */
  MOE_STAGE_COMBINE = 6,  /* inverse permutation and weighted sum */
  MOE_NUM_STAGES = 7
};

/* Profiling aid. With events set (2 * MOE_NUM_STAGES caller-created
 * hipEvent_t handles), moe_layer_forward and moe_layer_forward_replicated
 * on the calling thread record events[2 i] on their stream just before
 * stage i and events[2 i + 1] just after, so the caller can read each
 * stage's GPU time. A stage that launches no kernel in a call records
 * neither of its events (their old times stay). events = NULL turns
 * this off (the default). Error: n_events != 2 * MOE_NUM_STAGES. */
int moe_set_stage_events(void* const* events, int n_events);

/* *ran = 1 if the calling thread's last layer call with stage events set
 * recorded stage `stage`'s events, 0 if that stage launched nothing (or no
 * such call was made). Errors: ran NULL, stage outside [0, MOE_NUM_STAGES). */
int moe_stage_ran(int32_t stage, int32_t* ran);

/* Static description of a status code. */
const char* moe_status_string(int status);

/* Message of the last MOE_ERR_HIP (or argument error) on the calling thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
